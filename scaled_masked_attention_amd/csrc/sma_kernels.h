// Internal interface between the C-ABI host layer (sma_host.cpp) and the HIP
// kernels. Not installed; the public ABI is include/sma.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sma {

// Arguments of one attention-forward launch (one variant of dtype/head_dim/mask).
struct FwdArgs {
  const void* q;     // [bh][seq_q][d], f32, bf16 or fp16
  const void* k;     // [bh][seq_kv][d]
  const void* v;     // [bh][seq_kv][d]
  float* o;          // nsplit == 1: final O [bh][seq_q][d] fp32 (when o_bf16 is null)
  unsigned short* o_bf16;  // nsplit == 1: final O as 16 bits (round to nearest even), or null
  int32_t o_f16;           // the 16-bit O is fp16 (else bf16)
  float* lse;        // nsplit == 1: final LSE [bh][seq_q] (natural log), may be null
  float* part_o;     // nsplit > 1: per-split normalised O [nsplit][bh][seq_q][d]
  float* part_lse;   // nsplit > 1: per-split LSE in log2 units [nsplit][bh][seq_q]
  int64_t bh;        // batch * heads
  int32_t seq_q;
  int32_t seq_kv;
  int32_t nqb;       // query blocks per (batch, head)
  int32_t nsplit;    // key splits per query row (1 = none)
  int32_t split_len; // keys per split, a multiple of the kernel's key tile
  float c;           // |scale| * log2(e), rounded once to fp32
  int32_t negate_q;  // scale < 0: the kernel multiplies by -q and |scale|
  uint32_t nwg;      // bh * nqb * nsplit workgroups
  // Element strides (the head dim is contiguous): (batch, head, row) of Q and
  // O, and of K and V. [B,H,S,d] gives (H*S*d, S*d, d); [B,S,H,d] gives
  // (S*H*d, d, H*d).
  int64_t heads;
  int64_t qs_b, qs_h, qs_s;
  int64_t kvs_b, kvs_h, kvs_s;
  // Optional hard mask, packed: bit j % 32 of word (row, j / 32) admits key j
  // of query row `row`. mask_words words per row; word strides over batch and
  // head (0 broadcasts). Null when there is no mask.
  const uint32_t* mask_bits;
  int32_t mask_words;
  int64_t mbits_sb, mbits_sh;
  // The 16-bit kernel takes the mask packed by launch_mask_pack_cols instead:
  // mask_bits is then the column words (mask_words = key positions per 32-row
  // block, mbits_* slab strides in words) and mask_cls the per-tile classes
  // (mask_tiles per 32-row block, mcls_* slab strides in words).
  const uint32_t* mask_cls;
  int32_t mask_tiles;
  int64_t mcls_sb, mcls_sh;
};

// Column packing of a byte mask [slabs][seq_q][seq_kv] for the 16-bit kernel:
// per slab and 32-row block rb, one 32-bit word per key j, bit i admitting key
// j for row 32 rb + i (rows past seq_q admit, keys past seq_kv block). Words are
// stored at position (j & ~15) | ((j & 7) << 1) | ((j >> 3) & 1) of the block's
// kpad positions (kpad = seq_kv rounded up to 64), so that keys j and j + 8 of a
// 16-key group sit side by side: a 64-lane mask for the 32x32 MFMA's score
// layout. Each 64-key tile of each block gets a class: 0 nothing admitted, 1
// everything admitted, 2 mixed.
struct MaskColArgs {
  const unsigned char* mask;
  uint32_t* cols;     // [slabs][nrb][kpad]
  uint32_t* cls;      // [slabs][nrb][kpad / 64]
  int64_t slabs;
  int32_t seq_q, seq_kv, nrb, kpad;
};
hipError_t launch_mask_pack_cols(const MaskColArgs& a, hipStream_t s);

// Packing of a byte mask [mask_batches][mask_heads][seq_q][seq_kv] (nonzero
// admits) into the bit words above, one slab per (mask batch, mask head).
struct MaskPackArgs {
  const unsigned char* mask;
  uint32_t* bits;
  int64_t slabs;
  int32_t seq_q, seq_kv, words;
};
hipError_t launch_mask_pack(const MaskPackArgs& a, hipStream_t s);

// Arguments of the split-combine launch.
struct CombineArgs {
  const float* part_o;   // [nsplit][rows][d]
  const float* part_lse; // [nsplit][rows], log2 units
  float* o;              // [rows][d] fp32 (when o_bf16 is null)
  unsigned short* o_bf16; // [rows][d] as 16 bits (bf16, or fp16 when o_f16), or null
  int32_t o_f16;
  float* lse;            // [rows] natural log, may be null
  int64_t rows;          // bh * seq_q
  int32_t nsplit;
  int32_t seq_q;
  int64_t heads;         // O's strides, as FwdArgs
  int64_t os_b, os_h, os_s;
};

// Arguments of the attention-backward launches (fp32 or bf16 Q, K, V; fp32 O, dO and
// gradients). Tensors are addressed through the strides below.
struct BwdArgs {
  const float* q;     // Q rows
  const float* k;     // K rows
  const float* v;     // V rows
  const float* o;     // the forward's output, Q's layout
  const float* dout;  // upstream gradient dL/dO, Q's layout
  const float* lse;   // [bh][seq_q], the forward's log-sum-exp (natural log)
  float* dq;          // Q's layout
  float* dk;          // K's layout
  float* dv;          // K's layout
  float* meta;        // workspace [bh][nqb][64]: per 32-row query block, lse2 then D
  // 16-bit inputs (the 16-bit backward): q, k, v as bf16, or fp16 when in_f16, and the
  // workspace copy of dO rounded to that type ([bh][seq_q][d]); o and dout stay fp32.
  const unsigned short* q16;
  const unsigned short* k16;
  const unsigned short* v16;
  unsigned short* dout16;
  int32_t in_f16;
  int64_t bh;
  int32_t seq_q;
  int32_t seq_kv;
  int32_t nqb;        // 32-row query blocks per (batch, head)
  int32_t nkb;        // 32-row key blocks per (batch, head)
  float c;            // scale * log2(e) (signed), rounded once to fp32
  float scale;        // scale rounded to fp32
  uint32_t nwg;       // workgroups of the launch (set per launch)
  // Element strides (the head dim is contiguous), as in FwdArgs: (batch, head, row) of
  // Q, O, dO and dQ, and of K, V, dK and dV. The bf16 copy of dO is always [bh][seq_q][d].
  int64_t heads;
  int64_t qs_b, qs_h, qs_s;
  int64_t kvs_b, kvs_h, kvs_s;
  // Optional hard mask, packed as in FwdArgs (bit j % 32 of word (row, j / 32) admits key
  // j); null when there is none.
  const uint32_t* mask_bits;
  int32_t mask_words;
  int64_t mbits_sb, mbits_sh;
};

// Workgroup geometry the planner needs (must match the kernels).
constexpr int kF32QueriesPerWG = 128;
constexpr int kF32KeysPerTile = 32;
constexpr int kF32WsplitQueriesPerWG = 32;  // in-workgroup key-split kernel
constexpr int kBF16QueriesPerWG = 256;
constexpr int kBF16KeysPerTile = 64;
// The 16-bit kernel at head dim 128 (two 32-row blocks per wave, 32-key tiles).
constexpr int kBF16D128QueriesPerWG = 512;
constexpr int kBF16D128KeysPerTile = 32;
// The 16-bit kernel at head dim 256 (the role-split kernel: 6 pairs of 32 rows, 32-key tiles).
constexpr int kBF16D256QueriesPerWG = 192;
constexpr int kBF16D256KeysPerTile = 32;
constexpr int kThreadsPerWG = 256;

// Row primitives on a (rows x cols) fp32 matrix.
enum RowMode { kRowSoftmax = 0, kRowLse = 1, kRowMasked = 2, kRowScaled = 3 };
struct RowArgs {
  const float* in;          // [rows][cols]
  const float* mask;        // [rows][cols], kRowMasked only (nonzero = admitted)
  float* out;               // [rows][cols], or [rows] for kRowLse; may equal in
  int64_t rows;
  int32_t cols;
  int32_t rows_per_matrix;  // kRowScaled with causal: rows of each matrix (row r = i % this)
  int32_t causal;           // kRowScaled: bottom-right causal mask
  float c;                  // scale * log2(e) (log2(e) for the unscaled modes), rounded once
};
// How a row is mapped: `team` lanes per row holding per_lane vectors of
// `vec` floats each in registers, or two streaming passes.
struct RowPlan {
  int vec = 1, team = 64, per_lane = 1;
  bool stream = false;
};
constexpr int kRowMaxPerLane = 16;  // vectors per lane of a register-resident row
RowPlan plan_rows(int64_t cols, bool vec4);
hipError_t launch_rows(int mode, const RowArgs& a, const RowPlan& p, hipStream_t s);
// Softmax backward on (rows x cols) fp32: dx = scale * y * (dy - rowsum(y * dy)).
struct RowBwdArgs {
  const float* y;   // softmax output [rows][cols]
  const float* dy;  // upstream gradient [rows][cols]
  float* dx;        // [rows][cols]; may equal y or dy
  int64_t rows;
  int32_t cols;
  float scale;
};
hipError_t launch_rows_bwd(const RowBwdArgs& a, const RowPlan& p, hipStream_t s);

hipError_t launch_fwd_f32(const FwdArgs& a, int head_dim, bool causal, hipStream_t s);
hipError_t launch_fwd_f32_wsplit(const FwdArgs& a, int head_dim, bool causal, hipStream_t s);
// 16-bit inputs: bf16, or fp16 when f16.
hipError_t launch_fwd_bf16(const FwdArgs& a, int head_dim, bool causal, bool f16, hipStream_t s);
constexpr int kBwdRowsPerBlock = 32;         // query and key block of the backward kernels
constexpr int kBwdMetaFloats = 64;          // workspace floats per query block
hipError_t launch_bwd_f32(const BwdArgs& a, int head_dim, bool causal, hipStream_t s,
                          hipEvent_t ev_pre, hipEvent_t ev_dkdv);
// 16-bit inputs: bf16, or fp16 when a.in_f16.
hipError_t launch_bwd_bf16(const BwdArgs& a, int head_dim, bool causal, hipStream_t s,
                           hipEvent_t ev_pre, hipEvent_t ev_dkdv);
hipError_t launch_combine(const CombineArgs& a, int head_dim, hipStream_t s);

}  // namespace sma
