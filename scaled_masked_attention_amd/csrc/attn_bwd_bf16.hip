// Attention backward with bf16 or fp16 Q, K, V on 16-bit MFMA (v_mfma_f32_32x32x16_bf16,
// or _f16 under the F16 template flag; fp32 accumulation): dQ, dK and dV (fp32) of O = softmax(scale * Q K^T + causal mask) V, from
// the forward's fp32 O and log-sum-exp and an fp32 upstream gradient dO (oxicuda
// ComputeBackend `attention` for the forward; the softmax vector-Jacobian product of
// pulsatrix HIPBackend `softmax_rows_backward` and of MicroGPT's fused attention-softmax
// backward; the operand precision of oxicuda `gemm_mixed_precision`: 16-bit operands, fp32
// accumulation and result).
//
// The arithmetic and the three launches (preprocess, dK/dV, dQ) are those of the fp32
// backward, with workgroups shaped for 16-bit MFMA and two waves per SIMD (at head dim
// 256 the dQ work is split by role between the two waves of a SIMD):
//   P_ij = 2^(c s_ij - lse2_i), D_i = dO_i . O_i, dP_ij = dO_i . v_j, dS_ij = P_ij (dP_ij - D_i),
//   dV_j = sum_i P_ij dO_i,  dK_j = scale sum_i dS_ij q_i,  dQ_i = scale sum_j dS_ij k_j,
// with three roundings to the input type (nearest even) for the products: dO once, in
// the preprocess (D stays the fp32 dot product of the fp32 dO and O); P for dV; dS for dK
// and dQ. P and dS themselves are formed in fp32 from fp32 scores. fp16 is rounded the
// same way, with no rescaling: values past its range become infinite and those under its
// normal range lose bits, so the caller keeps dO (and with it dS) inside that range, as
// with loss scaling. The 16-bit registers below are typed bf16 and hold raw bits either
// way; only the MFMA and the roundings read them as numbers.
//
// MFMA layouts (lane = 32*h + m; accumulator register r of lane (n, h) holds row
// 8*(r/4) + 4*h + r%4 of output column n):
//  - The tiles that are A operands of the score products (Q and dO in the dK/dV kernel,
//    K and V in the dQ kernel) are stored with bits 2 and 3 of the row index swapped.
//    Register r of a score accumulator then holds original row 16*(r/8) + 8*h + r%8, so
//    registers 8t..8t+7 are the eight rows this lane supplies, as the B operand, to k-step
//    t of the next product (dV^T += dO^T P, dK^T += Q^T dS, dQ^T += K^T dS^T).
//  - The A operands of those products (dO^T, Q^T, K^T) come from the same tiles through
//    the transposing read ds_read_b64_tr_b16: tile rows 16t + 4h + 0..3 and
//    16t + 8 + 4h + 0..3 hold original rows 16t + 8h + 0..7.
//  - The B operands of the score products (K and V in the dK/dV kernel, Q and dO in the
//    dQ kernel) stay in registers for the whole pass, read once: K and V from unpermuted
//    LDS tiles, Q and dO straight from global memory.
//  - Every tile is XOR-swizzled in 16-byte chunks (swz below), which keeps both the
//    16-byte row reads (16 lanes, 16 consecutive rows, one chunk) and the transposing
//    reads (32 lanes, 4 consecutive rows, one 64-byte group) free of bank conflicts.
#include "attn_common.h"

namespace sma {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.44269504088896340736f;

template <int D>
struct HGeom {
  static constexpr int kRows = kBwdRowsPerBlock;    // rows per query / key block
  static constexpr int kSteps = D / 16;             // k-steps of the score products
  static constexpr int kNch = D / 32;               // 32-wide output chunks
  static constexpr int kRowBytes = 2 * D;           // one bf16 row
  static constexpr int kChunks = D / 8;             // 16-byte chunks per row
  static constexpr int kTileBytes = kRows * kRowBytes;
  static constexpr int kDmaPerTile = kTileBytes / 1024;
  static constexpr int kMetaBytes = kBwdMetaFloats * 4;
  static_assert(kRows == 32, "one 32x32 MFMA tile per block");
  static_assert(kBwdMetaFloats == 64, "one 4-byte direct-to-LDS load per block's lse2 and D");
};

template <bool F16>
__device__ __forceinline__ f32x16 mfma16(bf16x8 a, bf16x8 b, f32x16 c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                   __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// x rounded to nearest even in the input type, as the raw bits of one 16-bit lane.
template <bool F16>
__device__ __forceinline__ __bf16 round16(float x) {
  if constexpr (F16)
    return __builtin_bit_cast(__bf16, (_Float16)x);
  else
    return (__bf16)x;
}

// Original row held in accumulator register r of half h under the row permutation.
__device__ __forceinline__ int perm_acc_row(int r, int h) { return 16 * (r / 8) + 8 * h + (r % 8); }
// Bits 2 and 3 of a tile row swapped (its own inverse).
__device__ __forceinline__ int swap_bits_2_3(int p) {
  return (p & ~0xC) | ((p & 4) << 1) | ((p & 8) >> 1);
}
// Chunk swizzle of tile row p. d = 128 and 256 (rows of 256 bytes or more, every row
// on all 64 banks, chunk c on the banks of c mod 16): the 16 rows of a row read must
// land on 16 different chunks mod 16, and the 4 rows of a transposing read on 4
// different 64-byte groups; 4*(p&3) + ((p>>2)&3) does both.
// d = 64 (128-byte rows, two rows per bank cycle): the same over rows of one parity,
// 4*((p>>1)&1) + ((p>>2)&3). d = 32 (64-byte rows, four per bank cycle): rows p and
// p + 4k share banks, so (p>>2)&3 separates the four of a row read; the four rows of a
// transposing read are 256 consecutive bytes whatever the chunk order within them.
template <int D>
__device__ __forceinline__ int swz(int p) {
  static_assert(D == 32 || D == 64 || D == 128 || D == 256, "16-bit backward tile swizzle");
  return D >= 128 ? 4 * (p & 3) + ((p >> 2) & 3)
                  : D == 64 ? 4 * ((p >> 1) & 1) + ((p >> 2) & 3) : ((p >> 2) & 3);
}

// Byte offset, from the tile's first row in global memory (rows row_bytes apart), of the
// 16 bytes that lane `lane` of direct-to-LDS copy instruction t fetches: LDS chunk
// position P = 64t + lane is tile row p = P / chunks, chunk slot P % chunks, which holds
// logical chunk slot ^ swz(p) of source row p (or of row swap_bits_2_3(p) in a permuted
// tile).
template <int D, bool PERM>
__device__ __forceinline__ unsigned tile_src(int t, int lane, unsigned row_bytes) {
  constexpr int kC = D / 8;
  const int pos = 64 * t + lane;
  const int p = pos / kC;
  const int c = (pos % kC) ^ swz<D>(p);
  return (unsigned)(PERM ? swap_bits_2_3(p) : p) * row_bytes + 16u * (unsigned)c;
}

// The 8 bf16 at logical chunk c of tile row p (a row read).
template <int D>
__device__ __forceinline__ bf16x8 row_chunk(const unsigned char* tile, int p, int c) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                        tile + p * 2 * D + 16 * (c ^ swz<D>(p))));
}

// Transposed A operand of k-step t2 and output chunk cb from a permuted tile: lane
// (c, h) receives original rows 16*t2 + 8*h + 0..7 at head dim 32*cb + c. In each 16-lane
// group, lane role s reads 4 dims of tile row 16*t2 + 4*h + s/4 (elements 0..3) and of
// that row + 8 (elements 4..7).
template <int D>
__device__ __forceinline__ bf16x8 tr_operand(const unsigned char* tile, int lane, int t2, int cb) {
  const int s = lane & 15;
  const int colq = 2 * ((lane >> 4) & 1) + ((s & 3) >> 1);  // chunk within a 32-dim group
  const int half8 = 8 * (s & 1);
  const int r_lo = 16 * t2 + 4 * (lane >> 5) + s / 4;
  const int r_hi = r_lo + 8;
  const int chunk = 4 * cb + colq;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(tile + r_lo * 2 * D + 16 * (chunk ^ swz<D>(r_lo)) + half8));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(tile + r_hi * 2 * D + 16 * (chunk ^ swz<D>(r_hi)) + half8));
  const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
  return __builtin_bit_cast(bf16x8, u32x4{lo2[0], lo2[1], hi2[0], hi2[1]});
}

// The same reads from a tile whose LDS address is a multiple of 2*D bytes (D >= 128),
// with every address formed inside the step from one base register and a constant. The
// swizzle only flips bits 4..7 of a row's byte offset, so with the row's own part folded
// into the base, chunk 2*st + h of row p sits at (base ^ 32*(st % 8)) + 256*(st / 8), and
// the chunks of a transposing read at (base ^ 64*(cb % 4)) + 256*(cb / 4) + 32*D*t2 (the
// swizzle of rows 16*t2 + r does not depend on t2). The empty asm makes the base opaque,
// so the compiler cannot hoist one precomputed offset per chunk out of the step loop and
// hold them all in registers.
template <int D>
__device__ __forceinline__ unsigned row_base(unsigned tile, int p, int h) {
  static_assert(D >= 128, "swizzle confined to bits 4..7");
  unsigned b = tile + (unsigned)(p * 2 * D + 16 * (swz<D>(p) ^ h));
  asm volatile("" : "+v"(b));
  return b;
}
// The base again, opaque at this point of the program: a read formed from it cannot be
// hoisted above an earlier pin, which keeps streamed reads in their place.
__device__ __forceinline__ unsigned pin(unsigned& base) {
  asm volatile("" : "+v"(base));
  return base;
}
// An MFMA result, opaque at this point: the MFMA stays ahead of every later pin.
__device__ __forceinline__ void pin_acc(f32x16& c) { asm volatile("" : "+v"(c)); }
__device__ __forceinline__ bf16x8 row_read(unsigned base, int st) {
  const unsigned a = (base ^ (32u * (unsigned)(st & 7))) + 256u * (unsigned)(st >> 3);
  return __builtin_bit_cast(bf16x8, *(__attribute__((address_space(3))) const u32x4*)(size_t)a);
}
template <int D>
__device__ __forceinline__ unsigned tr_base(unsigned tile, int lane, bool hi) {
  static_assert(D >= 128, "swizzle confined to bits 4..7");
  const int s = lane & 15;
  const int colq = 2 * ((lane >> 4) & 1) + ((s & 3) >> 1);
  const int r = 4 * (lane >> 5) + s / 4 + (hi ? 8 : 0);
  unsigned b = tile + (unsigned)(r * 2 * D + 16 * (swz<D>(r) ^ colq) + 8 * (s & 1));
  asm volatile("" : "+v"(b));
  return b;
}
template <int D>
__device__ __forceinline__ bf16x8 tr_read(unsigned lo_base, unsigned hi_base, int t2, int cb) {
  const unsigned x = 64u * (unsigned)(cb & 3);
  const unsigned imm = 256u * (unsigned)(cb >> 2) + 32u * D * (unsigned)t2;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(size_t)((lo_base ^ x) + imm));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(size_t)((hi_base ^ x) + imm));
  const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
  return __builtin_bit_cast(bf16x8, u32x4{lo2[0], lo2[1], hi2[0], hi2[1]});
}

// N MFMAs, the i-th on the A operand op(i) (an LDS read) and run by mf(i, a); the reads
// are issued kPf MFMAs ahead of their use, and scheduling barriers keep them there.
template <int N, int kPf, typename Op, typename Mf>
__device__ __forceinline__ void mfma_stream(Op op, Mf mf) {
  bf16x8 buf[kPf + 1];
#pragma unroll
  for (int i = 0; i < kPf && i < N; ++i) buf[i] = op(i);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (i + kPf < N) buf[(i + kPf) % (kPf + 1)] = op(i + kPf);
    __builtin_amdgcn_sched_barrier(0);
    mf(i, buf[i % (kPf + 1)]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ---------------------------------------------------------------- preprocess

// Per 32-row query block: lse2 = LSE log2(e) (+inf for a row without admitted keys or past
// the end, which makes its P exactly 0) and D = dO . O in fp32, as 64 floats of meta; and
// dO rounded to the input type into the workspace copy the products read.
template <int D, bool F16>
__global__ __launch_bounds__(256) void attn_bwd_pre_bf16_kernel(BwdArgs a) {
  constexpr int kT = D / 4;  // threads per row, 4 head dims each
  constexpr int kRowsPerPass = 256 / kT;
  const int64_t blk = blockIdx.x;  // (batch*head, query block)
  const int64_t bh = blk / a.nqb;
  const int32_t i0 = (int32_t)(blk % a.nqb) * kBwdRowsPerBlock;
  const int tid = threadIdx.x;
  const int c4 = tid % kT;
  float* const meta = a.meta + blk * kBwdMetaFloats;
#pragma unroll
  for (int pass = 0; pass < kBwdRowsPerBlock / kRowsPerPass; ++pass) {
    const int r = pass * kRowsPerPass + tid / kT;
    const int32_t row = i0 + r;
    const bool live = row < a.seq_q;
    float d = 0.f;
    if (live) {
      const int64_t off = head_offset(bh, a.heads, a.qs_b, a.qs_h) + (int64_t)row * a.qs_s + 4 * c4;
      const f32x4 g = *reinterpret_cast<const f32x4*>(a.dout + off);
      const f32x4 o = *reinterpret_cast<const f32x4*>(a.o + off);
      d = g[0] * o[0] + g[1] * o[1] + g[2] * o[2] + g[3] * o[3];
      const size_t off16 = ((size_t)bh * a.seq_q + row) * D + 4 * c4;  // the copy is [bh][seq_q][d]
      *reinterpret_cast<u32x2*>(a.dout16 + off16) = u32x2{pack_out16(g[0], g[1], F16), pack_out16(g[2], g[3], F16)};
    }
#pragma unroll
    for (int w = kT / 2; w >= 1; w >>= 1) d += __shfl_xor(d, w);
    if (c4 == 0) {
      float l2 = INFINITY;
      if (live) {
        const float lse = a.lse[(size_t)bh * a.seq_q + row];
        l2 = lse == -INFINITY ? INFINITY : lse * kLog2e;
      }
      meta[r] = l2;
      meta[kBwdRowsPerBlock + r] = live ? d : 0.f;
    }
  }
}

// ---------------------------------------------------------------- dK, dV

// A workgroup owns 128 keys of one (batch, head), as four 32-key blocks, and 8 waves. For
// key block kb, wave kb (the P wave) forms S = Q K^T and P = 2^(c S - lse2) and
// accumulates dV^T += dO^T P; wave 4 + kb (the dS wave) forms dP = dO V^T, reads that P
// back from LDS, forms dS = P (dP - D) and accumulates dK^T += Q^T dS. A wave keeps only
// its key block's K or V (the B operand of S or dP) and one accumulator set in registers,
// so two waves fit a SIMD; the two waves of a key block share one, and one's MFMAs run
// while the other works on the VALU. At head dim 256 a wave holds 64 registers of K or V
// and 128 of accumulators, which leaves about 60 of the 256 that two waves per SIMD allow:
// there its operand reads are streamed two MFMAs ahead at addresses formed in the step
// (row_read, tr_read), so that no per-chunk offset or operand queue outgrows them.
//
// All the waves step through the query blocks together. Query block T's Q and dO tiles
// (permuted), its lse2/D and, with a hard mask, the four key blocks' mask words of its rows
// are copied straight into a ring of four LDS slots two steps ahead (three slots, one step
// ahead, at head dim 256, for the LDS), each wave issuing a share. In step T the P waves
// work on block T and the dS waves on block T - 1, whose P the P waves left in LDS (fp32,
// double buffered) in step T - 1. One barrier per step.
template <int D>
struct KVGeom {
  static constexpr int kWaves = 8;
  static constexpr int kKB = kWaves / 2;                        // 32-key blocks per workgroup
  static constexpr int kKeys = 32 * kKB;
  // Ring slots, and blocks copied ahead (a dS wave still reads block T - 1 in step T).
  static constexpr int kSlots = D == 256 ? 3 : 4;
  static constexpr int kAhead = kSlots - 2;
  static constexpr int kTileBytes = HGeom<D>::kTileBytes;
  static constexpr int kDma = HGeom<D>::kDmaPerTile;            // 1 KB copies per tile
  static constexpr int kTileCopies = 2 * kDma;                  // Q and dO of one block
  // Copies each wave issues per block: the same number for every wave, or (d = 32, four
  // copies) one for each of waves 0..3.
  static constexpr int kTileCopiesPerWave = kTileCopies >= kWaves ? kTileCopies / kWaves : 1;
  static constexpr int kXBytes = 16 * 64 * 4;                   // a wave's 16 P values per lane
  static_assert(kTileCopies < kWaves ? kTileCopies * 2 == kWaves : kTileCopiesPerWave * kWaves == kTileCopies,
                "copy split");
  static constexpr int kMaskWaves = kKB / 2;  // waves 1.. that copy mask words (32 rows x 2 key blocks each)
  static_assert(kMaskWaves < kKB, "the lse2/D and mask copies come from P waves (0 .. kKB - 1)");
};

// A vmcnt wait with a wave-uniform count (0..20; counts above 20 wait for 20, which is
// stricter and so still correct).
template <int N = 0>
__device__ __forceinline__ void wait_vmcnt_n(int n) {
  if constexpr (N >= 20) {
    wait_vmcnt<20>();
  } else {
    if (n == N) wait_vmcnt<N>();
    else wait_vmcnt_n<N + 1>(n);
  }
}

template <int D, bool CAUSAL, bool MASKED, bool F16>
__global__ __launch_bounds__(64 * KVGeom<D>::kWaves) void attn_bwd_dkdv_bf16_kernel(BwdArgs a) {
  using G = HGeom<D>;
  using W = KVGeom<D>;
  // Slot: Q tile, dO tile, lse2/D, and with a hard mask [key block][row] words.
  constexpr int kMaskBytes = MASKED ? W::kKB * G::kRows * 4 : 0;
  // Head dim 256 reads its tiles at XOR-formed addresses (row_read, tr_read): every tile
  // starts on a multiple of 512 bytes.
  constexpr int kAlign = D == 256 ? 2 * D : 16;
  constexpr int kSlotBytes = (2 * G::kTileBytes + G::kMetaBytes + kMaskBytes + kAlign - 1) / kAlign * kAlign;
  constexpr int kRingBytes = W::kSlots * kSlotBytes;
  constexpr int kLdsBytes = kRingBytes + 2 * W::kKB * W::kXBytes;
  static_assert(2 * W::kKB * G::kTileBytes <= kLdsBytes, "K and V stage through the LDS");
  __shared__ __attribute__((aligned(kAlign))) unsigned char lds[kLdsBytes];
  unsigned char* const xbuf = lds + kRingBytes;  // [key block][parity][4][64 lanes][4 floats]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kb = wave & (W::kKB - 1);
  const bool pwave = wave < W::kKB;
  const int lm = lane & 31;
  const int lh = lane >> 5;

  // Workgroups of a head are consecutive, the lowest keys (the most query blocks under a
  // causal mask) first.
  const uint32_t nkw = (uint32_t)(a.nkb + W::kKB - 1) / W::kKB;
  const uint32_t lam = xcd_remap(blockIdx.x, a.nwg);
  const int64_t bh = (int64_t)(lam / nkw);
  const int32_t j0 = (int32_t)(lam % nkw) * W::kKeys;
  const int32_t jk = j0 + 32 * kb;  // this wave's first key
  const int32_t delta = a.seq_kv - a.seq_q;
  // Query blocks holding a row that admits some key of the workgroup: row i admits key j0
  // iff i >= j0 - delta.
  int32_t qb_first = 0;
  if (CAUSAL) {
    const int32_t i_min = j0 - delta;
    qb_first = i_min <= 0 ? 0 : i_min / G::kRows;
  }
  const int32_t nblk = a.nqb > qb_first ? a.nqb - qb_first : 0;

  const int64_t q_off = head_offset(bh, a.heads, a.qs_b, a.qs_h);
  const int64_t kv_off = head_offset(bh, a.heads, a.kvs_b, a.kvs_h);
  const unsigned q_row = (unsigned)(a.qs_s * 2), kv_row = (unsigned)(a.kvs_s * 2);
  const unsigned g_row = (unsigned)G::kRowBytes;
  // Rows past the end of each array lie outside these ranges and read as zeros.
  const __amdgpu_buffer_rsrc_t q_rsrc = raw_buffer(a.q16 + q_off, strided_range(a.seq_q, a.qs_s, D, 2));
  const __amdgpu_buffer_rsrc_t g_rsrc =
      raw_buffer(a.dout16 + (size_t)bh * a.seq_q * D, (unsigned)a.seq_q * g_row);
  const __amdgpu_buffer_rsrc_t m_rsrc =
      raw_buffer(a.meta + (size_t)bh * a.nqb * kBwdMetaFloats, (unsigned)a.nqb * (unsigned)G::kMetaBytes);
  __amdgpu_buffer_rsrc_t w_rsrc;  // rows past seq_q read as 0: nothing admitted
  if (MASKED)
    w_rsrc = raw_buffer(a.mask_bits + head_offset(bh, a.heads, a.mbits_sb, a.mbits_sh),
                        (unsigned)a.seq_q * (unsigned)a.mask_words * 4u);

  // Copies of query block T (absolute block qb_first + T) into its ring slot: the Q and dO
  // tiles split over the waves; wave 0 adds lse2/D, waves 1 .. kKB/2 the mask words
  // (lane l of wave 1 + h: key block 2h + l / 32, row l % 32). These are P waves: `pw`
  // (std::true_type in their loop) compiles the lse2/D and mask copies out of the dS
  // waves' loop, whose registers they would otherwise hold.
  auto issue = [&](int32_t T, auto pw) {
    constexpr bool kP = decltype(pw)::value;
    const int32_t qb = qb_first + T;
    unsigned char* const slot = lds + (T % W::kSlots) * kSlotBytes;
#pragma unroll
    for (int u = 0; u < W::kTileCopiesPerWave; ++u) {
      const int c = u * W::kWaves + wave;  // 0 .. 2 kDma - 1: Q copies, then dO copies
      if (c >= W::kTileCopies) break;      // d = 32: waves 4..7 copy no tile
      if (c < W::kDma)
        dma_load_x4(q_rsrc, (unsigned)(G::kRows * qb) * q_row + tile_src<D, true>(c, lane, q_row),
                    lds_address(slot + 1024 * c));
      else
        dma_load_x4(g_rsrc, (unsigned)(G::kRows * qb) * g_row + tile_src<D, true>(c - W::kDma, lane, g_row),
                    lds_address(slot + 1024 * c));
    }
    if (kP && wave == 0)
      dma_load_x1(m_rsrc, (unsigned)qb * (unsigned)G::kMetaBytes + 4u * lane,
                  lds_address(slot + 2 * G::kTileBytes));
    if (MASKED && kP && wave >= 1 && wave <= W::kMaskWaves) {
      const int kbw = 2 * (wave - 1) + (lane >> 5);
      dma_load_x1(w_rsrc, ((unsigned)(G::kRows * qb + (lane & 31)) * (unsigned)a.mask_words +
                           (unsigned)(j0 / 32 + kbw)) * 4u,
                  lds_address(slot + 2 * G::kTileBytes + G::kMetaBytes + 256 * (wave - 1)));
    }
  };
  // Wait until this wave's copies of every block but the last one issued have landed.
  const int copies_per_block = (wave < W::kTileCopies ? W::kTileCopiesPerWave : 0) + (wave == 0 ? 1 : 0) +
                               (MASKED && wave >= 1 && wave <= W::kMaskWaves ? 1 : 0);
  auto wait_all_but_last_block = [&]() { wait_vmcnt_n(copies_per_block); };

  // The four key blocks' K and V tiles (unpermuted), staged through the ring (each wave
  // copies a share), into the B operands: the P wave of key block kb takes K, the dS wave
  // V; lane (key m, h) holds head dims 16*st + 8*h .. + 7 of key jk + m for k-step st.
  const unsigned kv_range = strided_range(a.seq_kv, a.kvs_s, D, 2);
  bf16x8 kv[G::kSteps];
  {
    const __amdgpu_buffer_rsrc_t k_rsrc = raw_buffer(a.k16 + kv_off, kv_range);
    const __amdgpu_buffer_rsrc_t v_rsrc = raw_buffer(a.v16 + kv_off, kv_range);
    constexpr int kCopies = 2 * W::kKB * W::kDma;  // K tiles, then V tiles
#pragma unroll
    for (int u = 0; u < kCopies / W::kWaves; ++u) {
      const int c = u * W::kWaves + wave;
      const int tensor = c / (W::kKB * W::kDma), kbc = (c / W::kDma) % W::kKB, t = c % W::kDma;
      const unsigned src = (unsigned)(j0 + 32 * kbc) * kv_row + tile_src<D, false>(t, lane, kv_row);
      dma_load_x4(tensor == 0 ? k_rsrc : v_rsrc, src, lds_address(lds + 1024 * c));
    }
    wait_vmcnt<0>();
    __syncthreads();
    const unsigned char* tile = lds + (pwave ? kb : W::kKB + kb) * G::kTileBytes;
#pragma unroll
    for (int st = 0; st < G::kSteps; ++st) kv[st] = row_chunk<D>(tile, lm, 2 * st + lh);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the operand reads have returned
    __syncthreads();                     // before the ring takes the space
  }

  f32x16 acc[G::kNch];  // dV (P waves) or dK (dS waves)
#pragma unroll
  for (int cb = 0; cb < G::kNch; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[cb][r] = 0.f;

  // Whether query block qb reaches this wave's keys at all, and whether some of its pairs
  // are masked by the causal bound (its last key past its first row's limit).
  auto reaches = [&](int32_t qb) {
    return jk < a.seq_kv && (!CAUSAL || G::kRows * qb + G::kRows - 1 + delta >= jk);
  };

  // The step loop (its waits, barrier and copies), run by every wave with its role's work.
  // Each role has its own copy of the loop, so that its accumulators keep their registers.
  auto run_steps = [&](auto pw, auto&& work) {
#pragma unroll
    for (int u = 0; u < W::kAhead; ++u)
      if (u < nblk) issue(u, pw);
    for (int32_t T = 0; T <= nblk; ++T) {
      if (W::kAhead == 2 && T + 1 < nblk) wait_all_but_last_block();
      else wait_vmcnt<0>();
      __syncthreads();  // block T has landed; step T - 1 is done with its slots and P
      if (T + W::kAhead < nblk) issue(T + W::kAhead, pw);
      work(T);
    }
  };
  if (pwave) {
    // The P wave runs a block's dV product at the start of the next step, ahead of the
    // next block's S MFMAs: its partner dS wave starts each step with MFMAs too, and the
    // P wave's softmax then meets the dS wave's dK MFMAs.
    bf16x8 pp_late[2];
    bool pending = false;
    const unsigned char* g_late = lds;
    run_steps(std::true_type{}, [&](int32_t T) {
      if (pending) {
        __builtin_amdgcn_s_setprio(1);
        if constexpr (D == 256) {
          unsigned tl = tr_base<D>(lds_address(g_late), lane, false);
          unsigned th = tr_base<D>(lds_address(g_late), lane, true);
          mfma_stream<2 * G::kNch, 2>(
              [&](int i) { return tr_read<D>(pin(tl), pin(th), i / G::kNch, i % G::kNch); },
              [&](int i, bf16x8 x) {
                acc[i % G::kNch] = mfma16<F16>(x, pp_late[i / G::kNch], acc[i % G::kNch]);
                pin_acc(acc[i % G::kNch]);
              });
        } else {
#pragma unroll
          for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
            for (int cb = 0; cb < G::kNch; ++cb) acc[cb] = mfma16<F16>(tr_operand<D>(g_late, lane, t2, cb), pp_late[t2], acc[cb]);
        }
        __builtin_amdgcn_s_setprio(0);
        pending = false;
      }
      const int32_t qb = qb_first + T;
      if (T < nblk && reaches(qb)) {
        const int32_t i0 = G::kRows * qb;
        const unsigned char* const q_slot = lds + (T % W::kSlots) * kSlotBytes;
        const unsigned char* const g_slot = q_slot + G::kTileBytes;
        const unsigned char* const m_slot = g_slot + G::kTileBytes;
        // lse2 of this lane's queries perm_acc_row(r, lh): rows 16t + 8h + 0..7, t = 0, 1.
        // Head dim 256 reads them after the score chain, which holds the most registers.
        f32x4 l2[4];
        if constexpr (D != 256) {
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4)
            l2[q4] = *reinterpret_cast<const f32x4*>(m_slot + 4 * (16 * (q4 / 2) + 8 * lh + 4 * (q4 % 2)));
        }
        f32x16 s;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = 0.f;
        __builtin_amdgcn_s_setprio(1);
        if constexpr (D == 256) {
          unsigned rb = row_base<D>(lds_address(q_slot), lm, lh);
          mfma_stream<G::kSteps, 2>([&](int st) { return row_read(pin(rb), st); },
                                    [&](int st, bf16x8 x) { s = mfma16<F16>(x, kv[st], s); pin_acc(s); });
        } else {
#pragma unroll
          for (int st = 0; st < G::kSteps; ++st) s = mfma16<F16>(row_chunk<D>(q_slot, lm, 2 * st + lh), kv[st], s);
        }
        __builtin_amdgcn_s_setprio(0);
        // With a hard mask at head dim 256, this lane's bits of the 16 rows' words are
        // gathered into one register (bit r: row perm_acc_row(r, lh)) before lse2 is read.
        uint32_t mbits = 0;
        if constexpr (D == 256 && MASKED) {
          unsigned wa = lds_address(m_slot + G::kMetaBytes + 4 * G::kRows * kb) + 32u * (unsigned)lh;
          pin(wa);
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const u32x4 w4 =
                *(__attribute__((address_space(3))) const u32x4*)(size_t)(wa + 4u * (16 * (q4 / 2) + 4 * (q4 % 2)));
#pragma unroll
            for (int e = 0; e < 4; ++e) mbits |= ((w4[e] >> lm) & 1u) << (4 * q4 + e);
          }
          asm volatile("" : "+v"(mbits));
        }
        if constexpr (D == 256) {
          unsigned ma = lds_address(m_slot) + 32u * (unsigned)lh;
          pin(ma);
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4)
            l2[q4] = *(__attribute__((address_space(3))) const f32x4*)(size_t)(ma + 4u * (16 * (q4 / 2) + 4 * (q4 % 2)));
        }
        const bool diag = CAUSAL && (jk + G::kRows - 1 > i0 + delta);
        uint32_t mw[16];  // mask word of query row perm_acc_row(r, lh); bit lm is this lane's key
        if (MASKED && D != 256) {
          const unsigned char* const w_slot = m_slot + G::kMetaBytes + 4 * G::kRows * kb;
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const u32x4 w4 = *reinterpret_cast<const u32x4*>(w_slot + 4 * (16 * (q4 / 2) + 8 * lh + 4 * (q4 % 2)));
#pragma unroll
            for (int e = 0; e < 4; ++e) mw[4 * q4 + e] = w4[e];
          }
        }
        float t[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) t[r] = s[r] * a.c - l2[r / 4][r % 4];
        if (diag) {
          // Key jk + lm is admitted to row i0 + perm_acc_row(r, lh) iff
          // 16 (r / 8) + r % 8 >= rel. The empty asm keeps the bound, and with it the
          // comparisons, inside this branch.
          int32_t rel = jk + lm - i0 - delta - 8 * lh;
          asm volatile("" : "+v"(rel));
#pragma unroll
          for (int r = 0; r < 16; ++r) t[r] = 16 * (r / 8) + r % 8 >= rel ? t[r] : -INFINITY;
        }
        if (MASKED) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            t[r] = (D == 256 ? (mbits >> r) & 1u : (mw[r] >> lm) & 1u) ? t[r] : -INFINITY;
        }
        f32x4 p32[4];
        bf16x8 pp[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(t[r]);
          p32[r / 4][r % 4] = p;
          pp[r / 8][r % 8] = round16<F16>(p);
        }
        unsigned char* const xp = xbuf + (2 * kb + (T & 1)) * W::kXBytes + 16 * lane;
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) *reinterpret_cast<f32x4*>(xp + 1024 * c4) = p32[c4];
        // dV^T += dO^T P, at the start of the next step
        pp_late[0] = pp[0];
        pp_late[1] = pp[1];
        g_late = g_slot;
        pending = true;
      }
    });
  } else {
    run_steps(std::false_type{}, [&](int32_t T) {
      const int32_t qb = qb_first + T - 1;
      if (T >= 1 && reaches(qb)) {
        const unsigned char* const q_slot = lds + ((T - 1) % W::kSlots) * kSlotBytes;
        const unsigned char* const g_slot = q_slot + G::kTileBytes;
        const unsigned char* const m_slot = g_slot + G::kTileBytes;
        f32x16 dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) dp[r] = 0.f;
        __builtin_amdgcn_s_setprio(1);
        if constexpr (D == 256) {
          unsigned rb = row_base<D>(lds_address(g_slot), lm, lh);
          mfma_stream<G::kSteps, 2>([&](int st) { return row_read(pin(rb), st); },
                                    [&](int st, bf16x8 x) { dp = mfma16<F16>(x, kv[st], dp); pin_acc(dp); });
        } else {
#pragma unroll
          for (int st = 0; st < G::kSteps; ++st) dp = mfma16<F16>(row_chunk<D>(g_slot, lm, 2 * st + lh), kv[st], dp);
        }
        __builtin_amdgcn_s_setprio(0);
        f32x4 dd[4];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          dd[q4] = *reinterpret_cast<const f32x4*>(m_slot + 4 * (G::kRows + 16 * (q4 / 2) + 8 * lh + 4 * (q4 % 2)));
        const unsigned char* const xp = xbuf + (2 * kb + ((T - 1) & 1)) * W::kXBytes + 16 * lane;
        bf16x8 pds[2];
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
          const f32x4 p4 = *reinterpret_cast<const f32x4*>(xp + 1024 * c4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * c4 + e;
            pds[r / 8][r % 8] = round16<F16>(p4[e] * (dp[r] - dd[c4][e]));
          }
        }
        // dK^T += Q^T dS (the scale is applied once, at the end)
        __builtin_amdgcn_s_setprio(1);
        if constexpr (D == 256) {
          unsigned tl = tr_base<D>(lds_address(q_slot), lane, false);
          unsigned th = tr_base<D>(lds_address(q_slot), lane, true);
          mfma_stream<2 * G::kNch, 2>(
              [&](int i) { return tr_read<D>(pin(tl), pin(th), i / G::kNch, i % G::kNch); },
              [&](int i, bf16x8 x) {
                acc[i % G::kNch] = mfma16<F16>(x, pds[i / G::kNch], acc[i % G::kNch]);
                pin_acc(acc[i % G::kNch]);
              });
        } else {
#pragma unroll
          for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
            for (int cb = 0; cb < G::kNch; ++cb) acc[cb] = mfma16<F16>(tr_operand<D>(q_slot, lane, t2, cb), pds[t2], acc[cb]);
        }
        __builtin_amdgcn_s_setprio(0);
      }
    });
  }

  // Lane (key m, h) holds head dims 32*cb + 8*g4 + 4*h .. + 3 of key jk + m.
  const int32_t j = jk + lm;
  if (j >= a.seq_kv) return;
  float* const out = (pwave ? a.dv : a.dk) + kv_off + (int64_t)j * a.kvs_s;
  const float mul = pwave ? 1.0f : a.scale;
#pragma unroll
  for (int cb = 0; cb < G::kNch; ++cb)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4)
      *reinterpret_cast<f32x4*>(out + 32 * cb + 8 * g4 + 4 * lh) =
          f32x4{acc[cb][4 * g4] * mul, acc[cb][4 * g4 + 1] * mul, acc[cb][4 * g4 + 2] * mul,
                acc[cb][4 * g4 + 3] * mul};
}

// Head dim 128: the same roles with two key blocks per wave, so that each Q or dO operand
// read from LDS (row or transposing) feeds two MFMAs, one per key block. A workgroup owns
// 256 keys as 8 key blocks and 8 waves: for pair p, the P wave p keeps K of key blocks
// 2p and 2p + 1 (64 registers) and their dV accumulators (128), the dS wave 4 + p their V
// and dK accumulators. Query block T's Q and dO tiles, lse2/D and, with a hard mask, the
// eight key blocks' words of its rows go through a 4-slot ring two steps ahead; P leaves
// the P wave through LDS (fp32, double buffered, per key block). Operand reads are
// streamed at XOR-formed addresses and lse2, D and the mask bits are read late and in
// small pieces, which keeps each role inside the 256 registers of two waves per SIMD.
struct KV2Geom {
  static constexpr int D = 128;
  static constexpr int kPairs = 4;
  static constexpr int kWaves = 2 * kPairs;
  static constexpr int kKBW = 2;                  // key blocks per wave
  static constexpr int kKB = kPairs * kKBW;       // key blocks per workgroup
  static constexpr int kKeys = 32 * kKB;
  static constexpr int kSlots = 4;
  static constexpr int kTileCopies = 2 * HGeom<D>::kDmaPerTile;  // Q and dO of one block
  static constexpr int kTileCopiesPerWave = kTileCopies / kWaves;
  static constexpr int kXBytes = 16 * 64 * 4;     // one key block's 16 P values per lane
  static_assert(kTileCopiesPerWave * kWaves == kTileCopies, "copy split");
  static_assert(kKB == 2 * kPairs && kPairs == 4, "mask copies: P wave w takes key blocks 2w, 2w + 1");
};

template <bool CAUSAL, bool MASKED, bool F16>
__global__ __launch_bounds__(64 * KV2Geom::kWaves) void attn_bwd_dkdv_bf16_kb2_kernel(BwdArgs a) {
  constexpr int D = KV2Geom::D;
  using G = HGeom<D>;
  using W = KV2Geom;
  // Slot: Q tile, dO tile, lse2/D, and with a hard mask [key block][row] words; every tile on
  // a multiple of 256 bytes (the XOR-formed addresses).
  constexpr int kMaskBytes = MASKED ? W::kKB * G::kRows * 4 : 0;
  constexpr int kSlotBytes = (2 * G::kTileBytes + G::kMetaBytes + kMaskBytes + 255) / 256 * 256;
  constexpr int kRingBytes = W::kSlots * kSlotBytes;
  constexpr int kLdsBytes = kRingBytes + 2 * W::kKB * W::kXBytes;
  static_assert(2 * W::kKB * G::kTileBytes <= kLdsBytes, "K and V stage through the LDS");
  __shared__ __attribute__((aligned(256))) unsigned char lds[kLdsBytes];
  unsigned char* const xbuf = lds + kRingBytes;  // [key block][parity][4][64 lanes][4 floats]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool pwave = wave < W::kPairs;
  const int pair = pwave ? wave : wave - W::kPairs;
  const int lm = lane & 31;
  const int lh = lane >> 5;

  const uint32_t nkw = (uint32_t)(a.nkb + W::kKB - 1) / W::kKB;
  const uint32_t lam = xcd_remap(blockIdx.x, a.nwg);
  const int64_t bh = (int64_t)(lam / nkw);
  const int32_t j0 = (int32_t)(lam % nkw) * W::kKeys;
  const int32_t jk0 = j0 + 64 * pair;  // this pair's first key (key blocks 2p, 2p + 1)
  const int32_t delta = a.seq_kv - a.seq_q;
  int32_t qb_first = 0;
  if (CAUSAL) {
    const int32_t i_min = j0 - delta;
    qb_first = i_min <= 0 ? 0 : i_min / G::kRows;
  }
  const int32_t nblk = a.nqb > qb_first ? a.nqb - qb_first : 0;

  const int64_t q_off = head_offset(bh, a.heads, a.qs_b, a.qs_h);
  const int64_t kv_off = head_offset(bh, a.heads, a.kvs_b, a.kvs_h);
  const unsigned q_row = (unsigned)(a.qs_s * 2), kv_row = (unsigned)(a.kvs_s * 2);
  const unsigned g_row = (unsigned)G::kRowBytes;
  const __amdgpu_buffer_rsrc_t q_rsrc = raw_buffer(a.q16 + q_off, strided_range(a.seq_q, a.qs_s, D, 2));
  const __amdgpu_buffer_rsrc_t g_rsrc =
      raw_buffer(a.dout16 + (size_t)bh * a.seq_q * D, (unsigned)a.seq_q * g_row);
  const __amdgpu_buffer_rsrc_t m_rsrc =
      raw_buffer(a.meta + (size_t)bh * a.nqb * kBwdMetaFloats, (unsigned)a.nqb * (unsigned)G::kMetaBytes);
  __amdgpu_buffer_rsrc_t w_rsrc;
  if (MASKED)
    w_rsrc = raw_buffer(a.mask_bits + head_offset(bh, a.heads, a.mbits_sb, a.mbits_sh),
                        (unsigned)a.seq_q * (unsigned)a.mask_words * 4u);

  // Copies of query block T into its ring slot: the Q and dO tiles split over the waves;
  // the P waves add lse2/D (wave 0) and the mask words (wave w: key blocks 2w + lane / 32,
  // row lane % 32). `pw` compiles those out of the dS waves' loop.
  // The lane's source offsets are formed again at each copy from an opaque lane index
  // rather than held in registers across the step loop. Wave w's copy of a tile (Q for
  // u = 0, dO for u = 1) is LDS rows 4 w + t (t = lane / 16), whose source rows are
  // swap_bits_2_3(4 w) + t and whose chunk position lane % 16 holds logical chunk
  // (lane % 16) ^ (4 t + w % 4): what tile_src gives, with only t per lane.
  static_assert(W::kTileCopiesPerWave == 2 && G::kDmaPerTile == W::kWaves && G::kChunks == 16,
                "one Q and one dO copy per wave, 16 chunks per row");
  const unsigned src_row0 = (unsigned)swap_bits_2_3(4 * wave);
  auto issue = [&](int32_t T, auto pw) {
    constexpr bool kP = decltype(pw)::value;
    unsigned ln = (unsigned)lane;
    asm volatile("" : "+v"(ln));
    const unsigned t = ln >> 4;
    const unsigned x = 16u * ((ln & 15u) ^ (4u * t + (unsigned)(wave & 3)));
    const unsigned r0 = (unsigned)(G::kRows * (qb_first + T)) + src_row0;
    unsigned char* const slot = lds + (T % W::kSlots) * kSlotBytes;
    dma_load_x4(q_rsrc, (r0 + t) * q_row + x, lds_address(slot + 1024 * wave));
    dma_load_x4(g_rsrc, (r0 + t) * g_row + x, lds_address(slot + 1024 * (G::kDmaPerTile + wave)));
    const int32_t qb = qb_first + T;
    if (kP && wave == 0)
      dma_load_x1(m_rsrc, (unsigned)qb * (unsigned)G::kMetaBytes + 4u * ln, lds_address(slot + 2 * G::kTileBytes));
    if (MASKED && kP) {
      const unsigned kbw = 2u * (unsigned)wave + (ln >> 5);
      dma_load_x1(w_rsrc, ((unsigned)(G::kRows * qb) + (ln & 31u)) * (unsigned)a.mask_words * 4u +
                              ((unsigned)(j0 / 32) + kbw) * 4u,
                  lds_address(slot + 2 * G::kTileBytes + G::kMetaBytes + 256 * wave));
    }
  };
  const int copies_per_block = W::kTileCopiesPerWave + (pwave && wave == 0 ? 1 : 0) + (MASKED && pwave ? 1 : 0);

  // K (P waves) or V (dS waves) of the pair's two key blocks, staged through the LDS, into
  // B operands: lane (key m, h) holds head dims 16 st + 8 h .. + 7 of key jk0 + 32 b + m.
  const unsigned kv_range = strided_range(a.seq_kv, a.kvs_s, D, 2);
  bf16x8 kv[W::kKBW][G::kSteps];
  {
    const __amdgpu_buffer_rsrc_t k_rsrc = raw_buffer(a.k16 + kv_off, kv_range);
    const __amdgpu_buffer_rsrc_t v_rsrc = raw_buffer(a.v16 + kv_off, kv_range);
    constexpr int kCopies = 2 * W::kKB * G::kDmaPerTile;  // K tiles, then V tiles
#pragma unroll
    for (int u = 0; u < kCopies / W::kWaves; ++u) {
      const int c = u * W::kWaves + wave;
      const int tensor = c / (W::kKB * G::kDmaPerTile), kbc = (c / G::kDmaPerTile) % W::kKB, t = c % G::kDmaPerTile;
      const unsigned src = (unsigned)(j0 + 32 * kbc) * kv_row + tile_src<D, false>(t, lane, kv_row);
      dma_load_x4(tensor == 0 ? k_rsrc : v_rsrc, src, lds_address(lds + 1024 * c));
    }
    wait_vmcnt<0>();
    __syncthreads();
#pragma unroll
    for (int b = 0; b < W::kKBW; ++b) {
      const unsigned char* tile = lds + ((pwave ? 0 : W::kKB) + 2 * pair + b) * G::kTileBytes;
#pragma unroll
      for (int st = 0; st < G::kSteps; ++st) kv[b][st] = row_chunk<D>(tile, lm, 2 * st + lh);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the operand reads have returned
    __syncthreads();                     // before the ring takes the space
  }

  f32x16 acc[W::kKBW][G::kNch];  // dV (P waves) or dK (dS waves) of the two key blocks
#pragma unroll
  for (int b = 0; b < W::kKBW; ++b)
#pragma unroll
    for (int cb = 0; cb < G::kNch; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[b][cb][r] = 0.f;

  // Whether query block qb admits a key of the pair (then the pair computes both key
  // blocks: the causal bound excludes what the second one does not admit).
  auto reaches = [&](int32_t qb) {
    return jk0 < a.seq_kv && (!CAUSAL || G::kRows * qb + G::kRows - 1 + delta >= jk0);
  };

  auto run_steps = [&](auto pw, auto&& work) {
    if (nblk > 0) issue(0, pw);
    if (nblk > 1) issue(1, pw);
    for (int32_t T = 0; T <= nblk; ++T) {
      if (T + 1 < nblk) wait_vmcnt_n(copies_per_block);
      else wait_vmcnt<0>();
      __syncthreads();  // block T has landed; step T - 1 is done with its slots and P
      if (T + 2 < nblk) issue(T + 2, pw);
      work(T);
    }
  };

  // Read bases from an opaque lane index, formed in each step (a few instructions) rather
  // than held in registers across it.
  auto opaque_lane = [&]() {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    return ln;
  };

  if (pwave) {
    bf16x8 pp_late[W::kKBW][2];
    bool pending = false;
    const unsigned char* g_late = lds;
    run_steps(std::true_type{}, [&](int32_t T) {
      if (pending) {  // dV^T += dO^T P of the previous block, for both key blocks
        __builtin_amdgcn_s_setprio(1);
        const int ln = opaque_lane();
        unsigned tl = tr_base<D>(lds_address(g_late), ln, false);
        unsigned th = tr_base<D>(lds_address(g_late), ln, true);
        mfma_stream<2 * G::kNch, 2>(
            [&](int i) { return tr_read<D>(pin(tl), pin(th), i / G::kNch, i % G::kNch); },
            [&](int i, bf16x8 x) {
#pragma unroll
              for (int b = 0; b < W::kKBW; ++b) {
                acc[b][i % G::kNch] = mfma16<F16>(x, pp_late[b][i / G::kNch], acc[b][i % G::kNch]);
                pin_acc(acc[b][i % G::kNch]);
              }
            });
        __builtin_amdgcn_s_setprio(0);
        pending = false;
      }
      const int32_t qb = qb_first + T;
      if (T < nblk && reaches(qb)) {
        const int32_t i0 = G::kRows * qb;
        const unsigned char* const q_slot = lds + (T % W::kSlots) * kSlotBytes;
        const unsigned char* const g_slot = q_slot + G::kTileBytes;
        const unsigned char* const m_slot = g_slot + G::kTileBytes;
        f32x16 s[W::kKBW];
#pragma unroll
        for (int b = 0; b < W::kKBW; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[b][r] = 0.f;
        __builtin_amdgcn_s_setprio(1);
        const int lq = opaque_lane();
        unsigned rb = row_base<D>(lds_address(q_slot), lq & 31, lq >> 5);
        mfma_stream<G::kSteps, 1>([&](int st) { return row_read(pin(rb), st); },
                                  [&](int st, bf16x8 x) {
#pragma unroll
                                    for (int b = 0; b < W::kKBW; ++b) {
                                      s[b] = mfma16<F16>(x, kv[b][st], s[b]);
                                      pin_acc(s[b]);
                                    }
                                  });
        __builtin_amdgcn_s_setprio(0);
        unsigned ma = lds_address(m_slot) + 32u * (unsigned)lh;  // lse2 of rows 16t + 8 lh + 0..7
        pin(ma);
        bf16x8 pp[W::kKBW][2];
#pragma unroll
        for (int b = 0; b < W::kKBW; ++b) {
          const int32_t jk = jk0 + 32 * b;
          uint32_t mbits = 0;  // bit r: row perm_acc_row(r, lh) admits key jk + lm
          if (MASKED) {
            unsigned wa = lds_address(m_slot + G::kMetaBytes + 4 * G::kRows * (2 * pair + b)) + 32u * (unsigned)lh;
            pin(wa);
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              const u32x4 w4 =
                  *(__attribute__((address_space(3))) const u32x4*)(size_t)(wa + 4u * (16 * (q4 / 2) + 4 * (q4 % 2)));
#pragma unroll
              for (int e = 0; e < 4; ++e) mbits |= ((w4[e] >> lm) & 1u) << (4 * q4 + e);
            }
            asm volatile("" : "+v"(mbits));
          }
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {  // exponents in place of the scores
            const f32x4 l4 =
                *(__attribute__((address_space(3))) const f32x4*)(size_t)(ma + 4u * (16 * (q4 / 2) + 4 * (q4 % 2)));
#pragma unroll
            for (int e = 0; e < 4; ++e) s[b][4 * q4 + e] = s[b][4 * q4 + e] * a.c - l4[e];
          }
          if (CAUSAL && jk + G::kRows - 1 > i0 + delta) {
            // Key jk + lm is admitted to row i0 + perm_acc_row(r, lh) iff
            // 16 (r / 8) + r % 8 >= rel. The empty asm keeps the bound, and with it the
            // comparisons, inside this branch.
            int32_t rel = jk + lm - i0 - delta - 8 * lh;
            asm volatile("" : "+v"(rel));
#pragma unroll
            for (int r = 0; r < 16; ++r) s[b][r] = 16 * (r / 8) + r % 8 >= rel ? s[b][r] : -INFINITY;
          }
          if (MASKED) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[b][r] = ((mbits >> r) & 1u) ? s[b][r] : -INFINITY;
          }
          unsigned char* const xp = xbuf + ((2 * (2 * pair + b)) + (T & 1)) * W::kXBytes + 16 * lane;
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            f32x4 p4;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 4 * q4 + e;
              const float p = __builtin_amdgcn_exp2f(s[b][r]);
              p4[e] = p;
              pp[b][r / 8][r % 8] = round16<F16>(p);
            }
            *reinterpret_cast<f32x4*>(xp + 1024 * q4) = p4;
          }
        }
#pragma unroll
        for (int b = 0; b < W::kKBW; ++b) {
          pp_late[b][0] = pp[b][0];
          pp_late[b][1] = pp[b][1];
        }
        g_late = g_slot;
        pending = true;
      }
    });
  } else {
    run_steps(std::false_type{}, [&](int32_t T) {
      const int32_t qb = qb_first + T - 1;
      if (T >= 1 && reaches(qb)) {
        const unsigned char* const q_slot = lds + ((T - 1) % W::kSlots) * kSlotBytes;
        const unsigned char* const g_slot = q_slot + G::kTileBytes;
        const unsigned char* const m_slot = g_slot + G::kTileBytes;
        f32x16 dp[W::kKBW];
#pragma unroll
        for (int b = 0; b < W::kKBW; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r) dp[b][r] = 0.f;
        __builtin_amdgcn_s_setprio(1);
        const int lq = opaque_lane();
        unsigned rb = row_base<D>(lds_address(g_slot), lq & 31, lq >> 5);
        mfma_stream<G::kSteps, 1>([&](int st) { return row_read(pin(rb), st); },
                                  [&](int st, bf16x8 x) {
#pragma unroll
                                    for (int b = 0; b < W::kKBW; ++b) {
                                      dp[b] = mfma16<F16>(x, kv[b][st], dp[b]);
                                      pin_acc(dp[b]);
                                    }
                                  });
        __builtin_amdgcn_s_setprio(0);
        unsigned da = lds_address(m_slot) + 4u * (unsigned)G::kRows + 32u * (unsigned)lh;  // D of the same rows
        pin(da);
        bf16x8 pds[W::kKBW][2];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 d4 =
              *(__attribute__((address_space(3))) const f32x4*)(size_t)(da + 4u * (16 * (q4 / 2) + 4 * (q4 % 2)));
#pragma unroll
          for (int b = 0; b < W::kKBW; ++b) {
            const f32x4 p4 = *reinterpret_cast<const f32x4*>(
                xbuf + ((2 * (2 * pair + b)) + ((T - 1) & 1)) * W::kXBytes + 16 * lane + 1024 * q4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 4 * q4 + e;
              pds[b][r / 8][r % 8] = round16<F16>(p4[e] * (dp[b][r] - d4[e]));
            }
          }
        }
        // dK^T += Q^T dS for both key blocks (the scale is applied once, at the end)
        __builtin_amdgcn_s_setprio(1);
        const int ln = opaque_lane();
        unsigned tl = tr_base<D>(lds_address(q_slot), ln, false);
        unsigned th = tr_base<D>(lds_address(q_slot), ln, true);
        mfma_stream<2 * G::kNch, 2>(
            [&](int i) { return tr_read<D>(pin(tl), pin(th), i / G::kNch, i % G::kNch); },
            [&](int i, bf16x8 x) {
#pragma unroll
              for (int b = 0; b < W::kKBW; ++b) {
                acc[b][i % G::kNch] = mfma16<F16>(x, pds[b][i / G::kNch], acc[b][i % G::kNch]);
                pin_acc(acc[b][i % G::kNch]);
              }
            });
        __builtin_amdgcn_s_setprio(0);
      }
    });
  }

  // Lane (key m, h) holds head dims 32 cb + 8 g4 + 4 h .. + 3 of key jk0 + 32 b + m.
  const float mul = pwave ? 1.0f : a.scale;
#pragma unroll
  for (int b = 0; b < W::kKBW; ++b) {
    const int32_t j = jk0 + 32 * b + lm;
    if (j >= a.seq_kv) continue;
    float* const out = (pwave ? a.dv : a.dk) + kv_off + (int64_t)j * a.kvs_s;
#pragma unroll
    for (int cb = 0; cb < G::kNch; ++cb)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *reinterpret_cast<f32x4*>(out + 32 * cb + 8 * g4 + 4 * lh) =
            f32x4{acc[b][cb][4 * g4] * mul, acc[b][cb][4 * g4 + 1] * mul, acc[b][cb][4 * g4 + 2] * mul,
                  acc[b][cb][4 * g4 + 3] * mul};
  }
}

// ---------------------------------------------------------------- dQ

// A workgroup owns 256 queries of one (batch, head), a 32-row block per wave; each wave
// keeps its rows' Q and dO in registers as the B operands of S^T = K Q^T and
// dP^T = V dO^T, and accumulates dQ^T += K^T dS^T. The waves step through the key blocks
// the workgroup's rows admit together: key block T's K and V tiles (permuted) and, with a
// hard mask, the rows' words of block T are copied straight into a ring of eight LDS
// slots, a pair of blocks at a time two steps ahead, each wave issuing a share; waves 4-7
// run each block's dQ product one step late, so that block stays in the ring a step
// longer. One barrier per pair of steps.
template <int D>
struct QGeom {
  static_assert(D <= 128, "head dim 256 runs attn_bwd_dq_bf16_rs_kernel");
  static constexpr int kWaves = 8;
  static constexpr int kQ = 32 * kWaves;  // queries per workgroup
  static constexpr int kSlots = 8;  // blocks T - 1 .. T + 3 live in step T
  static constexpr int kDma = HGeom<D>::kDmaPerTile;
  static constexpr int kTileCopies = 2 * kDma;  // K and V of one block
  // As for the dK/dV kernel: d = 32 has four copies, one for each of waves 0..3.
  static constexpr int kTileCopiesPerWave = kTileCopies >= kWaves ? kTileCopies / kWaves : 1;
  static_assert(kTileCopies < kWaves ? kTileCopies * 2 == kWaves : kTileCopiesPerWave * kWaves == kTileCopies,
                "copy split");
};

template <int D, bool CAUSAL, bool MASKED, bool F16>
__global__ __launch_bounds__(64 * QGeom<D>::kWaves) void attn_bwd_dq_bf16_kernel(BwdArgs a) {
  using G = HGeom<D>;
  using W = QGeom<D>;
  // Slot: K tile, V tile, and with a hard mask the workgroup rows' words of the key block.
  constexpr int kMaskBytes = MASKED ? 4 * W::kQ : 0;
  // Head dim 128 reads its tiles at XOR-formed addresses (row_read, tr_read): every tile
  // starts on a multiple of 256 bytes.
  constexpr int kAlign = D == 128 ? 2 * D : 16;
  constexpr int kSlotBytes = (2 * G::kTileBytes + kMaskBytes + kAlign - 1) / kAlign * kAlign;
  __shared__ __attribute__((aligned(kAlign))) unsigned char lds[W::kSlots * kSlotBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lm = lane & 31;
  const int lh = lane >> 5;

  // Workgroups of a head are consecutive, the last queries (the most key blocks under a
  // causal mask) first.
  const uint32_t nqw = (uint32_t)(a.nqb + W::kWaves - 1) / W::kWaves;
  const uint32_t lam = xcd_remap(blockIdx.x, a.nwg);
  const int64_t bh = (int64_t)(lam / nqw);
  const int32_t q0 = (int32_t)(nqw - 1 - lam % nqw) * W::kQ;
  const int32_t qw0 = q0 + 32 * wave;  // this wave's first row
  const bool wave_live = qw0 < a.seq_q;

  const int32_t my_row = qw0 + lm;
  const int32_t last_row = min(q0 + W::kQ - 1, a.seq_q - 1);
  const int32_t nblk = (key_limit<CAUSAL>(last_row, a.seq_q, a.seq_kv, a.seq_kv) + G::kRows - 1) / G::kRows;
  const int32_t lim = key_limit<CAUSAL>(my_row, a.seq_q, a.seq_kv, a.seq_kv);
  const int32_t wave_lo = key_limit<CAUSAL>(qw0, a.seq_q, a.seq_kv, a.seq_kv);
  const int32_t wave_hi = key_limit<CAUSAL>(min(qw0 + 31, a.seq_q - 1), a.seq_q, a.seq_kv, a.seq_kv);

  const int64_t q_off = head_offset(bh, a.heads, a.qs_b, a.qs_h);
  const int64_t kv_off = head_offset(bh, a.heads, a.kvs_b, a.kvs_h);
  const unsigned kv_row = (unsigned)(a.kvs_s * 2);
  const unsigned kv_range = strided_range(a.seq_kv, a.kvs_s, D, 2);
  const __amdgpu_buffer_rsrc_t k_rsrc = raw_buffer(a.k16 + kv_off, kv_range);
  const __amdgpu_buffer_rsrc_t v_rsrc = raw_buffer(a.v16 + kv_off, kv_range);
  __amdgpu_buffer_rsrc_t w_rsrc;  // rows past seq_q read as 0: nothing admitted
  if (MASKED)
    w_rsrc = raw_buffer(a.mask_bits + head_offset(bh, a.heads, a.mbits_sb, a.mbits_sh),
                        (unsigned)a.seq_q * (unsigned)a.mask_words * 4u);

  // Copies of key block T into its ring slot: the K and V tiles split over the waves;
  // with a hard mask waves 0 .. kQ/64 - 1 add the words of 64 rows each.
  auto issue = [&](int32_t T) {
    unsigned char* const slot = lds + (T % W::kSlots) * kSlotBytes;
    const unsigned row0 = (unsigned)(G::kRows * T) * kv_row;
#pragma unroll
    for (int u = 0; u < W::kTileCopiesPerWave; ++u) {
      const int c = u * W::kWaves + wave;  // K copies, then V copies
      if (c >= W::kTileCopies) break;      // d = 32: waves 4..7 copy no tile
      if (c < W::kDma)
        dma_load_x4(k_rsrc, row0 + tile_src<D, true>(c, lane, kv_row), lds_address(slot + 1024 * c));
      else
        dma_load_x4(v_rsrc, row0 + tile_src<D, true>(c - W::kDma, lane, kv_row), lds_address(slot + 1024 * c));
    }
    if (MASKED && wave < W::kQ / 64)
      dma_load_x1(w_rsrc, ((unsigned)(q0 + 64 * wave + lane) * (unsigned)a.mask_words + (unsigned)T) * 4u,
                  lds_address(slot + 2 * G::kTileBytes + 256 * wave));
  };

  // This wave's rows: lse2 and D (the preprocess pads past seq_q), and Q and dO as B
  // operands: lane (query m, h) holds head dims 16*st + 8*h .. + 7 of row qw0 + m (zeros
  // past seq_q).
  float my_l2 = INFINITY, my_d = 0.f;
  bf16x8 qr[G::kSteps], gr[G::kSteps];
  {
    const bool row_ok = my_row < a.seq_q;
    if (wave_live) {
      const float* const meta = a.meta + ((size_t)bh * a.nqb + qw0 / G::kRows) * kBwdMetaFloats;
      my_l2 = meta[lm];
      my_d = meta[G::kRows + lm];
    }
    const unsigned short* const qrow = a.q16 + q_off + (int64_t)(row_ok ? my_row : 0) * a.qs_s;
    const unsigned short* const grow = a.dout16 + ((size_t)bh * a.seq_q + (row_ok ? my_row : 0)) * D;
#pragma unroll
    for (int st = 0; st < G::kSteps; ++st) {
      const u32x4 zero = {0u, 0u, 0u, 0u};
      const u32x4 xq = row_ok ? *reinterpret_cast<const u32x4*>(qrow + 16 * st + 8 * lh) : zero;
      const u32x4 xg = row_ok ? *reinterpret_cast<const u32x4*>(grow + 16 * st + 8 * lh) : zero;
      qr[st] = __builtin_bit_cast(bf16x8, xq);
      gr[st] = __builtin_bit_cast(bf16x8, xg);
    }
  }

  constexpr int kPf = 3;  // MFMA operand reads in flight ahead of their MFMA
  f32x16 dq[G::kNch];
#pragma unroll
  for (int cb = 0; cb < G::kNch; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[cb][r] = 0.f;

  // dQ^T += K^T dS^T for the block in k_slot.
  auto dq_product = [&](const unsigned char* k_slot, const bf16x8 (&pds)[2]) {
    __builtin_amdgcn_s_setprio(1);
    if constexpr (D == 128) {
      unsigned tl = tr_base<D>(lds_address(k_slot), lane, false);
      unsigned th = tr_base<D>(lds_address(k_slot), lane, true);
      mfma_stream<2 * G::kNch, kPf>(
          [&](int i) { return tr_read<D>(pin(tl), pin(th), i / G::kNch, i % G::kNch); },
          [&](int i, bf16x8 x) {
            dq[i % G::kNch] = mfma16<F16>(x, pds[i / G::kNch], dq[i % G::kNch]);
            pin_acc(dq[i % G::kNch]);
          });
    } else {
      mfma_stream<2 * G::kNch, kPf>(
          [&](int i) { return tr_operand<D>(k_slot, lane, i / G::kNch, i % G::kNch); },
          [&](int i, bf16x8 x) { dq[i % G::kNch] = mfma16<F16>(x, pds[i / G::kNch], dq[i % G::kNch]); });
    }
    __builtin_amdgcn_s_setprio(0);
  };
  // Waves 4-7 (each sharing a SIMD with wave - 4) run their dQ product of block T at the
  // start of step T + 1, so that the two waves of a SIMD are half a step apart and one's
  // MFMAs meet the other's softmax.
  const bool late = wave >= 4;
  bf16x8 pds_late[2];
  bool pending = false;
  const unsigned char* late_slot = lds;
  // Blocks are copied a pair at a time, two steps ahead, with one barrier per pair: at an
  // even step T blocks T and T + 1 have landed (nothing else is in flight) and every wave
  // is done with step T - 1, so blocks T + 2 and T + 3 may take the slots of T - 6 and
  // T - 5 (a late wave still reads block T - 1 in step T).
  if (0 < nblk) issue(0);
  if (1 < nblk) issue(1);
  for (int32_t T = 0; T < nblk; ++T) {
    if ((T & 1) == 0) {
      wait_vmcnt<0>();
      __syncthreads();
      if (T + 2 < nblk) issue(T + 2);
      if (T + 3 < nblk) issue(T + 3);
    }
    if (late && pending) {
      dq_product(late_slot, pds_late);
      pending = false;
    }
    const int32_t j0 = G::kRows * T;
    if (!wave_live || j0 >= wave_hi) continue;
    const unsigned char* const k_slot = lds + (T % W::kSlots) * kSlotBytes;
    const unsigned char* const v_slot = k_slot + G::kTileBytes;
    f32x16 dp, s;
#pragma unroll
    for (int r = 0; r < 16; ++r) dp[r] = s[r] = 0.f;
    __builtin_amdgcn_s_setprio(1);
    // dP^T and S^T, their k-steps interleaved.
    if constexpr (D == 128) {
      unsigned kb = row_base<D>(lds_address(k_slot), lm, lh), vb = row_base<D>(lds_address(v_slot), lm, lh);
      mfma_stream<2 * G::kSteps, kPf>(
          [&](int i) { return row_read(i % 2 ? pin(kb) : pin(vb), i / 2); },
          [&](int i, bf16x8 x) {
            if (i % 2) {
              s = mfma16<F16>(x, qr[i / 2], s);
              pin_acc(s);
            } else {
              dp = mfma16<F16>(x, gr[i / 2], dp);
              pin_acc(dp);
            }
          });
    } else {
      mfma_stream<2 * G::kSteps, kPf>(
          [&](int i) { return row_chunk<D>(i % 2 ? k_slot : v_slot, lm, 2 * (i / 2) + lh); },
          [&](int i, bf16x8 x) {
            if (i % 2) s = mfma16<F16>(x, qr[i / 2], s);
            else dp = mfma16<F16>(x, gr[i / 2], dp);
          });
    }
    __builtin_amdgcn_s_setprio(0);
    float t[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) t[r] = s[r] * a.c - my_l2;
    if (j0 + G::kRows > wave_lo) {  // some key of the block lies past the first row's limit
      // Key j0 + perm_acc_row(r, lh) is admitted iff 16 (r / 8) + r % 8 < rel (the empty
      // asm keeps the comparisons inside this branch).
      int32_t rel = lim - j0 - 8 * lh;
      asm volatile("" : "+v"(rel));
#pragma unroll
      for (int r = 0; r < 16; ++r) t[r] = 16 * (r / 8) + r % 8 < rel ? t[r] : -INFINITY;
    }
    if (MASKED) {
      const uint32_t mw = *reinterpret_cast<const uint32_t*>(v_slot + G::kTileBytes + 4 * (32 * wave + lm));
#pragma unroll
      for (int r = 0; r < 16; ++r) t[r] = ((mw >> perm_acc_row(r, lh)) & 1u) ? t[r] : -INFINITY;
    }
    bf16x8 pds[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      // dS in fp32, then rounded to the input type. For fp16 the compiler would otherwise
      // round the exact product once (v_fma_mixlo_f16), which now and then differs from the
      // dS that the dK/dV kernel rounds: the empty asm keeps the fp32 product.
      const float p = __builtin_amdgcn_exp2f(t[r]);
      float ds = p * (dp[r] - my_d);
      if constexpr (F16) asm("" : "+v"(ds));
      pds[r / 8][r % 8] = round16<F16>(ds);
    }
    if (late) {
      pds_late[0] = pds[0];
      pds_late[1] = pds[1];
      late_slot = k_slot;
      pending = true;
    } else {
      dq_product(k_slot, pds);
    }
  }
  if (pending) dq_product(late_slot, pds_late);

  // Lane (query m, h) holds head dims 32*cb + 8*g4 + 4*h .. + 3 of row qw0 + m.
  if (!wave_live || my_row >= a.seq_q) return;
  float* const out = a.dq + q_off + (int64_t)my_row * a.qs_s;
#pragma unroll
  for (int cb = 0; cb < G::kNch; ++cb)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4)
      *reinterpret_cast<f32x4*>(out + 32 * cb + 8 * g4 + 4 * lh) =
          f32x4{dq[cb][4 * g4] * a.scale, dq[cb][4 * g4 + 1] * a.scale, dq[cb][4 * g4 + 2] * a.scale,
                dq[cb][4 * g4 + 3] * a.scale};
}

// Head dim 256, where a wave cannot hold its rows' Q and dO (128 registers) beside their
// dQ accumulators (128) at two waves per SIMD. The work of a 32-row query block is split by
// role between two waves that share a SIMD, as in the dK/dV kernel:
//  - the S wave keeps the rows' Q, forms S^T = K Q^T and P = 2^(c S - lse2) for key block
//    T and leaves P in LDS (fp32, double buffered);
//  - the dS wave keeps the rows' dO and the dQ accumulators and works on block T - 1: it
//    forms dP^T = V dO^T, reads that block's P, forms dS = P (dP - D) and accumulates
//    dQ^T += K^T dS^T.
// A workgroup owns 128 queries, 4 pairs (wave p and wave p + 4). Key block T's K and V tiles
// (permuted) and, with a hard mask, the rows' words are copied straight into a ring of
// three LDS slots one step ahead; the operand reads are streamed two MFMAs ahead at
// XOR-formed addresses (row_read, tr_read). One barrier per step.
struct QRGeom {
  static constexpr int D = 256;
  static constexpr int kPairs = 4;
  static constexpr int kWaves = 2 * kPairs;
  static constexpr int kQ = 32 * kPairs;  // queries per workgroup
  static constexpr int kSlots = 3;
  static constexpr int kDma = HGeom<D>::kDmaPerTile;
  static constexpr int kTileCopies = 2 * kDma;  // K and V of one block
  static constexpr int kTileCopiesPerWave = kTileCopies / kWaves;
  static constexpr int kXBytes = 16 * 64 * 4;  // a wave's 16 P values per lane
  static_assert(kTileCopiesPerWave * kWaves == kTileCopies, "copy split");
};

template <bool CAUSAL, bool MASKED, bool F16>
__global__ __launch_bounds__(64 * QRGeom::kWaves) void attn_bwd_dq_bf16_rs_kernel(BwdArgs a) {
  constexpr int D = QRGeom::D;
  using G = HGeom<D>;
  using W = QRGeom;
  // Slot: K tile, V tile, and with a hard mask the workgroup rows' words of the key block;
  // every tile on a multiple of 512 bytes (the XOR-formed addresses).
  constexpr int kMaskBytes = MASKED ? 4 * W::kQ : 0;
  constexpr int kSlotBytes = (2 * G::kTileBytes + kMaskBytes + 2 * D - 1) / (2 * D) * (2 * D);
  constexpr int kRingBytes = W::kSlots * kSlotBytes;
  __shared__ __attribute__((aligned(2 * D))) unsigned char lds[kRingBytes + 2 * W::kPairs * W::kXBytes];
  unsigned char* const xbuf = lds + kRingBytes;  // [pair][parity][4][64 lanes][4 floats]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool swave = wave < W::kPairs;
  const int pair = swave ? wave : wave - W::kPairs;
  const int lm = lane & 31;
  const int lh = lane >> 5;

  // Workgroups of a head are consecutive, the last queries (the most key blocks under a
  // causal mask) first.
  const uint32_t nqw = (uint32_t)(a.nqb + W::kPairs - 1) / W::kPairs;
  const uint32_t lam = xcd_remap(blockIdx.x, a.nwg);
  const int64_t bh = (int64_t)(lam / nqw);
  const int32_t q0 = (int32_t)(nqw - 1 - lam % nqw) * W::kQ;
  const int32_t qw0 = q0 + 32 * pair;  // the pair's first row
  const bool pair_live = qw0 < a.seq_q;

  const int32_t my_row = qw0 + lm;
  const int32_t last_row = min(q0 + W::kQ - 1, a.seq_q - 1);
  const int32_t nblk = (key_limit<CAUSAL>(last_row, a.seq_q, a.seq_kv, a.seq_kv) + G::kRows - 1) / G::kRows;
  const int32_t lim = key_limit<CAUSAL>(my_row, a.seq_q, a.seq_kv, a.seq_kv);
  const int32_t pair_lo = key_limit<CAUSAL>(qw0, a.seq_q, a.seq_kv, a.seq_kv);
  const int32_t pair_hi = key_limit<CAUSAL>(min(qw0 + 31, a.seq_q - 1), a.seq_q, a.seq_kv, a.seq_kv);
  // Whether key block T holds a key some row of the pair admits (the same for both waves).
  auto works = [&](int32_t T) { return pair_live && G::kRows * T < pair_hi; };

  const int64_t q_off = head_offset(bh, a.heads, a.qs_b, a.qs_h);
  const int64_t kv_off = head_offset(bh, a.heads, a.kvs_b, a.kvs_h);
  const unsigned kv_row = (unsigned)(a.kvs_s * 2);
  const unsigned kv_range = strided_range(a.seq_kv, a.kvs_s, D, 2);
  const __amdgpu_buffer_rsrc_t k_rsrc = raw_buffer(a.k16 + kv_off, kv_range);
  const __amdgpu_buffer_rsrc_t v_rsrc = raw_buffer(a.v16 + kv_off, kv_range);
  __amdgpu_buffer_rsrc_t w_rsrc;  // rows past seq_q read as 0: nothing admitted
  if (MASKED)
    w_rsrc = raw_buffer(a.mask_bits + head_offset(bh, a.heads, a.mbits_sb, a.mbits_sh),
                        (unsigned)a.seq_q * (unsigned)a.mask_words * 4u);

  // Copies of key block T into its ring slot: the K and V tiles split over the waves; with
  // a hard mask waves 0 .. kQ/64 - 1 (S waves) add the words of 64 rows each.
  auto issue = [&](int32_t T, auto sw) {
    constexpr bool kS = decltype(sw)::value;
    unsigned char* const slot = lds + (T % W::kSlots) * kSlotBytes;
    const unsigned row0 = (unsigned)(G::kRows * T) * kv_row;
#pragma unroll
    for (int u = 0; u < W::kTileCopiesPerWave; ++u) {
      const int c = u * W::kWaves + wave;  // K copies, then V copies
      if (c < W::kDma)
        dma_load_x4(k_rsrc, row0 + tile_src<D, true>(c, lane, kv_row), lds_address(slot + 1024 * c));
      else
        dma_load_x4(v_rsrc, row0 + tile_src<D, true>(c - W::kDma, lane, kv_row), lds_address(slot + 1024 * c));
    }
    if (MASKED && kS && wave < W::kQ / 64)
      dma_load_x1(w_rsrc, ((unsigned)(q0 + 64 * wave + lane) * (unsigned)a.mask_words + (unsigned)T) * 4u,
                  lds_address(slot + 2 * G::kTileBytes + 256 * wave));
  };
  static_assert(W::kQ / 64 <= W::kPairs, "the mask copies come from S waves");

  // The step loop, run by every wave with its role's work (one copy per role, so that its
  // registers stay put): block T lands, one barrier, block T + 1 is issued.
  auto run_steps = [&](auto sw, auto&& work) {
    if (nblk > 0) issue(0, sw);
    for (int32_t T = 0; T <= nblk; ++T) {
      wait_vmcnt<0>();
      __syncthreads();  // block T has landed; step T - 1 is done with block T - 2's slot and its P
      if (T + 1 < nblk) issue(T + 1, sw);
      work(T);
    }
  };

  // This pair's rows: lane (query m, h) holds head dims 16*st + 8*h .. + 7 of row qw0 + m
  // (zeros past seq_q) of Q (S wave) or dO (dS wave), as the B operands of the score
  // products; lse2 or D of row qw0 + m (the preprocess pads past seq_q).
  bf16x8 rows[G::kSteps];
  float my_meta = swave ? INFINITY : 0.f;
  {
    const bool row_ok = my_row < a.seq_q;
    if (pair_live) {
      const float* const meta = a.meta + ((size_t)bh * a.nqb + qw0 / G::kRows) * kBwdMetaFloats;
      my_meta = meta[(swave ? 0 : G::kRows) + lm];
    }
    const unsigned short* const src =
        swave ? a.q16 + q_off + (int64_t)(row_ok ? my_row : 0) * a.qs_s
              : a.dout16 + ((size_t)bh * a.seq_q + (row_ok ? my_row : 0)) * D;
#pragma unroll
    for (int st = 0; st < G::kSteps; ++st) {
      const u32x4 zero = {0u, 0u, 0u, 0u};
      const u32x4 x = row_ok ? *reinterpret_cast<const u32x4*>(src + 16 * st + 8 * lh) : zero;
      rows[st] = __builtin_bit_cast(bf16x8, x);
    }
  }

  if (swave) {
    run_steps(std::true_type{}, [&](int32_t T) {
      if (!works(T)) return;
      const int32_t j0 = G::kRows * T;
      const unsigned char* const k_slot = lds + (T % W::kSlots) * kSlotBytes;
      f32x16 s;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = 0.f;
      __builtin_amdgcn_s_setprio(1);
      unsigned rb = row_base<D>(lds_address(k_slot), lm, lh);
      mfma_stream<G::kSteps, 2>([&](int st) { return row_read(pin(rb), st); },
                                [&](int st, bf16x8 x) { s = mfma16<F16>(x, rows[st], s); pin_acc(s); });
      __builtin_amdgcn_s_setprio(0);
      float t[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) t[r] = s[r] * a.c - my_meta;
      if (j0 + G::kRows > pair_lo) {  // some key of the block lies past the first row's limit
        // Key j0 + perm_acc_row(r, lh) is admitted iff 16 (r / 8) + r % 8 < rel (the empty
        // asm keeps the comparisons inside this branch).
        int32_t rel = lim - j0 - 8 * lh;
        asm volatile("" : "+v"(rel));
#pragma unroll
        for (int r = 0; r < 16; ++r) t[r] = 16 * (r / 8) + r % 8 < rel ? t[r] : -INFINITY;
      }
      if (MASKED) {
        const uint32_t mw = *reinterpret_cast<const uint32_t*>(k_slot + 2 * G::kTileBytes + 4 * (32 * pair + lm));
#pragma unroll
        for (int r = 0; r < 16; ++r) t[r] = ((mw >> perm_acc_row(r, lh)) & 1u) ? t[r] : -INFINITY;
      }
      unsigned char* const xp = xbuf + (2 * pair + (T & 1)) * W::kXBytes + 16 * lane;
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4)
        *reinterpret_cast<f32x4*>(xp + 1024 * c4) =
            f32x4{__builtin_amdgcn_exp2f(t[4 * c4]), __builtin_amdgcn_exp2f(t[4 * c4 + 1]),
                  __builtin_amdgcn_exp2f(t[4 * c4 + 2]), __builtin_amdgcn_exp2f(t[4 * c4 + 3])};
    });
    return;  // the dS wave of the pair writes its dQ
  }

  f32x16 dq[G::kNch];
#pragma unroll
  for (int cb = 0; cb < G::kNch; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[cb][r] = 0.f;
  run_steps(std::false_type{}, [&](int32_t T) {
    if (T < 1 || !works(T - 1)) return;
    const unsigned char* const k_slot = lds + ((T - 1) % W::kSlots) * kSlotBytes;
    const unsigned char* const v_slot = k_slot + G::kTileBytes;
    f32x16 dp;
#pragma unroll
    for (int r = 0; r < 16; ++r) dp[r] = 0.f;
    __builtin_amdgcn_s_setprio(1);
    unsigned rb = row_base<D>(lds_address(v_slot), lm, lh);
    mfma_stream<G::kSteps, 2>([&](int st) { return row_read(pin(rb), st); },
                              [&](int st, bf16x8 x) { dp = mfma16<F16>(x, rows[st], dp); pin_acc(dp); });
    __builtin_amdgcn_s_setprio(0);
    const unsigned char* const xp = xbuf + (2 * pair + ((T - 1) & 1)) * W::kXBytes + 16 * lane;
    bf16x8 pds[2];
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) {
      const f32x4 p4 = *reinterpret_cast<const f32x4*>(xp + 1024 * c4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * c4 + e;
        pds[r / 8][r % 8] = round16<F16>(p4[e] * (dp[r] - my_meta));
      }
    }
    // dQ^T += K^T dS^T (the scale is applied once, at the end)
    __builtin_amdgcn_s_setprio(1);
    unsigned tl = tr_base<D>(lds_address(k_slot), lane, false);
    unsigned th = tr_base<D>(lds_address(k_slot), lane, true);
    mfma_stream<2 * G::kNch, 2>(
        [&](int i) { return tr_read<D>(pin(tl), pin(th), i / G::kNch, i % G::kNch); },
        [&](int i, bf16x8 x) {
          dq[i % G::kNch] = mfma16<F16>(x, pds[i / G::kNch], dq[i % G::kNch]);
          pin_acc(dq[i % G::kNch]);
        });
    __builtin_amdgcn_s_setprio(0);
  });

  // Lane (query m, h) holds head dims 32*cb + 8*g4 + 4*h .. + 3 of row qw0 + m.
  if (!pair_live || my_row >= a.seq_q) return;
  float* const out = a.dq + q_off + (int64_t)my_row * a.qs_s;
#pragma unroll
  for (int cb = 0; cb < G::kNch; ++cb)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4)
      *reinterpret_cast<f32x4*>(out + 32 * cb + 8 * g4 + 4 * lh) =
          f32x4{dq[cb][4 * g4] * a.scale, dq[cb][4 * g4 + 1] * a.scale, dq[cb][4 * g4 + 2] * a.scale,
                dq[cb][4 * g4 + 3] * a.scale};
}

template <int D, bool CAUSAL, bool MASKED, bool F16>
hipError_t launch_bwd_bf16_variant(const BwdArgs& a0, hipStream_t s, hipEvent_t ev_pre,
                                   hipEvent_t ev_dkdv) {
  BwdArgs a = a0;
  const uint32_t nq = (uint32_t)(a.bh * a.nqb), nk = (uint32_t)(a.bh * a.nkb);
  if (nq > 0) {
    hipLaunchKernelGGL((attn_bwd_pre_bf16_kernel<D, F16>), dim3(nq), dim3(256), 0, s, a);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  }
  if (ev_pre && hipEventRecord(ev_pre, s) != hipSuccess) return hipErrorInvalidValue;
  if (nk > 0) {
    if constexpr (D == 128) {
      a.nwg = (uint32_t)(a.bh * ((a.nkb + KV2Geom::kKB - 1) / KV2Geom::kKB));
      hipLaunchKernelGGL((attn_bwd_dkdv_bf16_kb2_kernel<CAUSAL, MASKED, F16>), dim3(a.nwg),
                         dim3(64 * KV2Geom::kWaves), 0, s, a);
    } else {
      a.nwg = (uint32_t)(a.bh * ((a.nkb + KVGeom<D>::kKB - 1) / KVGeom<D>::kKB));
      hipLaunchKernelGGL((attn_bwd_dkdv_bf16_kernel<D, CAUSAL, MASKED, F16>), dim3(a.nwg),
                         dim3(64 * KVGeom<D>::kWaves), 0, s, a);
    }
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  }
  if (ev_dkdv && hipEventRecord(ev_dkdv, s) != hipSuccess) return hipErrorInvalidValue;
  if (nq > 0) {
    if constexpr (D == 256) {
      a.nwg = (uint32_t)(a.bh * ((a.nqb + QRGeom::kPairs - 1) / QRGeom::kPairs));
      hipLaunchKernelGGL((attn_bwd_dq_bf16_rs_kernel<CAUSAL, MASKED, F16>), dim3(a.nwg),
                         dim3(64 * QRGeom::kWaves), 0, s, a);
    } else {
      a.nwg = (uint32_t)(a.bh * ((a.nqb + QGeom<D>::kWaves - 1) / QGeom<D>::kWaves));
      hipLaunchKernelGGL((attn_bwd_dq_bf16_kernel<D, CAUSAL, MASKED, F16>), dim3(a.nwg),
                         dim3(64 * QGeom<D>::kWaves), 0, s, a);
    }
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  }
  return hipSuccess;
}

template <int D, bool F16>
hipError_t launch_bwd_bf16_d(const BwdArgs& a, bool causal, hipStream_t s, hipEvent_t ev_pre,
                             hipEvent_t ev_dkdv) {
  if (a.mask_bits)
    return causal ? launch_bwd_bf16_variant<D, true, true, F16>(a, s, ev_pre, ev_dkdv)
                  : launch_bwd_bf16_variant<D, false, true, F16>(a, s, ev_pre, ev_dkdv);
  return causal ? launch_bwd_bf16_variant<D, true, false, F16>(a, s, ev_pre, ev_dkdv)
                : launch_bwd_bf16_variant<D, false, false, F16>(a, s, ev_pre, ev_dkdv);
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a, int head_dim, bool causal, hipStream_t s,
                           hipEvent_t ev_pre, hipEvent_t ev_dkdv) {
  if (head_dim == 32)
    return a.in_f16 ? launch_bwd_bf16_d<32, true>(a, causal, s, ev_pre, ev_dkdv)
                    : launch_bwd_bf16_d<32, false>(a, causal, s, ev_pre, ev_dkdv);
  if (head_dim == 64)
    return a.in_f16 ? launch_bwd_bf16_d<64, true>(a, causal, s, ev_pre, ev_dkdv)
                    : launch_bwd_bf16_d<64, false>(a, causal, s, ev_pre, ev_dkdv);
  if (head_dim == 128)
    return a.in_f16 ? launch_bwd_bf16_d<128, true>(a, causal, s, ev_pre, ev_dkdv)
                    : launch_bwd_bf16_d<128, false>(a, causal, s, ev_pre, ev_dkdv);
  if (head_dim == 256)
    return a.in_f16 ? launch_bwd_bf16_d<256, true>(a, causal, s, ev_pre, ev_dkdv)
                    : launch_bwd_bf16_d<256, false>(a, causal, s, ev_pre, ev_dkdv);
  return hipErrorInvalidValue;
}

}  // namespace sma
