// Attention backward, fp32 inputs and gradients: dQ, dK and dV of
// O = softmax(scale * Q K^T + causal mask) V, from Q, K, V, O, dO and the
// forward's per-row log-sum-exp (oxicuda ComputeBackend `attention` for the
// forward; the softmax vector-Jacobian product of pulsatrix HIPBackend
// `softmax_rows_backward` and of MicroGPT's fused attention-softmax backward).
//
// Per (batch, head), over admitted pairs (bottom-right causal: j <= i + Skv - Sq):
//   P_ij  = 2^(c s_ij - lse2_i),  c = scale log2(e), lse2 = LSE log2(e)
//   D_i   = dO_i . O_i            (= sum_j P_ij dP_ij)
//   dP_ij = dO_i . v_j,           dS_ij = P_ij (dP_ij - D_i)
//   dV_j  = sum_i P_ij dO_i,      dK_j = scale sum_i dS_ij q_i,   dQ_i = scale sum_j dS_ij k_j
//
// Three launches and no atomics, so the gradients are bitwise reproducible:
//  1. preprocess: per query row lse2 (+inf for a row with no admitted key or
//     past the end, which makes its P exactly 0) and D, stored per 32-row
//     query block as 64 floats in the workspace;
//  2. dK/dV: a workgroup owns 32 keys. Its 4 waves split the query blocks that
//     admit any of them into contiguous ranges; each streams its Q and dO
//     tiles (and the block's lse2/D) into private LDS slots with direct-to-LDS
//     loads, accumulates partial dK^T and dV^T in registers, and the partials
//     are summed through LDS at the end;
//  3. dQ: a workgroup owns 32 queries and its 4 waves split the key blocks, as
//     in the key-split forward kernel; the partial dQ^T are summed at the end.
// S and dP are formed in both 2 and 3: seven 32x32xD products per pair of
// blocks instead of five, the price of writing every gradient from one place.
//
// MFMA layouts (v_mfma_f32_32x32x2f32, lane = 32*h + m). "Row r" of a lane is
// 8*(r/4) + 4*h + r%4, r = 0..15, the rows its 16 accumulator registers hold.
//  dK/dV kernel (lane m <-> key j0 + m):
//    S = Q K^T, dP = dO V^T: A = Q / dO row m at head dims 8u + 4h + e (LDS),
//      B = K / V of key m at the same dims (registers); the lane then holds
//      key m's column for queries i0 + row r.
//    dV^T += dO^T P, dK^T += Q^T dS: step r takes A = dO / Q of query
//      i0 + row r at head dims (D/32)*m + chunk (LDS), B = P / dS register r.
//  dQ kernel (lane m <-> query q0 + m):
//    S^T = K Q^T, dP^T = V dO^T: A = K / V rows (LDS), B = Q / dO of query m
//      (registers); the lane holds query m's scores for keys j0 + row r.
//    dQ^T += K^T dS^T: step r takes A = K of key j0 + row r at head dims
//      (D/32)*m + chunk (LDS), B = dS^T register r.
#include "attn_common.h"

namespace sma {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// D/32 consecutive floats: a lane's share of one gradient row, or of one tile row.
template <int N>
struct FVecB {
  typedef float T __attribute__((ext_vector_type(N)));
};

constexpr float kLog2e = 1.44269504088896340736f;

template <int D>
struct BGeom {
  static constexpr int kWaves = 4;
  static constexpr int kRows = kBwdRowsPerBlock;     // rows per query / key block
  static constexpr int kNch = D / 32;                // accumulator chunks per lane
  static constexpr int kSteps = D / 8;               // MFMA groups of 4 over the head dims
  static constexpr int kRowBytes = 4 * D;
  static constexpr int kTileBytes = kRows * kRowBytes;
  static constexpr int kDmaPerTile = kTileBytes / 1024;
  static constexpr int kMetaBytes = kBwdMetaFloats * 4;
  static constexpr int kPStride = D + 4;             // padded partial-gradient row (floats)
  static constexpr int kPartBytes = kWaves * kRows * kPStride * 4;  // one gradient's partials
  static_assert(kRows == 32, "one 32x32 MFMA tile per block");
  static_assert(kDmaPerTile % kWaves == 0, "shared tile copies split evenly over the waves");
  static_assert(kBwdMetaFloats == 64, "one 4-byte direct-to-LDS load per block's lse2 and D");
};

// Row r of a lane of half h (see the layout notes above).
__device__ __forceinline__ int acc_row(int r, int h) { return 8 * (r / 4) + 4 * h + (r % 4); }

// ---------------------------------------------------------------- preprocess

template <int D>
__global__ __launch_bounds__(256) void attn_bwd_pre_kernel(BwdArgs a) {
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
    }
    // Sum over the kT aligned lanes of the row.
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

template <int D, bool CAUSAL, bool MASKED>
__global__ __launch_bounds__(256) void attn_bwd_dkdv_f32_kernel(BwdArgs a) {
  using G = BGeom<D>;
  using VecN = typename FVecB<G::kNch>::T;
  // Q tile, dO tile, lse2/D, and with a hard mask the block's 32 mask words (this key block's
  // word of each query row; the upper 32 lanes of the copy repeat them).
  constexpr int kSlotBytes = 2 * G::kTileBytes + G::kMetaBytes + (MASKED ? 256 : 0);
  constexpr int kStageBytes = G::kWaves * kSlotBytes;
  constexpr int kLdsBytes = kStageBytes > 2 * G::kPartBytes ? kStageBytes : 2 * G::kPartBytes;
  static_assert(2 * G::kTileBytes <= kSlotBytes, "K and V prologue tiles fit in wave 0's slot");
  __shared__ __attribute__((aligned(16))) unsigned char lds[kLdsBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lm = lane & 31;
  const int lh = lane >> 5;
  unsigned char* const q_slot = lds + wave * kSlotBytes;
  unsigned char* const g_slot = q_slot + G::kTileBytes;
  unsigned char* const m_slot = g_slot + G::kTileBytes;
  unsigned char* const w_slot = m_slot + G::kMetaBytes;  // mask words (MASKED)

  const uint32_t lam = xcd_remap(blockIdx.x, a.nwg);
  const int64_t bh = (int64_t)(lam / (uint32_t)a.nkb);
  const int32_t j0 = (int32_t)(lam % (uint32_t)a.nkb) * G::kRows;
  const int32_t delta = a.seq_kv - a.seq_q;
  // Query blocks holding a row that admits some key of this block: row i
  // admits key j0 iff i >= j0 - delta.
  int32_t qb_first = 0;
  if (CAUSAL) {
    const int32_t i_min = j0 - delta;
    qb_first = i_min <= 0 ? 0 : i_min / G::kRows;
  }
  const int32_t nq = a.nqb - qb_first;
  const int32_t b_begin = qb_first + (int32_t)(((int64_t)nq * wave) / G::kWaves);
  const int32_t b_end = qb_first + (int32_t)(((int64_t)nq * (wave + 1)) / G::kWaves);

  // Rows past the end of each array lie outside these ranges and read as zeros. Rows
  // are q_row / kv_row bytes apart (the layout's row strides).
  const int64_t q_off = head_offset(bh, a.heads, a.qs_b, a.qs_h);
  const int64_t kv_off = head_offset(bh, a.heads, a.kvs_b, a.kvs_h);
  const unsigned q_row = (unsigned)(a.qs_s * 4), kv_row = (unsigned)(a.kvs_s * 4);
  const unsigned q_range = strided_range(a.seq_q, a.qs_s, D, 4);
  const unsigned kv_range = strided_range(a.seq_kv, a.kvs_s, D, 4);
  const __amdgpu_buffer_rsrc_t q_rsrc = raw_buffer(a.q + q_off, q_range);
  const __amdgpu_buffer_rsrc_t g_rsrc = raw_buffer(a.dout + q_off, q_range);
  const __amdgpu_buffer_rsrc_t m_rsrc =
      raw_buffer(a.meta + (size_t)bh * a.nqb * kBwdMetaFloats, (unsigned)a.nqb * (unsigned)G::kMetaBytes);
  const __amdgpu_buffer_rsrc_t k_rsrc = raw_buffer(a.k + kv_off, kv_range);
  const __amdgpu_buffer_rsrc_t v_rsrc = raw_buffer(a.v + kv_off, kv_range);
  __amdgpu_buffer_rsrc_t w_rsrc;  // rows past seq_q read as 0: nothing admitted
  if (MASKED)
    w_rsrc = raw_buffer(a.mask_bits + head_offset(bh, a.heads, a.mbits_sb, a.mbits_sh),
                        (unsigned)a.seq_q * (unsigned)a.mask_words * 4u);

  auto copy_q = [&](int32_t qb) {
    const unsigned row0 = (unsigned)(G::kRows * qb) * q_row;
#pragma unroll
    for (int t = 0; t < G::kDmaPerTile; ++t)
      dma_load_x4(q_rsrc, row0 + tile_src_offset<D>(t, lane, q_row), lds_address(q_slot + 1024 * t));
  };
  auto copy_g = [&](int32_t qb) {  // dO tile, then the block's lse2 and D
    const unsigned row0 = (unsigned)(G::kRows * qb) * q_row;
#pragma unroll
    for (int t = 0; t < G::kDmaPerTile; ++t)
      dma_load_x4(g_rsrc, row0 + tile_src_offset<D>(t, lane, q_row), lds_address(g_slot + 1024 * t));
    dma_load_x1(m_rsrc, (unsigned)qb * (unsigned)G::kMetaBytes + 4u * lane, lds_address(m_slot));
    if (MASKED)
      dma_load_x1(w_rsrc, ((unsigned)(G::kRows * qb + (lane & 31)) * (unsigned)a.mask_words +
                           (unsigned)(j0 / G::kRows)) * 4u, lds_address(w_slot));
  };

  // This block's K and V tiles, staged through wave 0's slot (each wave copies
  // a quarter), into the B operands of S and dP.
  {
    unsigned char* const k_tile = lds;
    unsigned char* const v_tile = lds + G::kTileBytes;
    const unsigned row0 = (unsigned)j0 * kv_row;
#pragma unroll
    for (int i = 0; i < G::kDmaPerTile / G::kWaves; ++i) {
      const int t = i * G::kWaves + wave;
      dma_load_x4(k_rsrc, row0 + tile_src_offset<D>(t, lane, kv_row), lds_address(k_tile + 1024 * t));
      dma_load_x4(v_rsrc, row0 + tile_src_offset<D>(t, lane, kv_row), lds_address(v_tile + 1024 * t));
    }
    wait_vmcnt<0>();
    __syncthreads();
  }
  float kr[4 * G::kSteps], vr[4 * G::kSteps];  // group u, element e: head dim 8u + 4*lh + e of key lm
#pragma unroll
  for (int u = 0; u < G::kSteps; ++u) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(lds + tile_operand_offset<D>(lm, lh, u));
    const f32x4 y =
        *reinterpret_cast<const f32x4*>(lds + G::kTileBytes + tile_operand_offset<D>(lm, lh, u));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      kr[4 * u + e] = x[e];
      vr[4 * u + e] = y[e];
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the operand reads have returned
  __syncthreads();                     // before wave 0 reuses its slot

  f32x16 dv[G::kNch], dk[G::kNch];
#pragma unroll
  for (int cb = 0; cb < G::kNch; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) dv[cb][r] = dk[cb][r] = 0.f;

  if (b_begin < b_end) {
    copy_g(b_begin);
    copy_q(b_begin);
  }
  for (int32_t qb = b_begin; qb < b_end; ++qb) {
    const int32_t i0 = G::kRows * qb;
    // The dO tile and lse2/D of block qb have landed (its Q tile, issued after
    // them, may still be in flight).
    wait_vmcnt<G::kDmaPerTile>();
    f32x4 l2[4], dd[4];  // lse2 and D of rows i0 + 8*rq + 4*lh + 0..3
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      l2[rq] = *reinterpret_cast<const f32x4*>(m_slot + 4 * (8 * rq + 4 * lh));
      dd[rq] = *reinterpret_cast<const f32x4*>(m_slot + 4 * (G::kRows + 8 * rq + 4 * lh));
    }
    f32x16 dp;
#pragma unroll
    for (int r = 0; r < 16; ++r) dp[r] = 0.f;
#pragma unroll
    for (int u = 0; u < G::kSteps; ++u) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(g_slot + tile_operand_offset<D>(lm, lh, u));
#pragma unroll
      for (int e = 0; e < 4; ++e) dp = __builtin_amdgcn_mfma_f32_32x32x2f32(x[e], vr[4 * u + e], dp, 0, 0, 0);
    }
    wait_vmcnt<0>();  // the Q tile
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int u = 0; u < G::kSteps; ++u) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(q_slot + tile_operand_offset<D>(lm, lh, u));
#pragma unroll
      for (int e = 0; e < 4; ++e) s = __builtin_amdgcn_mfma_f32_32x32x2f32(x[e], kr[4 * u + e], s, 0, 0, 0);
    }
    // Some pair of this block is masked iff its last key lies past its first row's limit.
    const bool diag = CAUSAL && (j0 + G::kRows - 1 > i0 + delta);
    uint32_t mw[16];  // mask word of query row acc_row(r, lh); bit lm is this lane's key
    if (MASKED) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const u32x4 w4 = *reinterpret_cast<const u32x4*>(w_slot + 4 * (8 * rq + 4 * lh));
#pragma unroll
        for (int e = 0; e < 4; ++e) mw[4 * rq + e] = w4[e];
      }
    }
    float p[16], ds[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float t = s[r] * a.c - l2[r / 4][r % 4];
      if (diag) t = (j0 + lm <= i0 + acc_row(r, lh) + delta) ? t : -INFINITY;
      if (MASKED) t = ((mw[r] >> lm) & 1u) ? t : -INFINITY;
      p[r] = __builtin_amdgcn_exp2f(t);
      ds[r] = p[r] * (dp[r] - dd[r / 4][r % 4]);
    }
    // dV^T += dO^T P
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const VecN x = *reinterpret_cast<const VecN*>(g_slot + tile_row_offset<D>(acc_row(r, lh), lm));
#pragma unroll
      for (int cb = 0; cb < G::kNch; ++cb) dv[cb] = __builtin_amdgcn_mfma_f32_32x32x2f32(x[cb], p[r], dv[cb], 0, 0, 0);
    }
    if (qb + 1 < b_end) {
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): done reading the dO and lse2/D slots
      copy_g(qb + 1);
    }
    // dK^T += Q^T dS (the scale is applied once, at the end)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const VecN x = *reinterpret_cast<const VecN*>(q_slot + tile_row_offset<D>(acc_row(r, lh), lm));
#pragma unroll
      for (int cb = 0; cb < G::kNch; ++cb) dk[cb] = __builtin_amdgcn_mfma_f32_32x32x2f32(x[cb], ds[r], dk[cb], 0, 0, 0);
    }
    if (qb + 1 < b_end) {
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): done reading the Q slot
      copy_q(qb + 1);
    }
  }

  // Partials -> LDS as [wave][key][head dim], then summed over the waves.
  __syncthreads();
  float* const part_v = reinterpret_cast<float*>(lds);
  float* const part_k = part_v + G::kWaves * G::kRows * G::kPStride;
  {
    float* const vrow = part_v + (wave * G::kRows + lm) * G::kPStride;
    float* const krow = part_k + (wave * G::kRows + lm) * G::kPStride;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      VecN xv, xk;
#pragma unroll
      for (int cb = 0; cb < G::kNch; ++cb) {
        xv[cb] = dv[cb][r];
        xk[cb] = dk[cb][r];
      }
      *reinterpret_cast<VecN*>(vrow + G::kNch * acc_row(r, lh)) = xv;
      *reinterpret_cast<VecN*>(krow + G::kNch * acc_row(r, lh)) = xk;
    }
  }
  __syncthreads();
  constexpr int kThreadsPerRow = D / 4;
  constexpr int kRowsPerPass = 256 / kThreadsPerRow;
#pragma unroll
  for (int pass = 0; pass < G::kRows / kRowsPerPass; ++pass) {
    const int key = pass * kRowsPerPass + tid / kThreadsPerRow;
    const int c4 = tid % kThreadsPerRow;
    const int32_t j = j0 + key;
    f32x4 sv = {0.f, 0.f, 0.f, 0.f}, sk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < G::kWaves; ++w) {
      sv += *reinterpret_cast<const f32x4*>(part_v + (w * G::kRows + key) * G::kPStride + 4 * c4);
      sk += *reinterpret_cast<const f32x4*>(part_k + (w * G::kRows + key) * G::kPStride + 4 * c4);
    }
    if (j >= a.seq_kv) continue;
    const int64_t off = kv_off + (int64_t)j * a.kvs_s + 4 * c4;
    *reinterpret_cast<f32x4*>(a.dv + off) = sv;
    *reinterpret_cast<f32x4*>(a.dk + off) = sk * a.scale;
  }
}

// ---------------------------------------------------------------- dQ

template <int D, bool CAUSAL, bool MASKED>
__global__ __launch_bounds__(256) void attn_bwd_dq_f32_kernel(BwdArgs a) {
  using G = BGeom<D>;
  using VecN = typename FVecB<G::kNch>::T;
  // K tile, V tile, and with a hard mask each query row's word of the key block.
  constexpr int kSlotBytes = 2 * G::kTileBytes + (MASKED ? 256 : 0);
  constexpr int kStageBytes = G::kWaves * kSlotBytes;
  constexpr int kLdsBytes = kStageBytes > G::kPartBytes ? kStageBytes : G::kPartBytes;
  __shared__ __attribute__((aligned(16))) unsigned char lds[kLdsBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lm = lane & 31;
  const int lh = lane >> 5;
  unsigned char* const k_slot = lds + wave * kSlotBytes;
  unsigned char* const v_slot = k_slot + G::kTileBytes;
  unsigned char* const w_slot = v_slot + G::kTileBytes;  // mask words (MASKED)

  // Workgroup -> (batch*head, query block), the longest causal blocks first.
  const uint32_t lam = xcd_remap(blockIdx.x, a.nwg);
  const int64_t bh = (int64_t)(lam / (uint32_t)a.nqb);
  const int32_t qb = a.nqb - 1 - (int32_t)(lam % (uint32_t)a.nqb);
  const int32_t q0 = qb * G::kRows;

  const int32_t my_row = q0 + lm;
  const int32_t last_row = min(q0 + G::kRows - 1, a.seq_q - 1);
  const int32_t lim = key_limit<CAUSAL>(my_row, a.seq_q, a.seq_kv, a.seq_kv);
  const int32_t lo = key_limit<CAUSAL>(q0, a.seq_q, a.seq_kv, a.seq_kv);
  const int32_t hi = key_limit<CAUSAL>(last_row, a.seq_q, a.seq_kv, a.seq_kv);
  const int32_t nblocks = (hi + G::kRows - 1) / G::kRows;
  const int32_t b_begin = (int32_t)(((int64_t)nblocks * wave) / G::kWaves);
  const int32_t b_end = (int32_t)(((int64_t)nblocks * (wave + 1)) / G::kWaves);

  // lse2 and D of this lane's query (the preprocess pads past seq_q).
  const float* const meta = a.meta + ((size_t)bh * a.nqb + qb) * kBwdMetaFloats;
  const float my_l2 = meta[lm];
  const float my_d = meta[G::kRows + lm];

  const int64_t q_off = head_offset(bh, a.heads, a.qs_b, a.qs_h);
  const int64_t kv_off = head_offset(bh, a.heads, a.kvs_b, a.kvs_h);
  const unsigned q_row = (unsigned)(a.qs_s * 4), kv_row = (unsigned)(a.kvs_s * 4);
  const unsigned q_range = strided_range(a.seq_q, a.qs_s, D, 4);
  const unsigned kv_range = strided_range(a.seq_kv, a.kvs_s, D, 4);
  const __amdgpu_buffer_rsrc_t q_rsrc = raw_buffer(a.q + q_off, q_range);
  const __amdgpu_buffer_rsrc_t g_rsrc = raw_buffer(a.dout + q_off, q_range);
  const __amdgpu_buffer_rsrc_t k_rsrc = raw_buffer(a.k + kv_off, kv_range);
  const __amdgpu_buffer_rsrc_t v_rsrc = raw_buffer(a.v + kv_off, kv_range);
  __amdgpu_buffer_rsrc_t w_rsrc;  // rows past seq_q read as 0: nothing admitted
  if (MASKED)
    w_rsrc = raw_buffer(a.mask_bits + head_offset(bh, a.heads, a.mbits_sb, a.mbits_sh),
                        (unsigned)a.seq_q * (unsigned)a.mask_words * 4u);
  auto copy_k = [&](int32_t b) {  // K tile, then the rows' mask words of block b
    const unsigned row0 = (unsigned)(G::kRows * b) * kv_row;
#pragma unroll
    for (int t = 0; t < G::kDmaPerTile; ++t)
      dma_load_x4(k_rsrc, row0 + tile_src_offset<D>(t, lane, kv_row), lds_address(k_slot + 1024 * t));
    if (MASKED)
      dma_load_x1(w_rsrc, ((unsigned)(q0 + (lane & 31)) * (unsigned)a.mask_words + (unsigned)b) * 4u,
                  lds_address(w_slot));
  };
  auto copy_v = [&](int32_t b) {
    const unsigned row0 = (unsigned)(G::kRows * b) * kv_row;
#pragma unroll
    for (int t = 0; t < G::kDmaPerTile; ++t)
      dma_load_x4(v_rsrc, row0 + tile_src_offset<D>(t, lane, kv_row), lds_address(v_slot + 1024 * t));
  };

  // The Q and dO tiles of this block, staged through wave 0's slot, into the
  // B operands of S^T and dP^T.
  {
    const unsigned row0 = (unsigned)q0 * q_row;
#pragma unroll
    for (int i = 0; i < G::kDmaPerTile / G::kWaves; ++i) {
      const int t = i * G::kWaves + wave;
      dma_load_x4(q_rsrc, row0 + tile_src_offset<D>(t, lane, q_row), lds_address(lds + 1024 * t));
      dma_load_x4(g_rsrc, row0 + tile_src_offset<D>(t, lane, q_row),
                  lds_address(lds + G::kTileBytes + 1024 * t));
    }
    wait_vmcnt<0>();
    __syncthreads();
  }
  float qr[4 * G::kSteps], gr[4 * G::kSteps];  // head dim 8u + 4*lh + e of query lm
#pragma unroll
  for (int u = 0; u < G::kSteps; ++u) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(lds + tile_operand_offset<D>(lm, lh, u));
    const f32x4 y =
        *reinterpret_cast<const f32x4*>(lds + G::kTileBytes + tile_operand_offset<D>(lm, lh, u));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qr[4 * u + e] = x[e];
      gr[4 * u + e] = y[e];
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __syncthreads();                     // before wave 0 reuses its slot

  f32x16 dq[G::kNch];
#pragma unroll
  for (int cb = 0; cb < G::kNch; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[cb][r] = 0.f;

  if (b_begin < b_end) {
    copy_v(b_begin);
    copy_k(b_begin);
  }
  for (int32_t b = b_begin; b < b_end; ++b) {
    const int32_t j0 = G::kRows * b;
    wait_vmcnt<G::kDmaPerTile>();  // V block b (K block b may still be in flight)
    f32x16 dp;
#pragma unroll
    for (int r = 0; r < 16; ++r) dp[r] = 0.f;
#pragma unroll
    for (int u = 0; u < G::kSteps; ++u) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(v_slot + tile_operand_offset<D>(lm, lh, u));
#pragma unroll
      for (int e = 0; e < 4; ++e) dp = __builtin_amdgcn_mfma_f32_32x32x2f32(x[e], gr[4 * u + e], dp, 0, 0, 0);
    }
    if (b + 1 < b_end) {
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): done reading the V slot
      copy_v(b + 1);
      wait_vmcnt<G::kDmaPerTile>();        // K block b (V block b+1 may still be in flight)
    } else {
      wait_vmcnt<0>();
    }
    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int u = 0; u < G::kSteps; ++u) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(k_slot + tile_operand_offset<D>(lm, lh, u));
#pragma unroll
      for (int e = 0; e < 4; ++e) s = __builtin_amdgcn_mfma_f32_32x32x2f32(x[e], qr[4 * u + e], s, 0, 0, 0);
    }
    const bool edge = j0 + G::kRows > lo;  // some key of the block lies past the first row's limit
    const uint32_t mw = MASKED ? *reinterpret_cast<const uint32_t*>(w_slot + 4 * lm) : ~0u;
    float ds[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float t = s[r] * a.c - my_l2;
      if (edge) t = (j0 + acc_row(r, lh) < lim) ? t : -INFINITY;
      if (MASKED) t = ((mw >> acc_row(r, lh)) & 1u) ? t : -INFINITY;
      const float p = __builtin_amdgcn_exp2f(t);
      ds[r] = p * (dp[r] - my_d);
    }
    // dQ^T += K^T dS^T
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const VecN x = *reinterpret_cast<const VecN*>(k_slot + tile_row_offset<D>(acc_row(r, lh), lm));
#pragma unroll
      for (int cb = 0; cb < G::kNch; ++cb) dq[cb] = __builtin_amdgcn_mfma_f32_32x32x2f32(x[cb], ds[r], dq[cb], 0, 0, 0);
    }
    if (b + 1 < b_end) {
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): done reading the K slot
      copy_k(b + 1);
    }
  }

  __syncthreads();
  float* const part = reinterpret_cast<float*>(lds);
  {
    float* const row = part + (wave * G::kRows + lm) * G::kPStride;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      VecN x;
#pragma unroll
      for (int cb = 0; cb < G::kNch; ++cb) x[cb] = dq[cb][r];
      *reinterpret_cast<VecN*>(row + G::kNch * acc_row(r, lh)) = x;
    }
  }
  __syncthreads();
  constexpr int kThreadsPerRow = D / 4;
  constexpr int kRowsPerPass = 256 / kThreadsPerRow;
#pragma unroll
  for (int pass = 0; pass < G::kRows / kRowsPerPass; ++pass) {
    const int qi = pass * kRowsPerPass + tid / kThreadsPerRow;
    const int c4 = tid % kThreadsPerRow;
    const int32_t row = q0 + qi;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < G::kWaves; ++w)
      acc += *reinterpret_cast<const f32x4*>(part + (w * G::kRows + qi) * G::kPStride + 4 * c4);
    if (row >= a.seq_q) continue;
    *reinterpret_cast<f32x4*>(a.dq + q_off + (int64_t)row * a.qs_s + 4 * c4) = acc * a.scale;
  }
}

template <int D, bool CAUSAL, bool MASKED>
hipError_t launch_bwd_variant(const BwdArgs& a0, hipStream_t s, hipEvent_t ev_pre,
                              hipEvent_t ev_dkdv) {
  BwdArgs a = a0;
  const uint32_t nq = (uint32_t)(a.bh * a.nqb), nk = (uint32_t)(a.bh * a.nkb);
  if (nq > 0) {
    hipLaunchKernelGGL((attn_bwd_pre_kernel<D>), dim3(nq), dim3(256), 0, s, a);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  }
  if (ev_pre && hipEventRecord(ev_pre, s) != hipSuccess) return hipErrorInvalidValue;
  if (nk > 0) {
    a.nwg = nk;
    hipLaunchKernelGGL((attn_bwd_dkdv_f32_kernel<D, CAUSAL, MASKED>), dim3(nk), dim3(256), 0, s, a);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  }
  if (ev_dkdv && hipEventRecord(ev_dkdv, s) != hipSuccess) return hipErrorInvalidValue;
  if (nq > 0) {
    a.nwg = nq;
    hipLaunchKernelGGL((attn_bwd_dq_f32_kernel<D, CAUSAL, MASKED>), dim3(nq), dim3(256), 0, s, a);
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  }
  return hipSuccess;
}

template <int D>
hipError_t launch_bwd_d(const BwdArgs& a, bool causal, hipStream_t s, hipEvent_t ev_pre,
                        hipEvent_t ev_dkdv) {
  if (a.mask_bits)
    return causal ? launch_bwd_variant<D, true, true>(a, s, ev_pre, ev_dkdv)
                  : launch_bwd_variant<D, false, true>(a, s, ev_pre, ev_dkdv);
  return causal ? launch_bwd_variant<D, true, false>(a, s, ev_pre, ev_dkdv)
                : launch_bwd_variant<D, false, false>(a, s, ev_pre, ev_dkdv);
}

}  // namespace

hipError_t launch_bwd_f32(const BwdArgs& a, int head_dim, bool causal, hipStream_t s,
                          hipEvent_t ev_pre, hipEvent_t ev_dkdv) {
  if (head_dim == 32) return launch_bwd_d<32>(a, causal, s, ev_pre, ev_dkdv);
  if (head_dim == 64) return launch_bwd_d<64>(a, causal, s, ev_pre, ev_dkdv);
  if (head_dim == 128) return launch_bwd_d<128>(a, causal, s, ev_pre, ev_dkdv);
  return hipErrorInvalidValue;
}

}  // namespace sma
