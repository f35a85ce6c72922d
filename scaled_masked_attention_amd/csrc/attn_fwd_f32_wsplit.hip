// Attention forward, fp32 inputs: the default fp32 kernel whenever its
// 32-row grid fills the GPU (or rows are short). Same method and conventions
// as attn_fwd_f32.hip (oxicuda ComputeBackend `attention`;
// pulsatrix HIPBackend `softmax_rows`, `logsumexp_rows`; TorchLean hard-masked
// softmax).
//
// Workgroup: 32 query rows of one (batch, head) and 4 waves that split the
// keys the rows admit into four contiguous ranges of 32-key blocks. At the end
// the four partial results (running max m_w, denominator l_w and unnormalised
// output O_w, all relative to m_w) are merged through LDS:
//   M = max_w m_w,  L = sum_w 2^(m_w - M) l_w,  O = sum_w 2^(m_w - M) O_w / L,
// the log-sum-exp identity of the split-combine kernel, so no workspace and
// no second launch are needed.
//
// Data movement. The Q tile is copied once per workgroup into LDS, and each
// wave streams its K and V blocks into private LDS slots, all with coalesced
// direct-to-LDS loads (1 KB of consecutive rows per instruction); the MFMA
// operands are read back from LDS. Block b+1's K copy is in flight during
// block b's scores and softmax, its V copy during block b+1's scores; the
// first V copy overlaps the first block's scores.
//
// MFMA layouts (v_mfma_f32_32x32x2f32, lane = 32*h + m):
//   S^T = K Q^T: step (u, e) multiplies head dims 8u + 4h + e of key m (A) and
//     query m (B); lane (m, h) then holds the scores of query m for keys
//     8*(r/4) + 4*h + r%4, r = 0..15.
//   O^T += V^T P^T: step r pairs lane (m, h) with key 8*(r/4) + 4*h + r%4;
//     the A operand is V at head dims (D/32)*m + chunk.
#include "attn_common.h"

namespace sma {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// D/32 consecutive floats: a lane's share of one output row, or of one V row.
template <int N>
struct FVecW {
  typedef float T __attribute__((ext_vector_type(N)));
};

constexpr float kTauW = 8.0f;  // lazy running-max threshold, log2 units

template <int D>
struct WGeom {
  static constexpr int kWaves = 4;
  static constexpr int kQ = kF32WsplitQueriesPerWG;  // query rows per workgroup
  static constexpr int kNch = D / 32;                // O^T chunks per lane
  static constexpr int kSteps = D / 8;               // S^T MFMA groups of 4 (head dims 8u..8u+7)
  static constexpr int kRowBytes = 4 * D;
  static constexpr int kTileBytes = 32 * kRowBytes;  // one 32-row tile of Q or K
  static constexpr int kDmaPerTile = kTileBytes / 1024;
  static constexpr int kOStride = D + 4;             // padded partial-O row in LDS (floats)
  static constexpr int kStageBytes = kTileBytes * (1 + 2 * kWaves);  // Q tile + K and V slots per wave
  static constexpr int kOPartBytes = kWaves * kQ * kOStride * 4;
  static constexpr int kLdsBytes = kStageBytes > kOPartBytes ? kStageBytes : kOPartBytes;
  static_assert(kQ == 32, "one 32x32 MFMA tile of queries");
  static_assert(kDmaPerTile % kWaves == 0, "the Q tile copy splits evenly over the waves");
};

template <int D, bool CAUSAL, bool MASKED>
__global__ __launch_bounds__(256) void attn_fwd_f32_wsplit_kernel(FwdArgs a) {
  using G = WGeom<D>;
  using VecN = typename FVecW<G::kNch>::T;
  // Staging (Q tile, K and V slots) during the key loop; partial O afterwards.
  __shared__ __attribute__((aligned(16))) unsigned char lds[G::kLdsBytes];
  __shared__ float m_part[G::kWaves][G::kQ];
  __shared__ float l_part[G::kWaves][G::kQ];
  // With a hard mask: each wave's copy of its current block's mask words (one
  // per query row; the copy's upper 32 lanes repeat the lower ones).
  __shared__ uint32_t mask_lds[MASKED ? G::kWaves : 1][64];
  constexpr int kMaskOps = MASKED ? 1 : 0;  // loads issued with each K block

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int lm = lane & 31;
  const int lh = lane >> 5;
  unsigned char* const q_tile = lds;
  unsigned char* const k_slot = lds + G::kTileBytes * (1 + wave);
  unsigned char* const v_slot = lds + G::kTileBytes * (1 + G::kWaves + wave);

  // Workgroup -> (batch*head, 32-row query block), XCD-aware order.
  const uint32_t lam = xcd_remap(blockIdx.x, a.nwg);
  const int64_t bh = (int64_t)(lam / (uint32_t)a.nqb);
  const int32_t q0 = (int32_t)(lam % (uint32_t)a.nqb) * G::kQ;

  const int32_t my_row = q0 + lm;
  const int32_t last_row = min(q0 + G::kQ - 1, a.seq_q - 1);
  const int32_t lim = key_limit<CAUSAL>(my_row, a.seq_q, a.seq_kv, a.seq_kv);
  const int32_t lo = key_limit<CAUSAL>(q0, a.seq_q, a.seq_kv, a.seq_kv);        // first row's limit
  const int32_t hi = key_limit<CAUSAL>(last_row, a.seq_q, a.seq_kv, a.seq_kv);  // last row's limit
  const int32_t nblocks = (hi + 31) / 32;
  const int32_t b_begin = (int32_t)(((int64_t)nblocks * wave) / G::kWaves);
  const int32_t b_end = (int32_t)(((int64_t)nblocks * (wave + 1)) / G::kWaves);

  // Rows past the end of Q or K lie outside these ranges and read as zeros.
  // Rows are q_row / kv_row bytes apart (the layout's row strides).
  const unsigned q_row = (unsigned)(a.qs_s * 4), kv_row = (unsigned)(a.kvs_s * 4);
  const __amdgpu_buffer_rsrc_t q_rsrc =
      raw_buffer(static_cast<const float*>(a.q) + head_offset(bh, a.heads, a.qs_b, a.qs_h),
                 strided_range(a.seq_q, a.qs_s, D, 4));
  const int64_t kv_off = head_offset(bh, a.heads, a.kvs_b, a.kvs_h);
  const __amdgpu_buffer_rsrc_t k_rsrc =
      raw_buffer(static_cast<const float*>(a.k) + kv_off, strided_range(a.seq_kv, a.kvs_s, D, 4));
  const __amdgpu_buffer_rsrc_t v_rsrc =
      raw_buffer(static_cast<const float*>(a.v) + kv_off, strided_range(a.seq_kv, a.kvs_s, D, 4));
  // V rows are copied as they are (row-major, unswizzled): the operand reads
  // below take 16 or 8 consecutive bytes per lane along a row.
  auto copy_v_block = [&](int32_t b) {
    const unsigned row0 = (unsigned)(32 * b) * kv_row;
#pragma unroll
    for (int t = 0; t < G::kDmaPerTile; ++t)
      dma_load_x4(v_rsrc, row0 + tile_src_offset_linear<D>(t, lane, kv_row),
                  lds_address(v_slot + 1024 * t));
  };
  __amdgpu_buffer_rsrc_t m_rsrc;
  if (MASKED)
    m_rsrc = raw_buffer(a.mask_bits + head_offset(bh, a.heads, a.mbits_sb, a.mbits_sh),
                        (unsigned)a.seq_q * (unsigned)a.mask_words * 4u);
  auto copy_k_block = [&](int32_t b) {
    const unsigned row0 = (unsigned)(32 * b) * kv_row;
#pragma unroll
    for (int t = 0; t < G::kDmaPerTile; ++t)
      dma_load_x4(k_rsrc, row0 + tile_src_offset<D>(t, lane, kv_row), lds_address(k_slot + 1024 * t));
    if (MASKED)  // word b of rows q0 .. q0 + 31 (rows past seq_q read as 0)
      dma_load_x1(m_rsrc, ((unsigned)(q0 + (lane & 31)) * (unsigned)a.mask_words + (unsigned)b) * 4u,
                  lds_address(&mask_lds[MASKED ? wave : 0][0]));
  };

  // Q tile (the waves copy a quarter each) and this wave's first K and V blocks.
#pragma unroll
  for (int i = 0; i < G::kDmaPerTile / G::kWaves; ++i) {
    const int t = i * G::kWaves + wave;
    dma_load_x4(q_rsrc, (unsigned)q0 * q_row + tile_src_offset<D>(t, lane, q_row),
                lds_address(q_tile + 1024 * t));
  }
  if (b_begin < b_end) {
    copy_k_block(b_begin);
    copy_v_block(b_begin);
    // Q and the first K block (with its mask words); the first V block, not
    // needed before the first block's softmax, stays in flight.
    wait_vmcnt<G::kDmaPerTile>();
  } else {
    wait_vmcnt<0>();
  }
  __syncthreads();

  float qr[4 * G::kSteps];  // group u, element e: head dim 8u + 4*lh + e of query lm
#pragma unroll
  for (int u = 0; u < G::kSteps; ++u) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(q_tile + tile_operand_offset<D>(lm, lh, u));
    qr[4 * u + 0] = x[0];
    qr[4 * u + 1] = x[1];
    qr[4 * u + 2] = x[2];
    qr[4 * u + 3] = x[3];
  }
  if (a.negate_q) {
#pragma unroll
    for (int i = 0; i < 4 * G::kSteps; ++i) qr[i] = -qr[i];
  }

  f32x16 oacc[G::kNch];
#pragma unroll
  for (int cb = 0; cb < G::kNch; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[cb][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  for (int32_t b = b_begin; b < b_end; ++b) {
    const int32_t j0 = 32 * b;
    // K block b (and its mask words) have landed; V block b may still be in
    // flight: it was issued after them, and in-order completion lets the wait
    // leave it outstanding.
    if (b > b_begin) wait_vmcnt<G::kDmaPerTile>();
    f32x4 kk[G::kSteps];
#pragma unroll
    for (int u = 0; u < G::kSteps; ++u)
      kk[u] = *reinterpret_cast<const f32x4*>(k_slot + tile_operand_offset<D>(lm, lh, u));
    const uint32_t mword = MASKED ? mask_lds[MASKED ? wave : 0][lm] : ~0u;
    if (b + 1 < b_end) {
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the K reads have returned
      copy_k_block(b + 1);
    }

    f32x16 s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int u = 0; u < G::kSteps; ++u) {
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(kk[u][0], qr[4 * u + 0], s, 0, 0, 0);
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(kk[u][1], qr[4 * u + 1], s, 0, 0, 0);
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(kk[u][2], qr[4 * u + 2], s, 0, 0, 0);
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(kk[u][3], qr[4 * u + 3], s, 0, 0, 0);
    }
    float tv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) tv[r] = s[r] * a.c;
    if (j0 + 32 > lo) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int32_t j = j0 + 8 * (r / 4) + 4 * lh + (r % 4);
        tv[r] = j < lim ? tv[r] : -INFINITY;
      }
    }
    if (MASKED) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        tv[r] = (mword >> (8 * (r / 4) + 4 * lh + (r % 4))) & 1u ? tv[r] : -INFINITY;
    }
    float mx = tv[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, tv[r]);
    {
      // Lanes m and m + 32 hold the two key halves of query m: after the swap
      // the pair holds (own, partner) on both sides, in the same order.
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                       false, false);
      mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    if (__any(mx > m_run + kTauW)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - (m_new == -INFINITY ? 0.f : m_new));
      l_run *= alpha;
#pragma unroll
      for (int cb = 0; cb < G::kNch; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[cb][r] *= alpha;
      m_run = m_new;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      tv[r] = __builtin_amdgcn_exp2f(tv[r] - m_use);
      psum += tv[r];
    }
    l_run += psum;
    // V block b: wait for its copy (only the K copy of block b+1 may remain
    // in flight), read the operands, then reuse the slot for block b+1.
    if (b + 1 < b_end) wait_vmcnt<G::kDmaPerTile + kMaskOps>();
    else wait_vmcnt<0>();
    VecN vv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 8 * (r / 4) + 4 * lh + (r % 4);
      vv[r] = *reinterpret_cast<const VecN*>(v_slot + key * G::kRowBytes + 4 * G::kNch * lm);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
      for (int cb = 0; cb < G::kNch; ++cb)
        oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv[r][cb], tv[r], oacc[cb], 0, 0, 0);
    if (b + 1 < b_end) {
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the V reads have returned
      copy_v_block(b + 1);
    }
  }

  float l_tot;
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run),
                                                     false, false);
    l_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  // Every wave is done with the staging area before it becomes partial O.
  __syncthreads();
  {
    float* orow = reinterpret_cast<float*>(lds) + (wave * G::kQ + lm) * G::kOStride;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = 8 * (r / 4) + 4 * lh + (r % 4);
      VecN out;
#pragma unroll
      for (int cb = 0; cb < G::kNch; ++cb) out[cb] = oacc[cb][r];
      *reinterpret_cast<VecN*>(orow + G::kNch * m) = out;
    }
    if (lh == 0) {
      m_part[wave][lm] = m_run;
      l_part[wave][lm] = l_tot;
    }
  }
  __syncthreads();

  // Merge: thread -> (query, 4 consecutive head dims). O is written with
  // non-temporal stores: it is not read again by this launch (measured 1.5 %
  // faster on the 512 x 512, d = 64 shape).
  const float* o_part = reinterpret_cast<const float*>(lds);
  constexpr int kThreadsPerRow = D / 4;
  constexpr int kRowsPerPass = 256 / kThreadsPerRow;
#pragma unroll
  for (int pass = 0; pass < G::kQ / kRowsPerPass; ++pass) {
    const int q = pass * kRowsPerPass + tid / kThreadsPerRow;
    const int c4 = tid % kThreadsPerRow;
    const int32_t row = q0 + q;
    float mw[G::kWaves], M = -INFINITY;
#pragma unroll
    for (int w = 0; w < G::kWaves; ++w) {
      mw[w] = m_part[w][q];
      M = fmaxf(M, mw[w]);
    }
    float L = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < G::kWaves; ++w) {
        const float f = __builtin_amdgcn_exp2f(mw[w] - M);  // 0 for a wave with no keys
        L += f * l_part[w][q];
        const f32x4 x =
            *reinterpret_cast<const f32x4*>(o_part + (w * G::kQ + q) * G::kOStride + 4 * c4);
        acc[0] += f * x[0];
        acc[1] += f * x[1];
        acc[2] += f * x[2];
        acc[3] += f * x[3];
      }
    }
    if (row >= a.seq_q) continue;
    const bool empty = !(L > 0.f);
    const float inv = empty ? 0.f : 1.0f / L;
    f32x4 out;
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = empty ? 0.f : acc[e] * inv;
    const size_t row_id = (size_t)bh * a.seq_q + row;
    const int64_t o_off = head_offset(bh, a.heads, a.qs_b, a.qs_h) + (int64_t)row * a.qs_s + 4 * c4;
    if (a.o_bf16) {
      typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
      const u32x2_t packed = {pack_out16(out[0], out[1], a.o_f16), pack_out16(out[2], out[3], a.o_f16)};
      __builtin_nontemporal_store(packed, reinterpret_cast<u32x2_t*>(a.o_bf16 + o_off));
    } else {
      __builtin_nontemporal_store(out, reinterpret_cast<f32x4*>(a.o + o_off));
    }
    if (a.lse && c4 == 0)
      a.lse[row_id] = empty ? -INFINITY : (M + __builtin_amdgcn_logf(L)) * 0.69314718055994530942f;
  }
}

template <int D, bool CAUSAL>
hipError_t launch_wsplit_variant(const FwdArgs& a, hipStream_t s) {
  if (a.mask_bits)
    hipLaunchKernelGGL((attn_fwd_f32_wsplit_kernel<D, CAUSAL, true>), dim3(a.nwg), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((attn_fwd_f32_wsplit_kernel<D, CAUSAL, false>), dim3(a.nwg), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

// Head dims 32, 64 and 128. At 256 a wave's private K and V slots (32 KB
// each) for four waves, plus the Q tile, would take 288 KB of LDS.
hipError_t launch_fwd_f32_wsplit(const FwdArgs& a, int head_dim, bool causal, hipStream_t s) {
  switch (head_dim) {
    case 32: return causal ? launch_wsplit_variant<32, true>(a, s) : launch_wsplit_variant<32, false>(a, s);
    case 64: return causal ? launch_wsplit_variant<64, true>(a, s) : launch_wsplit_variant<64, false>(a, s);
    case 128: return causal ? launch_wsplit_variant<128, true>(a, s) : launch_wsplit_variant<128, false>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sma
