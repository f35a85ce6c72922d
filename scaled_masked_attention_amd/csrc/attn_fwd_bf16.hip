// Attention forward, bf16 inputs, bf16 MFMA with fp32 accumulation
// (v_mfma_f32_32x32x16_bf16), fp32 output, gfx950.
//
// Same method as the fp32 kernel (oxicuda ComputeBackend `attention`; pulsatrix
// HIPBackend `softmax_rows`, `logsumexp_rows`; TorchLean hard-masked softmax),
// with the operand precision of the oxicuda `gemm_mixed_precision` contract:
// 16-bit operands, fp32 accumulation and result. The probabilities are
// rounded to bf16 (nearest even) for the P V product; the row sums use the
// fp32 probabilities.
//
// Workgroup: 8 waves x 32 query rows = 256 rows, two waves per SIMD, so that
// one wave's softmax (VALU, transcendental) runs while the other's MFMAs
// issue. Key tiles of 64 rows are staged HBM/L2 -> registers -> LDS, double
// buffered: waves 0-3 stage K row-major, waves 4-7 stage V transposed
// (V^T[dim][key]), so both MFMA operands are plain 16-byte LDS reads.
//
// S^T = K Q^T: lane (m, h) supplies K[key m] and Q[query m] at head dims
// h*D/2 + 8*step .. + 7 and receives the scores of query (lane % 32). K rows
// are stored with bits 2 and 3 of the row index swapped, which makes
// accumulator register r hold key 16*(r/8) + 8*h + r%8: registers 8t..8t+7
// are the eight keys this lane supplies to k-step t of O^T += V^T P^T.
#include "attn_common.h"

namespace sma {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

template <int D>
struct BGeom {
  static constexpr int kThreads = 512;
  static constexpr int kWaves = 8;
  static constexpr int kQW = 32;                       // query rows per wave
  static constexpr int kQ = kWaves * kQW;              // query rows per workgroup
  static constexpr int kK = kBF16KeysPerTile;          // keys per LDS tile
  static constexpr int kKB = kK / 32;                  // 32-key sub-blocks per tile
  static constexpr int kKStride = D + 8;               // K row in LDS (bf16), 16 B pad
  static constexpr int kVtStride = kK + 8;             // V^T row (one head dim) in LDS, 16 B pad
  static constexpr int kHalf = D / 2;
  static constexpr int kSteps = D / 16;                // QK^T k-steps (8 dims per lane half)
  static constexpr int kNch = D / 32;                  // 32-wide output chunks
  static constexpr int kStagers = kThreads / 2;        // threads staging K (and as many for V)
  static constexpr int kKChunks = kK * D / 8 / kStagers;         // 16-byte K chunks per thread
  static constexpr int kVPatches = (kK / 4) * (D / 8);  // 4-key x 8-dim V patches, one per thread
  static_assert(kQ == kBF16QueriesPerWG, "planner geometry");
  static_assert(kKChunks * 8 * kStagers == kK * D, "K tile split");
  static_assert(kVPatches <= kStagers && kKChunks <= 4, "staging split");
};

constexpr float kTau = 8.0f;  // lazy running-max threshold, log2 units (see the fp32 kernel)

__device__ __forceinline__ int swap_bits_2_3(int r) {
  return (r & ~0xC) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// Low (sel = 0) or high (sel = 1) bf16 of two dwords packed into one dword: {a.sel, b.sel}.
__device__ __forceinline__ unsigned pack_lo(unsigned a, unsigned b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ unsigned pack_hi(unsigned a, unsigned b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(512) void attn_fwd_bf16_kernel(FwdArgs a) {
  using G = BGeom<D>;
  __shared__ __attribute__((aligned(16))) unsigned short k_lds[2][G::kK * G::kKStride];
  __shared__ __attribute__((aligned(16))) unsigned short vt_lds[2][D * G::kVtStride];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lm = lane & 31;
  const int lh = lane >> 5;

  const TileId t = decode_tile(blockIdx.x, a);
  const int32_t q0 = t.qb * G::kQ;
  const int32_t qw0 = q0 + wave * G::kQW;
  const int32_t ks = t.split * a.split_len;
  const int32_t split_end = min(a.seq_kv, ks + a.split_len);
  const int32_t wg_last_row = min(q0 + G::kQ - 1, a.seq_q - 1);
  const int32_t ke = key_limit<CAUSAL>(wg_last_row, a.seq_q, a.seq_kv, split_end);
  const int32_t ntiles = ke > ks ? (ke - ks + G::kK - 1) / G::kK : 0;

  const bool wave_live = qw0 < a.seq_q;
  const int32_t wave_lo = key_limit<CAUSAL>(qw0, a.seq_q, a.seq_kv, split_end);
  const int32_t wave_hi = key_limit<CAUSAL>(min(qw0 + G::kQW - 1, a.seq_q - 1), a.seq_q,
                                            a.seq_kv, split_end);
  const int32_t my_row = qw0 + lm;
  const int32_t lim = key_limit<CAUSAL>(my_row, a.seq_q, a.seq_kv, split_end);

  // Q operands in registers for the whole pass.
  bf16x8 qr[G::kSteps];
  {
    const unsigned short* qp = static_cast<const unsigned short*>(a.q) +
                               ((size_t)t.bh * a.seq_q + min(my_row, a.seq_q - 1)) * D + lh * G::kHalf;
    const unsigned flip = a.negate_q ? 0x80008000u : 0u;
#pragma unroll
    for (int s = 0; s < G::kSteps; ++s) {
      u32x4 x = *reinterpret_cast<const u32x4*>(qp + 8 * s);
      x ^= flip;
      qr[s] = __builtin_bit_cast(bf16x8, x);
    }
  }

  const unsigned short* kg = static_cast<const unsigned short*>(a.k) + (size_t)t.bh * a.seq_kv * D;
  const unsigned short* vg = static_cast<const unsigned short*>(a.v) + (size_t)t.bh * a.seq_kv * D;
  const bool k_stager = tid < G::kStagers;
  const int st = k_stager ? tid : tid - G::kStagers;
  const bool v_stager = !k_stager && st < G::kVPatches;
  u32x4 sreg[4];  // staged chunks: K (kKChunks of them) or the 4 key rows of a V patch

  auto load_tile = [&](int32_t tile) {
    const int32_t j0 = ks + tile * G::kK;
    if (k_stager) {
#pragma unroll
      for (int u = 0; u < G::kKChunks; ++u) {
        const int f = st + G::kStagers * u;
        const int row = f / (D / 8), c8 = f % (D / 8);
        const int32_t j = j0 + row;
        sreg[u] = j < a.seq_kv ? *reinterpret_cast<const u32x4*>(kg + (size_t)j * D + 8 * c8)
                               : u32x4{0u, 0u, 0u, 0u};
      }
    } else if (v_stager) {
      // patch: keys 4*kgp .. 4*kgp+3, head dims 8*cg .. 8*cg+7
      const int kgp = st % (G::kK / 4), cg = st / (G::kK / 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int32_t j = j0 + 4 * kgp + r;
        sreg[r] = j < a.seq_kv ? *reinterpret_cast<const u32x4*>(vg + (size_t)j * D + 8 * cg)
                               : u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_tile = [&](int buf) {
    if (k_stager) {
#pragma unroll
      for (int u = 0; u < G::kKChunks; ++u) {
        const int f = st + G::kStagers * u;
        const int row = f / (D / 8), c8 = f % (D / 8);
        const int krow = (row & ~31) | swap_bits_2_3(row & 31);
        *reinterpret_cast<u32x4*>(&k_lds[buf][krow * G::kKStride + 8 * c8]) = sreg[u];
      }
    } else if (v_stager) {
      const int kgp = st % (G::kK / 4), cg = st / (G::kK / 4);
      // sreg[r] holds dims 8cg..8cg+7 of key 4kgp+r as 4 dwords (2 dims each).
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const u32x2 even = {pack_lo(sreg[0][w], sreg[1][w]), pack_lo(sreg[2][w], sreg[3][w])};
        const u32x2 odd = {pack_hi(sreg[0][w], sreg[1][w]), pack_hi(sreg[2][w], sreg[3][w])};
        *reinterpret_cast<u32x2*>(&vt_lds[buf][(8 * cg + 2 * w) * G::kVtStride + 4 * kgp]) = even;
        *reinterpret_cast<u32x2*>(&vt_lds[buf][(8 * cg + 2 * w + 1) * G::kVtStride + 4 * kgp]) = odd;
      }
    }
  };

  f32x16 oacc[G::kNch];
#pragma unroll
  for (int cb = 0; cb < G::kNch; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[cb][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float c = a.c;

  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int32_t it = 0; it < ntiles; ++it) {
    const int buf = it & 1;
    if (it + 1 < ntiles) load_tile(it + 1);
    const int32_t j0 = ks + it * G::kK;
    if (wave_live && j0 < wave_hi) {
      f32x16 sacc[G::kKB];
#pragma unroll
      for (int kb = 0; kb < G::kKB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
        const unsigned short* krow = &k_lds[buf][(32 * kb + lm) * G::kKStride + lh * G::kHalf];
#pragma unroll
        for (int s = 0; s < G::kSteps; ++s) {
          const bf16x8 kop = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(krow + 8 * s));
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qr[s], sacc[kb], 0, 0, 0);
        }
      }

      // Row max of the raw scores (scale > 0 after the sign fold), masked keys excluded.
      const bool need_mask = j0 + G::kK > wave_lo;
      float mx = -INFINITY;
      if (need_mask) {
        const int32_t rel = lim - j0 - 8 * lh;  // key 32kb + 16(r/8) + r%8 allowed iff < rel
#pragma unroll
        for (int kb = 0; kb < G::kKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (32 * kb + 16 * (r / 8) + (r % 8) < rel) mx = fmaxf(mx, sacc[kb][r]);
      } else {
#pragma unroll
        for (int kb = 0; kb < G::kKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float tmax = mx == -INFINITY ? -INFINITY : mx * c;
      if (__any(tmax > m_run + kTau)) {
        const float m_new = fmaxf(m_run, tmax);
        const float alpha = __builtin_amdgcn_exp2f(m_run - (m_new == -INFINITY ? 0.f : m_new));
        l_run *= alpha;
#pragma unroll
        for (int cb = 0; cb < G::kNch; ++cb)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[cb][r] *= alpha;
        m_run = m_new;
      }
      const float neg_m = m_run == -INFINITY ? 0.f : -m_run;

      // p = 2^(s*c - m), rounded to bf16 for the PV product.
      bf16x8 pb[G::kKB][2];
      float psum = 0.f;
      if (need_mask) {
        const int32_t rel = lim - j0 - 8 * lh;
#pragma unroll
        for (int kb = 0; kb < G::kKB; ++kb)
#pragma unroll
          for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int key = 32 * kb + 16 * t2 + e;
              float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][8 * t2 + e], c, neg_m));
              p = key < rel ? p : 0.f;
              psum += p;
              pb[kb][t2][e] = (__bf16)p;
            }
      } else {
#pragma unroll
        for (int kb = 0; kb < G::kKB; ++kb)
#pragma unroll
          for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][8 * t2 + e], c, neg_m));
              psum += p;
              pb[kb][t2][e] = (__bf16)p;
            }
      }
      l_run += psum;

      // O^T += V^T P^T over the tile's 64 keys in k-steps of 16.
#pragma unroll
      for (int kb = 0; kb < G::kKB; ++kb)
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          const unsigned short* vp = &vt_lds[buf][lm * G::kVtStride + 32 * kb + 16 * t2 + 8 * lh];
#pragma unroll
          for (int cb = 0; cb < G::kNch; ++cb) {
            const bf16x8 aop =
                __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(vp + 32 * cb * G::kVtStride));
            oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, pb[kb][t2], oacc[cb], 0, 0, 0);
          }
        }
    }
    if (it + 1 < ntiles) store_tile((it + 1) & 1);
    __syncthreads();
  }

  // Epilogue (the cross-lane sum first, while all lanes run).
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!wave_live || my_row >= a.seq_q) return;
  const bool empty = !(l_tot > 0.f);
  const float inv = empty ? 0.f : 1.0f / l_tot;
  const float lse2 = empty ? -INFINITY : m_run + __builtin_amdgcn_logf(l_tot);
  const size_t row_id = (size_t)t.bh * a.seq_q + my_row;
  float* orow;
  if (a.nsplit == 1) {
    orow = a.o + row_id * D;
    if (a.lse && lh == 0) a.lse[row_id] = empty ? -INFINITY : lse2 * 0.69314718055994530942f;
  } else {
    const size_t prow = (size_t)t.split * ((size_t)a.bh * a.seq_q) + row_id;
    orow = a.part_o + prow * D;
    if (lh == 0) a.part_lse[prow] = lse2;
  }
#pragma unroll
  for (int cb = 0; cb < G::kNch; ++cb)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      f32x4 out;
#pragma unroll
      for (int e = 0; e < 4; ++e) out[e] = empty ? 0.f : oacc[cb][4 * g4 + e] * inv;
      *reinterpret_cast<f32x4*>(orow + 32 * cb + 8 * g4 + 4 * lh) = out;
    }
}

template <int D, bool CAUSAL>
hipError_t launch_bf16_variant(const FwdArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, CAUSAL>), dim3(a.nwg), dim3(BGeom<D>::kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, int head_dim, bool causal, hipStream_t s) {
  if (head_dim == 64) return causal ? launch_bf16_variant<64, true>(a, s) : launch_bf16_variant<64, false>(a, s);
  if (head_dim == 128) return causal ? launch_bf16_variant<128, true>(a, s) : launch_bf16_variant<128, false>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace sma
