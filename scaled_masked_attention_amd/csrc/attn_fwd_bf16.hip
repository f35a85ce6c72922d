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
// Workgroup: 4 waves x 64 query rows (two 32-row query tiles per wave, so
// every K/V operand read from LDS feeds two MFMAs) = 256 rows; key tiles of
// 64 rows, double buffered in LDS.
//
// S^T = K Q^T: lane (m, h) supplies K[key m] and Q[query m] at head dims
// h*D/2 + 8*step .. + 7 and receives the scores of query (lane % 32). K rows
// are stored in LDS with bits 2 and 3 of the row index swapped, which makes
// accumulator register r hold key 16*(r/8) + 8*h + r%8: registers 8t..8t+7
// are then exactly the eight keys this lane supplies to k-step t of
// O^T += V^T P^T. The V^T operand comes straight from row-major V in LDS
// through the gfx950 transposing read ds_read_b64_tr_b16.
#include "attn_common.h"

namespace sma {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

template <int D>
struct BGeom {
  static constexpr int kWaves = 4;
  static constexpr int kQT = 2;                        // 32-row query tiles per wave
  static constexpr int kQW = 32 * kQT;                 // query rows per wave
  static constexpr int kQ = kWaves * kQW;              // query rows per workgroup
  static constexpr int kK = kBF16KeysPerTile;          // keys per LDS tile
  static constexpr int kKB = kK / 32;                  // 32-key sub-blocks per tile
  static constexpr int kKStride = D + 8;               // K row in LDS (bf16), 16 B pad
  static constexpr int kVStride = D + 16;              // V row in LDS (bf16), 32 B pad
  static constexpr int kHalf = D / 2;
  static constexpr int kSteps = D / 16;                // QK^T k-steps (8 dims per lane half)
  static constexpr int kNch = D / 32;                  // 32-wide output chunks
  static constexpr int kChunksPerThread = kK * D / 8 / kThreadsPerWG;  // 16-byte chunks
  static_assert(kQ == kBF16QueriesPerWG, "planner geometry");
  static_assert(kChunksPerThread * 8 * kThreadsPerWG == kK * D, "tile split");
};

constexpr float kTau = 8.0f;  // lazy running-max threshold, log2 units (see the fp32 kernel)

__device__ __forceinline__ int swap_bits_2_3(int r) {
  return (r & ~0xC) | ((r & 4) << 1) | ((r & 8) >> 1);
}

__device__ __forceinline__ s16x4 lds_read_tr16(const unsigned short* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void attn_fwd_bf16_kernel(FwdArgs a) {
  using G = BGeom<D>;
  __shared__ __attribute__((aligned(16))) unsigned short k_lds[2][G::kK * G::kKStride];
  __shared__ __attribute__((aligned(16))) unsigned short v_lds[2][G::kK * G::kVStride];

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
  int32_t my_row[G::kQT], lim[G::kQT];
#pragma unroll
  for (int qt = 0; qt < G::kQT; ++qt) {
    my_row[qt] = qw0 + 32 * qt + lm;
    lim[qt] = key_limit<CAUSAL>(my_row[qt], a.seq_q, a.seq_kv, split_end);
  }

  // Q operands in registers for the whole pass.
  bf16x8 qr[G::kQT][G::kSteps];
  {
    const unsigned short* qbase = static_cast<const unsigned short*>(a.q) + (size_t)t.bh * a.seq_q * D;
    const unsigned flip = a.negate_q ? 0x80008000u : 0u;
#pragma unroll
    for (int qt = 0; qt < G::kQT; ++qt) {
      const int32_t ld_row = min(my_row[qt], a.seq_q - 1);
      const unsigned short* qp = qbase + (size_t)ld_row * D + lh * G::kHalf;
#pragma unroll
      for (int s = 0; s < G::kSteps; ++s) {
        u32x4 x = *reinterpret_cast<const u32x4*>(qp + 8 * s);
        x ^= flip;
        qr[qt][s] = __builtin_bit_cast(bf16x8, x);
      }
    }
  }

  const unsigned short* kg = static_cast<const unsigned short*>(a.k) + (size_t)t.bh * a.seq_kv * D;
  const unsigned short* vg = static_cast<const unsigned short*>(a.v) + (size_t)t.bh * a.seq_kv * D;
  u32x4 kreg[G::kChunksPerThread], vreg[G::kChunksPerThread];

  auto load_tile = [&](int32_t tile) {
    const int32_t j0 = ks + tile * G::kK;
#pragma unroll
    for (int u = 0; u < G::kChunksPerThread; ++u) {
      const int f = tid + kThreadsPerWG * u;
      const int row = f / (D / 8), c8 = f % (D / 8);
      const int32_t j = j0 + row;
      if (j < a.seq_kv) {
        kreg[u] = *reinterpret_cast<const u32x4*>(kg + (size_t)j * D + 8 * c8);
        vreg[u] = *reinterpret_cast<const u32x4*>(vg + (size_t)j * D + 8 * c8);
      } else {
        kreg[u] = u32x4{0u, 0u, 0u, 0u};
        vreg[u] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int u = 0; u < G::kChunksPerThread; ++u) {
      const int f = tid + kThreadsPerWG * u;
      const int row = f / (D / 8), c8 = f % (D / 8);
      const int krow = (row & ~31) | swap_bits_2_3(row & 31);
      *reinterpret_cast<u32x4*>(&k_lds[buf][krow * G::kKStride + 8 * c8]) = kreg[u];
      *reinterpret_cast<u32x4*>(&v_lds[buf][row * G::kVStride + 8 * c8]) = vreg[u];
    }
  };

  f32x16 oacc[G::kQT][G::kNch];
#pragma unroll
  for (int qt = 0; qt < G::kQT; ++qt)
#pragma unroll
    for (int cb = 0; cb < G::kNch; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[qt][cb][r] = 0.f;
  float m_run[G::kQT], l_run[G::kQT];
#pragma unroll
  for (int qt = 0; qt < G::kQT; ++qt) {
    m_run[qt] = -INFINITY;
    l_run[qt] = 0.f;
  }

  // Transposing-read addressing for the V^T operand (see the header comment):
  // in each 16-lane group, lane role s reads 4 dims of V row 8*h + s/4.
  const int tr_row = 8 * lh + (lane & 15) / 4;
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

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
      f32x16 sacc[G::kQT][G::kKB];
#pragma unroll
      for (int qt = 0; qt < G::kQT; ++qt)
#pragma unroll
        for (int kb = 0; kb < G::kKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[qt][kb][r] = 0.f;
#pragma unroll
      for (int kb = 0; kb < G::kKB; ++kb) {
        const unsigned short* krow = &k_lds[buf][(32 * kb + lm) * G::kKStride + lh * G::kHalf];
#pragma unroll
        for (int s = 0; s < G::kSteps; ++s) {
          const bf16x8 kop = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(krow + 8 * s));
#pragma unroll
          for (int qt = 0; qt < G::kQT; ++qt)
            sacc[qt][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qr[qt][s], sacc[qt][kb], 0, 0, 0);
        }
      }

      const bool need_mask = j0 + G::kK > wave_lo;
      bf16x8 pb[G::kQT][G::kKB][2];
#pragma unroll
      for (int qt = 0; qt < G::kQT; ++qt) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < G::kKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float tv = sacc[qt][kb][r] * a.c;
            if (need_mask) {
              const int32_t j = j0 + 32 * kb + 16 * (r / 8) + 8 * lh + (r % 8);
              tv = j < lim[qt] ? tv : -INFINITY;
            }
            sacc[qt][kb][r] = tv;
            mx = fmaxf(mx, tv);
          }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const bool raise = mx > m_run[qt] + kTau;
        if (__any(raise)) {
          const float m_new = fmaxf(m_run[qt], mx);
          const float m_use = m_new == -INFINITY ? 0.f : m_new;
          const float alpha = __builtin_amdgcn_exp2f(m_run[qt] - m_use);
          l_run[qt] *= alpha;
#pragma unroll
          for (int cb = 0; cb < G::kNch; ++cb)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[qt][cb][r] *= alpha;
          m_run[qt] = m_new;
        }
        const float m_use = m_run[qt] == -INFINITY ? 0.f : m_run[qt];
        float psum = 0.f;
#pragma unroll
        for (int kb = 0; kb < G::kKB; ++kb)
#pragma unroll
          for (int t2 = 0; t2 < 2; ++t2) {
            bf16x8 pv;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float p = __builtin_amdgcn_exp2f(sacc[qt][kb][8 * t2 + e] - m_use);
              psum += p;
              pv[e] = (__bf16)p;
            }
            pb[qt][kb][t2] = pv;
          }
        l_run[qt] += psum;
      }

      // O^T += V^T P^T over the tile's 64 keys in k-steps of 16.
#pragma unroll
      for (int kb = 0; kb < G::kKB; ++kb)
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          const unsigned short* vp = &v_lds[buf][(32 * kb + 16 * t2 + tr_row) * G::kVStride + tr_col];
#pragma unroll
          for (int cb = 0; cb < G::kNch; ++cb) {
            const s16x4 lo = lds_read_tr16(vp + 32 * cb);
            const s16x4 hi = lds_read_tr16(vp + 4 * G::kVStride + 32 * cb);
            const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
            const bf16x8 aop = __builtin_bit_cast(bf16x8, u32x4{lo2[0], lo2[1], hi2[0], hi2[1]});
#pragma unroll
            for (int qt = 0; qt < G::kQT; ++qt)
              oacc[qt][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, pb[qt][kb][t2], oacc[qt][cb], 0, 0, 0);
          }
        }
    }
    if (it + 1 < ntiles) store_tile((it + 1) & 1);
    __syncthreads();
  }

  // Epilogue per query tile (the cross-lane sums first, while all lanes run).
  float l_tot_q[G::kQT];
#pragma unroll
  for (int qt = 0; qt < G::kQT; ++qt) l_tot_q[qt] = l_run[qt] + __shfl_xor(l_run[qt], 32);
  if (!wave_live) return;
#pragma unroll
  for (int qt = 0; qt < G::kQT; ++qt) {
    const float l_tot = l_tot_q[qt];
    if (my_row[qt] >= a.seq_q) continue;
    const bool empty = !(l_tot > 0.f);
    const float inv = empty ? 0.f : 1.0f / l_tot;
    const float lse2 = empty ? -INFINITY : m_run[qt] + __builtin_amdgcn_logf(l_tot);
    const size_t row_id = (size_t)t.bh * a.seq_q + my_row[qt];
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
        for (int e = 0; e < 4; ++e) out[e] = empty ? 0.f : oacc[qt][cb][4 * g4 + e] * inv;
        *reinterpret_cast<f32x4*>(orow + 32 * cb + 8 * g4 + 4 * lh) = out;
      }
  }
}

template <int D, bool CAUSAL>
hipError_t launch_bf16_variant(const FwdArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, CAUSAL>), dim3(a.nwg), dim3(kThreadsPerWG), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, int head_dim, bool causal, hipStream_t s) {
  if (head_dim == 64) return causal ? launch_bf16_variant<64, true>(a, s) : launch_bf16_variant<64, false>(a, s);
  if (head_dim == 128) return causal ? launch_bf16_variant<128, true>(a, s) : launch_bf16_variant<128, false>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace sma
