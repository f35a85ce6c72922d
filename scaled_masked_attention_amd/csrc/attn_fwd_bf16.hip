// Attention forward, 16-bit inputs: bf16 (v_mfma_f32_32x32x16_bf16) or fp16
// (v_mfma_f32_32x32x16_f16, the F16 template flag), fp32 accumulation, fp32,
// bf16 or fp16 output, gfx950.
//
// Same method as the fp32 kernel (oxicuda ComputeBackend `attention`; pulsatrix
// HIPBackend `softmax_rows`, `logsumexp_rows`; TorchLean hard-masked softmax),
// with the operand precision of the oxicuda `gemm_mixed_precision` contract:
// 16-bit operands, fp32 accumulation and result (its MixedPrecision BF16 and
// F16). The probabilities are rounded to the input's 16-bit type (nearest
// even) for the P V product; the row sums use the fp32 probabilities.
//
// Head dims 32 and 64, and 128 with a hard mask: 8 waves x 32 query rows = 256
// rows, two waves per SIMD. Key tiles of 64 rows go HBM/L2 -> LDS through
// buffer-resource direct-to-LDS loads into a ring of five slots, each two steps ahead
// of its use and one workgroup barrier per pair of steps, without passing through
// registers; loads past the last key return zeros. Head dim 128 otherwise runs the same scheme with two 32-row blocks per wave
// (512 rows, 32-key tiles) so that each operand read from LDS feeds two MFMAs
// (attn_fwd_bf16_rb2_kernel), and head dim 256 the role-split kernel
// (attn_fwd_bf16_rs_kernel), both further down.
//
// S^T = K Q^T: lane (m, h) supplies K[key m] and Q[query m] at head dims
// h*D/2 + 8*step .. + 7 and receives the scores of query (lane % 32). K rows
// are placed with bits 2 and 3 of the row index swapped, which makes
// accumulator register r hold key 16*(r/8) + 8*h + r%8: registers 8t..8t+7
// are the eight keys this lane supplies to k-step t of O^T += V^T P^T. V stays
// row-major in LDS and the V^T operand is read with the gfx950 transposing
// read ds_read_b64_tr_b16. Both tiles are XOR-swizzled in 16-byte chunks so
// that these reads are free of bank conflicts (see k_swz / v_swz).
//
// The two waves sharing a SIMD (w and w+4) run half a step apart: waves 0-3
// do S(t), softmax(t), PV(t); waves 4-7 do PV(t-1), S(t), softmax(t). One
// wave's softmax (VALU, transcendental) then meets the other's MFMAs in two
// of the three phases.
//
// The library is built with VGPR-form MFMAs (accumulators in the architectural
// registers).
#include "attn_common.h"


namespace sma {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// The 16-bit element type: operand vectors, the rounding of P, and the MFMA.
template <bool F16>
struct Half;
template <>
struct Half<false> {
  typedef __bf16 E;
  typedef bf16x8 V8;
  static __device__ __forceinline__ f32x16 mfma(V8 a, V8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <>
struct Half<true> {
  typedef _Float16 E;
  typedef f16x8 V8;
  static __device__ __forceinline__ f32x16 mfma(V8 a, V8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// Geometry per head dim (32, 64, 128). At d = 32 a tensor's tile is 256 chunks:
// waves 0-3 copy K, waves 4-7 copy V.
template <int D>
struct BGeom {
  static_assert(D == 32 || D == 64 || D == 128, "the 32-row kernel's head dims (128 with a hard mask)");
  static constexpr int kWaves = 8;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kQW = 32;                     // query rows per wave
  static constexpr int kQ = kWaves * kQW;            // query rows per workgroup
  static constexpr int kK = kBF16KeysPerTile;        // keys per tile
  static constexpr int kKB = kK / 32;                // 32-key blocks per tile
  // Five slots (all 160 KB of LDS at head dim 128): see the step loop.
  static constexpr int kSlots = 5;                   // LDS ring of K/V tiles
  static constexpr int kChunksPerRow = D / 8;        // 16-byte chunks per K or V row
  static constexpr int kTileChunks = kK * kChunksPerRow;
  static constexpr bool kSplitKV = kTileChunks < kThreads;      // half the waves per tensor
  static constexpr int kCopyWaves = kSplitKV ? kWaves / 2 : kWaves;  // waves copying a tensor
  static constexpr int kLoadsPerThread = kTileChunks / (64 * kCopyWaves);  // per copied tensor
  static constexpr int kLoadsPerTile = kSplitKV ? kLoadsPerThread : 2 * kLoadsPerThread;
  static constexpr int kHalf = D / 2;
  static constexpr int kSteps = D / 16;              // QK^T k-steps (8 dims per lane half)
  static constexpr int kNch = D / 32;                // 32-wide output chunks
  static_assert(kQ == kBF16QueriesPerWG, "planner geometry");
  static_assert(kLoadsPerThread >= 1 && kLoadsPerThread * 64 * kCopyWaves == kTileChunks,
                "tile split");
};

// A load through the constant address space: with a wave-uniform address it
// becomes a scalar (s_load) load into SGPRs. Only for memory no kernel of the
// launch writes.
template <typename T>
__device__ __forceinline__ T scalar_load(const void* p) {
  return *(const __attribute__((address_space(4))) T*)p;
}

constexpr float kTau = 8.0f;  // lazy running-max threshold, log2 units (see the fp32 kernel)

__device__ __forceinline__ int swap_bits_2_3(int r) {
  return (r & ~0xC) | ((r & 4) << 1) | ((r & 8) >> 1);
}
// 16-byte chunk swizzles (XOR on the chunk index within a row). gfx950's LDS
// has 64 four-byte banks and serves a ds_read_b128 in groups of 16 lanes and
// a ds_read_b64_tr_b16 in groups of 32 lanes, so:
//  - K: the 16 lanes of a group read 16 consecutive rows at one logical
//    chunk; with rows of 256 bytes or more (d >= 128) the chunk is XORed with
//    row & 15, with 128-byte rows (d = 64, two rows per bank cycle) with
//    (row >> 1) & 7, with 64-byte rows (d = 32, four rows per bank cycle)
//    with (row >> 2) & 3;
//  - V: a 32-lane group reads 4 consecutive rows x 4 chunks of one 64-byte
//    group; the four rows must use four different 64-byte bank groups, so the
//    chunk is XORed with 4*(row & 3) (d >= 128) or 4*((row >> 1) & 1) (d = 64);
//    at d = 32 the four 64-byte rows are already 256 consecutive bytes.
template <int D>
__device__ __forceinline__ int k_swz(int rho) {
  return D >= 128 ? (rho & 15) : D == 64 ? ((rho >> 1) & 7) : ((rho >> 2) & 3);
}
template <int D>
__device__ __forceinline__ int v_swz(int r) {
  return D >= 128 ? 4 * (r & 3) : D == 64 ? 4 * ((r >> 1) & 1) : 0;
}

template <int D, bool CAUSAL, bool F16, bool MASKED>
__global__ __launch_bounds__(BGeom<D>::kThreads) void attn_fwd_bf16_kernel(FwdArgs a) {
  using G = BGeom<D>;
  using H = Half<F16>;
  using V8 = typename H::V8;
  __shared__ __attribute__((aligned(16))) u32x4 k_lds[G::kSlots][G::kTileChunks];
  __shared__ __attribute__((aligned(16))) u32x4 v_lds[G::kSlots][G::kTileChunks];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
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
  V8 qr[G::kSteps];
  {
    const unsigned short* qp = static_cast<const unsigned short*>(a.q) +
                               head_offset(t.bh, a.heads, a.qs_b, a.qs_h) +
                               (int64_t)min(my_row, a.seq_q - 1) * a.qs_s + lh * G::kHalf;
    const unsigned flip = a.negate_q ? 0x80008000u : 0u;
#pragma unroll
    for (int s = 0; s < G::kSteps; ++s) {
      u32x4 x = *reinterpret_cast<const u32x4*>(qp + 8 * s);
      x ^= flip;
      qr[s] = __builtin_bit_cast(V8, x);
    }
  }
  // The tile loads below are invisible to the compiler's load counting, so
  // none of its own loads may still be in flight when they start.
  wait_vmcnt<0>();

  // Buffer resources over this (batch, head)'s K and V: rows past the last key
  // fall outside the byte range and read as zeros.
  const unsigned kv_bytes = strided_range(a.seq_kv, a.kvs_s, D, 2);
  const unsigned kv_row = (unsigned)(a.kvs_s * 2);  // bytes between consecutive key rows
  const int64_t kv_off = head_offset(t.bh, a.heads, a.kvs_b, a.kvs_h);
  const __amdgpu_buffer_rsrc_t k_rsrc =
      raw_buffer(static_cast<const unsigned short*>(a.k) + kv_off, kv_bytes);
  const __amdgpu_buffer_rsrc_t v_rsrc =
      raw_buffer(static_cast<const unsigned short*>(a.v) + kv_off, kv_bytes);
  // Each wave-wide load fills 64 consecutive LDS chunks: position
  // p = (u*copy_waves + w)*64 + lane (w the wave's index among the waves that
  // copy this tensor) is row rho = p / chunks_per_row, chunk p % chunks_per_row;
  // the lane fetches the global chunk that belongs there under the K row
  // permutation and the swizzles, which depend on the lane and on u only.
  constexpr int kRowsPerU = G::kCopyWaves * 64 / G::kChunksPerRow;
  static_assert(D == 32 || D == 64 || D == 128 || D == 256, "swizzles are defined for these");
  const int cw = G::kSplitKV ? wave % G::kCopyWaves : wave;  // index among the copying waves
  const bool copies_k = !G::kSplitKV || wave < G::kCopyWaves;
  const bool copies_v = !G::kSplitKV || wave >= G::kCopyWaves;
  const int rho0 = (cw * 64 + lane) / G::kChunksPerRow;
  const int pc = lane % G::kChunksPerRow;
  auto k_src = [&](int u) {
    const int rho = rho0 + u * kRowsPerU;
    return (unsigned)((rho & ~31) | swap_bits_2_3(rho & 31)) * kv_row + 16u * (unsigned)(pc ^ k_swz<D>(rho));
  };
  auto v_src = [&](int u) {
    const int rho = rho0 + u * kRowsPerU;
    return (unsigned)rho * kv_row + 16u * (unsigned)(pc ^ v_swz<D>(rho));
  };

  // A hard mask, packed by columns (MaskColArgs): this wave's 32-row block has
  // one row-bit word per key and a class per 64-key tile (0 nothing admitted,
  // 1 everything admitted, 2 mixed). Both are read with scalar loads: a tile
  // that admits nothing is skipped, one that admits everything runs unmasked,
  // and in a mixed tile two key words side by side are the 64-lane mask of one
  // score register, applied with a single v_cndmask.
  const uint32_t* mcols = nullptr;
  const uint32_t* mcls = nullptr;
  if (MASKED) {
    const int64_t rb = qw0 / 32;
    mcols = a.mask_bits + head_offset(t.bh, a.heads, a.mbits_sb, a.mbits_sh) + rb * a.mask_words;
    mcls = a.mask_cls + head_offset(t.bh, a.heads, a.mcls_sb, a.mcls_sh) + rb * a.mask_tiles;
  }
  auto issue_tile = [&](int32_t T, int slot) {
    const unsigned row0 = (unsigned)(ks + T * G::kK);
#pragma unroll
    for (int u = 0; u < G::kLoadsPerThread; ++u) {
      const int base = (u * G::kCopyWaves + cw) * 64;
      const unsigned tile_ofs = row0 * kv_row;
      if (copies_k) dma_load_x4(k_rsrc, k_src(u) + tile_ofs, lds_address(&k_lds[slot][base]));
      if (copies_v) dma_load_x4(v_rsrc, v_src(u) + tile_ofs, lds_address(&v_lds[slot][base]));
    }
  };

  f32x16 oacc[G::kNch];
#pragma unroll
  for (int cb = 0; cb < G::kNch; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[cb][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  // c = |scale| log2 e, kept positive so that an excluded score (-inf) gives
  // -inf, never NaN: with scale 0 every allowed |s| c is then below 2^-26 for
  // |s| < 2^100, and 2^(s c - m) rounds to 1, the uniform weights of scale 0.
  const float c = fmaxf(a.c, 1.17549435e-38f);

  // O^T += V^T P^T over a tile's 64 keys in k-steps of 16. In each 16-lane
  // group, lane role s reads 4 dims of V row 16*t2 + 8*h + s/4 (and +4).
  const int srole = lane & 15;
  const int colq = 2 * ((lane >> 4) & 1) + ((srole & 3) >> 1);  // chunk within a 32-dim group
  const int half8 = 8 * (srole & 1);
  auto pv_tile = [&](int slot, const V8 (&pb)[G::kKB][2]) {
    const unsigned char* vtile = reinterpret_cast<const unsigned char*>(&v_lds[slot][0]);
    // MFMA i = 4 (2 kb + t2) + cb: output chunk cb, keys 32 kb + 16 t2 .. + 15.
    auto v_operand = [&](int i) {
      const int kb = i / (2 * G::kNch), t2 = (i / G::kNch) % 2, cb = i % G::kNch;
      const int r_lo = 32 * kb + 16 * t2 + 8 * lh + srole / 4;
      const int r_hi = r_lo + 4;
      const int chunk = 4 * cb + colq;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(vtile + r_lo * (2 * D) +
                                                     16 * (chunk ^ v_swz<D>(r_lo)) + half8));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(vtile + r_hi * (2 * D) +
                                                     16 * (chunk ^ v_swz<D>(r_hi)) + half8));
      const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
      return __builtin_bit_cast(V8, u32x4{lo2[0], lo2[1], hi2[0], hi2[1]});
    };
    constexpr int kN = 2 * G::kKB * G::kNch;  // MFMAs per tile
    constexpr int kPf = 3;                    // operands in flight ahead of the MFMAs
    V8 vop[kPf + 1];
#pragma unroll
    for (int i = 0; i < kPf; ++i) vop[i] = v_operand(i);
    __builtin_amdgcn_s_setprio(1);  // as for the score MFMAs
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      if (i + kPf < kN) vop[(i + kPf) % (kPf + 1)] = v_operand(i + kPf);
      __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of this MFMA
      const int kb = i / (2 * G::kNch), t2 = (i / G::kNch) % 2, cb = i % G::kNch;
      oacc[cb] = H::mfma(vop[i % (kPf + 1)], pb[kb][t2], oacc[cb]);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // Scores, lazy running max and probabilities of tile T (in ring slot
  // `slot`); returns the bf16 probabilities for the PV product.
  auto scores_and_p = [&](int32_t T, int slot, V8 (&pb)[G::kKB][2], uint32_t cls) {
    const int32_t j0 = ks + T * G::kK;
    // The k-steps of the key blocks interleave, and the K operands of step
    // st + kPf are read before the MFMAs of step st, so that every LDS read has
    // 2 kPf MFMAs' time to land.
    f32x16 sacc[G::kKB];
    const unsigned char* ktile = reinterpret_cast<const unsigned char*>(&k_lds[slot][0]);
    auto k_operand = [&](int kb, int st) {
      const int rho = 32 * kb + lm;
      const int chunk = lh * G::kSteps + st;
      return __builtin_bit_cast(V8, *reinterpret_cast<const u32x4*>(
                                        ktile + rho * (2 * D) + 16 * (chunk ^ k_swz<D>(rho))));
    };
    constexpr int kPf = 2;  // k-steps of K operands in flight ahead of the MFMAs
    V8 kop[kPf + 1][G::kKB];
#pragma unroll
    for (int kb = 0; kb < G::kKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
    for (int st = 0; st < kPf; ++st)
#pragma unroll
      for (int kb = 0; kb < G::kKB; ++kb) kop[st][kb] = k_operand(kb, st);
    // While a wave issues its MFMAs it runs at raised priority, so that the
    // other wave on the SIMD (in its softmax, on the VALU) fills the issue
    // slots between them rather than competing for the matrix core.
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int st = 0; st < G::kSteps; ++st) {
      if (st + kPf < G::kSteps)
#pragma unroll
        for (int kb = 0; kb < G::kKB; ++kb) kop[(st + kPf) % (kPf + 1)][kb] = k_operand(kb, st + kPf);
      __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of these MFMAs
#pragma unroll
      for (int kb = 0; kb < G::kKB; ++kb)
        sacc[kb] = H::mfma(kop[st % (kPf + 1)][kb], qr[st], sacc[kb]);
      __builtin_amdgcn_sched_barrier(0);
    }

    __builtin_amdgcn_s_setprio(0);

    // Boundary tiles (the causal diagonal, the end of the keys): excluded
    // scores become -inf, so that they enter neither the max nor the sum
    // (2^-inf = 0; c > 0). The empty asm keeps the bound, and with it the
    // comparisons, inside this branch instead of on every tile.
    if (j0 + G::kK > wave_lo) {
      int32_t rel = lim - j0 - 8 * lh;  // key 32kb + 16(r/8) + r%8 allowed iff < rel
      asm volatile("" : "+v"(rel));
#pragma unroll
      for (int kb = 0; kb < G::kKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          sacc[kb][r] = (32 * kb + 16 * (r / 8) + (r % 8) < rel) ? sacc[kb][r] : -INFINITY;
    }
    // A mixed tile of the hard mask: score register r of key block kb holds key
    // 16(r/8) + r%8 (lanes 0-31) and that key + 8 (lanes 32-63) of the block;
    // their two column words, stored side by side, are its lane mask.
    if (MASKED && cls == 2u) {
      const float ninf = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < G::kKB; ++kb)
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          typedef unsigned u32x16 __attribute__((ext_vector_type(16)));
          const u32x16 w = scalar_load<u32x16>(mcols + (j0 + 32 * kb + 16 * g));
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const uint64_t lanes = (uint64_t)w[2 * i] | ((uint64_t)w[2 * i + 1] << 32);
            float x = sacc[kb][8 * g + i];
            asm("v_cndmask_b32_e64 %0, %1, %0, %2" : "+v"(x) : "v"(ninf), "s"(lanes));
            sacc[kb][8 * g + i] = x;
          }
        }
    }

    // Row max of the raw scores (scale > 0 after the sign fold).
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < G::kKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
    {  // lanes m and m + 32 hold the two key halves of query m (a VALU swap, not an LDS round trip)
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                       false, false);
      // scores are never NaN: a plain v_max_f32, without fmaxf's canonicalizing maxes
      asm("v_max_f32 %0, %1, %2" : "=v"(mx) : "v"(__uint_as_float(sw[0])), "v"(__uint_as_float(sw[1])));
    }
    const float tmax = mx * c;  // c > 0: -inf stays -inf
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
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < G::kKB; ++kb)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][8 * t2 + e], c, neg_m));
          psum += p;
          pb[kb][t2][e] = (typename H::E)p;
        }
    l_run += psum;
  };

  const bool late = wave >= G::kWaves / 2;
  V8 pb_late[G::kKB][2];
  bool late_pending = false;
  int late_slot = 0;

  // Tile T is copied in step T-2 and used in step T (and in step T+1 by the
  // late waves' PV), with one barrier per pair of steps: at an even step T
  // tiles T and T+1 are resident (nothing else is in flight). The last
  // barrier before step T leaves every wave done with step T-2 at least, so
  // the slot of tile T-3 is free for T+2; tiles T-1 .. T+2 are live.
  if (ntiles > 0) issue_tile(0, 0);
  if (ntiles > 1) issue_tile(1, 1);
  int slot = 0, slot2 = 2;  // the slots of tiles T and T+2 (ring positions, wave-uniform)
  for (int32_t T = 0; T < ntiles; ++T) {
    if ((T & 1) == 0) {
      wait_vmcnt<0>();
      __syncthreads();
    }
    if (T + 2 < ntiles) issue_tile(T + 2, slot2);
    if (late && late_pending) {
      pv_tile(late_slot, pb_late);
      late_pending = false;
    }
    // The tile's mask class (1 without a mask); a tile the mask closes is skipped.
    uint32_t cls = 1u;
    if (MASKED && wave_live && ks + T * G::kK < wave_hi)
      cls = scalar_load<uint32_t>(mcls + (ks + T * G::kK) / 64);  // the class of its 64-key tile
    if (wave_live && ks + T * G::kK < wave_hi && cls != 0u) {
      V8 pb[G::kKB][2];
      scores_and_p(T, slot, pb, cls);
      if (late) {
#pragma unroll
        for (int kb = 0; kb < G::kKB; ++kb)
#pragma unroll
          for (int t2 = 0; t2 < 2; ++t2) pb_late[kb][t2] = pb[kb][t2];
        late_pending = true;
        late_slot = slot;
      } else {
        pv_tile(slot, pb);
      }
    }
    slot = slot + 1 == G::kSlots ? 0 : slot + 1;
    slot2 = slot2 + 1 == G::kSlots ? 0 : slot2 + 1;
  }
  if (late_pending) pv_tile(late_slot, pb_late);

  // Epilogue (the cross-lane sum first, while all lanes run).
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!wave_live || my_row >= a.seq_q) return;
  const bool empty = !(l_tot > 0.f);
  const float inv = empty ? 0.f : 1.0f / l_tot;
  const float lse2 = empty ? -INFINITY : m_run + __builtin_amdgcn_logf(l_tot);
  const size_t row_id = (size_t)t.bh * a.seq_q + my_row;
  float* orow = nullptr;
  unsigned short* orow16 = nullptr;
  if (a.nsplit == 1) {
    const int64_t o_off = head_offset(t.bh, a.heads, a.qs_b, a.qs_h) + (int64_t)my_row * a.qs_s;
    if (a.o_bf16) orow16 = a.o_bf16 + o_off;
    else orow = a.o + o_off;
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
      if (orow16)
        *reinterpret_cast<u32x2*>(orow16 + 32 * cb + 8 * g4 + 4 * lh) =
            u32x2{pack_out16(out[0], out[1], a.o_f16), pack_out16(out[2], out[3], a.o_f16)};
      else
        *reinterpret_cast<f32x4*>(orow + 32 * cb + 8 * g4 + 4 * lh) = out;
    }
}

// ---------------------------------------------------------------- role-split kernel
// Head dim 256, where one wave holding both Q (64 registers) and all of O (128) would
// leave a SIMD a single wave. A workgroup of 12 waves is 6 pairs and 192 query rows. For
// pair p (rows q0 + 32p .. + 31), wave p (the S wave) holds Q, forms S^T = K Q^T, the
// lazy running max, the probabilities and the row sums, and leaves P (in the input's
// 16-bit type, already in the B-operand layout of the P V product) and the tile's
// rescale factor in LDS; wave 6 + p (the O wave) holds O and forms
// O^T = alpha O^T + V^T P^T one tile behind. Neither role needs more than 168
// registers, so three waves share each SIMD, and one wave's MFMAs run while another
// works on the VALU. K tiles of 32 keys come through a 3-slot ring and V tiles through a
// 4-slot ring, both two tiles ahead of the S waves, copied by waves 0-7; one barrier per
// tile.
template <int D>
struct RGeom {
  static constexpr int kPairs = 6;
  static constexpr int kWaves = 2 * kPairs;
  static constexpr int kCopyWaves = 8;  // waves 0-7 issue the tile copies
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kQW = 32;
  static constexpr int kQ = kPairs * kQW;
  static constexpr int kK = kBF16D256KeysPerTile;
  static constexpr int kKB = kK / 32;
  static constexpr int kKSlots = 3;
  static constexpr int kVSlots = 4;
  static constexpr int kChunksPerRow = D / 8;
  static constexpr int kTileChunks = kK * kChunksPerRow;
  static constexpr int kLoadsPerThread = kTileChunks / (64 * kCopyWaves);  // per tensor and tile
  static constexpr int kLoadsPerTile = 2 * kLoadsPerThread;
  static constexpr int kHalf = D / 2;
  static constexpr int kSteps = D / 16;
  static constexpr int kNch = D / 32;
  static_assert(kQ == kBF16D256QueriesPerWG, "planner geometry");
  static_assert(D == 256, "role-split geometry");
  static_assert(kLoadsPerThread >= 1 && kLoadsPerThread * 64 * kCopyWaves == kTileChunks, "tile split");
};

template <int D, bool CAUSAL, bool F16, bool MASKED>
__global__ __launch_bounds__(RGeom<D>::kThreads) void attn_fwd_bf16_rs_kernel(FwdArgs a) {
  using G = RGeom<D>;
  using H = Half<F16>;
  using V8 = typename H::V8;
  __shared__ __attribute__((aligned(16))) u32x4 k_lds[G::kKSlots][G::kTileChunks];
  __shared__ __attribute__((aligned(16))) u32x4 v_lds[G::kVSlots][G::kTileChunks];
  // P of a tile per pair and parity: [2 kb + t2][lane] holds lane's B operand of P V
  // k-step (kb, t2); the rescale factor per lane (1 when the max did not move); and
  // the S waves' final row sums.
  __shared__ __attribute__((aligned(16))) u32x4 p_lds[G::kPairs][2][2 * G::kKB][64];
  __shared__ float a_lds[G::kPairs][2][64];
  __shared__ float l_lds[G::kPairs][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool swave = wave < G::kPairs;
  const int pair = swave ? wave : wave - G::kPairs;
  const int lm = lane & 31;
  const int lh = lane >> 5;

  const TileId t = decode_tile(blockIdx.x, a);
  const int32_t q0 = t.qb * G::kQ;
  const int32_t qw0 = q0 + pair * G::kQW;
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

  const unsigned kv_bytes = strided_range(a.seq_kv, a.kvs_s, D, 2);
  const unsigned kv_row = (unsigned)(a.kvs_s * 2);
  const int64_t kv_off = head_offset(t.bh, a.heads, a.kvs_b, a.kvs_h);
  const __amdgpu_buffer_rsrc_t k_rsrc =
      raw_buffer(static_cast<const unsigned short*>(a.k) + kv_off, kv_bytes);
  const __amdgpu_buffer_rsrc_t v_rsrc =
      raw_buffer(static_cast<const unsigned short*>(a.v) + kv_off, kv_bytes);
  // As in the kernel above: position p = (u*waves + wave)*64 + lane of a tile is row
  // p / chunks_per_row, chunk p % chunks_per_row, under the K row permutation and the
  // swizzles.
  constexpr int kRowsPerU = G::kCopyWaves * 64 / G::kChunksPerRow;
  const int rho0 = (wave * 64 + lane) / G::kChunksPerRow;
  const int pc = lane % G::kChunksPerRow;
  auto k_src = [&](int u) {
    const int rho = rho0 + u * kRowsPerU;
    return (unsigned)((rho & ~31) | swap_bits_2_3(rho & 31)) * kv_row + 16u * (unsigned)(pc ^ k_swz<D>(rho));
  };
  auto v_src = [&](int u) {
    const int rho = rho0 + u * kRowsPerU;
    return (unsigned)rho * kv_row + 16u * (unsigned)(pc ^ v_swz<D>(rho));
  };
  auto issue_tile = [&](int32_t T) {
    const unsigned tile_ofs = (unsigned)(ks + T * G::kK) * kv_row;
    const int ksl = T % G::kKSlots, vsl = T % G::kVSlots;
    if (wave >= G::kCopyWaves) return;
#pragma unroll
    for (int u = 0; u < G::kLoadsPerThread; ++u) {
      const int base = (u * G::kCopyWaves + wave) * 64;
      dma_load_x4(k_rsrc, k_src(u) + tile_ofs, lds_address(&k_lds[ksl][base]));
      dma_load_x4(v_rsrc, v_src(u) + tile_ofs, lds_address(&v_lds[vsl][base]));
    }
  };

  // The hard mask, packed by columns as for the kernel above (one 32-row block per pair).
  const uint32_t* mcols = nullptr;
  const uint32_t* mcls = nullptr;
  if (MASKED) {
    const int64_t rb = qw0 / 32;
    mcols = a.mask_bits + head_offset(t.bh, a.heads, a.mbits_sb, a.mbits_sh) + rb * a.mask_words;
    mcls = a.mask_cls + head_offset(t.bh, a.heads, a.mcls_sb, a.mcls_sh) + rb * a.mask_tiles;
  }
  // Whether tile T holds keys of this pair's rows that are not all closed by the mask
  // (both waves of the pair evaluate it alike), and the tile's mask class.
  auto tile_class = [&](int32_t T) -> uint32_t {
    if (!wave_live || ks + T * G::kK >= wave_hi) return 0u;
    return MASKED ? scalar_load<uint32_t>(mcls + (ks + T * G::kK) / 64) : 1u;
  };

  // The step loop (its waits, barrier and copies), run by every wave with its role's
  // work; each role has its own copy of the loop, so that its registers stay put.
  auto run_steps = [&](auto&& work) {
    if (ntiles > 0) issue_tile(0);
    if (ntiles > 1) issue_tile(1);
    for (int32_t T = 0; T <= ntiles; ++T) {
      if (T + 1 < ntiles) wait_vmcnt<G::kLoadsPerTile>();
      else wait_vmcnt<0>();
      __syncthreads();  // tile T has landed; step T - 1 is done with its slots and P
      if (T + 2 < ntiles) issue_tile(T + 2);
      work(T);
    }
  };

  const float c = fmaxf(a.c, 1.17549435e-38f);  // as in the kernel above
  const size_t row_id = (size_t)t.bh * a.seq_q + my_row;

  if (swave) {
    // Q operands in registers (the copies below are invisible to the compiler's load
    // counting, so its own loads must be done first).
    V8 qr[G::kSteps];
    {
      const unsigned short* qp = static_cast<const unsigned short*>(a.q) +
                                 head_offset(t.bh, a.heads, a.qs_b, a.qs_h) +
                                 (int64_t)min(my_row, a.seq_q - 1) * a.qs_s + lh * G::kHalf;
      const unsigned flip = a.negate_q ? 0x80008000u : 0u;
#pragma unroll
      for (int s = 0; s < G::kSteps; ++s) {
        u32x4 x = *reinterpret_cast<const u32x4*>(qp + 8 * s);
        x ^= flip;
        qr[s] = __builtin_bit_cast(V8, x);
      }
    }
    wait_vmcnt<0>();
    float m_run = -INFINITY, l_run = 0.f;
    run_steps([&](int32_t T) {
      if (T >= ntiles) return;
      const uint32_t cls = tile_class(T);
      if (cls == 0u) return;
      const int32_t j0 = ks + T * G::kK;
      const unsigned char* ktile = reinterpret_cast<const unsigned char*>(&k_lds[T % G::kKSlots][0]);
      auto k_operand = [&](int kb, int st) {
        const int rho = 32 * kb + lm;
        const int chunk = lh * G::kSteps + st;
        return __builtin_bit_cast(V8, *reinterpret_cast<const u32x4*>(
                                          ktile + rho * (2 * D) + 16 * (chunk ^ k_swz<D>(rho))));
      };
      f32x16 sacc[G::kKB];
#pragma unroll
      for (int kb = 0; kb < G::kKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
      constexpr int kPf = 2;
      V8 kop[kPf + 1][G::kKB];
#pragma unroll
      for (int st = 0; st < kPf; ++st)
#pragma unroll
        for (int kb = 0; kb < G::kKB; ++kb) kop[st][kb] = k_operand(kb, st);
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int st = 0; st < G::kSteps; ++st) {
        if (st + kPf < G::kSteps)
#pragma unroll
          for (int kb = 0; kb < G::kKB; ++kb) kop[(st + kPf) % (kPf + 1)][kb] = k_operand(kb, st + kPf);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kb = 0; kb < G::kKB; ++kb) sacc[kb] = H::mfma(kop[st % (kPf + 1)][kb], qr[st], sacc[kb]);
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_setprio(0);

      if (j0 + G::kK > wave_lo) {
        int32_t rel = lim - j0 - 8 * lh;  // key 32kb + 16(r/8) + r%8 allowed iff < rel
        asm volatile("" : "+v"(rel));
#pragma unroll
        for (int kb = 0; kb < G::kKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            sacc[kb][r] = (32 * kb + 16 * (r / 8) + (r % 8) < rel) ? sacc[kb][r] : -INFINITY;
      }
      if (MASKED && cls == 2u) {
        const float ninf = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < G::kKB; ++kb)
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            typedef unsigned u32x16 __attribute__((ext_vector_type(16)));
            const u32x16 w = scalar_load<u32x16>(mcols + (j0 + 32 * kb + 16 * g));
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const uint64_t lanes = (uint64_t)w[2 * i] | ((uint64_t)w[2 * i + 1] << 32);
              float x = sacc[kb][8 * g + i];
              asm("v_cndmask_b32_e64 %0, %1, %0, %2" : "+v"(x) : "v"(ninf), "s"(lanes));
              sacc[kb][8 * g + i] = x;
            }
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < G::kKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
      {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                         false, false);
        asm("v_max_f32 %0, %1, %2" : "=v"(mx) : "v"(__uint_as_float(sw[0])), "v"(__uint_as_float(sw[1])));
      }
      const float tmax = mx * c;  // c > 0: -inf stays -inf
      float alpha = 1.f;
      if (__any(tmax > m_run + kTau)) {
        const float m_new = fmaxf(m_run, tmax);
        alpha = __builtin_amdgcn_exp2f(m_run - (m_new == -INFINITY ? 0.f : m_new));
        l_run *= alpha;
        m_run = m_new;
      }
      const float neg_m = m_run == -INFINITY ? 0.f : -m_run;
      float psum = 0.f;
      V8 pb[G::kKB][2];
#pragma unroll
      for (int kb = 0; kb < G::kKB; ++kb)
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][8 * t2 + e], c, neg_m));
            psum += p;
            pb[kb][t2][e] = (typename H::E)p;
          }
      l_run += psum;
      const int par = T & 1;
#pragma unroll
      for (int kb = 0; kb < G::kKB; ++kb)
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) p_lds[pair][par][2 * kb + t2][lane] = __builtin_bit_cast(u32x4, pb[kb][t2]);
      a_lds[pair][par][lane] = alpha;
    });
    // Epilogue: the row sums for the O wave, and the LSE.
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    l_lds[pair][lane] = l_tot;
    __syncthreads();
    if (!wave_live || my_row >= a.seq_q || lh != 0) return;
    const bool empty = !(l_tot > 0.f);
    const float lse2 = empty ? -INFINITY : m_run + __builtin_amdgcn_logf(l_tot);
    if (a.nsplit == 1) {
      if (a.lse) a.lse[row_id] = empty ? -INFINITY : lse2 * 0.69314718055994530942f;
    } else {
      a.part_lse[(size_t)t.split * ((size_t)a.bh * a.seq_q) + row_id] = lse2;
    }
  } else {
    f32x16 oacc[G::kNch];
#pragma unroll
    for (int cb = 0; cb < G::kNch; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[cb][r] = 0.f;
    const int srole = lane & 15;
    const int colq = 2 * ((lane >> 4) & 1) + ((srole & 3) >> 1);
    const int half8 = 8 * (srole & 1);
    run_steps([&](int32_t T) {
      if (T == 0 || tile_class(T - 1) == 0u) return;
      const int par = (T - 1) & 1;
      const float alpha = a_lds[pair][par][lane];
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int cb = 0; cb < G::kNch; ++cb)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[cb][r] *= alpha;
      }
      V8 pb[G::kKB][2];
#pragma unroll
      for (int kb = 0; kb < G::kKB; ++kb)
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) pb[kb][t2] = __builtin_bit_cast(V8, p_lds[pair][par][2 * kb + t2][lane]);
      const unsigned char* vtile = reinterpret_cast<const unsigned char*>(&v_lds[(T - 1) % G::kVSlots][0]);
      auto v_operand = [&](int i) {
        const int kb = i / (2 * G::kNch), t2 = (i / G::kNch) % 2, cb = i % G::kNch;
        const int r_lo = 32 * kb + 16 * t2 + 8 * lh + srole / 4;
        const int r_hi = r_lo + 4;
        const int chunk = 4 * cb + colq;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(vtile + r_lo * (2 * D) +
                                                       16 * (chunk ^ v_swz<D>(r_lo)) + half8));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(vtile + r_hi * (2 * D) +
                                                       16 * (chunk ^ v_swz<D>(r_hi)) + half8));
        const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
        return __builtin_bit_cast(V8, u32x4{lo2[0], lo2[1], hi2[0], hi2[1]});
      };
      constexpr int kN = 2 * G::kKB * G::kNch;
      constexpr int kPf = 1;  // one operand ahead: the O wave has 40 registers beside its accumulators
      V8 vop[kPf + 1];
#pragma unroll
      for (int i = 0; i < kPf; ++i) vop[i] = v_operand(i);
#pragma unroll
      for (int i = 0; i < kN; ++i) {
        if (i + kPf < kN) vop[(i + kPf) % (kPf + 1)] = v_operand(i + kPf);
        __builtin_amdgcn_sched_barrier(0);
        const int kb = i / (2 * G::kNch), t2 = (i / G::kNch) % 2, cb = i % G::kNch;
        oacc[cb] = H::mfma(vop[i % (kPf + 1)], pb[kb][t2], oacc[cb]);
        __builtin_amdgcn_sched_barrier(0);
      }
    });
    __syncthreads();  // the S waves' row sums
    const float l_tot = l_lds[pair][lane];
    if (!wave_live || my_row >= a.seq_q) return;
    const bool empty = !(l_tot > 0.f);
    const float inv = empty ? 0.f : 1.0f / l_tot;
    float* orow = nullptr;
    unsigned short* orow16 = nullptr;
    if (a.nsplit == 1) {
      const int64_t o_off = head_offset(t.bh, a.heads, a.qs_b, a.qs_h) + (int64_t)my_row * a.qs_s;
      if (a.o_bf16) orow16 = a.o_bf16 + o_off;
      else orow = a.o + o_off;
    } else {
      orow = a.part_o + ((size_t)t.split * ((size_t)a.bh * a.seq_q) + row_id) * D;
    }
#pragma unroll
    for (int cb = 0; cb < G::kNch; ++cb)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        f32x4 out;
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = empty ? 0.f : oacc[cb][4 * g4 + e] * inv;
        if (orow16)
          *reinterpret_cast<u32x2*>(orow16 + 32 * cb + 8 * g4 + 4 * lh) =
              u32x2{pack_out16(out[0], out[1], a.o_f16), pack_out16(out[2], out[3], a.o_f16)};
        else
          *reinterpret_cast<f32x4*>(orow + 32 * cb + 8 * g4 + 4 * lh) = out;
      }
  }
}

template <bool CAUSAL>
hipError_t launch_bf16_rs(const FwdArgs& a, bool f16, hipStream_t s) {
  constexpr int D = 256;
  const dim3 grid(a.nwg), block(RGeom<D>::kThreads);
  if (a.mask_bits) {
    if (f16) hipLaunchKernelGGL((attn_fwd_bf16_rs_kernel<D, CAUSAL, true, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((attn_fwd_bf16_rs_kernel<D, CAUSAL, false, true>), grid, block, 0, s, a);
  } else {
    if (f16) hipLaunchKernelGGL((attn_fwd_bf16_rs_kernel<D, CAUSAL, true, false>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((attn_fwd_bf16_rs_kernel<D, CAUSAL, false, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- two row blocks per wave
// Head dim 128 without a hard mask: each wave owns 64 query rows as two 32-row blocks,
// so that every K operand of the score product and every V^T operand of the P V product
// read from LDS feeds two MFMAs (one per row block) instead of one. 8 waves x 64 rows =
// 512 rows per workgroup, two waves per SIMD; key tiles of 32 rows (a wave's two score
// blocks then take 32 registers) in a ring of eight LDS slots, copied a pair at a time
// two tiles ahead, with one workgroup barrier per pair of tiles. LDS
// addresses are formed inside the step from one base register and an XOR constant (the
// swizzles only flip bits 4..7 of a row's byte offset), and the operand reads are
// streamed ahead of their MFMAs, pinned there by empty asm.
struct B2Geom {
  static constexpr int D = 128;
  static_assert(kBF16D128QueriesPerWG == 8 * 64 && kBF16D128KeysPerTile == 32, "planner geometry");
  static constexpr int kWaves = 8;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kRB = 2;                      // 32-row blocks per wave
  static constexpr int kQW = 32 * kRB;               // query rows per wave
  static constexpr int kQ = kWaves * kQW;            // query rows per workgroup
  static constexpr int kK = 32;                      // keys per tile
  static constexpr int kSlots = 8;                  // tiles T-1 .. T+3 live at step T
  static constexpr int kChunksPerRow = D / 8;        // 16
  static constexpr int kTileChunks = kK * kChunksPerRow;  // 512: one per thread and tensor
  static constexpr int kTileBytes = 16 * kTileChunks;
  static constexpr int kHalf = D / 2;
  static constexpr int kSteps = D / 16;              // 8
  static constexpr int kNch = D / 32;                // 4
  static_assert(kTileChunks == kThreads, "one K and one V chunk per thread and tile");
};

__device__ __forceinline__ unsigned pin_u(unsigned& x) {
  asm volatile("" : "+v"(x));
  return x;
}
__device__ __forceinline__ void pin_f16x(f32x16& c) { asm volatile("" : "+v"(c)); }

template <bool CAUSAL, bool F16>
__global__ __launch_bounds__(B2Geom::kThreads) void attn_fwd_bf16_rb2_kernel(FwdArgs a) {
  using G = B2Geom;
  constexpr int D = G::D;
  using H = Half<F16>;
  using V8 = typename H::V8;
  __shared__ __attribute__((aligned(1024))) unsigned char k_lds[G::kSlots][G::kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char v_lds[G::kSlots][G::kTileBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  const int32_t wave_hi = key_limit<CAUSAL>(min(qw0 + G::kQW - 1, a.seq_q - 1), a.seq_q, a.seq_kv, split_end);
  int32_t rb_lo[G::kRB], lim[G::kRB];
#pragma unroll
  for (int rb = 0; rb < G::kRB; ++rb) {
    rb_lo[rb] = key_limit<CAUSAL>(min(qw0 + 32 * rb, a.seq_q - 1), a.seq_q, a.seq_kv, split_end);
    lim[rb] = key_limit<CAUSAL>(qw0 + 32 * rb + lm, a.seq_q, a.seq_kv, split_end);
  }

  // Q operands of both row blocks in registers for the whole pass.
  V8 qr[G::kRB][G::kSteps];
  {
    const unsigned flip = a.negate_q ? 0x80008000u : 0u;
#pragma unroll
    for (int rb = 0; rb < G::kRB; ++rb) {
      const unsigned short* qp = static_cast<const unsigned short*>(a.q) +
                                 head_offset(t.bh, a.heads, a.qs_b, a.qs_h) +
                                 (int64_t)min(qw0 + 32 * rb + lm, a.seq_q - 1) * a.qs_s + lh * G::kHalf;
#pragma unroll
      for (int st = 0; st < G::kSteps; ++st) {
        u32x4 x = *reinterpret_cast<const u32x4*>(qp + 8 * st);
        x ^= flip;
        qr[rb][st] = __builtin_bit_cast(V8, x);
      }
    }
  }
  wait_vmcnt<0>();

  const unsigned kv_bytes = strided_range(a.seq_kv, a.kvs_s, D, 2);
  const unsigned kv_row = (unsigned)(a.kvs_s * 2);
  const int64_t kv_off = head_offset(t.bh, a.heads, a.kvs_b, a.kvs_h);
  const __amdgpu_buffer_rsrc_t k_rsrc = raw_buffer(static_cast<const unsigned short*>(a.k) + kv_off, kv_bytes);
  const __amdgpu_buffer_rsrc_t v_rsrc = raw_buffer(static_cast<const unsigned short*>(a.v) + kv_off, kv_bytes);
  // Thread (wave, lane) fills LDS chunk p = 64 wave + lane of each tile: row rho = p / 16,
  // position pc = p % 16, holding logical chunk pc ^ swizzle of the (permuted) row.
  // The lane's source offsets are formed again at each copy from an opaque lane index
  // rather than held in registers across the step loop. LDS chunk 64 wave + lane is tile
  // row rho = 4 wave + t (t = lane / 16), position lane % 16: with bits 2 and 3 of rho
  // swapped for K, that row is 4 swap01(wave) + t, and the K swizzle 4 (wave % 4) + t and
  // the V swizzle 4 t are XORed into the position. Only t and what depends on it are
  // per lane; the rest is wave-uniform.
  static_assert(G::kChunksPerRow == 16, "row and chunk of a copied LDS chunk by shifts");
  const unsigned uw = (unsigned)wave;
  const unsigned k_row0 = 4u * ((uw & 4u) | ((uw & 1u) << 1) | ((uw & 2u) >> 1));
  auto issue_tile = [&](int32_t T) {
    unsigned ln = (unsigned)lane;
    asm volatile("" : "+v"(ln));
    const unsigned t = ln >> 4, pc = ln & 15u;
    const unsigned tk = t * kv_row;
    const unsigned tile_ofs = (unsigned)(ks + T * G::kK) * kv_row;
    const int slot = T % G::kSlots;
    dma_load_x4(k_rsrc, tk + 16u * (pc ^ (4u * (uw & 3u) + t)) + (tile_ofs + k_row0 * kv_row),
                lds_address(&k_lds[slot][1024 * wave]));
    dma_load_x4(v_rsrc, tk + 16u * (pc ^ (4u * t)) + (tile_ofs + 4u * uw * kv_row),
                lds_address(&v_lds[slot][1024 * wave]));
  };

  f32x16 oacc[G::kRB][G::kNch];
#pragma unroll
  for (int rb = 0; rb < G::kRB; ++rb)
#pragma unroll
    for (int cb = 0; cb < G::kNch; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[rb][cb][r] = 0.f;
  float m_run[G::kRB], l_run[G::kRB];
#pragma unroll
  for (int rb = 0; rb < G::kRB; ++rb) {
    m_run[rb] = -INFINITY;
    l_run[rb] = 0.f;
  }
  const float c = fmaxf(a.c, 1.17549435e-38f);

  // Lane parts of the LDS addresses (tile bases are multiples of 1 KB):
  //  - K row read, logical chunk lh*8 + st of row lm: position (lh*8 + st) ^ (lm & 15), so
  //    the byte offset is k_lane ^ 16 st;
  //  - V^T transposing read of k-step t2 and output chunk cb: rows 16 t2 + 8 lh + s/4 (and
  //    + 4), chunk 4 cb + colq, swizzled by 4 (s/4); the byte offset is
  //    (v_lane ^ 64 cb) + 4096 t2 (+ 1024 for the second row).
  const int srole = lane & 15;
  const int colq = 2 * ((lane >> 4) & 1) + ((srole & 3) >> 1);
  const unsigned k_lane = (unsigned)(lm * 2 * D + 16 * (8 * lh ^ (lm & 15)));
  const unsigned v_lane = (unsigned)((8 * lh + srole / 4) * 2 * D + 64 * (srole / 4) + 16 * colq + 8 * (srole & 1));

  // O^T += V^T P^T for both row blocks: each V^T operand feeds two MFMAs.
  auto pv_tile = [&](int slot, const V8 (&pb)[G::kRB][2]) {
    unsigned vb = lds_address(&v_lds[slot][0]) + v_lane;
    auto v_operand = [&](int i) {  // i = 4 t2 + cb
      const int t2 = i / G::kNch, cb = i % G::kNch;
      const unsigned x = (pin_u(vb) ^ (64u * (unsigned)cb)) + 4096u * (unsigned)t2;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(size_t)x);
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(size_t)(x + 1024u));
      const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
      return __builtin_bit_cast(V8, u32x4{lo2[0], lo2[1], hi2[0], hi2[1]});
    };
    constexpr int kN = 2 * G::kNch;  // V^T operands per tile
    constexpr int kPf = 2;
    V8 vop[kPf + 1];
#pragma unroll
    for (int i = 0; i < kPf; ++i) vop[i] = v_operand(i);
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      if (i + kPf < kN) vop[(i + kPf) % (kPf + 1)] = v_operand(i + kPf);
      __builtin_amdgcn_sched_barrier(0);
      const int t2 = i / G::kNch, cb = i % G::kNch;
#pragma unroll
      for (int rb = 0; rb < G::kRB; ++rb) {
        oacc[rb][cb] = H::mfma(vop[i % (kPf + 1)], pb[rb][t2], oacc[rb][cb]);
        pin_f16x(oacc[rb][cb]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // Scores of both row blocks, lazy running max and probabilities of tile T.
  auto scores_and_p = [&](int32_t T, int slot, V8 (&pb)[G::kRB][2]) {
    const int32_t j0 = ks + T * G::kK;
    f32x16 sacc[G::kRB];
#pragma unroll
    for (int rb = 0; rb < G::kRB; ++rb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[rb][r] = 0.f;
    unsigned kb = lds_address(&k_lds[slot][0]) + k_lane;
    auto k_operand = [&](int st) {
      const unsigned x = pin_u(kb) ^ (16u * (unsigned)st);
      return __builtin_bit_cast(V8, *(__attribute__((address_space(3))) const u32x4*)(size_t)x);
    };
    constexpr int kPf = 1;  // each K operand feeds two MFMAs: one step ahead is two MFMAs
    V8 kop[kPf + 1];
#pragma unroll
    for (int st = 0; st < kPf; ++st) kop[st] = k_operand(st);
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int st = 0; st < G::kSteps; ++st) {
      if (st + kPf < G::kSteps) kop[(st + kPf) % (kPf + 1)] = k_operand(st + kPf);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int rb = 0; rb < G::kRB; ++rb) {
        sacc[rb] = H::mfma(kop[st % (kPf + 1)], qr[rb][st], sacc[rb]);
        pin_f16x(sacc[rb]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);

#pragma unroll
    for (int rb = 0; rb < G::kRB; ++rb) {
      if (j0 + G::kK > rb_lo[rb]) {
        int32_t rel = lim[rb] - j0 - 8 * lh;  // key 16(r/8) + r%8 (+ 8 lh) allowed iff < rel
        asm volatile("" : "+v"(rel));
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[rb][r] = (16 * (r / 8) + (r % 8) < rel) ? sacc[rb][r] : -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[rb][r]);
      {
        // The two key halves of query m (lanes m and m + 32). Scores are never NaN, so a
        // plain v_max_f32 does without the canonicalizing maxes fmaxf would add.
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        asm("v_max_f32 %0, %1, %2" : "=v"(mx) : "v"(__uint_as_float(sw[0])), "v"(__uint_as_float(sw[1])));
      }
      const float tmax = mx * c;  // c > 0: -inf stays -inf
      if (__any(tmax > m_run[rb] + kTau)) {
        const float m_new = fmaxf(m_run[rb], tmax);
        const float alpha = __builtin_amdgcn_exp2f(m_run[rb] - (m_new == -INFINITY ? 0.f : m_new));
        l_run[rb] *= alpha;
#pragma unroll
        for (int cb = 0; cb < G::kNch; ++cb)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[rb][cb][r] *= alpha;
        m_run[rb] = m_new;
      }
      const float neg_m = m_run[rb] == -INFINITY ? 0.f : -m_run[rb];
      float psum = 0.f;
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[rb][8 * t2 + e], c, neg_m));
          psum += p;
          pb[rb][t2][e] = (typename H::E)p;
        }
      l_run[rb] += psum;
    }
  };

  // Waves 4-7 (each sharing a SIMD with wave - 4) run a tile's P V product at the start of
  // the next step. Each role has its own copy of the step loop, so that the late waves'
  // held probabilities are not live across the other role's score chain.
  auto run_steps = [&](auto late_c) {
    constexpr bool kLate = decltype(late_c)::value;
    V8 pb_late[G::kRB][2];
    bool late_pending = false;
    int late_slot = 0;
    if (ntiles > 0) issue_tile(0);
    if (ntiles > 1) issue_tile(1);
    for (int32_t T = 0; T < ntiles; ++T) {
      // One barrier per pair of tiles: at an even step both tiles of the pair have
      // landed (nothing else is in flight) and the next pair goes into slots whose
      // tiles every wave finished two or more steps ago.
      if ((T & 1) == 0) {
        wait_vmcnt<0>();
        __syncthreads();
        if (T + 2 < ntiles) issue_tile(T + 2);
        if (T + 3 < ntiles) issue_tile(T + 3);
      }
      if (kLate && late_pending) {
        pv_tile(late_slot, pb_late);
        late_pending = false;
      }
      const int slot = T % G::kSlots;
      if (wave_live && ks + T * G::kK < wave_hi) {
        V8 pb[G::kRB][2];
        scores_and_p(T, slot, pb);
        if constexpr (kLate) {
#pragma unroll
          for (int rb = 0; rb < G::kRB; ++rb)
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2) pb_late[rb][t2] = pb[rb][t2];
          late_pending = true;
          late_slot = slot;
        } else {
          pv_tile(slot, pb);
        }
      }
    }
    if (kLate && late_pending) pv_tile(late_slot, pb_late);
  };
  if (wave >= G::kWaves / 2) run_steps(std::true_type{});
  else run_steps(std::false_type{});

#pragma unroll
  for (int rb = 0; rb < G::kRB; ++rb) {
    const float l_tot = l_run[rb] + __shfl_xor(l_run[rb], 32);
    const int32_t row = qw0 + 32 * rb + lm;
    if (!wave_live || row >= a.seq_q) continue;
    const bool empty = !(l_tot > 0.f);
    const float inv = empty ? 0.f : 1.0f / l_tot;
    const float lse2 = empty ? -INFINITY : m_run[rb] + __builtin_amdgcn_logf(l_tot);
    const size_t row_id = (size_t)t.bh * a.seq_q + row;
    float* orow = nullptr;
    unsigned short* orow16 = nullptr;
    if (a.nsplit == 1) {
      const int64_t o_off = head_offset(t.bh, a.heads, a.qs_b, a.qs_h) + (int64_t)row * a.qs_s;
      if (a.o_bf16) orow16 = a.o_bf16 + o_off;
      else orow = a.o + o_off;
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
        for (int e = 0; e < 4; ++e) out[e] = empty ? 0.f : oacc[rb][cb][4 * g4 + e] * inv;
        if (orow16)
          *reinterpret_cast<u32x2*>(orow16 + 32 * cb + 8 * g4 + 4 * lh) =
              u32x2{pack_out16(out[0], out[1], a.o_f16), pack_out16(out[2], out[3], a.o_f16)};
        else
          *reinterpret_cast<f32x4*>(orow + 32 * cb + 8 * g4 + 4 * lh) = out;
      }
  }
}

template <bool CAUSAL>
hipError_t launch_bf16_rb2(const FwdArgs& a, bool f16, hipStream_t s) {
  const dim3 grid(a.nwg), block(B2Geom::kThreads);
  if (f16) hipLaunchKernelGGL((attn_fwd_bf16_rb2_kernel<CAUSAL, true>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((attn_fwd_bf16_rb2_kernel<CAUSAL, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_bf16_variant(const FwdArgs& a, bool f16, hipStream_t s) {
  const dim3 grid(a.nwg), block(BGeom<D>::kThreads);
  if (a.mask_bits) {
    if (f16) hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, CAUSAL, true, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, CAUSAL, false, true>), grid, block, 0, s, a);
  } else if constexpr (D == 128) {  // head dim 128 without a mask runs attn_fwd_bf16_rb2_kernel
    return hipErrorInvalidValue;
  } else {
    if (f16) hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, CAUSAL, true, false>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, CAUSAL, false, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, int head_dim, bool causal, bool f16, hipStream_t s) {
  switch (head_dim) {
    case 32: return causal ? launch_bf16_variant<32, true>(a, f16, s) : launch_bf16_variant<32, false>(a, f16, s);
    case 64: return causal ? launch_bf16_variant<64, true>(a, f16, s) : launch_bf16_variant<64, false>(a, f16, s);
    case 128:  // with a hard mask the 32-row kernel (the planner's geometry follows)
      if (a.mask_bits) return causal ? launch_bf16_variant<128, true>(a, f16, s) : launch_bf16_variant<128, false>(a, f16, s);
      return causal ? launch_bf16_rb2<true>(a, f16, s) : launch_bf16_rb2<false>(a, f16, s);
    case 256: return causal ? launch_bf16_rs<true>(a, f16, s) : launch_bf16_rs<false>(a, f16, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sma
