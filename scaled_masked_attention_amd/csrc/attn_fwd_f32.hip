// Attention forward, fp32 inputs, fp32 MFMA (v_mfma_f32_32x32x2_f32), gfx950.
//
// Computes, per (batch, head), O = softmax(scale * Q K^T + mask) V with the
// max-subtracted row softmax streamed over key tiles (online softmax), the
// bottom-right causal mask, and all-zero rows where no key is admitted
// (oxicuda ComputeBackend `attention`; pulsatrix HIPBackend `softmax_rows`,
// `logsumexp_rows`; TorchLean hard-masked softmax).
//
// Workgroup: 4 waves x 32 query rows = 128 rows of one (batch, head), with a
// range of keys (all of them, or one split). Key tiles of 32 rows stream
// HBM/L2 -> LDS with direct-to-LDS loads (no registers on the way; double
// buffered, one barrier per tile): tile t+1 is in flight while tile t is used.
//
// Each wave computes S^T = K Q^T for its 32 queries and a 32-key tile: lane
// (m, h) = (lane % 32, lane / 32) supplies K[key m] and Q[query m] along head
// dims h*D/2 .. h*D/2 + D/2 - 1, and receives the scores of query (lane % 32)
// for keys 8*(r/4) + 4*h + r%4, r = 0..15. The row max therefore needs one
// exchange with lane ^ 32, and the probabilities are already in the layout
// of the B operand of O^T += V^T P^T, in which register r is the key step.
// Head dim c of the output is mapped as c = (D/32) * m + chunk, so each lane
// reads the V operands of all chunks with one contiguous LDS load.
#include "attn_common.h"

namespace sma {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

template <int D>
struct F32Geom {
  static constexpr int kWaves = 4;
  static constexpr int kQW = 32;                    // query rows per wave
  static constexpr int kQ = kWaves * kQW;           // query rows per workgroup
  static constexpr int kK = kF32KeysPerTile;        // keys per tile
  static constexpr int kHalf = D / 2;               // head dims per lane half in QK^T
  static constexpr int kNch = D / 32;               // 32-wide output chunks
  static constexpr int kChunks = D / 4;             // 16-byte chunks per row
  static constexpr int kDma = kK * D * 4 / 1024;    // 1 KB copy instructions per tile and tensor
  static constexpr int kDmaPerWave = kDma / kWaves;
  static constexpr int kRowsPerDma = 64 / kChunks;  // rows one copy instruction covers
  static_assert(kQ == kF32QueriesPerWG, "planner geometry");
  static_assert(kDmaPerWave >= 1 && kDmaPerWave * kWaves == kDma, "tile split");
};

// K tiles in LDS use the fp32 tile swizzle (tile_swz: row r's 16-byte chunk
// c at position c ^ tile_swz(r)), so the 16 lanes of each ds_read_b128 group
// in the QK^T operand read hit 64 different banks. V tiles are stored as they
// are: a half-wave reads one whole row, the other half the row 4 below, and
// each group of 16 lanes reads 256 consecutive bytes.

// D/32 consecutive floats: a lane's share of one output row, or of one V row.
template <int N>
struct FVec {
  typedef float T __attribute__((ext_vector_type(N)));
};

// Lazy max: the running max moves only when a tile raises it by more than
// this many log2 units, so most tiles skip the rescale of O. Probabilities
// stay below 2^kTau, far from fp32 overflow; the result is unchanged because
// numerator and denominator share the stale max.
constexpr float kTau = 8.0f;

template <int D, bool CAUSAL, bool MASKED>
__global__ __launch_bounds__(256) void attn_fwd_f32_kernel(FwdArgs a) {
  using G = F32Geom<D>;
  using VecN = typename FVec<G::kNch>::T;
  __shared__ __attribute__((aligned(16))) float k_lds[2][G::kK * D];
  __shared__ __attribute__((aligned(16))) float v_lds[2][G::kK * D];

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

  // Keys this workgroup must visit: up to the limit of its last real row.
  const int32_t wg_last_row = min(q0 + G::kQ - 1, a.seq_q - 1);
  const int32_t ke = key_limit<CAUSAL>(wg_last_row, a.seq_q, a.seq_kv, split_end);
  const int32_t ntiles = ke > ks ? (ke - ks + G::kK - 1) / G::kK : 0;

  const bool wave_live = qw0 < a.seq_q;
  const int32_t my_row = qw0 + lm;
  const int32_t ld_row = min(my_row, a.seq_q - 1);
  const int32_t lim = key_limit<CAUSAL>(my_row, a.seq_q, a.seq_kv, split_end);
  const int32_t wave_lo = key_limit<CAUSAL>(qw0, a.seq_q, a.seq_kv, split_end);
  const int32_t wave_hi = key_limit<CAUSAL>(min(qw0 + G::kQW - 1, a.seq_q - 1), a.seq_q,
                                            a.seq_kv, split_end);

  // This lane's half of its query row, kept in registers for the whole pass.
  float qr[G::kHalf];
  {
    const float* qp = static_cast<const float*>(a.q) + head_offset(t.bh, a.heads, a.qs_b, a.qs_h) +
                      (int64_t)ld_row * a.qs_s + lh * G::kHalf;
#pragma unroll
    for (int u = 0; u < G::kHalf / 4; ++u) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(qp + 4 * u);
      qr[4 * u + 0] = x[0];
      qr[4 * u + 1] = x[1];
      qr[4 * u + 2] = x[2];
      qr[4 * u + 3] = x[3];
    }
    if (a.negate_q) {
#pragma unroll
      for (int i = 0; i < G::kHalf; ++i) qr[i] = -qr[i];
    }
  }

  const int64_t kv_off = head_offset(t.bh, a.heads, a.kvs_b, a.kvs_h);
  // With a hard mask: this row's packed admission words (one per 32 keys).
  const uint32_t* mrow = nullptr;
  if (MASKED)
    mrow = a.mask_bits + head_offset(t.bh, a.heads, a.mbits_sb, a.mbits_sh) +
           (int64_t)ld_row * a.mask_words;
  const float* kg = static_cast<const float*>(a.k) + kv_off;
  const float* vg = static_cast<const float*>(a.v) + kv_off;
  const unsigned kv_row = (unsigned)(a.kvs_s * 4);  // bytes between key rows

  // Copy key tile `tile` into LDS buffer `buf`. The buffer resources start at
  // the tile's first row and end after its last real one, so rows past seq_kv
  // read as zeros (such keys are always excluded) and the 32-bit offsets stay
  // within one tile. Lane l of instruction i (of this wave) fills LDS chunk
  // position p = 64*(i*waves + wave) + l: row p / chunks, position p % chunks.
  auto issue_tile = [&](int32_t tile, int buf) {
    const int32_t j0 = ks + tile * G::kK;
    const int32_t rows = min(G::kK, a.seq_kv - j0);
    const unsigned bytes = strided_range(rows, a.kvs_s, D, 4);
    const __amdgpu_buffer_rsrc_t k_rsrc = raw_buffer(kg + (int64_t)j0 * a.kvs_s, bytes);
    const __amdgpu_buffer_rsrc_t v_rsrc = raw_buffer(vg + (int64_t)j0 * a.kvs_s, bytes);
#pragma unroll
    for (int i = 0; i < G::kDmaPerWave; ++i) {
      const int ti = i * G::kWaves + wave;
      const int r = ti * G::kRowsPerDma + lane / G::kChunks;
      const int c = lane % G::kChunks;
      dma_load_x4(k_rsrc, (unsigned)r * kv_row + 16u * (unsigned)(c ^ tile_swz<D>(r)),
                  lds_address(&k_lds[buf][256 * ti]));
      dma_load_x4(v_rsrc, (unsigned)r * kv_row + 16u * (unsigned)c, lds_address(&v_lds[buf][256 * ti]));
    }
  };

  f32x16 oacc[G::kNch];
#pragma unroll
  for (int cb = 0; cb < G::kNch; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[cb][r] = 0.f;
  float m_run = -INFINITY;  // running row max, log2 units (shared by both lane halves)
  float l_run = 0.f;        // this lane half's share of the row denominator

  // The mask word of the tile about to be used is loaded one tile ahead, so
  // that its wait (which the compiler places, counting only its own loads)
  // never waits for a tile copy as well.
  uint32_t mword_next = 0u;
  if (ntiles > 0) {
    issue_tile(0, 0);
    if (MASKED) mword_next = mrow[ks >> 5];
    wait_vmcnt<0>();
  }
  __syncthreads();

  for (int32_t it = 0; it < ntiles; ++it) {
    const int buf = it & 1;
    uint32_t mword = ~0u;
    if (MASKED) {
      mword = mword_next;
      asm volatile("" : "+v"(mword));  // consumed here: no copy is in flight yet
    }
    // Buffer buf ^ 1 was last read in the previous iteration, before its barrier.
    if (it + 1 < ntiles) issue_tile(it + 1, buf ^ 1);
    const int32_t j0 = ks + it * G::kK;
    if (wave_live && j0 < wave_hi) {
      // S^T tile = K Q^T over the head dim.
      f32x16 s;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = 0.f;
      const float* krow = &k_lds[buf][lm * D];
#pragma unroll
      for (int u = 0; u < G::kHalf / 4; ++u) {
        const int c = lh * (G::kHalf / 4) + u;  // this lane half's chunk u
        const f32x4 kk = *reinterpret_cast<const f32x4*>(krow + 4 * (c ^ tile_swz<D>(lm)));
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(kk[0], qr[4 * u + 0], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(kk[1], qr[4 * u + 1], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(kk[2], qr[4 * u + 2], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(kk[3], qr[4 * u + 3], s, 0, 0, 0);
      }
      // Scale into log2 units, then exclude masked keys from max and sum.
      float tv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) tv[r] = s[r] * a.c;
      if (j0 + G::kK > wave_lo) {
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
      {  // lanes m and m + 32 hold the two key halves of query m (VALU swap, no LDS round trip)
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                         false, false);
        mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      }
      const bool raise = mx > m_run + kTau;
      if (__any(raise)) {
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
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
      // O^T += V^T P^T: key step r pairs this lane's probability with V row
      // 8*(r/4) + 4*h + r%4; its head dims (D/32)*m .. + D/32 - 1 are contiguous.
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int vrow = 8 * (r / 4) + 4 * lh + (r % 4);
        const VecN vv = *reinterpret_cast<const VecN*>(&v_lds[buf][vrow * D + G::kNch * lm]);
#pragma unroll
        for (int cb = 0; cb < G::kNch; ++cb)
          oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv[cb], tv[r], oacc[cb], 0, 0, 0);
      }
    }
    if (it + 1 < ntiles) {
      if (MASKED) mword_next = mrow[(j0 + G::kK) >> 5];
      wait_vmcnt<0>();  // this wave's copies of tile it + 1 (and the mask word) have landed
    }
    __syncthreads();  // everyone's copies landed; everyone is done with buffer buf
  }

  // Epilogue: combine the two lane halves' denominators, normalise, write.
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
  for (int r = 0; r < 16; ++r) {
    const int m = 8 * (r / 4) + 4 * lh + (r % 4);
    VecN out;
#pragma unroll
    for (int cb = 0; cb < G::kNch; ++cb) out[cb] = empty ? 0.f : oacc[cb][r] * inv;
    if (orow16) {
      if constexpr (G::kNch == 1) {
        orow16[m] = (unsigned short)(pack_out16(out[0], 0.f, a.o_f16) & 0xffffu);
      } else {
        typedef unsigned PackedT __attribute__((ext_vector_type(G::kNch / 2)));
        PackedT packed;
#pragma unroll
        for (int i = 0; i < G::kNch / 2; ++i) packed[i] = pack_out16(out[2 * i], out[2 * i + 1], a.o_f16);
        *reinterpret_cast<PackedT*>(orow16 + G::kNch * m) = packed;
      }
    } else {
      *reinterpret_cast<VecN*>(orow + G::kNch * m) = out;
    }
  }
}

template <int D, bool CAUSAL>
hipError_t launch_f32_variant(const FwdArgs& a, hipStream_t s) {
  if (a.mask_bits)
    hipLaunchKernelGGL((attn_fwd_f32_kernel<D, CAUSAL, true>), dim3(a.nwg), dim3(kThreadsPerWG), 0, s, a);
  else
    hipLaunchKernelGGL((attn_fwd_f32_kernel<D, CAUSAL, false>), dim3(a.nwg), dim3(kThreadsPerWG), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, int head_dim, bool causal, hipStream_t s) {
  switch (head_dim) {
    case 32: return causal ? launch_f32_variant<32, true>(a, s) : launch_f32_variant<32, false>(a, s);
    case 64: return causal ? launch_f32_variant<64, true>(a, s) : launch_f32_variant<64, false>(a, s);
    case 128: return causal ? launch_f32_variant<128, true>(a, s) : launch_f32_variant<128, false>(a, s);
    case 256: return causal ? launch_f32_variant<256, true>(a, s) : launch_f32_variant<256, false>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sma
