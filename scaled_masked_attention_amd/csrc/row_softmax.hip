// Row primitives on a materialised (rows x cols) fp32 score matrix, gfx950:
//   softmax_rows / logsumexp_rows (pulsatrix HIPBackend: max-subtracted row
//   softmax and per-row log-sum-exp), the hard-masked row softmax (TorchLean
//   "CUDA Buffer Kernels FFI": max and denominator over admitted entries,
//   blocked entries exactly zero, a row admitting nothing all zeros) and the
//   fused scale + causal mask + softmax (MicroGPT CuBLASBackend
//   `fused_attn_softmax`, bottom-right causal alignment as in attention),
//   and the softmax backward from the forward's output (pulsatrix
//   `softmax_rows_backward`; with a scale, the backward of MicroGPT's fused
//   scale + mask + softmax): dx_j = scale * y_j * (dy_j - sum_k y_k dy_k).
//
// HBM-bound: a row is read once and written once when it fits in the
// registers of its team (a wave for rows up to 4096 floats, a 256-thread
// workgroup up to 16384), else read twice (online max and sum, then the
// normalised write). Arithmetic per admitted entry, with sgn = sign(scale):
//   s = sgn * x (an input of -infinity stays -infinity), m = max s,
//   p = 2^((s - m) * |c|) / sum, c = scale * log2(e),
// so the max is subtracted in input units before scaling (exact for nearby
// values) and -infinity inputs weigh an exact zero whatever the scale.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sma_kernels.h"

namespace sma {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLn2 = 0.69314718055994530942f;

template <int N>
struct Vec;
template <>
struct Vec<1> {
  typedef float T;
  static __device__ __forceinline__ float get(const T& v, int) { return v; }
  static __device__ __forceinline__ void set(T& v, int, float x) { v = x; }
};
template <>
struct Vec<4> {
  typedef f32x4 T;
  static __device__ __forceinline__ float get(const T& v, int e) { return v[e]; }
  static __device__ __forceinline__ void set(T& v, int e, float x) { v[e] = x; }
};

// Streaming memory access. Every output row is written with non-temporal
// stores (it is not read again by this launch), which measured 12-17 %
// faster on 512-column rows and no slower elsewhere. A register-resident row
// of a 256-thread team is also read with non-temporal loads (1-3 % faster
// there); shorter rows, and logsumexp (no store stream), use ordinary loads,
// which measured faster for them.
template <bool NT, class T>
__device__ __forceinline__ T load_row(const float* p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const T*>(p));
  else return *reinterpret_cast<const T*>(p);
}
template <class T>
__device__ __forceinline__ void store_row(float* p, const T& v) {
  __builtin_nontemporal_store(v, reinterpret_cast<T*>(p));
}

// Keys j < limit are admitted by the causal mask (bottom-right: j <= r + cols
// - rows_per_matrix for row r of its matrix); every key without the mask.
__device__ __forceinline__ int32_t causal_limit(const RowArgs& a, int64_t row) {
  if (!a.causal) return a.cols;
  const int64_t r = row % a.rows_per_matrix;
  const int64_t hi = r + (int64_t)a.cols - (int64_t)a.rows_per_matrix + 1;
  return (int32_t)(hi < 0 ? 0 : (hi > a.cols ? a.cols : hi));
}

// Admission of element j (mask entry already loaded as mval; lim from causal_limit).
template <int MODE>
__device__ __forceinline__ bool admitted(int32_t j, float mval, int32_t lim) {
  if (MODE == kRowMasked) return mval != 0.0f;
  if (MODE == kRowScaled) return j < lim;
  return true;
}

// Signed score in input units: -infinity for an input of -infinity.
__device__ __forceinline__ float signed_score(float x, float sgn) {
  return x == -INFINITY ? -INFINITY : sgn * x;
}

// Reduction over a team of TEAM lanes (a wave, or a 256-thread workgroup via LDS).
template <int TEAM>
__device__ __forceinline__ float team_max(float v, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  if (TEAM == 256) {
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    v = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  }
  return v;
}
template <int TEAM>
__device__ __forceinline__ float team_sum(float v, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  if (TEAM == 256) {
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[4 + w] = v;
    __syncthreads();
    v = (red[4] + red[5]) + (red[6] + red[7]);
  }
  return v;
}

// Register-resident rows: each lane holds E vectors of VEC floats of its row,
// element j = VEC * (lane_in_team + TEAM * k) + e.
template <int MODE, int VEC, int E, int TEAM>
__global__ __launch_bounds__(256) void row_softmax_kernel(RowArgs a) {
  using V = Vec<VEC>;
  using VT = typename V::T;
  __shared__ float red[8];
  constexpr int kRowsPerWG = 256 / TEAM;
  const int t = threadIdx.x % TEAM;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerWG + threadIdx.x / TEAM;
  const bool live = row < a.rows;  // uniform per team
  const float sgn = a.c < 0.f ? -1.f : 1.f;
  const float cabs = fabsf(a.c);
  const float* xr = a.in + (live ? row : 0) * (int64_t)a.cols;
  const float* mr = MODE == kRowMasked ? a.mask + (live ? row : 0) * (int64_t)a.cols : nullptr;
  const int32_t lim = MODE == kRowScaled ? causal_limit(a, live ? row : 0) : a.cols;

  constexpr bool kNtLoad = TEAM == 256 && MODE != kRowLse;
  VT s[E];
  float m = -INFINITY;
#pragma unroll
  for (int k = 0; k < E; ++k) {
    const int32_t j0 = VEC * (t + TEAM * k);
    VT x, mv;
    if (live && j0 < a.cols) {
      x = load_row<kNtLoad, VT>(xr + j0);
      if (MODE == kRowMasked) mv = load_row<kNtLoad, VT>(mr + j0);
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) V::set(x, e, -INFINITY);
      if (MODE == kRowMasked) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) V::set(mv, e, 0.f);
      }
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const int32_t j = j0 + e;
      const float mval = MODE == kRowMasked ? V::get(mv, e) : 1.f;
      const bool ok = j < a.cols && admitted<MODE>(j, mval, lim);
      const float sc = ok ? signed_score(V::get(x, e), sgn) : -INFINITY;
      V::set(s[k], e, sc);
      m = fmaxf(m, sc);
    }
  }
  m = team_max<TEAM>(m, red);
  const bool empty = m == -INFINITY;
  float l = 0.f;
#pragma unroll
  for (int k = 0; k < E; ++k)
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const float sc = V::get(s[k], e);
      const float p = (empty || sc == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((sc - m) * cabs);
      V::set(s[k], e, p);
      l += p;
    }
  l = team_sum<TEAM>(l, red);
  if (!live) return;
  if (MODE == kRowLse) {
    if (t == 0) a.out[row] = empty ? -INFINITY : m + __builtin_amdgcn_logf(l) * kLn2;
    return;
  }
  const float inv = empty ? 0.f : 1.0f / l;
  float* orow = a.out + row * (int64_t)a.cols;
#pragma unroll
  for (int k = 0; k < E; ++k) {
    const int32_t j0 = VEC * (t + TEAM * k);
    if (j0 < a.cols) {
      VT o;
#pragma unroll
      for (int e = 0; e < VEC; ++e) V::set(o, e, V::get(s[k], e) * inv);
      store_row(orow + j0, o);
    }
  }
}

// Rows longer than a team's registers: a workgroup per row, two passes.
template <int MODE, int VEC>
__global__ __launch_bounds__(256) void row_softmax_stream_kernel(RowArgs a) {
  using V = Vec<VEC>;
  using VT = typename V::T;
  __shared__ float red[8];
  const int t = threadIdx.x;
  const int64_t row = blockIdx.x;
  const float sgn = a.c < 0.f ? -1.f : 1.f;
  const float cabs = fabsf(a.c);
  const float* xr = a.in + row * (int64_t)a.cols;
  const float* mr = MODE == kRowMasked ? a.mask + row * (int64_t)a.cols : nullptr;
  const int32_t lim = MODE == kRowScaled ? causal_limit(a, row) : a.cols;
  constexpr int kStep = 256 * VEC;

  // Pass 1: running max and sum per lane (sum relative to the lane's max).
  float m = -INFINITY, l = 0.f;
  for (int32_t j0 = VEC * t; j0 < a.cols; j0 += kStep) {
    const VT x = *reinterpret_cast<const VT*>(xr + j0);
    VT mv;
    if (MODE == kRowMasked) mv = *reinterpret_cast<const VT*>(mr + j0);
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const int32_t j = j0 + e;
      const float mval = MODE == kRowMasked ? V::get(mv, e) : 1.f;
      if (!admitted<MODE>(j, mval, lim)) continue;
      const float sc = signed_score(V::get(x, e), sgn);
      if (sc == -INFINITY) continue;
      if (sc > m) {
        l = (m == -INFINITY ? 0.f : l * __builtin_amdgcn_exp2f((m - sc) * cabs)) + 1.f;
        m = sc;
      } else {
        l += __builtin_amdgcn_exp2f((sc - m) * cabs);
      }
    }
  }
  const float mt = team_max<256>(m, red);
  l = team_sum<256>(m == -INFINITY ? 0.f : l * __builtin_amdgcn_exp2f((m - mt) * cabs), red);
  m = mt;
  const bool empty = m == -INFINITY;
  if (MODE == kRowLse) {
    if (t == 0) a.out[row] = empty ? -INFINITY : m + __builtin_amdgcn_logf(l) * kLn2;
    return;
  }
  // Pass 2: normalised probabilities (each element is read before its own write).
  const float inv = empty ? 0.f : 1.0f / l;
  float* orow = a.out + row * (int64_t)a.cols;
  for (int32_t j0 = VEC * t; j0 < a.cols; j0 += kStep) {
    const VT x = *reinterpret_cast<const VT*>(xr + j0);
    VT mv;
    if (MODE == kRowMasked) mv = *reinterpret_cast<const VT*>(mr + j0);
    VT o;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const int32_t j = j0 + e;
      const float mval = MODE == kRowMasked ? V::get(mv, e) : 1.f;
      const bool ok = admitted<MODE>(j, mval, lim);
      const float sc = ok ? signed_score(V::get(x, e), sgn) : -INFINITY;
      const float p = (empty || sc == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((sc - m) * cabs) * inv;
      V::set(o, e, p);
    }
    store_row(orow + j0, o);
  }
}

// Softmax backward, register-resident rows: each lane holds E vectors of VEC
// floats of y and of dy (element j = VEC * (lane_in_team + TEAM * k) + e),
// the row's dot product is reduced over the team, and dx is written from
// the registers. Every input is read before any output is written, so dx
// may be y or dy.
template <int VEC, int E, int TEAM>
__global__ __launch_bounds__(256) void row_softmax_bwd_kernel(RowBwdArgs a) {
  using V = Vec<VEC>;
  using VT = typename V::T;
  __shared__ float red[8];
  constexpr int kRowsPerWG = 256 / TEAM;
  const int t = threadIdx.x % TEAM;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerWG + threadIdx.x / TEAM;
  const bool live = row < a.rows;  // uniform per team
  const float* yr = a.y + (live ? row : 0) * (int64_t)a.cols;
  const float* gr = a.dy + (live ? row : 0) * (int64_t)a.cols;
  VT y[E], g[E];
  float dot = 0.f;
#pragma unroll
  for (int k = 0; k < E; ++k) {
    const int32_t j0 = VEC * (t + TEAM * k);
    if (live && j0 < a.cols) {
      y[k] = load_row<TEAM == 256, VT>(yr + j0);
      g[k] = load_row<TEAM == 256, VT>(gr + j0);
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        V::set(y[k], e, 0.f);
        V::set(g[k], e, 0.f);
      }
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) dot = __builtin_fmaf(V::get(y[k], e), V::get(g[k], e), dot);
  }
  dot = team_sum<TEAM>(dot, red);
  if (!live) return;
  float* orow = a.dx + row * (int64_t)a.cols;
#pragma unroll
  for (int k = 0; k < E; ++k) {
    const int32_t j0 = VEC * (t + TEAM * k);
    if (j0 < a.cols) {
      VT o;
#pragma unroll
      for (int e = 0; e < VEC; ++e)
        V::set(o, e, a.scale * (V::get(y[k], e) * (V::get(g[k], e) - dot)));
      store_row(orow + j0, o);
    }
  }
}

// Softmax backward of rows longer than a team's registers: a workgroup per
// row, the dot product in a first pass, dx in a second (each element is read
// by the thread that then writes it, after the first pass has ended).
template <int VEC>
__global__ __launch_bounds__(256) void row_softmax_bwd_stream_kernel(RowBwdArgs a) {
  using V = Vec<VEC>;
  using VT = typename V::T;
  __shared__ float red[8];
  const int t = threadIdx.x;
  const int64_t row = blockIdx.x;
  const float* yr = a.y + row * (int64_t)a.cols;
  const float* gr = a.dy + row * (int64_t)a.cols;
  constexpr int kStep = 256 * VEC;
  float dot = 0.f;
  for (int32_t j0 = VEC * t; j0 < a.cols; j0 += kStep) {
    const VT y = *reinterpret_cast<const VT*>(yr + j0);
    const VT g = *reinterpret_cast<const VT*>(gr + j0);
#pragma unroll
    for (int e = 0; e < VEC; ++e) dot = __builtin_fmaf(V::get(y, e), V::get(g, e), dot);
  }
  dot = team_sum<256>(dot, red);
  float* orow = a.dx + row * (int64_t)a.cols;
  for (int32_t j0 = VEC * t; j0 < a.cols; j0 += kStep) {
    const VT y = *reinterpret_cast<const VT*>(yr + j0);
    const VT g = *reinterpret_cast<const VT*>(gr + j0);
    VT o;
#pragma unroll
    for (int e = 0; e < VEC; ++e) V::set(o, e, a.scale * (V::get(y, e) * (V::get(g, e) - dot)));
    store_row(orow + j0, o);
  }
}

template <int VEC, int E, int TEAM>
hipError_t launch_bwd_resident(const RowBwdArgs& a, hipStream_t st) {
  const int64_t nwg = (a.rows + (256 / TEAM) - 1) / (256 / TEAM);
  hipLaunchKernelGGL((row_softmax_bwd_kernel<VEC, E, TEAM>), dim3((uint32_t)nwg), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int VEC, int TEAM>
hipError_t launch_bwd_team(const RowBwdArgs& a, int e, hipStream_t st) {
  switch (e) {
    case 1: return launch_bwd_resident<VEC, 1, TEAM>(a, st);
    case 2: return launch_bwd_resident<VEC, 2, TEAM>(a, st);
    case 4: return launch_bwd_resident<VEC, 4, TEAM>(a, st);
    case 8: return launch_bwd_resident<VEC, 8, TEAM>(a, st);
    case 16: return launch_bwd_resident<VEC, 16, TEAM>(a, st);
    default: return hipErrorInvalidValue;
  }
}

template <int VEC>
hipError_t launch_bwd_vec(const RowBwdArgs& a, const RowPlan& p, hipStream_t st) {
  if (p.stream) {
    hipLaunchKernelGGL((row_softmax_bwd_stream_kernel<VEC>), dim3((uint32_t)a.rows), dim3(256), 0, st, a);
    return hipGetLastError();
  }
  return p.team == 64 ? launch_bwd_team<VEC, 64>(a, p.per_lane, st)
                      : launch_bwd_team<VEC, 256>(a, p.per_lane, st);
}

template <int MODE, int VEC, int E, int TEAM>
hipError_t launch_resident(const RowArgs& a, hipStream_t st) {
  const int64_t nwg = (a.rows + (256 / TEAM) - 1) / (256 / TEAM);
  hipLaunchKernelGGL((row_softmax_kernel<MODE, VEC, E, TEAM>), dim3((uint32_t)nwg), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int MODE, int VEC, int TEAM>
hipError_t launch_team(const RowArgs& a, int e, hipStream_t st) {
  switch (e) {
    case 1: return launch_resident<MODE, VEC, 1, TEAM>(a, st);
    case 2: return launch_resident<MODE, VEC, 2, TEAM>(a, st);
    case 4: return launch_resident<MODE, VEC, 4, TEAM>(a, st);
    case 8: return launch_resident<MODE, VEC, 8, TEAM>(a, st);
    case 16: return launch_resident<MODE, VEC, 16, TEAM>(a, st);
    default: return hipErrorInvalidValue;
  }
}

template <int MODE, int VEC>
hipError_t launch_vec(const RowArgs& a, const RowPlan& p, hipStream_t st) {
  if (p.stream) {
    hipLaunchKernelGGL((row_softmax_stream_kernel<MODE, VEC>), dim3((uint32_t)a.rows), dim3(256), 0, st, a);
    return hipGetLastError();
  }
  return p.team == 64 ? launch_team<MODE, VEC, 64>(a, p.per_lane, st)
                      : launch_team<MODE, VEC, 256>(a, p.per_lane, st);
}

template <int MODE>
hipError_t launch_mode(const RowArgs& a, const RowPlan& p, hipStream_t st) {
  return p.vec == 4 ? launch_vec<MODE, 4>(a, p, st) : launch_vec<MODE, 1>(a, p, st);
}

}  // namespace

RowPlan plan_rows(int64_t cols, bool vec4) {
  RowPlan p;
  p.vec = vec4 ? 4 : 1;
  for (int team : {64, 256}) {
    const int64_t per = (int64_t)team * p.vec;  // floats per vector slot of the team
    if (cols <= per * kRowMaxPerLane) {
      int e = 1;
      while ((int64_t)e * per < cols) e *= 2;
      p.team = team;
      p.per_lane = e;
      p.stream = false;
      return p;
    }
  }
  p.team = 256;
  p.per_lane = 0;
  p.stream = true;
  return p;
}

hipError_t launch_rows_bwd(const RowBwdArgs& a, const RowPlan& p, hipStream_t st) {
  return p.vec == 4 ? launch_bwd_vec<4>(a, p, st) : launch_bwd_vec<1>(a, p, st);
}

hipError_t launch_rows(int mode, const RowArgs& a, const RowPlan& p, hipStream_t st) {
  switch (mode) {
    case kRowSoftmax: return launch_mode<kRowSoftmax>(a, p, st);
    case kRowLse: return launch_mode<kRowLse>(a, p, st);
    case kRowMasked: return launch_mode<kRowMasked>(a, p, st);
    case kRowScaled: return launch_mode<kRowScaled>(a, p, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sma
