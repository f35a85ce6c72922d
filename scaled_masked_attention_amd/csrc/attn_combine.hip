// Combine of key splits: each split s of a query row holds its own normalised
// output O_s and log-sum-exp L_s (log2 units) over its keys. Since the
// log-sum-exp of a union is the log of the summed exponentials (pulsatrix
// HIPBackend `logsumexp_rows` definition), the full row is
//   L = log2 sum_s 2^L_s,   O = sum_s 2^(L_s - L) O_s,
// with empty splits (L_s = -inf) weighing zero and a row empty in every split
// written as O = +0.0, LSE = -inf. HBM-bound: it reads nsplit*(d+1) floats per
// row and writes d+1 (the output in fp32 or, rounded to nearest even, bf16 or fp16),
// the output with non-temporal stores (written once, not read here again).
#include "attn_common.h"

namespace sma {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(CombineArgs a) {
  constexpr int kThreadsPerRow = D / 4;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid / kThreadsPerRow;
  const int c4 = (int)(gid % kThreadsPerRow);
  if (row >= a.rows) return;
  float mx = -INFINITY;
  for (int s = 0; s < a.nsplit; ++s) mx = fmaxf(mx, a.part_lse[(int64_t)s * a.rows + row]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float lse2 = -INFINITY;
  if (mx != -INFINITY) {
    float sum = 0.f;
    for (int s = 0; s < a.nsplit; ++s)
      sum += __builtin_amdgcn_exp2f(a.part_lse[(int64_t)s * a.rows + row] - mx);
    lse2 = mx + __builtin_amdgcn_logf(sum);
    for (int s = 0; s < a.nsplit; ++s) {
      const float w = __builtin_amdgcn_exp2f(a.part_lse[(int64_t)s * a.rows + row] - lse2);
      const f32x4 x =
          *reinterpret_cast<const f32x4*>(a.part_o + ((int64_t)s * a.rows + row) * D + 4 * c4);
      acc[0] += w * x[0];
      acc[1] += w * x[1];
      acc[2] += w * x[2];
      acc[3] += w * x[3];
    }
  }
  const int64_t bh = row / a.seq_q;
  const int64_t o_off = head_offset(bh, a.heads, a.os_b, a.os_h) + (row - bh * a.seq_q) * a.os_s + 4 * c4;
  if (a.o_bf16) {
    typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
    __builtin_nontemporal_store(u32x2_t{pack_out16(acc[0], acc[1], a.o_f16), pack_out16(acc[2], acc[3], a.o_f16)},
                                reinterpret_cast<u32x2_t*>(a.o_bf16 + o_off));
  } else {
    __builtin_nontemporal_store(acc, reinterpret_cast<f32x4*>(a.o + o_off));
  }
  if (a.lse && c4 == 0) a.lse[row] = mx == -INFINITY ? -INFINITY : lse2 * 0.69314718055994530942f;
}

template <int D>
hipError_t launch_combine_variant(const CombineArgs& a, hipStream_t s) {
  const int64_t threads = a.rows * (D / 4);
  const int64_t blocks = (threads + 255) / 256;
  hipLaunchKernelGGL((attn_combine_kernel<D>), dim3((uint32_t)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, int head_dim, hipStream_t s) {
  switch (head_dim) {
    case 32: return launch_combine_variant<32>(a, s);
    case 64: return launch_combine_variant<64>(a, s);
    case 128: return launch_combine_variant<128>(a, s);
    case 256: return launch_combine_variant<256>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sma
