// Packing of a hard attention mask (TorchLean hard-masked softmax: an entry is
// admitted or blocked) from one byte per (query, key), nonzero admitting, into
// one bit per pair: bit j % 32 of 32-bit word j / 32 of the query's row. The
// attention kernels then fetch a 32-key block's admissions for a row as one
// word. HBM-bound: reads seq_q * seq_kv bytes per slab, writes an eighth.
#include "attn_common.h"

namespace sma {
namespace {

// One thread per output word: it reads the word's 32 mask bytes (two 16-byte
// loads where the row allows them, else byte by byte) and sets bit i when
// byte i is nonzero. Consecutive threads read consecutive 32-byte runs.
__global__ __launch_bounds__(256) void mask_pack_kernel(MaskPackArgs a) {
  typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = a.slabs * a.seq_q * a.words;
  if (gid >= total) return;
  const int64_t row = gid / a.words;
  const int32_t w = (int32_t)(gid % a.words);
  const int32_t j0 = 32 * w;
  const int32_t n = a.seq_kv - j0 < 32 ? a.seq_kv - j0 : 32;  // keys of this word (>= 1)
  const unsigned char* src = a.mask + row * a.seq_kv + j0;
  uint32_t bits = 0;
  if (n == 32 && ((uintptr_t)src & 15) == 0) {
    const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(src);
    const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(src + 16);
    const unsigned dw[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
    for (int i = 0; i < 32; ++i) bits |= (((dw[i / 4] >> (8 * (i % 4))) & 0xFFu) != 0u ? 1u : 0u) << i;
  } else {
    for (int i = 0; i < n; ++i) bits |= (src[i] != 0 ? 1u : 0u) << i;
  }
  a.bits[gid] = bits;
}

}  // namespace

hipError_t launch_mask_pack(const MaskPackArgs& a, hipStream_t s) {
  const int64_t words = a.slabs * a.seq_q * a.words;
  const int64_t blocks = (words + 255) / 256;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(mask_pack_kernel, dim3((uint32_t)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace sma
