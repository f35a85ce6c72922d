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

// Column packing: one wave per (slab, 32-row block, 512-key chunk). Lane l
// takes keys j = 512 c + 8 l .. + 7: for each of the block's 32 rows it reads
// their 8 mask bytes (a row's 512 bytes in one wave-wide load), sets row bit i
// of each key's word, and writes the words at their paired positions. Eight
// lanes cover a 64-key tile, whose class the wave's votes give.
constexpr int kColKeysPerLane = 8;
constexpr int kColChunk = 64 * kColKeysPerLane;

__global__ __launch_bounds__(256) void mask_pack_cols_kernel(MaskColArgs a) {
  typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
  constexpr int K = kColKeysPerLane;
  const int lane = threadIdx.x & 63;
  const int64_t wv = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int32_t nchunk = (a.kpad + kColChunk - 1) / kColChunk;
  const int64_t total = a.slabs * a.nrb * nchunk;
  if (wv >= total) return;  // whole waves leave together
  const int32_t chunk = (int32_t)(wv % nchunk);
  const int64_t blk = wv / nchunk;  // slab * nrb + rb
  const int32_t rb = (int32_t)(blk % a.nrb);
  const int64_t slab = blk / a.nrb;
  const int32_t j0 = kColChunk * chunk + K * lane;
  uint32_t word[K];
#pragma unroll
  for (int e = 0; e < K; ++e) word[e] = 0u;
  const unsigned char* base = a.mask + (slab * a.seq_q) * (int64_t)a.seq_kv;
  const bool vec = (a.seq_kv & (K - 1)) == 0 && j0 + K <= a.seq_kv && ((uintptr_t)base & (K - 1)) == 0;
  for (int i = 0; i < 32; ++i) {
    const int32_t row = 32 * rb + i;
    u32x2_t b8 = {0x01010101u, 0x01010101u};  // rows past seq_q admit
    if (row < a.seq_q) {
      const unsigned char* src = base + (int64_t)row * a.seq_kv + j0;
      if (vec) {
        b8 = *reinterpret_cast<const u32x2_t*>(src);
      } else {
        b8 = u32x2_t{0u, 0u};
        for (int e = 0; e < K; ++e)
          if (j0 + e < a.seq_kv) b8[e / 4] |= (uint32_t)src[e] << (8 * (e % 4));
      }
    }
#pragma unroll
    for (int e = 0; e < K; ++e) word[e] |= (((b8[e / 4] >> (8 * (e % 4))) & 0xFFu) != 0u ? 1u : 0u) << i;
  }
  uint32_t any_w = 0u, all_w = ~0u;
#pragma unroll
  for (int e = 0; e < K; ++e) {
    const int32_t j = j0 + e;
    if (j >= a.seq_kv) word[e] = 0u;  // keys past seq_kv block
    if (j < a.kpad) a.cols[blk * a.kpad + ((j & ~15) | ((j & 7) << 1) | ((j >> 3) & 1))] = word[e];
    any_w |= word[e];
    all_w &= word[e];
  }
  const uint64_t any = __ballot(any_w != 0u);
  const uint64_t full = __ballot(all_w == ~0u);
  constexpr int kLanesPerTile = 64 / K;
  constexpr uint64_t kTileLanes = (1ull << kLanesPerTile) - 1;
  if (lane < K) {
    const int32_t tile = K * chunk + lane;
    if (64 * tile < a.kpad) {
      const uint64_t any_t = (any >> (kLanesPerTile * lane)) & kTileLanes;
      const uint64_t full_t = (full >> (kLanesPerTile * lane)) & kTileLanes;
      a.cls[blk * (a.kpad / 64) + tile] = any_t == 0 ? 0u : (full_t == kTileLanes ? 1u : 2u);
    }
  }
}

}  // namespace

hipError_t launch_mask_pack_cols(const MaskColArgs& a, hipStream_t s) {
  const int64_t waves = a.slabs * a.nrb * ((a.kpad + kColChunk - 1) / kColChunk);
  const int64_t blocks = (waves + 3) / 4;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(mask_pack_cols_kernel, dim3((uint32_t)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_mask_pack(const MaskPackArgs& a, hipStream_t s) {
  const int64_t words = a.slabs * a.seq_q * a.words;
  const int64_t blocks = (words + 255) / 256;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(mask_pack_kernel, dim3((uint32_t)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace sma
