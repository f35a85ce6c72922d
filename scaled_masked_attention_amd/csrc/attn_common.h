// Device helpers shared by the attention-forward kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sma_kernels.h"

namespace sma {

// MI355X dispatches consecutive workgroup ids round-robin over its 8 XCDs,
// each with its own L2. Remap so that XCD x runs one contiguous range of
// logical tiles: neighbouring query blocks of a head (which stream the same
// K/V tiles) then share an L2.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t wg, uint32_t nwg) {
  constexpr uint32_t kXcds = 8;
  const uint32_t per = nwg / kXcds, rem = nwg % kXcds;
  const uint32_t x = wg % kXcds, slot = wg / kXcds;
  return x * per + (x < rem ? x : rem) + slot;
}

// Element offset of the first row of (batch*head index bh) under strides (sb, sh).
__device__ __forceinline__ int64_t head_offset(int64_t bh, int64_t heads, int64_t sb, int64_t sh) {
  return (bh / heads) * sb + (bh % heads) * sh;
}

struct TileId {
  int64_t bh;
  int32_t qb;
  int32_t split;
};

// Logical tile order: heads outermost, then query blocks from the last (the
// longest under a causal mask) to the first, then key splits.
__device__ __forceinline__ TileId decode_tile(uint32_t wg, const FwdArgs& a) {
  const uint32_t lam = xcd_remap(wg, a.nwg);
  TileId t;
  t.split = (int32_t)(lam % (uint32_t)a.nsplit);
  const uint32_t rest = lam / (uint32_t)a.nsplit;
  t.qb = a.nqb - 1 - (int32_t)(rest % (uint32_t)a.nqb);
  t.bh = (int64_t)(rest / (uint32_t)a.nqb);
  return t;
}

// Keys j < key_limit(i) are admitted for query row i (bottom-right causal:
// j <= i + seq_kv - seq_q), further bounded by the end of the key split.
template <bool CAUSAL>
__device__ __forceinline__ int32_t key_limit(int32_t row, int32_t seq_q, int32_t seq_kv,
                                             int32_t split_end) {
  if (!CAUSAL) return split_end;
  int32_t hi = row + (seq_kv - seq_q) + 1;
  hi = hi < 0 ? 0 : hi;
  return hi < split_end ? hi : split_end;
}

// Wait until at most N vector-memory operations of this wave are in flight
// (expcnt and lgkmcnt left unconstrained).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// One 16-byte-per-lane direct-to-LDS load through a buffer resource: lane i's
// chunk lands at LDS byte address lds_addr + 16*i (lds_addr wave-uniform, in
// M0). Issued as inline asm so that the compiler adds no conservative waits
// for it before unrelated LDS reads; the kernel waits explicitly (wait_vmcnt)
// before a tile is used. The s_nop covers the M0-write hazard.
__device__ __forceinline__ void dma_load_x4(__amdgpu_buffer_rsrc_t rsrc, unsigned voffset,
                                            unsigned lds_addr) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voffset), "s"(rsrc), "{m0}"(lds_addr)
               : "memory");
}

// The 4-byte form: lane i's dword lands at lds_addr + 4*i (256 bytes per instruction).
__device__ __forceinline__ void dma_load_x1(__amdgpu_buffer_rsrc_t rsrc, unsigned voffset,
                                            unsigned lds_addr) {
  asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :
               : "v"(voffset), "s"(rsrc), "{m0}"(lds_addr)
               : "memory");
}

__device__ __forceinline__ unsigned lds_address(const void* p) {
  return (unsigned)(size_t)(__attribute__((address_space(3))) const void*)p;
}

// Buffer resource over `bytes` bytes at `base`: loads at byte offsets at or
// past `bytes` return zeros. Word 3 selects a raw (untyped) buffer on gfx9.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_buffer(const void* base, unsigned bytes) {
  constexpr int kRsrcWord3 = 0x00020000;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRsrcWord3);
}

// Two floats rounded to bf16 (nearest even, the hardware conversion), packed
// low word first: the storage order of consecutive bf16 elements.
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(unsigned, v);
}
// The same for fp16 (the hardware conversion under the default rounding mode, nearest even).
__device__ __forceinline__ unsigned pack_f16x2(float lo, float hi) {
  typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
  const f16x2_t v = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(unsigned, v);
}
// A 16-bit output pair: fp16 when f16, else bf16.
__device__ __forceinline__ unsigned pack_out16(float lo, float hi, bool f16) {
  return f16 ? pack_f16x2(lo, hi) : pack_bf16x2(lo, hi);
}

// A 32-row fp32 tile (of Q, K, dO or V) in LDS: row r's 16-byte chunk c is
// stored at chunk position c ^ tile_swz<D>(r) of the row. The operand reads
// take one chunk from each of 16 consecutive rows per ds_read_b128 group of 16
// lanes; rows of 256 bytes or more all start at bank 0, so XOR with r & 15
// spreads those 16 lanes over the 64 banks, while 128-byte rows (d = 32)
// alternate between the two bank halves, so XOR with (r >> 1) & 7 does.
// A direct-to-LDS instruction fills 1 KB of consecutive positions, so lane l
// of copy instruction t fetches the global chunk that belongs at position
// p = 64t + l.
template <int D>
__device__ __forceinline__ int tile_swz(int r) {
  static_assert(D == 32 || D == 64 || D == 128 || D == 256, "fp32 tile swizzle");
  return D >= 64 ? (r & 15) : ((r >> 1) & 7);
}
template <int D>
__device__ __forceinline__ unsigned tile_src_offset(int t, int lane) {
  constexpr int kChunks = D / 4;  // 16-byte chunks per row
  const int p = 64 * t + lane;
  const int r = p / kChunks;
  const int c = (p % kChunks) ^ tile_swz<D>(r);
  return (unsigned)(r * 4 * D + 16 * c);
}
// The same with rows row_bytes apart in global memory (a strided layout).
template <int D>
__device__ __forceinline__ unsigned tile_src_offset(int t, int lane, unsigned row_bytes) {
  constexpr int kChunks = D / 4;
  const int p = 64 * t + lane;
  const int r = p / kChunks;
  const int c = (p % kChunks) ^ tile_swz<D>(r);
  return (unsigned)r * row_bytes + 16u * (unsigned)c;
}
// Unswizzled copy: lane l of instruction t fetches chunk p = 64t + l in row order.
template <int D>
__device__ __forceinline__ unsigned tile_src_offset_linear(int t, int lane, unsigned row_bytes) {
  constexpr int kChunks = D / 4;
  const int p = 64 * t + lane;
  return (unsigned)(p / kChunks) * row_bytes + 16u * (unsigned)(p % kChunks);
}
// Bytes a buffer resource must span to cover `rows` rows of `row_elems`
// elements each, `stride_elems` apart: the last row ends the range.
__device__ __forceinline__ unsigned strided_range(int32_t rows, int64_t stride_elems,
                                                  int row_elems, int elem_bytes) {
  return rows > 0 ? (unsigned)(((int64_t)(rows - 1) * stride_elems + row_elems) * elem_bytes) : 0u;
}

// LDS byte offset, within a tile, of the 16 bytes holding head dims
// 8u + 4h .. 8u + 4h + 3 of row m (the operand of MFMA group u).
template <int D>
__device__ __forceinline__ unsigned tile_operand_offset(int m, int h, int u) {
  return (unsigned)(m * 4 * D + 16 * ((2 * u + h) ^ tile_swz<D>(m)));
}

// LDS byte offset, within such a tile, of the D/32 consecutive floats at head
// dims (D/32)*j .. (D/32)*j + D/32 - 1 of row `row` (j = 0..31: one 32-lane half
// of a wave reads one whole row).
template <int D>
__device__ __forceinline__ unsigned tile_row_offset(int row, int j) {
  constexpr int kLaneBytes = 4 * (D / 32);
  const int byte = kLaneBytes * j;
  return (unsigned)(row * 4 * D + 16 * ((byte >> 4) ^ tile_swz<D>(row)) + (byte & 15));
}

}  // namespace sma
