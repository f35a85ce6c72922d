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

}  // namespace sma
