// Reading per-row tile lists: the uint16 per-key-tile query-block lists of the
// backward, and the set rule every kernel applies to a caller's int32 lists.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace sla {

// Entry e of a uint16 array at a wave-uniform index, through a scalar load of
// the aligned dword that holds it: there is no 16-bit scalar load, and a
// vector load would be waited for at once (its value is needed in a scalar
// register), which also drains every load in flight.  The dword holds entries
// 2 (e / 2) and 2 (e / 2) + 1: the array must start 4-byte aligned and have
// room for an even number of entries (the backward workspace rounds each of
// its regions up to 256 bytes).
__device__ __forceinline__ int u16_entry(const uint16_t* __restrict__ base, int64_t e) {
  const uint32_t w = reinterpret_cast<const uint32_t*>(base)[e >> 1];
  return (int)((e & 1) ? (w >> 16) : (w & 0xFFFFu));
}

// A list of key tiles is a set: an entry outside [0, nkb) is ignored, and so
// is an entry equal to an earlier one (the tile is attended once, at its
// first position).  Lists from the block-mask kernel are strictly ascending
// and in range ("canonical"); every entry of such a list is used, so the
// per-entry test below reduces to a range check.

// Whether the first `count` entries of `list` are strictly ascending and in
// [0, nkb).  Every lane of the wave gets the same answer (64 entries per step).
__device__ __forceinline__ bool list_is_canonical(const int32_t* __restrict__ list, int count,
                                                  int nkb, int lane) {
  for (int t0 = 0; t0 < count; t0 += 64) {
    const int t = t0 + lane;
    bool bad = false;
    if (t < count) {
      const int j = list[t];
      bad = j < 0 || j >= nkb || (t + 1 < count && list[t + 1] <= j);
    }
    if (__ballot(bad)) return false;
  }
  return true;
}

// Whether entry t (value j) of a list is used under the set rule; `canonical`
// from list_is_canonical.  Wave-uniform arguments give a wave-uniform answer;
// the scan of earlier entries runs only for lists that are not canonical.
__device__ __forceinline__ bool list_entry_used(const int32_t* __restrict__ list, int t, int j,
                                                int nkb, bool canonical) {
  if (j < 0 || j >= nkb) return false;
  if (canonical) return true;
  for (int u = 0; u < t; ++u)
    if (list[u] == j) return false;
  return true;
}

// Query block run by the workgroup at position pos (< nqb) of its head's
// sequence: pos itself, or entry pos of the head's row order (a permutation of
// the head's query blocks, as sla_row_order writes; -1 for an entry outside
// [0, nqb), whose workgroup then does nothing).
__device__ __forceinline__ int ordered_block(const int32_t* __restrict__ order, int64_t bh,
                                             int nqb, int pos) {
  if (!order) return pos;
  const int qb = order[bh * nqb + pos];
  return qb >= 0 && qb < nqb ? qb : -1;
}

}  // namespace sla
