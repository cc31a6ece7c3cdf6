// Reading the per-key-tile query-block lists (uint16 entries) of the backward.
#pragma once
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

}  // namespace sla
