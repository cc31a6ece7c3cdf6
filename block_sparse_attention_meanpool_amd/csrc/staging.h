// Staging of bf16 tiles from global memory into LDS by 8 x 8 sub-blocks, for
// the kernels that need a tile both row-major and transposed (the backward
// kernels for d = 64 or 64-token blocks).
#pragma once

#include "common.h"

namespace sla {

// A tile of R rows x F bf16 features (row stride F elements), rows
// [row0, row0 + R) of a buffer resource, into LDS by 8 x 8 sub-blocks: one
// global read per 16-byte chunk, stored row-major (rows != nullptr; chunks
// placed as row_offset<F / 8>) and/or transposed (tr != nullptr; feature rows
// of R tokens placed as tr_offset<R>).  xf(chunk, r) maps each chunk of 8
// values of tile row r before it is stored; rows past the resource's range
// read as zeros.  NT threads, tid = threadIdx.x.
template <int R, int F, int NT, class XF>
__device__ __forceinline__ void stage_subblocks(const __amdgpu_buffer_rsrc_t& rs, int row0,
                                                char* rows, char* tr, int tid, XF xf) {
  constexpr int NSUB = (R / 8) * (F / 8);
#pragma unroll
  for (int s0 = 0; s0 < NSUB; s0 += NT) {
    const int s = s0 + tid;
    if (NSUB % NT == 0 || s < NSUB) {
      int tc, fc;
      subblock_coords<R>(s, tc, fc);
      u32x4 in[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        in[e] = xf(buf_load16(rs, (uint32_t)((row0 + 8 * tc + e) * F + 8 * fc) * 2), 8 * tc + e);
      if (rows) {
#pragma unroll
        for (int e = 0; e < 8; ++e) *(u32x4*)(rows + row_offset<F / 8>(8 * tc + e, fc)) = in[e];
      }
      if (tr) {
        u32x4 out[8];
        transpose8x8(in, out);
#pragma unroll
        for (int f = 0; f < 8; ++f) *(u32x4*)(tr + tr_offset<R>(8 * fc + f, tc)) = out[f];
      }
    }
  }
}

struct KeepChunk {
  __device__ u32x4 operator()(u32x4 x, int) const { return x; }
};

}  // namespace sla
