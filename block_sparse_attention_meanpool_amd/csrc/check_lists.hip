// Per-query-block tile lists (the Veda article's per-query sets of key
// tiles): validation of lists supplied by a caller, and a locality-aware order
// in which to run the query blocks.
//
// Validation (the lists the block-mask kernel writes always pass): every
// entry in [0, nkb), no repeated entry, ascending order, and a count in
// [0, width].  The kernels that read lists treat a list as a set of tiles
// whatever it holds; this check tells a caller that its lists were not in the
// documented form.  A row order must be, per head, a permutation of the query
// blocks; a second check tells a caller when one is not.
//
// Row order: query blocks sorted by the median tile of their lists.  Blocks
// whose lists sit around the same tiles then run next to each other on one
// XCD and find those tiles in its L2; the order changes nothing in any result
// (each query block is computed on its own).
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/sla.h"
#include "launch.h"

namespace sla {

// One wave per row.  A per-wave bitmap in LDS (nkb <= 4096 bits) finds
// repeated entries in any order; neighbouring entries give the order check.
__global__ __launch_bounds__(256) void check_lists_kernel(const int32_t* __restrict__ idx,
                                                          const int32_t* __restrict__ cnt,
                                                          int64_t rows, int width, int nkb,
                                                          int32_t* __restrict__ err_flag) {
  __shared__ uint32_t seen[4][128];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * 4 + wv;
  if (row >= rows) return;
  seen[wv][lane] = 0u;
  seen[wv][lane + 64] = 0u;
  __builtin_amdgcn_wave_barrier();
  int flags = 0;
  const int c0 = cnt[row];
  if (c0 < 0 || c0 > width) flags |= SLA_FLAG_LIST_COUNT;
  const int c = min(max(c0, 0), width);
  const int32_t* list = idx + row * (int64_t)width;
  for (int t0 = 0; t0 < c; t0 += 64) {
    const int t = t0 + lane;
    if (t < c) {
      const int j = list[t];
      if (j < 0 || j >= nkb) {
        flags |= SLA_FLAG_LIST_RANGE;
      } else {
        const uint32_t bit = 1u << (j & 31);
        if (atomicOr(&seen[wv][j >> 5], bit) & bit) flags |= SLA_FLAG_LIST_REPEAT;
      }
      if (t + 1 < c && list[t + 1] < j) flags |= SLA_FLAG_LIST_ORDER;
    }
  }
  if (flags) atomicOr(err_flag, flags);
}

hipError_t launch_check_lists(const int32_t* idx, const int32_t* cnt, int64_t rows, int width,
                              int nkb, int32_t* err_flag, hipStream_t s) {
  check_lists_kernel<<<dim3((unsigned)((rows + 3) / 4)), 256, 0, s>>>(idx, cnt, rows, width, nkb,
                                                                     err_flag);
  return hipGetLastError();
}

// One workgroup per head: every entry of the head's row order in [0, nqb) and
// none repeated, i.e. a permutation (nqb <= 4096: a 4096-bit LDS bitmap).
__global__ __launch_bounds__(256) void check_order_kernel(const int32_t* __restrict__ order, int nqb,
                                                          int32_t* __restrict__ err_flag) {
  __shared__ uint32_t seen[128];
  if (threadIdx.x < 128) seen[threadIdx.x] = 0u;
  __syncthreads();
  const int32_t* row = order + (int64_t)blockIdx.x * nqb;
  bool bad = false;
  for (int i = threadIdx.x; i < nqb; i += 256) {
    const int v = row[i];
    if (v < 0 || v >= nqb) {
      bad = true;
    } else {
      const uint32_t bit = 1u << (v & 31);
      if (atomicOr(&seen[v >> 5], bit) & bit) bad = true;
    }
  }
  if (bad) atomicOr(err_flag, SLA_FLAG_ORDER_PERM);
}

hipError_t launch_check_order(const int32_t* order, int64_t BH, int nqb, int32_t* err_flag,
                              hipStream_t s) {
  check_order_kernel<<<dim3((unsigned)BH), 256, 0, s>>>(order, nqb, err_flag);
  return hipGetLastError();
}

// One workgroup per head: a bitonic sort in LDS of the keys
// (median entry << 12) | query block, so equal medians keep index order
// (nqb <= 4096; an empty row sorts last with key 4096).
__global__ __launch_bounds__(1024) void row_order_kernel(const int32_t* __restrict__ idx,
                                                         const int32_t* __restrict__ cnt, int nqb,
                                                         int width, int32_t* __restrict__ order) {
  __shared__ uint32_t key[4096];
  const int64_t bh = blockIdx.x;
  int P = 1;
  while (P < nqb) P <<= 1;
  for (int i = threadIdx.x; i < P; i += 1024) {
    uint32_t kk = 0xffffffffu;  // padding sorts after every real key
    if (i < nqb) {
      const int64_t row = bh * nqb + i;
      const int c = min(cnt[row], width);
      uint32_t m = 4096u;
      if (c > 0) m = (uint32_t)min(max(idx[row * width + c / 2], 0), 4095);
      kk = (m << 12) | (uint32_t)i;
    }
    key[i] = kk;
  }
  __syncthreads();
  for (int size = 2; size <= P; size <<= 1)
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < P; i += 1024) {
        const int j = i ^ stride;
        if (j > i) {
          const bool up = (i & size) == 0;
          const uint32_t a = key[i], b = key[j];
          if ((a > b) == up) {
            key[i] = b;
            key[j] = a;
          }
        }
      }
      __syncthreads();
    }
  for (int i = threadIdx.x; i < nqb; i += 1024) order[bh * nqb + i] = (int32_t)(key[i] & 0xfffu);
}

hipError_t launch_row_order(const int32_t* idx, const int32_t* cnt, int64_t BH, int nqb, int width,
                            int32_t* order, hipStream_t s) {
  row_order_kernel<<<dim3((unsigned)BH), 1024, 0, s>>>(idx, cnt, nqb, width, order);
  return hipGetLastError();
}

// The flag word that builds with SLA_DEBUG_CHECKS report list violations in
// (each device holds its own), addressed through hipGetSymbolAddress as for
// any device symbol: the name itself is a host-side stand-in.
static __device__ int32_t debug_flag;

namespace {
std::mutex g_dbg_mu;
void* g_dbg_ptr[64] = {};
}  // namespace

hipError_t debug_flag_ptr(int32_t** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_dbg_mu);
  if (!g_dbg_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(debug_flag));
    if (e != hipSuccess) return e;
    g_dbg_ptr[dev] = p;
  }
  *ptr = static_cast<int32_t*>(g_dbg_ptr[dev]);
  return hipSuccess;
}

}  // namespace sla
