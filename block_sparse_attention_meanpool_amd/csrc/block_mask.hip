// Class map -> compact ascending lists of the key tiles each query block needs
// (Veda article, "what happened": the kernel works only on the selected key
// tiles of each query).  One wave per row; ballots give each selected block
// its position, so the lists come out in ascending order with no sort.
#include "common.h"
#include "launch.h"

namespace sla {

__global__ __launch_bounds__(256) void block_mask_kernel(
    const uint8_t* __restrict__ cls, int64_t rows, int nkb, int32_t* __restrict__ crit_idx,
    int32_t* __restrict__ crit_cnt, int kc_max, int32_t* __restrict__ marg_idx,
    int32_t* __restrict__ marg_cnt, int km_max, int32_t* __restrict__ err_flag) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const uint8_t* crow = cls + row * nkb;
  int32_t* ci = crit_idx + row * kc_max;
  int32_t* mi = marg_idx ? marg_idx + row * km_max : nullptr;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int nc = 0, nm = 0;
  bool bad = false;
  for (int j0 = 0; j0 < nkb; j0 += 64) {
    const int j = j0 + lane;
    const int c = j < nkb ? crow[j] : 0;
    bad |= c > 2;
    const uint64_t mc = __ballot(c == 2);
    const uint64_t mm = __ballot(c == 1);
    if (c == 2) {
      const int pos = nc + __popcll(mc & below);
      if (pos < kc_max) ci[pos] = j;
    }
    if (c == 1 && mi) {
      const int pos = nm + __popcll(mm & below);
      if (pos < km_max) mi[pos] = j;
    }
    nc += __popcll(mc);
    nm += __popcll(mm);
  }
  for (int p = nc + lane; p < kc_max; p += 64) ci[p] = -1;
  if (mi)
    for (int p = nm + lane; p < km_max; p += 64) mi[p] = -1;
  const bool any_bad = __ballot(bad) != 0;
  if (lane == 0) {
    int flag = 0;
    if (any_bad) flag |= 1;
    if (nc > kc_max || (mi && nm > km_max)) flag |= 2;
    crit_cnt[row] = min(nc, kc_max);
    if (mi) marg_cnt[row] = min(nm, km_max);
    if (flag && err_flag) atomicOr(err_flag, flag);
  }
}

hipError_t launch_block_mask(const uint8_t* cls, int64_t rows, int nkb, int32_t* crit_idx,
                             int32_t* crit_cnt, int kc_max, int32_t* marg_idx, int32_t* marg_cnt,
                             int km_max, int32_t* err_flag, hipStream_t s) {
  dim3 grid((unsigned)((rows + 3) / 4));
  block_mask_kernel<<<grid, 256, 0, s>>>(cls, rows, nkb, crit_idx, crit_cnt, kc_max, marg_idx,
                                         marg_cnt, km_max, err_flag);
  return hipGetLastError();
}

}  // namespace sla
