// Mask quality (Veda article: fidelity to the structure of dense attention,
// reported as recall): the share of each query's dense softmax mass that the
// kept tiles hold, exp(LSE over the kept keys - LSE over all keys).
#include "common.h"
#include "launch.h"

namespace sla {

__global__ __launch_bounds__(256) void recall_kernel(const float* __restrict__ lse_kept,
                                                     const float* __restrict__ lse_all,
                                                     float* __restrict__ recall, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const float a = lse_kept[i];
  recall[i] = a == -INFINITY ? 0.f : __expf(a - lse_all[i]);
}

RecallWs recall_ws_layout(int64_t BH, int N, int d) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  RecallWs w;
  w.o_bytes = up((size_t)BH * N * d * 2);
  w.lse_bytes = up((size_t)BH * N * 4);
  w.total = w.o_bytes + 2 * w.lse_bytes;
  return w;
}

hipError_t launch_recall(const uint16_t* q, const uint16_t* k, int64_t BH, int N, int d, int block,
                         int nb, const int32_t* idx, const int32_t* cnt, int kmax, float scale,
                         float* recall, void* ws, hipStream_t s) {
  const RecallWs lw = recall_ws_layout(BH, N, d);
  char* p = static_cast<char*>(ws);
  void* o = p;
  float* lse_all = reinterpret_cast<float*>(p + lw.o_bytes);
  float* lse_kept = reinterpret_cast<float*>(p + lw.o_bytes + lw.lse_bytes);
  // V does not enter the LSE: K stands in for it, and O goes to the workspace.
  hipError_t e = launch_attn(q, k, k, BH, N, d, block, nb, nullptr, nullptr, nb, scale, o, 0,
                             lse_all, nullptr, nullptr, s);
  if (e != hipSuccess) return e;
  e = launch_attn(q, k, k, BH, N, d, block, nb, idx, cnt, kmax, scale, o, 0, lse_kept, nullptr,
                  nullptr, s);
  if (e != hipSuccess) return e;
  const int64_t n = BH * N;
  recall_kernel<<<dim3((unsigned)((n + 255) / 256)), 256, 0, s>>>(lse_kept, lse_all, recall, n);
  return hipGetLastError();
}

}  // namespace sla
