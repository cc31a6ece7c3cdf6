// The output side of the linear-attention branch (SLA post: intermediate
// blocks go through linear attention, phi(x) = elu(x) + 1), shared by the
// standalone apply kernel and the fused epilogue of the softmax kernels.
#pragma once

#include "common.h"

namespace sla {

__device__ __forceinline__ float phi(float x) { return x > 0.f ? x + 1.f : __expf(x); }

// phi of 8 bf16 values, rounded back to bf16; tokens past the end give 0.
__device__ __forceinline__ u32x4 phi8(u32x4 x, bool valid) {
  u32x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float a = valid ? phi(bf16_bits_to_f32(x[e] & 0xffffu)) : 0.f;
    const float b = valid ? phi(bf16_bits_to_f32(x[e] >> 16)) : 0.f;
    r[e] = pack_bf16x2(a, b);
  }
  return r;
}

// O_lin^T = S_i^T phi(Q)^T for one wave's 32 queries, on bf16 MFMA.
//   St    S_i^T of the query block, bf16, row d2 holding d1 = 0..D-1
//   zt    zeta_i, fp32 [D]
//   qf    Q in the B-operand layout: lane holds Q[query l32][16 ks + 8 hf + 0..7]
//   lacc  out, in the layout of the softmax branch's O^T accumulators:
//         register r of block db holds feature 32 db + 8 (r / 4) + 4 hf + r % 4
//         of query l32
//   St_lo with HILO: the low bf16 part of S_i^T (same layout), multiplied
//         into the same accumulators, so S_i enters with about 16 bits
// Returns 1 / (phi(q) . zeta_i), or 0 when that dot product is not positive
// (a query block with no marginal tile has S_i = 0 and zeta_i = 0).
template <int D, bool HILO = false>
__device__ __forceinline__ float linear_apply(const uint16_t* __restrict__ St,
                                              const float* __restrict__ zt,
                                              const u32x4 (&qf)[D / 16], int l32, int hf,
                                              f32x16 (&lacc)[D / 32],
                                              const uint16_t* __restrict__ St_lo = nullptr) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db) lacc[db] = f32x16{};
  float den = 0.f;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const u32x4 pq = phi8(qf[ks], true);
    const f32x4 z0 = *(const f32x4*)(zt + 16 * ks + 8 * hf);
    const f32x4 z1 = *(const f32x4*)(zt + 16 * ks + 8 * hf + 4);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      den = fmaf(bf16_bits_to_f32(pq[e] & 0xffffu), z0[2 * e], den);
      den = fmaf(bf16_bits_to_f32(pq[e] >> 16), z0[2 * e + 1], den);
      den = fmaf(bf16_bits_to_f32(pq[2 + e] & 0xffffu), z1[2 * e], den);
      den = fmaf(bf16_bits_to_f32(pq[2 + e] >> 16), z1[2 * e + 1], den);
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const u32x4 a = *(const u32x4*)(St + (32 * db + l32) * D + 16 * ks + 8 * hf);
      lacc[db] = mfma32x32x16(a, pq, lacc[db]);
      if constexpr (HILO) {
        const u32x4 al = *(const u32x4*)(St_lo + (32 * db + l32) * D + 16 * ks + 8 * hf);
        lacc[db] = mfma32x32x16(al, pq, lacc[db]);
      }
    }
  }
  den = sum_halves(den);
  return den > 0.f ? 1.f / den : 0.f;
}

}  // namespace sla
