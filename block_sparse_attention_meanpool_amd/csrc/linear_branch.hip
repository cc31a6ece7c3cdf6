// Linear-attention branch over the marginal key tiles (SLA post: intermediate
// blocks go through linear attention), phi(x) = elu(x) + 1, and the final sum
// of the two branches.
//
// state:  per key tile j, H_j = phi(K_j)^T V_j (d x d) and z_j = sum phi(K_j),
//         one workgroup per tile; both operands are staged token-contiguous in
//         LDS (the contraction runs over tokens) and multiplied on bf16 MFMA.
// apply:  per query block i, S_i = sum_{j in marg_i} H_j and zeta_i = sum z_j
//         (fp32), then O_lin^T = S_i^T phi(Q_i)^T on bf16 MFMA, one query per
//         lane, divided by phi(q) . zeta_i.
#include "common.h"
#include "launch.h"

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

template <int D, int BLK>
__global__ __launch_bounds__(256) void lin_state_kernel(const uint16_t* __restrict__ k,
                                                        const uint16_t* __restrict__ v, int N,
                                                        int nkb, float* __restrict__ Hs,
                                                        float* __restrict__ Zs) {
  constexpr int NT = 256;
  __shared__ __attribute__((aligned(16))) uint16_t Kt[D * BLK];  // phi(K)^T
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * BLK];  // V^T
  const int64_t bh = blockIdx.x / nkb;
  const int j = blockIdx.x % nkb;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int64_t head_off = bh * (int64_t)N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + head_off, head_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + head_off, head_bytes);

  constexpr int NSUB = (BLK / 8) * (D / 8);
#pragma unroll
  for (int s0 = 0; s0 < NSUB; s0 += NT) {
    const int s = s0 + tid;
    if (NSUB % NT == 0 || s < NSUB) {
      int tc, fc;
      subblock_coords<BLK, D>(s, tc, fc);
      u32x4 ink[8], inv[8], out[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int tok = j * BLK + 8 * tc + r;
        const uint32_t off = (uint32_t)(tok * D + 8 * fc) * 2;
        ink[r] = phi8(buf_load16(rk, off), tok < N);
        inv[r] = buf_load16(rv, off);
      }
      transpose8x8(ink, out);
#pragma unroll
      for (int f = 0; f < 8; ++f) *(u32x4*)((char*)Kt + tr_offset<BLK>(8 * fc + f, tc)) = out[f];
      transpose8x8(inv, out);
#pragma unroll
      for (int f = 0; f < 8; ++f) *(u32x4*)((char*)Vt + tr_offset<BLK>(8 * fc + f, tc)) = out[f];
    }
  }
  __syncthreads();

  // z_j: row sums of phi(K)^T (the same bf16 values the product uses).
  if (tid < D) {
    float z = 0.f;
#pragma unroll
    for (int c = 0; c < BLK / 8; ++c) {
      const u32x4 x = *(const u32x4*)((const char*)Kt + tr_offset<BLK>(tid, c));
#pragma unroll
      for (int e = 0; e < 4; ++e) z += bf16_bits_to_f32(x[e] & 0xffffu) + bf16_bits_to_f32(x[e] >> 16);
    }
    Zs[(bh * nkb + j) * D + tid] = z;
  }

  // H = phi(K)^T V: (D/32)^2 output blocks of 32x32 spread over 4 waves.
  constexpr int NB = (D / 32) * (D / 32);
  constexpr int PERW = NB / 4;
  f32x16 acc[PERW];
#pragma unroll
  for (int u = 0; u < PERW; ++u) acc[u] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < BLK / 16; ++ks) {
#pragma unroll
    for (int u = 0; u < PERW; ++u) {
      const int blkid = w * PERW + u;
      const int db1 = blkid / (D / 32), db2 = blkid % (D / 32);
      const u32x4 a = *(const u32x4*)((const char*)Kt + tr_offset<BLK>(32 * db1 + l32, 2 * ks + hf));
      const u32x4 b = *(const u32x4*)((const char*)Vt + tr_offset<BLK>(32 * db2 + l32, 2 * ks + hf));
      acc[u] = mfma32x32x16(a, b, acc[u]);
    }
  }
  float* Hj = Hs + (bh * nkb + j) * (int64_t)D * D;
#pragma unroll
  for (int u = 0; u < PERW; ++u) {
    const int blkid = w * PERW + u;
    const int db1 = blkid / (D / 32), db2 = blkid % (D / 32);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int d1 = 32 * db1 + 8 * (r / 4) + 4 * hf + (r % 4);
      Hj[d1 * D + 32 * db2 + l32] = acc[u][r];
    }
  }
}

template <int D, int BLK>
__global__ __launch_bounds__(256) void lin_apply_kernel(const uint16_t* __restrict__ q, int N,
                                                        int nqb, int nkb,
                                                        const int32_t* __restrict__ idx,
                                                        const int32_t* __restrict__ cnt, int kmax,
                                                        const float* __restrict__ Hs,
                                                        const float* __restrict__ Zs,
                                                        float* __restrict__ o_lin) {
  constexpr int NT = 256;
  constexpr int PER = D * D / 4 / NT;  // float4 chunks of S per thread
  __shared__ __attribute__((aligned(16))) uint16_t St[D * D];  // S^T as bf16 [d2][d1]
  __shared__ float zs[D];
  const int64_t bh = blockIdx.x / nqb;
  const int qb = blockIdx.x % nqb;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int64_t head_off = bh * (int64_t)N * D;
  const int count = min(cnt[bh * nqb + qb], kmax);
  const int32_t* list = idx + (bh * nqb + qb) * (int64_t)kmax;

  f32x4 sacc[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) sacc[u] = f32x4{};
  float zacc = 0.f;
  int used = 0;
  for (int t = 0; t < count; ++t) {
    const int j = list[t];
    if (j < 0 || j >= nkb) continue;
    ++used;
    const f32x4* Hj = (const f32x4*)(Hs + (bh * nkb + j) * (int64_t)D * D);
#pragma unroll
    for (int u = 0; u < PER; ++u) sacc[u] += Hj[tid + NT * u];
    if (tid < D) zacc += Zs[(bh * nkb + j) * D + tid];
  }
  if (tid < D) zs[tid] = zacc;
  // S^T into LDS, bf16, rows d2, columns d1 (d1-contiguous chunks).
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int e = 4 * (tid + NT * u);
    const int d1 = e / D, d2 = e % D;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t off = tr_offset<D>(d2 + c, d1 / 8) + 2 * (d1 % 8);
      *(uint16_t*)((char*)St + off) = (uint16_t)f32_to_bf16_bits(sacc[u][c]);
    }
  }
  __syncthreads();
  if (32 * w >= BLK) return;

  const int qrow = qb * BLK + 32 * w + l32;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + head_off, (uint32_t)N * D * 2);
  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
  float den = 0.f;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const u32x4 pq = phi8(buf_load16(rq, (uint32_t)(qrow * D + 16 * ks + 8 * hf) * 2), true);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int d1 = 16 * ks + 8 * hf + 2 * e;
      den = fmaf(bf16_bits_to_f32(pq[e] & 0xffffu), zs[d1], den);
      den = fmaf(bf16_bits_to_f32(pq[e] >> 16), zs[d1 + 1], den);
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const u32x4 a = *(const u32x4*)((const char*)St + tr_offset<D>(32 * db + l32, 2 * ks + hf));
      oacc[db] = mfma32x32x16(a, pq, oacc[db]);
    }
  }
  den = sum_halves(den);
  const float inv = (used > 0 && den > 0.f) ? 1.f / den : 0.f;
  if (qrow < N) {
    float* orow = o_lin + head_off + (int64_t)qrow * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * hf;
        *(f32x4*)(orow + d0) = f32x4{oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv,
                                     oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv};
      }
  }
}

__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ o_s, int o_s_fp32,
                                                      const float* __restrict__ o_lin,
                                                      uint16_t* __restrict__ o, int64_t n8) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  float x[8];
  if (o_s_fp32) {
    const f32x4* p = (const f32x4*)o_s + 2 * i;
    const f32x4 a = p[0], b = p[1];
#pragma unroll
    for (int e = 0; e < 4; ++e) { x[e] = a[e]; x[4 + e] = b[e]; }
  } else {
    const u32x4 a = ((const u32x4*)o_s)[i];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = bf16_bits_to_f32(a[e] & 0xffffu);
      x[2 * e + 1] = bf16_bits_to_f32(a[e] >> 16);
    }
  }
  if (o_lin) {
    const f32x4* p = (const f32x4*)o_lin + 2 * i;
    const f32x4 a = p[0], b = p[1];
#pragma unroll
    for (int e = 0; e < 4; ++e) { x[e] += a[e]; x[4 + e] += b[e]; }
  }
  ((u32x4*)o)[i] = u32x4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                         pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])};
}

template <int D, int BLK>
static hipError_t launch_linear_t(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                  int64_t BH, int N, int nb, const int32_t* idx, const int32_t* cnt,
                                  int kmax, float* o_lin, float* Hs, float* Zs, hipStream_t s) {
  lin_state_kernel<D, BLK><<<dim3((unsigned)(BH * nb)), 256, 0, s>>>(k, v, N, nb, Hs, Zs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  lin_apply_kernel<D, BLK><<<dim3((unsigned)(BH * nb)), 256, 0, s>>>(q, N, nb, nb, idx, cnt, kmax,
                                                                    Hs, Zs, o_lin);
  return hipGetLastError();
}

hipError_t launch_linear(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t BH, int N,
                         int d, int block, int nb, const int32_t* idx, const int32_t* cnt, int kmax,
                         float* o_lin, float* Hs, float* Zs, hipStream_t s) {
  if (d == 128 && block == 128)
    return launch_linear_t<128, 128>(q, k, v, BH, N, nb, idx, cnt, kmax, o_lin, Hs, Zs, s);
  if (d == 128 && block == 64)
    return launch_linear_t<128, 64>(q, k, v, BH, N, nb, idx, cnt, kmax, o_lin, Hs, Zs, s);
  if (d == 64 && block == 128)
    return launch_linear_t<64, 128>(q, k, v, BH, N, nb, idx, cnt, kmax, o_lin, Hs, Zs, s);
  return launch_linear_t<64, 64>(q, k, v, BH, N, nb, idx, cnt, kmax, o_lin, Hs, Zs, s);
}

hipError_t launch_combine(const void* o_s, int o_s_fp32, const float* o_lin, uint16_t* o,
                          int64_t n_elems, hipStream_t s) {
  const int64_t n8 = n_elems / 8;
  if (n8 == 0) return hipSuccess;
  combine_kernel<<<dim3((unsigned)((n8 + 255) / 256)), 256, 0, s>>>(o_s, o_s_fp32, o_lin, o, n8);
  return hipGetLastError();
}

}  // namespace sla
