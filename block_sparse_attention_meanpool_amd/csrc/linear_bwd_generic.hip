// Backward pass of the linear-attention branch for the shapes other than
// d = 128 with 128-token blocks (d in {64, 128}, blocks of 64 or 128 tokens).
// Same gradients as the tuned kernels (SLA post: intermediate blocks via
// linear attention, phi = elu + 1; results: the method is trainable), with
// a = phi(q), w_n = a_n . zeta_i, O_lin_n = a_n^T S_i / w_n:
//   g_n = dO_n / w_n,  h_n = -(dO_n . O_lin_n) / w_n
//   dq_n += (S_i g_n + zeta_i h_n) * phi'(q_n)
//   dS_i  = A_i^T G_i,  dzeta_i = A_i^T h        (query side, per block)
//   dH_j, dz_j: sums of dS_i, dzeta_i over the query blocks whose marginal
//               list holds j (the gather kernels of the forward)
//   dk_m += (dH_j v_m + dz_j) * phi'(k_m),  dv_m += dH_j^T phi(k_m)
// Tiles are staged through LDS by 8 x 8 sub-blocks, row-major and/or
// transposed as each MFMA operand needs; dq, dk, dv are fp32 and accumulated
// into.
#include "common.h"
#include "launch.h"
#include "staging.h"
#include "linear_apply.h"

namespace sla {
namespace glbwd {

__device__ __forceinline__ float dphi(float x) { return x > 0.f ? 1.f : __expf(x); }

struct PhiChunk {  // phi of the 8 values, rows at or past `valid` give 0
  int valid;
  __device__ u32x4 operator()(u32x4 x, int r) const { return phi8(x, r < valid); }
};

struct ScaleChunk {  // the 8 values times a per-row factor, rounded to bf16 (as g above)
  const float* f;
  __device__ u32x4 operator()(u32x4 x, int r) const {
    const float s = f[r];
    u32x4 y;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      y[e] = pack_bf16x2(bf16_bits_to_f32(x[e] & 0xffffu) * s, bf16_bits_to_f32(x[e] >> 16) * s);
    return y;
  }
};

// One workgroup per query block, BLK/32 waves of 32 queries (one per lane).
// As in the tuned kernel, dq's two nearly cancelling terms get S_i (C, C_lo),
// O_lin and g as hi + lo bf16 pairs.
template <int D, int BLK>
__global__ __launch_bounds__(BLK * 2) void query_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ d_o, int N, int nqb,
    const uint16_t* __restrict__ C, const uint16_t* __restrict__ C_lo,
    const float* __restrict__ zeta, float* __restrict__ dq, uint16_t* __restrict__ dS,
    float* __restrict__ dzeta) {
  constexpr int NT = BLK * 2, W = BLK / 32, KS = D / 16, DB = D / 32;
  __shared__ __attribute__((aligned(16))) char Sr[D * D * 2];    // S_i: rows c, e contiguous
  __shared__ __attribute__((aligned(16))) char Sl[D * D * 2];    // its low part, same layout
  __shared__ __attribute__((aligned(16))) char At[D * BLK * 2];  // phi(Q)^T: rows c, n contiguous
  __shared__ __attribute__((aligned(16))) char Gt[D * BLK * 2];  // G^T: rows e, n contiguous
  __shared__ float winv[BLK], hs[BLK];
  const int64_t bh = blockIdx.x / nqb;
  const int qb = blockIdx.x % nqb;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int64_t head_off = bh * (int64_t)N * D;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + head_off, (uint32_t)N * D * 2);
  const __amdgpu_buffer_rsrc_t rdo = make_rsrc(d_o + head_off, (uint32_t)N * D * 2);
  const int64_t row = bh * nqb + qb;
  const uint16_t* St = C + row * D * D;  // S_i^T: row e holds c = 0..D-1
  const uint16_t* St_lo = C_lo + row * D * D;
  const float* zt = zeta + row * D;
  const int n = 32 * w + l32;  // query within the block
  const int qrow = qb * BLK + n;

  u32x4 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) qf[ks] = buf_load16(rq, (uint32_t)(qrow * D + 16 * ks + 8 * hf) * 2);
  float linv, hdot = 0.f;
  {
    f32x16 acc[DB];
    linv = linear_apply<D, true>(St, zt, qf, l32, hf, acc, St_lo);  // acc * linv = O_lin^T
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * hf;
        const uint32_t off = (uint32_t)(qrow * D + d0) * 2;
        const uint32_t x0 = __builtin_amdgcn_raw_buffer_load_b32(rdo, off, 0, 0);
        const uint32_t x1 = __builtin_amdgcn_raw_buffer_load_b32(rdo, off + 4, 0, 0);
        hdot = fmaf(bf16_bits_to_f32(x0 & 0xffffu), acc[db][4 * g], hdot);
        hdot = fmaf(bf16_bits_to_f32(x0 >> 16), acc[db][4 * g + 1], hdot);
        hdot = fmaf(bf16_bits_to_f32(x1 & 0xffffu), acc[db][4 * g + 2], hdot);
        hdot = fmaf(bf16_bits_to_f32(x1 >> 16), acc[db][4 * g + 3], hdot);
      }
  }
  hdot = sum_halves(hdot);
  const float hn = -hdot * linv * linv;  // -(dO . O_lin) / w
  if (hf == 0) {
    winv[n] = linv;
    hs[n] = hn;
  }
  // g_n = dO_n / w_n as the B operand, a hi + lo bf16 pair: lane holds
  // g[n][16 ks + 8 hf + 0..7]
  u32x4 gb[KS], gl[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const u32x4 x = buf_load16(rdo, (uint32_t)(qrow * D + 16 * ks + 8 * hf) * 2);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float g0 = bf16_bits_to_f32(x[e] & 0xffffu) * linv;
      const float g1 = bf16_bits_to_f32(x[e] >> 16) * linv;
      gb[ks][e] = pack_bf16x2(g0, g1);
      gl[ks][e] = pack_bf16x2_lo(g0, g1);
    }
  }
  __syncthreads();  // winv and hs written
  // S_i (the transpose of the stored S_i^T), phi(Q)^T and G^T into LDS; the
  // block's rows past N read as zeros and get phi = 0
  const int valid = min(BLK, N - qb * BLK);
  const uint32_t blk_bytes = (uint32_t)valid * D * 2;
  const int64_t blk_off = head_off + (int64_t)qb * BLK * D;
  stage_subblocks<D, D, NT>(make_rsrc(St, D * D * 2), 0, nullptr, Sr, tid, KeepChunk{});
  stage_subblocks<D, D, NT>(make_rsrc(St_lo, D * D * 2), 0, nullptr, Sl, tid, KeepChunk{});
  stage_subblocks<BLK, D, NT>(make_rsrc(q + blk_off, blk_bytes), 0, nullptr, At, tid,
                              PhiChunk{valid});
  stage_subblocks<BLK, D, NT>(make_rsrc(d_o + blk_off, blk_bytes), 0, nullptr, Gt, tid,
                              ScaleChunk{winv});
  __syncthreads();

  // da^T = S_i G^T: A = S_i [c x e] rows from Sr (and Sl), B = G^T from
  // registers; hi g_hi + hi g_lo + lo g_hi
  {
    f32x16 dacc[DB];
#pragma unroll
    for (int cb = 0; cb < DB; ++cb) dacc[cb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int cb = 0; cb < DB; ++cb) {
        const uint32_t off = tr_offset<D>(32 * cb + l32, 2 * ks + hf);
        const u32x4 sh = *(const u32x4*)(Sr + off), sl = *(const u32x4*)(Sl + off);
        dacc[cb] = mfma32x32x16(sh, gb[ks], dacc[cb]);
        dacc[cb] = mfma32x32x16(sh, gl[ks], dacc[cb]);
        dacc[cb] = mfma32x32x16(sl, gb[ks], dacc[cb]);
      }
    if (qrow < N) {
      float* drow = dq + head_off + (int64_t)qrow * D;
#pragma unroll
      for (int cb = 0; cb < DB; ++cb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c0 = 32 * cb + 8 * g + 4 * hf;
          const uint32_t off = (uint32_t)(qrow * D + c0) * 2;
          const uint32_t x0 = __builtin_amdgcn_raw_buffer_load_b32(rq, off, 0, 0);
          const uint32_t x1 = __builtin_amdgcn_raw_buffer_load_b32(rq, off + 4, 0, 0);
          const float qv[4] = {bf16_bits_to_f32(x0 & 0xffffu), bf16_bits_to_f32(x0 >> 16),
                               bf16_bits_to_f32(x1 & 0xffffu), bf16_bits_to_f32(x1 >> 16)};
          f32x4 cur = *(f32x4*)(drow + c0);
#pragma unroll
          for (int r = 0; r < 4; ++r)
            cur[r] += fmaf(zt[c0 + r], hn, dacc[cb][4 * g + r]) * dphi(qv[r]);
          *(f32x4*)(drow + c0) = cur;
        }
    }
  }

  // dS_i [c x e] = A^T G over the block's queries: (D/32)^2 blocks of 32 x 32
  // spread over the waves; stored like the forward states, dS[row][e * D + c]
  uint16_t* dSi = dS + row * D * D;
#pragma unroll
  for (int u = w; u < DB * DB; u += W) {
    const int cb = u / DB, eb = u % DB;
    f32x16 acc = f32x16{};
#pragma unroll
    for (int ks = 0; ks < BLK / 16; ++ks)
      acc = mfma32x32x16(*(const u32x4*)(At + tr_offset<BLK>(32 * cb + l32, 2 * ks + hf)),
                         *(const u32x4*)(Gt + tr_offset<BLK>(32 * eb + l32, 2 * ks + hf)), acc);
    const int e = 32 * eb + l32;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c = 32 * cb + 8 * g + 4 * hf;
      *(u32x2*)(dSi + e * D + c) = u32x2{pack_bf16x2(acc[4 * g], acc[4 * g + 1]),
                                         pack_bf16x2(acc[4 * g + 2], acc[4 * g + 3])};
    }
  }
  // dzeta_i[c] = sum_n a_n[c] h_n, in query order
  if (tid < D) {
    float z = 0.f;
    for (int m = 0; m < BLK; ++m) {
      const uint16_t a = *(const uint16_t*)(At + tr_offset<BLK>(tid, m >> 3) + 2 * (m & 7));
      z = fmaf(bf16_bits_to_f32(a), hs[m], z);
    }
    dzeta[row * D + tid] = z;
  }
}

// One workgroup per key tile, BLK/32 waves of 32 keys (one per lane).
template <int D, int BLK>
__global__ __launch_bounds__(BLK * 2) void key_kernel(const uint16_t* __restrict__ k,
                                                      const uint16_t* __restrict__ v, int N,
                                                      int nkb, const uint16_t* __restrict__ dHt,
                                                      const float* __restrict__ dz,
                                                      float* __restrict__ dk,
                                                      float* __restrict__ dv) {
  constexpr int NT = BLK * 2, KS = D / 16, DB = D / 32;
  __shared__ __attribute__((aligned(16))) char Hr[D * D * 2];  // dH_j^T: rows e, c contiguous
  __shared__ __attribute__((aligned(16))) char Ht[D * D * 2];  // dH_j: rows c, e contiguous
  const int64_t bh = blockIdx.x / nkb;
  const int j = blockIdx.x % nkb;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int64_t head_off = bh * (int64_t)N * D;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + head_off, (uint32_t)N * D * 2);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + head_off, (uint32_t)N * D * 2);
  const int64_t row = bh * nkb + j;
  stage_subblocks<D, D, NT>(make_rsrc(dHt + row * D * D, D * D * 2), 0, Hr, Ht, tid, KeepChunk{});
  const int key = j * BLK + 32 * w + l32;
  u32x4 vf[KS], pk[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const uint32_t off = (uint32_t)(key * D + 16 * ks + 8 * hf) * 2;
    vf[ks] = buf_load16(rv, off);
    pk[ks] = phi8(buf_load16(rk, off), key < N);
  }
  __syncthreads();

  // dPhi^T [c x m] = dH_j [c x e] V^T
  f32x16 pacc[DB];
#pragma unroll
  for (int cb = 0; cb < DB; ++cb) pacc[cb] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int cb = 0; cb < DB; ++cb)
      pacc[cb] = mfma32x32x16(*(const u32x4*)(Ht + tr_offset<D>(32 * cb + l32, 2 * ks + hf)), vf[ks],
                              pacc[cb]);
  if (key < N) {
    float* krow = dk + head_off + (int64_t)key * D;
    const float* zr = dz + row * D;
#pragma unroll
    for (int cb = 0; cb < DB; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c0 = 32 * cb + 8 * g + 4 * hf;
        const uint32_t off = (uint32_t)(key * D + c0) * 2;
        const uint32_t x0 = __builtin_amdgcn_raw_buffer_load_b32(rk, off, 0, 0);
        const uint32_t x1 = __builtin_amdgcn_raw_buffer_load_b32(rk, off + 4, 0, 0);
        const float kv[4] = {bf16_bits_to_f32(x0 & 0xffffu), bf16_bits_to_f32(x0 >> 16),
                             bf16_bits_to_f32(x1 & 0xffffu), bf16_bits_to_f32(x1 >> 16)};
        f32x4 cur = *(f32x4*)(krow + c0);
#pragma unroll
        for (int r = 0; r < 4; ++r) cur[r] += (pacc[cb][4 * g + r] + zr[c0 + r]) * dphi(kv[r]);
        *(f32x4*)(krow + c0) = cur;
      }
  }
  // dV^T [e x m] = dH_j^T [e x c] Phi^T
  f32x16 vacc[DB];
#pragma unroll
  for (int eb = 0; eb < DB; ++eb) vacc[eb] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int eb = 0; eb < DB; ++eb)
      vacc[eb] = mfma32x32x16(*(const u32x4*)(Hr + row_offset<D / 8>(32 * eb + l32, 2 * ks + hf)),
                              pk[ks], vacc[eb]);
  if (key < N) {
    float* vrow = dv + head_off + (int64_t)key * D;
#pragma unroll
    for (int eb = 0; eb < DB; ++eb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int e0 = 32 * eb + 8 * g + 4 * hf;
        f32x4 cur = *(f32x4*)(vrow + e0);
#pragma unroll
        for (int r = 0; r < 4; ++r) cur[r] += vacc[eb][4 * g + r];
        *(f32x4*)(vrow + e0) = cur;
      }
  }
}

}  // namespace glbwd

hipError_t launch_linear_bwd_query_generic(const uint16_t* q, const uint16_t* d_o, int64_t BH,
                                           int N, int d, int block, int nb, const uint16_t* C,
                                           const uint16_t* C_lo, const float* zeta, float* dq,
                                           uint16_t* dS, float* dzeta, hipStream_t s) {
  const dim3 grid((unsigned)(BH * nb));
  if (d == 64 && block == 64)
    glbwd::query_kernel<64, 64><<<grid, 128, 0, s>>>(q, d_o, N, nb, C, C_lo, zeta, dq, dS, dzeta);
  else if (d == 64 && block == 128)
    glbwd::query_kernel<64, 128><<<grid, 256, 0, s>>>(q, d_o, N, nb, C, C_lo, zeta, dq, dS, dzeta);
  else if (d == 128 && block == 64)
    glbwd::query_kernel<128, 64><<<grid, 128, 0, s>>>(q, d_o, N, nb, C, C_lo, zeta, dq, dS, dzeta);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_linear_bwd_key_generic(const uint16_t* k, const uint16_t* v, int64_t BH, int N,
                                         int d, int block, int nb, const uint16_t* dH,
                                         const float* dz, float* dk, float* dv, hipStream_t s) {
  const dim3 grid((unsigned)(BH * nb));
  if (d == 64 && block == 64)
    glbwd::key_kernel<64, 64><<<grid, 128, 0, s>>>(k, v, N, nb, dH, dz, dk, dv);
  else if (d == 64 && block == 128)
    glbwd::key_kernel<64, 128><<<grid, 256, 0, s>>>(k, v, N, nb, dH, dz, dk, dv);
  else if (d == 128 && block == 64)
    glbwd::key_kernel<128, 64><<<grid, 128, 0, s>>>(k, v, N, nb, dH, dz, dk, dv);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace sla
