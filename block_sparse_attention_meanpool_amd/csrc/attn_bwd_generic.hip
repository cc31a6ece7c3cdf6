// Backward pass of the softmax branch for the shapes other than d = 128 with
// 128-token blocks: d in {64, 128}, blocks of 64 or 128 tokens.  Same
// gradients as the pipelined kernels (SLA post, results: the method is
// trainable), with P recomputed from the forward's LSE over each query
// block's critical keys:
//   D_n = dO_n . O_s_n,   dS = P * (dO V^T - D)
//   dQ = scale dS K,      dK = scale dS^T Q,      dV = P^T dO
//
// The layout follows the generic forward kernel: tiles are staged through
// LDS by ordinary loads, each tile once row-major (16-byte chunks XOR-
// swizzled per row) for the MFMA operands that run along the feature axis
// and, where needed, once transposed (feature rows, token-contiguous) for the
// operands that run along the token axis.  One global read feeds both copies.
//
// dq:   one workgroup per query block, BLK/32 waves of 32 queries (one query
//       per lane column): S^T = K Q^T, dP^T = V dO^T, dQ^T += K^T dS^T; it
//       also writes D for the second kernel.
// dkdv: one workgroup per key tile, BLK/32 waves of 32 keys: over the query
//       blocks whose critical list holds the tile, S = Q K^T, dP = dO V^T,
//       dV^T += dO^T P, dK^T += Q^T dS.
#include "common.h"
#include "launch.h"
#include "lists.h"
#include "staging.h"

namespace sla {
namespace gbwd {

// Tile rows [row0, row0 + BLK) of a [N, D] bf16 tensor into LDS: row-major
// (rows != nullptr) and/or transposed (tr != nullptr).  Rows past the
// resource's range read as zeros.
template <int D, int BLK>
__device__ __forceinline__ void stage(const __amdgpu_buffer_rsrc_t& r, int row0, char* rows,
                                      char* tr, int tid) {
  stage_subblocks<BLK, D, BLK * 2>(r, row0, rows, tr, tid, KeepChunk{});
}

// d = 64 with 64-token blocks fits three waves per SIMD without spills (10%
// faster than two); the other shapes keep two.
template <int D, int BLK>
__global__ __launch_bounds__(BLK * 2) __attribute__((amdgpu_waves_per_eu(
    D == 64 && BLK == 64 ? 3 : 2, D == 64 && BLK == 64 ? 3 : 2))) void dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const void* __restrict__ o_s, int o_fp32, const float* __restrict__ lse,
    const uint16_t* __restrict__ d_o, int N, int nqb, int nkb, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ cnt, int kmax, float sl2, float scale, float* __restrict__ dq,
    float* __restrict__ Dbuf, int seg, const int32_t* __restrict__ order) {
  constexpr int CH = D / 8, KS = D / 16, KB = BLK / 32;
  __shared__ __attribute__((aligned(16))) char Ks[BLK * D * 2];
  __shared__ __attribute__((aligned(16))) char Kt[D * BLK * 2];
  __shared__ __attribute__((aligned(16))) char Vs[BLK * D * 2];

  const int xcd = blockIdx.x & 7;
  const int slot = blockIdx.x >> 3;
  const int64_t bh = slot / seg;
  const int pos = xcd * seg + slot % seg;
  if (pos >= nqb) return;
  const int qb = ordered_block(order, bh, nqb, pos);
  if (qb < 0) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int64_t head_off = bh * (int64_t)N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + head_off, head_bytes);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + head_off, head_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + head_off, head_bytes);
  const __amdgpu_buffer_rsrc_t rdo = make_rsrc(d_o + head_off, head_bytes);

  // Q and dO as B operands: lane holds row qrow, features 16 ks + 8 hf + 0..7.
  const int qrow = qb * BLK + 32 * w + l32;
  u32x4 qf[KS], dof[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const uint32_t off = (uint32_t)(qrow * D + 16 * ks + 8 * hf) * 2;
    qf[ks] = buf_load16(rq, off);
    dof[ks] = buf_load16(rdo, off);
  }
  // D_n = dO_n . O_s_n over this lane's D/2 features, then both halves.
  float dn = 0.f;
  if (o_fp32) {
    const __amdgpu_buffer_rsrc_t ro = make_rsrc((const float*)o_s + head_off, (uint32_t)N * D * 4);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint32_t off = (uint32_t)(qrow * D + 16 * ks + 8 * hf) * 4;
      const u32x4 a = buf_load16(ro, off), b = buf_load16(ro, off + 16);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        dn = fmaf(bf16_bits_to_f32(dof[ks][e] & 0xffffu), __uint_as_float(a[2 * e]), dn);
        dn = fmaf(bf16_bits_to_f32(dof[ks][e] >> 16), __uint_as_float(a[2 * e + 1]), dn);
        dn = fmaf(bf16_bits_to_f32(dof[ks][2 + e] & 0xffffu), __uint_as_float(b[2 * e]), dn);
        dn = fmaf(bf16_bits_to_f32(dof[ks][2 + e] >> 16), __uint_as_float(b[2 * e + 1]), dn);
      }
    }
  } else {
    const __amdgpu_buffer_rsrc_t ro = make_rsrc((const uint16_t*)o_s + head_off, head_bytes);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 a = buf_load16(ro, (uint32_t)(qrow * D + 16 * ks + 8 * hf) * 2);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dn = fmaf(bf16_bits_to_f32(dof[ks][e] & 0xffffu), bf16_bits_to_f32(a[e] & 0xffffu), dn);
        dn = fmaf(bf16_bits_to_f32(dof[ks][e] >> 16), bf16_bits_to_f32(a[e] >> 16), dn);
      }
    }
  }
  dn = sum_halves(dn);
  const float lse2 = qrow < N ? lse[bh * N + qrow] * kLog2e : 0.f;
  if (hf == 0 && qrow < N) Dbuf[bh * N + qrow] = dn;

  const int count = min(cnt[bh * nqb + qb], kmax);
  const int32_t* list = idx + (bh * nqb + qb) * (int64_t)kmax;
  const bool canon = __builtin_amdgcn_readfirstlane(list_is_canonical(list, count, nkb, lane));
  f32x16 dqacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) dqacc[db] = f32x16{};
  const int krow = swap_bits_2_3(l32);

  for (int t = 0; t < count; ++t) {
    const int j = list[t];
    if (!list_entry_used(list, t, j, nkb, canon)) continue;  // the list is a set of tiles
    __syncthreads();  // the previous tile's LDS reads are done
    stage<D, BLK>(rk, j * BLK, Ks, Kt, tid);
    stage<D, BLK>(rv, j * BLK, Vs, nullptr, tid);
    __syncthreads();

    // S^T = K Q^T and dP^T = V dO^T: KB blocks of 32 keys.
    f32x16 sacc[KB], dpacc[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) sacc[kb] = dpacc[kb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const uint32_t off = row_offset<CH>(32 * kb + krow, 2 * ks + hf);
        sacc[kb] = mfma32x32x16(*(const u32x4*)(Ks + off), qf[ks], sacc[kb]);
        dpacc[kb] = mfma32x32x16(*(const u32x4*)(Vs + off), dof[ks], dpacc[kb]);
      }
    if ((j + 1) * BLK > N) {
      // register r of block kb holds key j BLK + 8 hf + (32 kb + r + 8 [r >= 8])
      const int lim = N - j * BLK - 8 * hf;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * kb + r + (r >= 8 ? 8 : 0) >= lim) sacc[kb][r] = -INFINITY;
    }
    // dS^T = P^T (dP^T - D), as B operands of 16 keys each.
    u32x4 dsb[BLK / 16];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int hs = 0; hs < 2; ++hs)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int r = 8 * hs + 2 * p;
          const float p0 = fast_exp2(fmaf(sacc[kb][r], sl2, -lse2));
          const float p1 = fast_exp2(fmaf(sacc[kb][r + 1], sl2, -lse2));
          dsb[2 * kb + hs][p] = pack_bf16x2(p0 * (dpacc[kb][r] - dn), p1 * (dpacc[kb][r + 1] - dn));
        }
    // dQ^T += K^T dS^T.
#pragma unroll
    for (int ks2 = 0; ks2 < BLK / 16; ++ks2)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const u32x4 a = *(const u32x4*)(Kt + tr_offset<BLK>(32 * db + l32, 2 * ks2 + hf));
        dqacc[db] = mfma32x32x16(a, dsb[ks2], dqacc[db]);
      }
  }

  if (qrow < N) {
    float* orow = dq + head_off + (int64_t)qrow * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * hf;
        *(f32x4*)(orow + d0) = f32x4{dqacc[db][4 * g] * scale, dqacc[db][4 * g + 1] * scale,
                                     dqacc[db][4 * g + 2] * scale, dqacc[db][4 * g + 3] * scale};
      }
  }
}

// Two waves per SIMD where the registers allow it; d = 128 (its dK and dV
// accumulators alone take 128 registers) runs at one.
template <int D, int BLK>
__global__ __launch_bounds__(BLK * 2) __attribute__((amdgpu_waves_per_eu(D == 128 ? 1 : 2, 2))) void dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ lse, const float* __restrict__ Dbuf,
    const uint16_t* __restrict__ d_o, int N, int nqb, int nkb,
    const uint16_t* __restrict__ col_idx, const int32_t* __restrict__ col_cnt, int width,
    float sl2, float scale, float* __restrict__ dk, float* __restrict__ dv, int seg) {
  constexpr int CH = D / 8, KS = D / 16;
  __shared__ __attribute__((aligned(16))) char Qs[BLK * D * 2];
  __shared__ __attribute__((aligned(16))) char Qt[D * BLK * 2];
  __shared__ __attribute__((aligned(16))) char Os[BLK * D * 2];
  __shared__ __attribute__((aligned(16))) char Ot[D * BLK * 2];
  __shared__ __attribute__((aligned(16))) float Ls[BLK], Es[BLK];

  const int xcd = blockIdx.x & 7;
  const int slot = blockIdx.x >> 3;
  const int64_t bh = slot / seg;
  const int kt = xcd * seg + slot % seg;
  if (kt >= nkb) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int64_t head_off = bh * (int64_t)N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + head_off, head_bytes);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + head_off, head_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + head_off, head_bytes);
  const __amdgpu_buffer_rsrc_t rdo = make_rsrc(d_o + head_off, head_bytes);

  // K and V as B operands: lane holds key `key`, features 16 ks + 8 hf + 0..7.
  const int key = kt * BLK + 32 * w + l32;
  u32x4 kf[KS], vf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const uint32_t off = (uint32_t)(key * D + 16 * ks + 8 * hf) * 2;
    kf[ks] = buf_load16(rk, off);
    vf[ks] = buf_load16(rv, off);
  }
  f32x16 dkacc[D / 32], dvacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) dkacc[db] = dvacc[db] = f32x16{};
  const int qrowp = swap_bits_2_3(l32);
  const int count = col_cnt[bh * nkb + kt];
  const int64_t list0 = (bh * nkb + kt) * (int64_t)width;  // first entry of this tile's list

  for (int t = 0; t < count; ++t) {
    const int i = u16_entry(col_idx, list0 + t);
    __syncthreads();  // the previous block's LDS reads are done
    stage<D, BLK>(rq, i * BLK, Qs, Qt, tid);
    stage<D, BLK>(rdo, i * BLK, Os, Ot, tid);
    if (tid < BLK) {
      // queries past N: LSE and D read as 0; their Q and dO rows are zeros,
      // so they add nothing to dK or dV
      const int n = i * BLK + tid;
      Ls[tid] = n < N ? lse[bh * N + n] * kLog2e : 0.f;
      Es[tid] = n < N ? Dbuf[bh * N + n] : 0.f;
    }
    __syncthreads();

#pragma unroll
    for (int qb2 = 0; qb2 < BLK / 32; ++qb2) {
      f32x16 sacc = f32x16{}, dpacc = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint32_t off = row_offset<CH>(32 * qb2 + qrowp, 2 * ks + hf);
        sacc = mfma32x32x16(*(const u32x4*)(Qs + off), kf[ks], sacc);
        dpacc = mfma32x32x16(*(const u32x4*)(Os + off), vf[ks], dpacc);
      }
      // register r holds query 32 qb2 + 16 (r / 8) + 8 hf + r % 8 of the block
#pragma unroll
      for (int hs = 0; hs < 2; ++hs) {
        const int q0 = 32 * qb2 + 16 * hs + 8 * hf;
        u32x4 pb, dsb;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int r = 8 * hs + 2 * p;
          const float p0 = fast_exp2(fmaf(sacc[r], sl2, -Ls[q0 + 2 * p]));
          const float p1 = fast_exp2(fmaf(sacc[r + 1], sl2, -Ls[q0 + 2 * p + 1]));
          pb[p] = pack_bf16x2(p0, p1);
          dsb[p] = pack_bf16x2(p0 * (dpacc[r] - Es[q0 + 2 * p]), p1 * (dpacc[r + 1] - Es[q0 + 2 * p + 1]));
        }
        const int ks2 = 2 * qb2 + hs;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const uint32_t off = tr_offset<BLK>(32 * db + l32, 2 * ks2 + hf);
          dvacc[db] = mfma32x32x16(*(const u32x4*)(Ot + off), pb, dvacc[db]);
          dkacc[db] = mfma32x32x16(*(const u32x4*)(Qt + off), dsb, dkacc[db]);
        }
      }
    }
  }

  if (key < N) {
    float* krow_out = dk + head_off + (int64_t)key * D;
    float* vrow_out = dv + head_off + (int64_t)key * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * hf;
        *(f32x4*)(krow_out + d0) = f32x4{dkacc[db][4 * g] * scale, dkacc[db][4 * g + 1] * scale,
                                         dkacc[db][4 * g + 2] * scale, dkacc[db][4 * g + 3] * scale};
        *(f32x4*)(vrow_out + d0) = f32x4{dvacc[db][4 * g], dvacc[db][4 * g + 1],
                                         dvacc[db][4 * g + 2], dvacc[db][4 * g + 3]};
      }
  }
}

template <int D, int BLK>
static hipError_t launch_t(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t BH,
                           int N, int nb, const int32_t* idx, const int32_t* cnt, int kmax,
                           float scale, const void* o_s, int o_fp32, const float* lse,
                           const uint16_t* d_o, float* dq, float* dk, float* dv, float* Dbuf,
                           const uint16_t* col_idx, const int32_t* col_cnt, const int32_t* order,
                           hipStream_t s) {
  const int seg = (nb + 7) / 8;
  const dim3 grid((unsigned)(BH * seg * 8));
  const float sl2 = scale * kLog2e;
  dq_kernel<D, BLK><<<grid, BLK * 2, 0, s>>>(q, k, v, o_s, o_fp32, lse, d_o, N, nb, nb, idx, cnt,
                                              kmax, sl2, scale, dq, Dbuf, seg, order);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dkdv_kernel<D, BLK><<<grid, BLK * 2, 0, s>>>(q, k, v, lse, Dbuf, d_o, N, nb, nb, col_idx, col_cnt,
                                                nb, sl2, scale, dk, dv, seg);
  return hipGetLastError();
}

}  // namespace gbwd

hipError_t launch_attn_bwd_generic(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                   int64_t BH, int N, int d, int block, int nb,
                                   const int32_t* idx, const int32_t* cnt, int kmax, float scale,
                                   const void* o_s, int o_fp32, const float* lse,
                                   const uint16_t* d_o, float* dq, float* dk, float* dv,
                                   float* Dbuf, const uint16_t* col_idx, const int32_t* col_cnt,
                                   const int32_t* order, hipStream_t s) {
  if (d == 64 && block == 64)
    return gbwd::launch_t<64, 64>(q, k, v, BH, N, nb, idx, cnt, kmax, scale, o_s, o_fp32, lse, d_o,
                                  dq, dk, dv, Dbuf, col_idx, col_cnt, order, s);
  if (d == 64 && block == 128)
    return gbwd::launch_t<64, 128>(q, k, v, BH, N, nb, idx, cnt, kmax, scale, o_s, o_fp32, lse,
                                   d_o, dq, dk, dv, Dbuf, col_idx, col_cnt, order, s);
  if (d == 128 && block == 64)
    return gbwd::launch_t<128, 64>(q, k, v, BH, N, nb, idx, cnt, kmax, scale, o_s, o_fp32, lse,
                                   d_o, dq, dk, dv, Dbuf, col_idx, col_cnt, order, s);
  return hipErrorInvalidValue;
}

}  // namespace sla
