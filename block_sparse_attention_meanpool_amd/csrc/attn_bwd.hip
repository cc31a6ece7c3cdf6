// Backward pass of the softmax branch with the class map held fixed (SLA
// post, results: the method is trainable with a short fine-tuning).  With P
// recomputed from the forward's LSE over each query block's critical keys:
//   D_n = dO_n . O_s_n,   dS = P * (dO V^T - D)
//   dQ = scale dS K,      dK = scale dS^T Q,      dV = P^T dO
// d = 128, 128-token blocks.
//
// col bits / lists: the query blocks whose critical list holds key tile j,
//        ascending (a bit matrix scattered from the row lists, then one wave
//        per key tile compacts its column).
// dq:    one workgroup per query block, as in the forward: S^T = K Q^T and
//        dP^T = V dO^T with one query per lane, dQ^T += K^T dS^T; it also
//        writes D for the dK/dV pass.
// dkdv:  one workgroup per key tile, one key per lane: S = Q K^T and
//        dP = dO V^T over the query blocks of the tile's column list, then
//        dV^T += dO^T P and dK^T += Q^T dS.
// K and V (dq) and Q and dO (dkdv) are read both by rows and transposed, so
// their LDS tiles use the dual swizzle; they arrive by asynchronous
// LDS-direct loads into double buffers of 64-row halves, rows past N landing
// as zeros.
#include "common.h"
#include "launch.h"
#include "lists.h"

namespace sla {
namespace bwd {

constexpr int D = 128, BLK = 128, HALF = 64, NT = 256;
constexpr int BUFB = HALF * 256;  // 64 rows of 256 bytes

__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t* __restrict__ p, int64_t n,
                                                       uint32_t value) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = value;
}

// Bit (j, i) of the column bit matrix for every entry j of query block i's
// list; entries outside [0, nkb) are dropped.
__global__ __launch_bounds__(256) void col_bits_kernel(const int32_t* __restrict__ idx,
                                                       const int32_t* __restrict__ cnt, int kmax,
                                                       int64_t rows, int nqb, int nkb, int WC,
                                                       uint32_t* __restrict__ bitsT) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= rows * kmax) return;
  const int64_t row = t / kmax;
  const int pos = (int)(t % kmax);
  if (pos >= min(cnt[row], kmax)) return;
  const int j = idx[t];
  if (j < 0 || j >= nkb) return;
  const int64_t bh = row / nqb;
  const int i = (int)(row % nqb);
  atomicOr(&bitsT[(bh * nkb + j) * WC + (i >> 5)], 1u << (i & 31));
}

// One wave per column: its set bits as an ascending list of query blocks.
__global__ __launch_bounds__(256) void col_lists_kernel(const uint32_t* __restrict__ bitsT,
                                                        int64_t cols, int WC, int width,
                                                        uint16_t* __restrict__ col_idx,
                                                        int32_t* __restrict__ col_cnt) {
  const int lane = threadIdx.x & 63;
  const int64_t col = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (col >= cols) return;
  const uint32_t* wrow = bitsT + col * WC;
  uint32_t w0 = lane < WC ? wrow[lane] : 0u;
  uint32_t w1 = lane + 64 < WC ? wrow[lane + 64] : 0u;
  const int c0 = __popc(w0), c1 = __popc(w1);
  int s0 = c0, s1 = c1;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t0 = __shfl_up(s0, o), t1 = __shfl_up(s1, o);
    if (lane >= o) {
      s0 += t0;
      s1 += t1;
    }
  }
  const int tot0 = __shfl(s0, 63);
  const int total = tot0 + __shfl(s1, 63);
  int p0 = s0 - c0, p1 = tot0 + s1 - c1;
  uint16_t* out = col_idx + col * width;
  while (w0) {
    out[p0++] = (uint16_t)(32 * lane + __ffs(w0) - 1);
    w0 &= w0 - 1u;
  }
  while (w1) {
    out[p1++] = (uint16_t)(32 * (lane + 64) + __ffs(w1) - 1);
    w1 &= w1 - 1u;
  }
  if (lane == 0) col_cnt[col] = total;
}

// Rows [row0, row0 + 64) of two d = 128 bf16 tensors into dual-swizzled LDS
// halves: each wave moves 4 KB of each, lane-contiguous in LDS, the global
// chunk each lane fetches implementing the swizzle.  Rows past the buffer
// range land as zeros.
__device__ __forceinline__ void issue_rows(const __amdgpu_buffer_rsrc_t& ra,
                                           const __amdgpu_buffer_rsrc_t& rb, int row0, char* abuf,
                                           char* bbuf, int lane, int w) {
  // the wave index, known uniform: the LDS destinations stay scalar
  const int wu = __builtin_amdgcn_readfirstlane(w);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int inst = 4 * wu + e;
    const int row = 4 * inst + (lane >> 4);
    const int ch = (lane & 15) ^ dual_swz(row);
    const uint32_t off = (uint32_t)((row0 + row) * D + ch * 8) * 2;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void_ptr)(abuf + inst * 1024), 16, off, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void_ptr)(bbuf + inst * 1024), 16, off, 0, 0, 0);
  }
}

// ---------------------------------------------------------------------------
// dQ (and D), one workgroup per query block
// ---------------------------------------------------------------------------

// One 64-key half of a critical tile: S^T = K Q^T, dP^T = V dO^T,
// dS^T = P^T (dP^T - D), dQ^T += K^T dS^T.
__device__ __forceinline__ void dq_half(const char* kbuf, const char* vbuf, const u32x4 (&qf)[8],
                                        const u32x4 (&dof)[8], f32x16 (&dqacc)[4], float lse2,
                                        float dn, int key0, int N, float sl2, int hf, int krow,
                                        int lane) {
  f32x16 sacc[2] = {f32x16{}, f32x16{}};
  f32x16 dpacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = mfma32x32x16(dual_row_read(kbuf, 32 * kb + krow, 2 * ks + hf), qf[ks], sacc[kb]);
      dpacc[kb] = mfma32x32x16(dual_row_read(vbuf, 32 * kb + krow, 2 * ks + hf), dof[ks], dpacc[kb]);
    }
  }
  // Scheduling hints (LLVM's interleave strategies) for the MFMA chains with
  // their LDS reads and for the exp2 softmax with the dQ MFMAs; instruction
  // order only, results bit-identical.
  __builtin_amdgcn_iglp_opt(1);
  if (key0 + HALF > N) {
    // register r of block kb holds key key0 + 8 hf + (32 kb + r + 8 [r >= 8])
    const int lim = N - key0 - 8 * hf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (32 * kb + r + (r >= 8 ? 8 : 0) >= lim) sacc[kb][r] = -INFINITY;
  }
  u32x4 dsb[4];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int hs = 0; hs < 2; ++hs)
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int r = 8 * hs + 2 * p;
        const float p0 = fast_exp2(fmaf(sacc[kb][r], sl2, -lse2));
        const float p1 = fast_exp2(fmaf(sacc[kb][r + 1], sl2, -lse2));
        dsb[2 * kb + hs][p] = pack_bf16x2(p0 * (dpacc[kb][r] - dn), p1 * (dpacc[kb][r + 1] - dn));
      }
#pragma unroll
  for (int ks2 = 0; ks2 < 4; ++ks2)
#pragma unroll
    for (int db = 0; db < 4; ++db)
      dqacc[db] = mfma32x32x16(tr_operand<DualSwz>(kbuf, 16 * ks2, 32 * db, lane), dsb[ks2], dqacc[db]);
  __builtin_amdgcn_iglp_opt(2);
}

__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const void* __restrict__ o_s, int o_fp32, const float* __restrict__ lse,
    const uint16_t* __restrict__ d_o, int N, int nqb, int nkb, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ cnt, int kmax, float sl2, float scale, float* __restrict__ dq,
    float* __restrict__ Dbuf, float* __restrict__ L2buf, int seg, const int32_t* __restrict__ order) {
  __shared__ __attribute__((aligned(1024))) char K0[BUFB];
  __shared__ __attribute__((aligned(1024))) char V0[BUFB];
  __shared__ __attribute__((aligned(1024))) char K1[BUFB];
  __shared__ __attribute__((aligned(1024))) char V1[BUFB];

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

  const int count = min(cnt[bh * nqb + qb], kmax);
  const int32_t* list = idx + (bh * nqb + qb) * (int64_t)kmax;
  int j_cur = count > 0 ? list[0] : 0;
  auto clampj = [&](int j) { return min(max(j, 0), nkb - 1); };
  if (count > 0) issue_rows(rk, rv, clampj(j_cur) * BLK, K0, V0, lane, w);

  const int qrow = qb * BLK + 32 * w + l32;
  u32x4 qf[8], dof[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const uint32_t off = (uint32_t)(qrow * D + 16 * ks + 8 * hf) * 2;
    qf[ks] = buf_load16(rq, off);
    dof[ks] = buf_load16(rdo, off);
  }
  // D_n = dO_n . O_s_n: this lane's 64 features, then both halves.
  float dn = 0.f;
  if (o_fp32) {
    const __amdgpu_buffer_rsrc_t ro = make_rsrc((const float*)o_s + head_off, (uint32_t)N * D * 4);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
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
    for (int ks = 0; ks < 8; ++ks) {
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
  if (hf == 0 && qrow < N) {
    Dbuf[bh * N + qrow] = dn;
    L2buf[bh * N + qrow] = lse2;  // LSE log2 e, as the dK/dV pass uses it
  }

  f32x16 dqacc[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
  const int krow = swap_bits_2_3(l32);
  const bool canon = __builtin_amdgcn_readfirstlane(list_is_canonical(list, count, nkb, lane));
  for (int t = 0; t < count; ++t) {
    const bool ok = list_entry_used(list, t, j_cur, nkb, canon);  // the list is a set of tiles
    const int j_next = (t + 1 < count) ? list[t + 1] : 0;
    wait_vmcnt0();
    __syncthreads();  // buffer 0 complete; every wave is done with buffer 1
    issue_rows(rk, rv, clampj(j_cur) * BLK + HALF, K1, V1, lane, w);
    if (ok) dq_half(K0, V0, qf, dof, dqacc, lse2, dn, j_cur * BLK, N, sl2, hf, krow, lane);
    wait_vmcnt0();
    __syncthreads();  // buffer 1 complete; every wave is done with buffer 0
    if (t + 1 < count) issue_rows(rk, rv, clampj(j_next) * BLK, K0, V0, lane, w);
    if (ok && j_cur * BLK + HALF < N)
      dq_half(K1, V1, qf, dof, dqacc, lse2, dn, j_cur * BLK + HALF, N, sl2, hf, krow, lane);
    j_cur = j_next;
  }

  if (qrow < N) {
    float* orow = dq + head_off + (int64_t)qrow * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * hf;
        *(f32x4*)(orow + d0) = f32x4{dqacc[db][4 * g] * scale, dqacc[db][4 * g + 1] * scale,
                                     dqacc[db][4 * g + 2] * scale, dqacc[db][4 * g + 3] * scale};
      }
  }
}

// ---------------------------------------------------------------------------
// dK, dV, one workgroup per key tile, two waves per SIMD
// ---------------------------------------------------------------------------
// A workgroup runs the query blocks that list its key tile in list order, each
// as four 32-query stages: S = Q K^T, dP = dO V^T, P = exp2(S sl2 - LSE log2 e),
// dS = P (dP - D); dV^T += dO^T P, dK^T += Q^T dS.  K stays in registers; V
// (the tile's 128 rows) sits in LDS for the dP products; Q and dO come in
// 32-row stages through two alternating buffers chosen at run time, which
// keeps the swizzled LDS addresses loop-variant instead of one register per
// address.  65 KB of LDS and at most 256 registers let two workgroups share a
// CU, so each SIMD runs two waves.

// dV += P^T dO and dK += dS^T Q over a stage's 32 queries.
__device__ __forceinline__ void acc_block(const char* qbuf, const char* obuf, int lane,
                                          const u32x4 (&pb)[2], const u32x4 (&dsb)[2],
                                          f32x16 (&dkacc)[4], f32x16 (&dvacc)[4]) {
#pragma unroll
  for (int hs = 0; hs < 2; ++hs) {
    const int k0 = 16 * hs;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      dvacc[db] = mfma32x32x16(tr_operand<DualSwz>(obuf, k0, 32 * db, lane), pb[hs], dvacc[db]);
      dkacc[db] = mfma32x32x16(tr_operand<DualSwz>(qbuf, k0, 32 * db, lane), dsb[hs], dkacc[db]);
    }
  }
}

// One softmax step: P = exp2(S sl2 - LSE log2 e) and dS = P (dP - D) for the
// register pair r = 8 hs + 2 p (stage queries 16 hs + 8 hf + 2 p and the
// next), packed into the bf16 B operands pb[hs] and dsb[hs].
__device__ __forceinline__ void pds_step(const float* lbuf, const float* ebuf, int hf,
                                         float sl2, const f32x16& sacc, const f32x16& dpacc,
                                         int hs, int p, u32x4 (&pb)[2], u32x4 (&dsb)[2]) {
  const int q0 = 16 * hs + 8 * hf + 2 * p;
  const f32x2 lp = *(const f32x2*)(lbuf + q0), ep = *(const f32x2*)(ebuf + q0);
  const float l0 = lp[0], l1 = lp[1], e0 = ep[0], e1 = ep[1];
  const int r = 8 * hs + 2 * p;
  const float p0 = fast_exp2(fmaf(sacc[r], sl2, -l0));
  const float p1 = fast_exp2(fmaf(sacc[r + 1], sl2, -l1));
  pb[hs][p] = pack_bf16x2(p0, p1);
  dsb[hs][p] = pack_bf16x2(p0 * (dpacc[r] - e0), p1 * (dpacc[r + 1] - e1));
}

constexpr int SROWS = 32, SBUF = SROWS * 256;  // 8 KB per stage buffer

// Rows [row0, row0 + 32) of Q and dO into a dual-swizzled stage (2 KB of each
// per wave), and their LSE log2 e and D (wave 0 and 1, 64 entries each; the 32
// past the stage are never read).  The dQ pass writes LSE log2 e beside D, so
// the stage's exponent is one fma.
__device__ __forceinline__ void issue_stage(const __amdgpu_buffer_rsrc_t& rq,
                                            const __amdgpu_buffer_rsrc_t& rdo,
                                            const __amdgpu_buffer_rsrc_t& rl,
                                            const __amdgpu_buffer_rsrc_t& re, int row0, char* qbuf,
                                            char* obuf, float* lbuf, float* ebuf, int lane, int wu) {
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int inst = 2 * wu + e;
    const int row = 4 * inst + (lane >> 4);
    const int ch = (lane & 15) ^ dual_swz(row);
    const uint32_t off = (uint32_t)((row0 + row) * D + ch * 8) * 2;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (lds_void_ptr)(qbuf + inst * 1024), 16, off, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rdo, (lds_void_ptr)(obuf + inst * 1024), 16, off, 0, 0, 0);
  }
  const uint32_t off = (uint32_t)(row0 + lane) * 4;
  if (wu == 0)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (lds_void_ptr)lbuf, 4, off, 0, 0, 0);
  else if (wu == 1)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(re, (lds_void_ptr)ebuf, 4, off, 0, 0, 0);
}

__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ L2buf, const float* __restrict__ Dbuf,
    const uint16_t* __restrict__ d_o, int N, int nqb, int nkb,
    const uint16_t* __restrict__ col_idx, const int32_t* __restrict__ col_cnt, int width,
    float sl2, float scale, float* __restrict__ dk, float* __restrict__ dv, int seg) {
  __shared__ __attribute__((aligned(1024))) char Vt[BLK * 256];
  __shared__ __attribute__((aligned(1024))) char QS[2][SBUF];
  __shared__ __attribute__((aligned(1024))) char OS[2][SBUF];
  __shared__ __attribute__((aligned(256))) float LS[2][64], ES[2][64];

  const int xcd = blockIdx.x & 7;
  const int slot = blockIdx.x >> 3;
  const int64_t bh = slot / seg;
  // Each XCD takes a contiguous range of a head's key tiles (their column lists
  // overlap, which its L2 serves), and the range rotates from head to head:
  // tiles in some positions are listed by many more query blocks than others,
  // and a fixed range per XCD left some XCDs idle at the end.
  const int kt = (int)((xcd + bh) & 7) * seg + slot % seg;
  if (kt >= nkb) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int l32 = lane & 31, hf = lane >> 5;
  const int64_t head_off = bh * (int64_t)N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + head_off, head_bytes);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + head_off, head_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(v + head_off, head_bytes);
  const __amdgpu_buffer_rsrc_t rdo = make_rsrc(d_o + head_off, head_bytes);
  const __amdgpu_buffer_rsrc_t rl = make_rsrc(L2buf + bh * N, (uint32_t)N * 4);
  const __amdgpu_buffer_rsrc_t re = make_rsrc(Dbuf + bh * N, (uint32_t)N * 4);

  const int count = col_cnt[bh * nkb + kt];
  const int64_t list0 = (bh * nkb + kt) * (int64_t)width;
  const int nst = 4 * count;  // stages: 4 per listed query block
  // this tile's V rows, row-major with the K tiles' swizzle (8 KB per wave);
  // nothing is loaded for an empty list, so no load outlives the workgroup
  if (nst > 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int inst = 8 * wu + e;
      const int row = 4 * inst + (lane >> 4);
      const uint32_t off =
          (uint32_t)((kt * BLK + row) * D + ((lane & 15) ^ row_swz<16>(row)) * 8) * 2;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_ptr)(Vt + inst * 1024), 16, off, 0, 0, 0);
    }
  }
  int i_cur = count > 0 ? u16_entry(col_idx, list0) : 0;
  if (nst > 0) issue_stage(rq, rdo, rl, re, i_cur * BLK, QS[0], OS[0], LS[0], ES[0], lane, wu);

  const int key = kt * BLK + 32 * w + l32;
  u32x4 kf[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) kf[ks] = buf_load16(rk, (uint32_t)(key * D + 16 * ks + 8 * hf) * 2);
  f32x16 dkacc[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
  f32x16 dvacc[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
  const int qrowp = swap_bits_2_3(l32);
  const int vrow = 32 * w + l32;

#pragma unroll 1
  for (int u = 0; u < nst; ++u) {
    const int t = u >> 2, st = u & 3, b = u & 1;
    int i_nx = i_cur;
    if (st == 3) i_nx = (t + 1 < count) ? u16_entry(col_idx, list0 + t + 1) : 0;
    wait_vmcnt0();
    __syncthreads();  // stage u complete in buffer b; every wave is done with buffer b ^ 1
    if (u + 1 < nst)
      issue_stage(rq, rdo, rl, re, i_nx * BLK + SROWS * ((st + 1) & 3), QS[b ^ 1], OS[b ^ 1],
                  LS[b ^ 1], ES[b ^ 1], lane, wu);
    if (i_cur * BLK + SROWS * st < N) {
      const char* qbuf = QS[b];
      const char* obuf = OS[b];
      f32x16 sacc = f32x16{}, dpacc = f32x16{};
      // S's chain, then dP's, with LLVM's MFMA / LDS-read interleave strategy
      // for the stage (instruction order only: 1-2% off the backward against
      // the two chains interleaved, same bits)
      __builtin_amdgcn_iglp_opt(1);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        sacc = mfma32x32x16(dual_row_read(qbuf, qrowp, 2 * ks + hf), kf[ks], sacc);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const u32x4 vb = *(const u32x4*)(Vt + row_offset<16>(vrow, 2 * ks + hf));
        dpacc = mfma32x32x16(dual_row_read(obuf, qrowp, 2 * ks + hf), vb, dpacc);
      }
      u32x4 pb[2], dsb[2];
#pragma unroll
      for (int hs = 0; hs < 2; ++hs)
#pragma unroll
        for (int p = 0; p < 4; ++p) pds_step(LS[b], ES[b], hf, sl2, sacc, dpacc, hs, p, pb, dsb);
      acc_block(qbuf, obuf, lane, pb, dsb, dkacc, dvacc);
    }
    i_cur = i_nx;
  }

  if (key < N) {
    float* krow_out = dk + head_off + (int64_t)key * D;
    float* vrow_out = dv + head_off + (int64_t)key * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
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

}  // namespace bwd

hipError_t launch_col_bits(const int32_t* idx, const int32_t* cnt, int kmax, int64_t BH, int nrows,
                           int ncols, int WC, uint32_t* bitsT, hipStream_t s) {
  const int64_t nwords = BH * ncols * WC;
  const int64_t fill_blocks = (nwords + 255) / 256;
  bwd::fill_u32_kernel<<<dim3((unsigned)(fill_blocks < 65536 ? fill_blocks : 65536)), 256, 0, s>>>(
      bitsT, nwords, 0u);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows = BH * nrows;
  bwd::col_bits_kernel<<<dim3((unsigned)((rows * kmax + 255) / 256)), 256, 0, s>>>(
      idx, cnt, kmax, rows, nrows, ncols, WC, bitsT);
  return hipGetLastError();
}

AttnBwdWs attn_bwd_ws_layout(int64_t BH, int N, int nb) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  AttnBwdWs w;
  w.wc = 2 * ((nb + 63) / 64);
  w.d_bytes = 2 * up((size_t)BH * N * 4);  // D, then LSE log2 e
  w.bits_bytes = up((size_t)BH * nb * w.wc * 4);
  w.cnt_bytes = up((size_t)BH * nb * 4);
  w.idx_bytes = up((size_t)BH * nb * nb * 2);
  w.total = w.d_bytes + w.bits_bytes + w.cnt_bytes + w.idx_bytes;
  return w;
}

hipError_t launch_attn_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t BH,
                           int N, int d, int block, int nb, const int32_t* idx, const int32_t* cnt,
                           int kmax,
                           float scale, const void* o_s, int o_fp32, const float* lse,
                           const uint16_t* d_o, float* dq, float* dk, float* dv, void* ws,
                           const int32_t* order, hipStream_t s) {
  const AttnBwdWs lw = attn_bwd_ws_layout(BH, N, nb);
  char* p = static_cast<char*>(ws);
  float* Dbuf = reinterpret_cast<float*>(p);
  float* L2buf = reinterpret_cast<float*>(p + lw.d_bytes / 2);
  uint32_t* bitsT = reinterpret_cast<uint32_t*>(p + lw.d_bytes);
  int32_t* col_cnt = reinterpret_cast<int32_t*>(p + lw.d_bytes + lw.bits_bytes);
  uint16_t* col_idx = reinterpret_cast<uint16_t*>(p + lw.d_bytes + lw.bits_bytes + lw.cnt_bytes);

  hipError_t e = launch_col_bits(idx, cnt, kmax, BH, nb, nb, lw.wc, bitsT, s);
  if (e != hipSuccess) return e;
  const int64_t rows = BH * nb;
  bwd::col_lists_kernel<<<dim3((unsigned)((rows + 3) / 4)), 256, 0, s>>>(bitsT, rows, lw.wc, nb,
                                                                          col_idx, col_cnt);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (d != bwd::D || block != bwd::BLK)
    return launch_attn_bwd_generic(q, k, v, BH, N, d, block, nb, idx, cnt, kmax, scale, o_s, o_fp32,
                                   lse, d_o, dq, dk, dv, Dbuf, col_idx, col_cnt, order, s);
  const int seg = (nb + 7) / 8;
  const dim3 grid((unsigned)(BH * seg * 8));
  const float sl2 = scale * kLog2e;
  bwd::attn_bwd_dq_kernel<<<grid, bwd::NT, 0, s>>>(q, k, v, o_s, o_fp32, lse, d_o, N, nb, nb, idx,
                                                   cnt, kmax, sl2, scale, dq, Dbuf, L2buf, seg, order);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  bwd::attn_bwd_dkdv_kernel<<<grid, bwd::NT, 0, s>>>(q, k, v, L2buf, Dbuf, d_o, N, nb, nb, col_idx,
                                                      col_cnt, nb, sl2, scale, dk, dv, seg);
  return hipGetLastError();
}

}  // namespace sla
