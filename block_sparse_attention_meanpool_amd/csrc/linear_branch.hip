// Linear-attention branch over the marginal key tiles (SLA post: intermediate
// blocks go through linear attention), phi(x) = elu(x) + 1, and the final sum
// of the two branches.
//
// state:  per key tile j, H_j = phi(K_j)^T V_j (d x d) and z_j = sum phi(K_j),
//         one workgroup per tile; both operands are staged token-contiguous in
//         LDS (the contraction runs over tokens) and multiplied on bf16 MFMA.
//         H_j is stored transposed, bf16, as a row of the head's state matrix
//         Ht[j][d2 * d + d1].
// bits:   each query block's marginal list as a row of a bit matrix.
// gather: S_i^T = sum over marginal j of H_j^T for every query block at once:
//         C = M Ht with M the 0/1 marginal mask (exact in bf16), a GEMM on
//         MFMA.  Ht is streamed through double-buffered LDS by asynchronous
//         LDS-direct loads and read as the transposed operand; the mask bits
//         become the bf16 1.0 / 0.0 operand in registers.
// apply:  O_lin^T = S_i^T phi(Q_i)^T on MFMA, one query per lane, divided by
//         phi(q) . zeta_i with zeta_i = sum over marginal j of z_j (fp32).
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
                                                        int nkb, uint16_t* __restrict__ Ht,
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
  // H^T row of tile j: Ht[j][d2 * D + d1]; a lane holds 4 consecutive d1 per group.
  uint16_t* Hj = Ht + (bh * nkb + j) * (int64_t)D * D;
#pragma unroll
  for (int u = 0; u < PERW; ++u) {
    const int blkid = w * PERW + u;
    const int db1 = blkid / (D / 32), db2 = blkid % (D / 32);
    const int d2 = 32 * db2 + l32;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d1 = 32 * db1 + 8 * g + 4 * hf;
      *(u32x2*)(Hj + d2 * D + d1) = u32x2{pack_bf16x2(acc[u][4 * g], acc[u][4 * g + 1]),
                                          pack_bf16x2(acc[u][4 * g + 2], acc[u][4 * g + 3])};
    }
  }
}

// Marginal list of each query block -> row of a bit matrix (W 32-bit words per
// row, W even, W <= 128).  One wave per row; entries outside [0, nkb) are
// dropped.
__global__ __launch_bounds__(256) void lin_bits_kernel(const int32_t* __restrict__ idx,
                                                       const int32_t* __restrict__ cnt, int kmax,
                                                       int64_t rows, int nkb, int W,
                                                       uint32_t* __restrict__ bits) {
  __shared__ uint32_t words[4][128];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * 4 + wv;
  if (row >= rows) return;
  for (int x = lane; x < W; x += 64) words[wv][x] = 0u;
  __builtin_amdgcn_wave_barrier();
  const int c = min(cnt[row], kmax);
  const int32_t* list = idx + row * kmax;
  for (int t = lane; t < c; t += 64) {
    const int j = list[t];
    if (j >= 0 && j < nkb) atomicOr(&words[wv][j >> 5], 1u << (j & 31));
  }
  __builtin_amdgcn_wave_barrier();
  for (int x = lane; x < W; x += 64) bits[row * W + x] = words[wv][x];
}

// 8 mask bits -> 8 bf16 values 1.0 / 0.0 (the B operand of the gather GEMM).
__device__ __forceinline__ u32x4 bits_to_bf16(uint32_t b8) {
  u32x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    r[e] = (((b8 >> (2 * e)) & 1u) * 0x3f80u) | (((b8 >> (2 * e + 1)) & 1u) * 0x3f800000u);
  return r;
}

// Gather GEMM, one 128 (query blocks) x 128 (state columns) tile per
// workgroup: C^T tile = Ht^T M^T, i.e. per wave 32 query blocks x 128
// columns, K = key tiles in chunks of 64 streamed through LDS.
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void lin_gather_kernel(
    const uint16_t* __restrict__ Ht, const uint32_t* __restrict__ bits, int nqb, int nkb, int W,
    int rowtiles, int coltiles, int per_xcd, int64_t tiles, uint16_t* __restrict__ C) {
  constexpr int DD = D * D;
  constexpr int CHUNK = 64, COLS = 128, BUFB = CHUNK * COLS * 2;  // 16 KB
  __shared__ __attribute__((aligned(1024))) char B0[BUFB];
  __shared__ __attribute__((aligned(1024))) char B1[BUFB];
  extern __shared__ uint32_t mbits[];  // this tile's 128 mask rows, pitch W + 1 words
  const int Wp = W + 1;                // odd pitch: the 32 rows a wave reads hit distinct banks

  // XCD-aware order: logical tiles [x * per_xcd, (x+1) * per_xcd) run on XCD x,
  // row tiles fastest, so the row tiles sharing one column slice of Ht meet in
  // one L2.
  const int64_t L = (int64_t)(blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (L >= tiles) return;
  const int rt = (int)(L % rowtiles);
  const int64_t rest = L / rowtiles;
  const int ct = (int)(rest % coltiles);
  const int64_t bh = rest / coltiles;
  const int i0 = rt * 128, c0 = ct * COLS;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  for (int x = tid; x < 128 * W; x += 256) {
    const int r = x / W, c = x % W;
    mbits[r * Wp + c] = (i0 + r < nqb) ? bits[((int64_t)bh * nqb + i0 + r) * W + c] : 0u;
  }

  const __amdgpu_buffer_rsrc_t rh = make_rsrc(Ht + bh * (int64_t)nkb * DD, (uint32_t)nkb * DD * 2);
  const int wu = __builtin_amdgcn_readfirstlane(w);
  uint32_t voff[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int row = 4 * (4 * w + e) + (lane >> 4);
    voff[e] = (uint32_t)(row * DD + ((lane & 15) ^ trs_swz(row)) * 8) * 2;
  }
  // Rows past nkb fall outside the buffer range and land in LDS as zeros.
  auto issue = [&](int chunk, char* buf) {
    const int soff = (chunk * CHUNK * DD + c0) * 2;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rh, (lds_void_ptr)(buf + (4 * wu + e) * 1024), 16,
                                               voff[e], soff, 0, 0);
  };

  f32x16 acc[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
  const int nchunk = (nkb + CHUNK - 1) / CHUNK;
  const int myrow = 32 * w + l32;
  auto compute = [&](int chunk, const char* buf) {
    const uint32_t lo = mbits[myrow * Wp + 2 * chunk], hi = mbits[myrow * Wp + 2 * chunk + 1];
#pragma unroll
    for (int ks2 = 0; ks2 < 4; ++ks2) {
      const int sh = 16 * ks2 + 8 * hf;
      const uint32_t b8 = (sh < 32 ? lo >> sh : hi >> (sh - 32)) & 0xffu;
      const u32x4 b = bits_to_bf16(b8);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
        acc[cb] = mfma32x32x16(tr_operand(buf, 16 * ks2, 32 * cb, lane), b, acc[cb]);
    }
  };

  issue(0, B0);
  for (int ch = 0; ch < nchunk; ch += 2) {
    wait_vmcnt0();
    __syncthreads();  // B0 holds chunk ch; every wave is done with B1
    if (ch + 1 < nchunk) issue(ch + 1, B1);
    compute(ch, B0);
    if (ch + 1 < nchunk) {
      wait_vmcnt0();
      __syncthreads();  // B1 holds chunk ch + 1; every wave is done with B0
      if (ch + 2 < nchunk) issue(ch + 2, B0);
      compute(ch + 1, B1);
    }
  }

  // C[i][c0 + col] (bf16): a lane holds query block i0 + myrow, 4 consecutive
  // columns per register group.
  const int i = i0 + myrow;
  if (i < nqb) {
    uint16_t* crow = C + ((int64_t)bh * nqb + i) * DD + c0;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = 32 * cb + 8 * g + 4 * hf;
        *(u32x2*)(crow + col) = u32x2{pack_bf16x2(acc[cb][4 * g], acc[cb][4 * g + 1]),
                                      pack_bf16x2(acc[cb][4 * g + 2], acc[cb][4 * g + 3])};
      }
  }
}

template <int D, int BLK>
__global__ __launch_bounds__(256) void lin_apply_kernel(const uint16_t* __restrict__ q, int N,
                                                        int nqb, int nkb,
                                                        const int32_t* __restrict__ idx,
                                                        const int32_t* __restrict__ cnt, int kmax,
                                                        const uint16_t* __restrict__ C,
                                                        const float* __restrict__ Zs,
                                                        float* __restrict__ o_lin) {
  __shared__ float zs[D];
  __shared__ int used_s;
  const int64_t bh = blockIdx.x / nqb;
  const int qb = blockIdx.x % nqb;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int64_t head_off = bh * (int64_t)N * D;
  const int count = min(cnt[bh * nqb + qb], kmax);
  const int32_t* list = idx + (bh * nqb + qb) * (int64_t)kmax;

  // zeta_i = sum of z_j over the marginal list (fp32)
  if (tid < D) {
    float zacc = 0.f;
    int used = 0;
    for (int t = 0; t < count; ++t) {
      const int j = list[t];
      if (j < 0 || j >= nkb) continue;
      ++used;
      zacc += Zs[(bh * nkb + j) * D + tid];
    }
    zs[tid] = zacc;
    if (tid == 0) used_s = used;
  }
  __syncthreads();
  if (32 * w >= BLK) return;

  // O_lin^T = S_i^T phi(Q_i)^T; S_i^T rows (d2) come straight from C, d1-contiguous.
  const uint16_t* St = C + (bh * nqb + qb) * (int64_t)D * D;
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
      const u32x4 a = *(const u32x4*)(St + (32 * db + l32) * D + 16 * ks + 8 * hf);
      oacc[db] = mfma32x32x16(a, pq, oacc[db]);
    }
  }
  den = sum_halves(den);
  const float inv = (used_s > 0 && den > 0.f) ? 1.f / den : 0.f;
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

LinearWs linear_ws_layout(int64_t BH, int nb, int d) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  LinearWs w;
  w.words = 2 * ((nb + 63) / 64);
  w.ht_bytes = up((size_t)BH * nb * d * d * 2);
  w.z_bytes = up((size_t)BH * nb * d * 4);
  w.bits_bytes = up((size_t)BH * nb * w.words * 4);
  w.c_bytes = up((size_t)BH * nb * d * d * 2);
  w.total = w.ht_bytes + w.z_bytes + w.bits_bytes + w.c_bytes;
  return w;
}

template <int D, int BLK>
static hipError_t launch_linear_t(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                  int64_t BH, int N, int nb, const int32_t* idx, const int32_t* cnt,
                                  int kmax, float* o_lin, void* ws, hipStream_t s) {
  const LinearWs lw = linear_ws_layout(BH, nb, D);
  char* p = static_cast<char*>(ws);
  uint16_t* Ht = reinterpret_cast<uint16_t*>(p);
  float* Zs = reinterpret_cast<float*>(p + lw.ht_bytes);
  uint32_t* bits = reinterpret_cast<uint32_t*>(p + lw.ht_bytes + lw.z_bytes);
  uint16_t* C = reinterpret_cast<uint16_t*>(p + lw.ht_bytes + lw.z_bytes + lw.bits_bytes);

  lin_state_kernel<D, BLK><<<dim3((unsigned)(BH * nb)), 256, 0, s>>>(k, v, N, nb, Ht, Zs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows = BH * nb;
  lin_bits_kernel<<<dim3((unsigned)((rows + 3) / 4)), 256, 0, s>>>(idx, cnt, kmax, rows, nb,
                                                                   lw.words, bits);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rowtiles = (nb + 127) / 128, coltiles = D * D / 128;
  const int64_t tiles = BH * rowtiles * coltiles;
  const int per_xcd = (int)((tiles + 7) / 8);
  const size_t mbytes = (size_t)128 * (lw.words + 1) * sizeof(uint32_t);
  lin_gather_kernel<D><<<dim3((unsigned)(per_xcd * 8)), 256, mbytes, s>>>(
      Ht, bits, nb, nb, lw.words, rowtiles, coltiles, per_xcd, tiles, C);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  lin_apply_kernel<D, BLK><<<dim3((unsigned)(BH * nb)), 256, 0, s>>>(q, N, nb, nb, idx, cnt, kmax,
                                                                    C, Zs, o_lin);
  return hipGetLastError();
}

hipError_t launch_linear(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t BH, int N,
                         int d, int block, int nb, const int32_t* idx, const int32_t* cnt, int kmax,
                         float* o_lin, void* ws, hipStream_t s) {
  if (d == 128 && block == 128)
    return launch_linear_t<128, 128>(q, k, v, BH, N, nb, idx, cnt, kmax, o_lin, ws, s);
  if (d == 128 && block == 64)
    return launch_linear_t<128, 64>(q, k, v, BH, N, nb, idx, cnt, kmax, o_lin, ws, s);
  if (d == 64 && block == 128)
    return launch_linear_t<64, 128>(q, k, v, BH, N, nb, idx, cnt, kmax, o_lin, ws, s);
  return launch_linear_t<64, 64>(q, k, v, BH, N, nb, idx, cnt, kmax, o_lin, ws, s);
}

hipError_t launch_combine(const void* o_s, int o_s_fp32, const float* o_lin, uint16_t* o,
                          int64_t n_elems, hipStream_t s) {
  const int64_t n8 = n_elems / 8;
  if (n8 == 0) return hipSuccess;
  combine_kernel<<<dim3((unsigned)((n8 + 255) / 256)), 256, 0, s>>>(o_s, o_s_fp32, o_lin, o, n8);
  return hipGetLastError();
}

}  // namespace sla
