// Mean pooling of Q and K over blocks, pooled block scores and per-row block
// selection (SLA post: the mean-pooling step that marks blocks; NABLA post,
// points 2-3: compressed Q/K and the 1 - thr cumulative softmax cut; Veda
// article, "what happened": top-k over key tiles).
#include "common.h"
#include "launch.h"

namespace sla {

// ---------------------------------------------------------------------------
// Pool: one workgroup per (tensor, batch*head, block).  256 threads; thread t
// owns the 16-byte feature chunk t % (D/8) and walks the block's rows with a
// stride of 256 / (D/8).  fp32 sums, reduced across row groups in LDS.
// HBM-bound: each workgroup streams block*D*2 bytes once.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void pool_kernel(const uint16_t* __restrict__ q,
                                                   const uint16_t* __restrict__ k,
                                                   float* __restrict__ qp, float* __restrict__ kp,
                                                   int N, int block, int nb) {
  constexpr int CH = D / 8;          // 16-byte chunks per row
  constexpr int RS = 256 / CH;       // rows per sweep
  __shared__ float part[RS][D + 1];
  const int blk = blockIdx.x;
  const int64_t bh = blockIdx.y;
  const uint16_t* src = (blockIdx.z == 0 ? q : k) + bh * (int64_t)N * D;
  float* dst = (blockIdx.z == 0 ? qp : kp) + (bh * nb + blk) * D;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(src, (uint32_t)N * D * 2);
  const int t = threadIdx.x;
  const int c = t % CH, r0 = t / CH;
  const int row0 = blk * block;
  const int valid = min(block, N - row0);
  // All of this thread's rows (at most 128 / RS) are loaded before the first
  // add, so their latencies overlap; rows past the block's end read as 0 and
  // the sums run in row order as before.
  constexpr int MAXS = 128 / RS;
  u32x4 xs[MAXS];
#pragma unroll
  for (int s = 0; s < MAXS; ++s) {
    const int r = r0 + s * RS;
    xs[s] = r < valid ? buf_load16(rs, (uint32_t)((row0 + r) * D + c * 8) * 2) : u32x4{};
  }
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int s = 0; s < MAXS; ++s) {
    if (r0 + s * RS >= valid) break;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += bf16_bits_to_f32(xs[s][e] & 0xffffu);
      acc[2 * e + 1] += bf16_bits_to_f32(xs[s][e] >> 16);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[r0][c * 8 + e] = acc[e];
  __syncthreads();
  if (t < D) {
    float s = 0.f;
#pragma unroll 8
    for (int r = 0; r < RS; ++r) s += part[r][t];
    dst[t] = s / (float)valid;
  }
}

// ---------------------------------------------------------------------------
// Scores: S[bh][i][j] = scale * qbar_i . kbar_j in fp32 on the matrix cores
// (v_mfma_f32_32x32x2_f32: fp32 products, fp32 sums; the feature order of the
// sums is the instruction's, not a plain chain).  TS x TS output tile per
// workgroup (TS = 64 or 128), four waves in a 2 x 2 arrangement, each wave
// WB x WB blocks of 32 x 32 (WB = TS / 64).  Operands come straight from
// global memory (the pooled tensors are small and L2-resident): in each
// chunk of 8 features, lane half h holds features 4h + 0..3 of its row
// (16 bytes), and MFMA step u pairs feature u (half 0) with 4 + u (half 1);
// Q and K use the same pairing, so every feature enters each dot product once.
// Rows past nb load as zeros (buffer range) and are not stored.
// ---------------------------------------------------------------------------
template <int D, int TS>
__global__ __launch_bounds__(256) void score_kernel(const float* __restrict__ qp,
                                                    const float* __restrict__ kp,
                                                    float* __restrict__ S, int nb, float scale) {
  constexpr int WB = TS / 64, CH = D / 8;
  const int64_t bh = blockIdx.z;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int i0 = blockIdx.y * TS + (w >> 1) * (TS / 2);
  const int j0 = blockIdx.x * TS + (w & 1) * (TS / 2);
  const uint32_t head_bytes = (uint32_t)nb * D * 4;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(qp + bh * nb * D, head_bytes);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kp + bh * nb * D, head_bytes);
  uint32_t qoff[WB], koff[WB];
#pragma unroll
  for (int b = 0; b < WB; ++b) {
    qoff[b] = (uint32_t)((i0 + 32 * b + l32) * D + 4 * hf) * 4;
    koff[b] = (uint32_t)((j0 + 32 * b + l32) * D + 4 * hf) * 4;
  }
  f32x16 acc[WB][WB];
#pragma unroll
  for (int a = 0; a < WB; ++a)
#pragma unroll
    for (int b = 0; b < WB; ++b) acc[a][b] = f32x16{};
  f32x4 qa[WB], kb[WB];
#pragma unroll
  for (int b = 0; b < WB; ++b) {
    qa[b] = __builtin_bit_cast(f32x4, buf_load16(rq, qoff[b]));
    kb[b] = __builtin_bit_cast(f32x4, buf_load16(rk, koff[b]));
  }
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    f32x4 qn[WB], kn[WB];
    if (c + 1 < CH) {
#pragma unroll
      for (int b = 0; b < WB; ++b) {
        qn[b] = __builtin_bit_cast(f32x4, buf_load16(rq, qoff[b] + 32 * (c + 1)));
        kn[b] = __builtin_bit_cast(f32x4, buf_load16(rk, koff[b] + 32 * (c + 1)));
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int a = 0; a < WB; ++a)
#pragma unroll
        for (int b = 0; b < WB; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x2f32(qa[a][u], kb[b][u], acc[a][b], 0, 0, 0);
    if (c + 1 < CH) {
#pragma unroll
      for (int b = 0; b < WB; ++b) {
        qa[b] = qn[b];
        kb[b] = kn[b];
      }
    }
  }
  // C layout: register r of a lane holds row 8 (r / 4) + 4 hf + r % 4, column l32
  float* Sh = S + bh * (int64_t)nb * nb;
#pragma unroll
  for (int a = 0; a < WB; ++a)
#pragma unroll
    for (int b = 0; b < WB; ++b) {
      const int gj = j0 + 32 * b + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int gi = i0 + 32 * a + 8 * (r / 4) + 4 * hf + r % 4;
        if (gi < nb && gj < nb) Sh[(int64_t)gi * nb + gj] = scale * acc[a][b][r];
      }
    }
}

// ---------------------------------------------------------------------------
// Select: one wave per row of S.  Each lane keeps the row's entries
// j = lane + 64*t as 44-bit keys (order-preserving fp32 bits << 12 |
// 4095 - j), so that a larger key means "earlier in the descending order,
// ties to the lower j".  All keys are distinct, and a bit-by-bit search finds
//   - a threshold that admits exactly the k largest keys (top-k and the two
//     cuts of the three-way split);
//   - the largest key T whose prefix {key >= T} holds softmax mass >= 1 - thr
//     (the NABLA cut), which is exactly the smallest such prefix.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t order_key(float s, int j) {
  uint32_t u = __float_as_uint(s + 0.0f);  // -0 -> +0
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 12) | (uint64_t)(4095 - j);
}

__device__ __forceinline__ float wave_sum_f(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ float wave_max_f(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

// A threshold T with exactly k keys >= T.  The search fixes bits from the
// top while at least k keys stay above the candidate; once exactly k do, the
// candidate already separates the k largest from the rest (the same set the
// k-th largest key itself would select), so the remaining bits are skipped.
// The k-th largest key of a row spread over a wave (slot t of lane l holds
// entry l + 64 t; absent entries hold key 0, below every candidate).  The
// count of keys at or above a candidate is one compare per slot, its ballot
// counted on the scalar unit.  Every slot is compared (no branch per slot),
// so the compares issue back to back; the launch picks MC close to nb / 64.
template <int MC>
__device__ __forceinline__ uint64_t kth_largest(const uint64_t (&key)[MC], int k) {
  uint64_t T = 0;
  for (int bit = 43; bit >= 0; --bit) {
    const uint64_t cand = T | (1ull << bit);
    int c = 0;
#pragma unroll
    for (int g = 0; g < MC; g += 4) {  // four ballots live at once: no wait between compares
      uint64_t b[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) b[t] = __builtin_amdgcn_ballot_w64(key[g + t] >= cand);
#pragma unroll
      for (int t = 0; t < 4; ++t) c += __popcll(b[t]);
    }
    if (c >= k) {
      T = cand;
      if (c == k) break;
    }
  }
  return T;
}

template <int MC>
__global__ __launch_bounds__(256) void select_kernel(const float* __restrict__ S,
                                                     uint8_t* __restrict__ cls, int64_t rows,
                                                     int nb, int mode, int kc, int km, float thr) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const float* srow = S + row * nb;
  uint8_t* crow = cls + row * nb;
  uint64_t key[MC];
  float sv[MC];
  int n_here = 0;
#pragma unroll
  for (int t = 0; t < MC; ++t) {
    const int j = lane + 64 * t;
    if (j < nb) {
      sv[t] = srow[j];
      key[t] = order_key(sv[t], j);
      n_here = t + 1;
    } else {
      sv[t] = -INFINITY;
      key[t] = 0;
    }
  }
  uint64_t t_crit, t_marg = ~0ull;
  if (mode == 1) {  // NABLA cut
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < MC; ++t) mx = fmaxf(mx, sv[t]);
    mx = wave_max_f(mx);
    float e[MC];
    float z = 0.f;
#pragma unroll
    for (int t = 0; t < MC; ++t) {
      e[t] = (t < n_here && lane + 64 * t < nb) ? expf(sv[t] - mx) : 0.f;
      z += e[t];
    }
    z = wave_sum_f(z);
    const float target = (1.0f - thr) * z;
    uint64_t T = 0;
    for (int bit = 43; bit >= 0; --bit) {
      const uint64_t cand = T | (1ull << bit);
      float m = 0.f;
#pragma unroll
      for (int t = 0; t < MC; ++t) m += (key[t] >= cand) ? e[t] : 0.f;
      if (wave_sum_f(m) >= target) T = cand;
    }
    t_crit = T;
  } else {
    t_crit = kth_largest<MC>(key, kc);
    if (mode == 2 && km > 0) t_marg = kth_largest<MC>(key, kc + km);
  }
#pragma unroll
  for (int t = 0; t < MC; ++t) {
    const int j = lane + 64 * t;
    if (j < nb) {
      uint8_t c = 0;
      if (key[t] >= t_crit) c = 2;
      else if (key[t] >= t_marg) c = 1;
      crow[j] = c;
    }
  }
}

// ---------------------------------------------------------------------------
hipError_t launch_pool(const uint16_t* q, const uint16_t* k, float* qp, float* kp, int64_t BH,
                       int N, int d, int block, int nb, hipStream_t s) {
  dim3 grid(nb, (unsigned)BH, 2);
  if (d == 128) pool_kernel<128><<<grid, 256, 0, s>>>(q, k, qp, kp, N, block, nb);
  else pool_kernel<64><<<grid, 256, 0, s>>>(q, k, qp, kp, N, block, nb);
  return hipGetLastError();
}

hipError_t launch_scores(const float* qp, const float* kp, float* S, int64_t BH, int d, int nb,
                         float scale, hipStream_t s) {
  // 128 x 128 tiles when they still give two workgroups per CU (256 CUs),
  // else 64 x 64 tiles for more parallelism
  const int64_t t128 = (int64_t)((nb + 127) / 128) * ((nb + 127) / 128) * BH;
  if (t128 >= 512) {
    const dim3 grid((nb + 127) / 128, (nb + 127) / 128, (unsigned)BH);
    if (d == 128) score_kernel<128, 128><<<grid, 256, 0, s>>>(qp, kp, S, nb, scale);
    else score_kernel<64, 128><<<grid, 256, 0, s>>>(qp, kp, S, nb, scale);
  } else {
    const dim3 grid((nb + 63) / 64, (nb + 63) / 64, (unsigned)BH);
    if (d == 128) score_kernel<128, 64><<<grid, 256, 0, s>>>(qp, kp, S, nb, scale);
    else score_kernel<64, 64><<<grid, 256, 0, s>>>(qp, kp, S, nb, scale);
  }
  return hipGetLastError();
}

hipError_t launch_select(const float* S, uint8_t* cls, int64_t rows, int nb, int mode, int kc,
                         int km, float thr, hipStream_t s) {
  dim3 grid((unsigned)((rows + 3) / 4));
  // MC = slots per lane: the smallest of these that holds nb keys
  if (nb <= 256) select_kernel<4><<<grid, 256, 0, s>>>(S, cls, rows, nb, mode, kc, km, thr);
  else if (nb <= 512) select_kernel<8><<<grid, 256, 0, s>>>(S, cls, rows, nb, mode, kc, km, thr);
  else if (nb <= 768) select_kernel<12><<<grid, 256, 0, s>>>(S, cls, rows, nb, mode, kc, km, thr);
  else if (nb <= 1024) select_kernel<16><<<grid, 256, 0, s>>>(S, cls, rows, nb, mode, kc, km, thr);
  else if (nb <= 1536) select_kernel<24><<<grid, 256, 0, s>>>(S, cls, rows, nb, mode, kc, km, thr);
  else if (nb <= 2048) select_kernel<32><<<grid, 256, 0, s>>>(S, cls, rows, nb, mode, kc, km, thr);
  else if (nb <= 3072) select_kernel<48><<<grid, 256, 0, s>>>(S, cls, rows, nb, mode, kc, km, thr);
  else select_kernel<64><<<grid, 256, 0, s>>>(S, cls, rows, nb, mode, kc, km, thr);
  return hipGetLastError();
}

}  // namespace sla
