// Linear-attention branch over the marginal key tiles (SLA post: intermediate
// blocks go through linear attention), phi(x) = elu(x) + 1, and the final sum
// of the two branches.
//
// state:  per key tile j, H_j = phi(K_j)^T V_j (d x d) and z_j = sum phi(K_j),
//         one workgroup per tile; both operands are staged token-contiguous in
//         LDS (the contraction runs over tokens) and multiplied on bf16 MFMA.
//         At d = 128 with 128-token tiles, lin_state_pipe_kernel computes the
//         same states with the tiles streamed through LDS-direct loads.
//         H_j is stored transposed, bf16, as a row of the head's state matrix
//         Ht[j][d2 * d + d1].
// mask:   each query block's marginal list as a row of a bit matrix, and
//         zeta_i = sum over the marked j of z_j (fp32, ascending j).
// gather: S_i^T = sum over marginal j of H_j^T for every query block at once:
//         C = M Ht with M the 0/1 marginal mask (exact in bf16), a GEMM on
//         MFMA.  Ht is streamed through double-buffered LDS by asynchronous
//         LDS-direct loads and read as the transposed operand; the mask bits
//         become the bf16 1.0 / 0.0 operand in registers.
// apply:  O_lin^T = S_i^T phi(Q_i)^T on MFMA, one query per lane, divided by
//         phi(q) . zeta_i (linear_apply.h; the fused softmax kernels run the
//         same step in their epilogue).
#include "common.h"
#include "launch.h"
#include "linear_apply.h"

namespace sla {

// LO: store the low part H_j - bf16(H_j) of each state instead (a hi + lo
// pair with the states above; z_j is not written).
template <int D, int BLK, bool LO = false>
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
      subblock_coords<BLK>(s, tc, fc);
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
  if (!LO && tid < D) {
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
      if (LO)
        *(u32x2*)(Hj + d2 * D + d1) = u32x2{pack_bf16x2_lo(acc[u][4 * g], acc[u][4 * g + 1]),
                                            pack_bf16x2_lo(acc[u][4 * g + 2], acc[u][4 * g + 3])};
      else
        *(u32x2*)(Hj + d2 * D + d1) = u32x2{pack_bf16x2(acc[u][4 * g], acc[u][4 * g + 1]),
                                            pack_bf16x2(acc[u][4 * g + 2], acc[u][4 * g + 3])};
    }
  }
}

// d = 128, 128-token tiles: the same states, streamed.  Each workgroup takes
// two consecutive tiles of one head and reads them as four 64-token halves
// through double-buffered LDS by LDS-direct loads (K and V rows, row-major,
// with the transpose-read swizzle), the next half's loads in flight while the
// current half's MFMAs run.  Transpose reads give a lane 8 consecutive tokens
// of one feature: the layout of both MFMA operands of a product that
// contracts over tokens.  phi is applied to the K operand in registers
// (tokens at or past N load as zeros and give 0).  The two tiles accumulate in
// separate registers, so the first tile's stores go out while the second
// tile's first half is computed, and the wait before its second half (a full
// drain, as loads and stores in flight together may complete in any order)
// finds them done.  H_j, z_j and their summation orders are those of
// lin_state_kernel, bit for bit.
namespace lstate {

constexpr int D = 128, BLK = 128, HALF = 64, NT = 256;
constexpr int BUFB = HALF * D * 2;  // 16 KB: one 64-token half of K or V

struct Ctx {
  __amdgpu_buffer_rsrc_t rk, rv;
  int wu;           // the wave index, known uniform
  uint32_t off[4];  // per-lane byte offsets of the 4 rows a lane loads
};

__device__ __forceinline__ void issue(const Ctx& c, int tile, int hh, char* kb, char* vb) {
  const uint32_t t = (uint32_t)(tile * BLK + HALF * hh) * D * 2;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rk, (lds_void_ptr)(kb + (4 * c.wu + e) * 1024), 16,
                                             c.off[e] + t, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rv, (lds_void_ptr)(vb + (4 * c.wu + e) * 1024), 16,
                                             c.off[e] + t, 0, 0, 0);
  }
}

// phi of 8 bf16 values of tokens tok0 .. tok0 + 7 (low half of each dword
// first); tokens at or past N give 0.
__device__ __forceinline__ u32x4 phi8_tokens(u32x4 x, int tok0, int N) {
  u32x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float a = tok0 + 2 * e < N ? phi(bf16_bits_to_f32(x[e] & 0xffffu)) : 0.f;
    const float b = tok0 + 2 * e + 1 < N ? phi(bf16_bits_to_f32(x[e] >> 16)) : 0.f;
    r[e] = pack_bf16x2(a, b);
  }
  return r;
}

// One 64-token half into the wave's four 32x32 blocks of H (rows d1 of block
// w, every d2) and into z of feature 32 w + lane % 32, summed in token order
// by the lane of the lower 32 (it takes the upper lane's 8 tokens after its own).
__device__ __forceinline__ void half(const char* kb, const char* vb, int tok0, int N, int w,
                                     int lane, int hf, f32x16 (&acc)[4], float& z) {
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const u32x4 a = phi8_tokens(tr_operand(kb, 16 * ks, 32 * w, lane), tok0 + 16 * ks + 8 * hf, N);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      acc[u] = mfma32x32x16(a, tr_operand(vb, 16 * ks, 32 * u, lane), acc[u]);
    // every lane gets both lanes' dwords: the lower lane's 8 tokens, then the upper lane's
    uint32_t lo8[4], hi8[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const auto sw = __builtin_amdgcn_permlane32_swap(a[e], a[e], false, false);
      lo8[e] = sw[0];
      hi8[e] = sw[1];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) z += bf16_bits_to_f32(lo8[e] & 0xffffu) + bf16_bits_to_f32(lo8[e] >> 16);
#pragma unroll
    for (int e = 0; e < 4; ++e) z += bf16_bits_to_f32(hi8[e] & 0xffffu) + bf16_bits_to_f32(hi8[e] >> 16);
  }
}

// H^T row of a tile (lin_state_kernel's layout) and z (lanes of the lower 32);
// with LO the low parts H - bf16(H) and no z.
template <bool LO>
__device__ __forceinline__ void store_tile(uint16_t* __restrict__ Ht, float* __restrict__ Zs,
                                           int64_t row, const f32x16 (&acc)[4], float z, int w,
                                           int l32, int hf) {
  uint16_t* Hj = Ht + row * (int64_t)D * D;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int d2 = 32 * u + l32;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d1 = 32 * w + 8 * g + 4 * hf;
      if (LO)
        *(u32x2*)(Hj + d2 * D + d1) = u32x2{pack_bf16x2_lo(acc[u][4 * g], acc[u][4 * g + 1]),
                                            pack_bf16x2_lo(acc[u][4 * g + 2], acc[u][4 * g + 3])};
      else
        *(u32x2*)(Hj + d2 * D + d1) = u32x2{pack_bf16x2(acc[u][4 * g], acc[u][4 * g + 1]),
                                            pack_bf16x2(acc[u][4 * g + 2], acc[u][4 * g + 3])};
    }
  }
  if (!LO && hf == 0) Zs[row * D + 32 * w + l32] = z;
}

template <bool LO>
__global__ __launch_bounds__(NT) void lin_state_pipe_kernel(const uint16_t* __restrict__ k,
                                                            const uint16_t* __restrict__ v, int N,
                                                            int nkb, int npairs,
                                                            uint16_t* __restrict__ Ht,
                                                            float* __restrict__ Zs) {
  __shared__ __attribute__((aligned(1024))) char K0[BUFB];
  __shared__ __attribute__((aligned(1024))) char V0[BUFB];
  __shared__ __attribute__((aligned(1024))) char K1[BUFB];
  __shared__ __attribute__((aligned(1024))) char V1[BUFB];
  const int64_t bh = blockIdx.x / npairs;
  const int t0 = 2 * (blockIdx.x % npairs);
  const bool two = t0 + 1 < nkb;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int64_t head_off = bh * (int64_t)N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  Ctx c;
  c.rk = make_rsrc(k + head_off, head_bytes);
  c.rv = make_rsrc(v + head_off, head_bytes);
  c.wu = __builtin_amdgcn_readfirstlane(w);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int row = 4 * (4 * w + e) + (lane >> 4);  // row within the half
    c.off[e] = (uint32_t)(row * D + ((lane & 15) ^ trs_swz(row)) * 8) * 2;
  }
  f32x16 acc0[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
  f32x16 acc1[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
  float z0 = 0.f, z1 = 0.f;
  const int64_t row0 = bh * nkb + t0;

  issue(c, t0, 0, K0, V0);
  wait_vmcnt0();
  __syncthreads();
  issue(c, t0, 1, K1, V1);
  half(K0, V0, t0 * BLK, N, w, lane, hf, acc0, z0);
  wait_vmcnt0();
  __syncthreads();  // every wave is done with buffer 0
  if (two) issue(c, t0 + 1, 0, K0, V0);
  half(K1, V1, t0 * BLK + HALF, N, w, lane, hf, acc0, z0);
  if (two) {
    wait_vmcnt0();
    __syncthreads();  // every wave is done with buffer 1
    issue(c, t0 + 1, 1, K1, V1);
    store_tile<LO>(Ht, Zs, row0, acc0, z0, w, l32, hf);
    half(K0, V0, (t0 + 1) * BLK, N, w, lane, hf, acc1, z1);
    wait_vmcnt0();
    __syncthreads();  // the first tile's stores are done too
    half(K1, V1, (t0 + 1) * BLK + HALF, N, w, lane, hf, acc1, z1);
    store_tile<LO>(Ht, Zs, row0 + 1, acc1, z1, w, l32, hf);
  } else {
    store_tile<LO>(Ht, Zs, row0, acc0, z0, w, l32, hf);
  }
}

}  // namespace lstate

// Sum of the rows src[j] (fp32, D features) over the set bits j of a bit row
// held in LDS (W <= 128 words), strictly in ascending j: the set bits are
// compacted into a list first (popcount prefix over the lanes), then summed
// with 8 loads in flight.  One wave; each lane owns D / 64 features.
template <int D>
__device__ __forceinline__ void bitrow_sum(const uint32_t* words, int W, uint16_t* js,
                                           const float* __restrict__ src, float* __restrict__ out,
                                           int lane) {
  constexpr int PER = D / 64;
  uint32_t w0 = lane < W ? words[lane] : 0u;
  uint32_t w1 = lane + 64 < W ? words[lane + 64] : 0u;
  const int c0 = __popc(w0), c1 = __popc(w1);
  int s0 = c0, s1 = c1;  // inclusive prefix sums over lanes
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
  while (w0) {
    js[p0++] = (uint16_t)(32 * lane + __ffs(w0) - 1);
    w0 &= w0 - 1u;
  }
  while (w1) {
    js[p1++] = (uint16_t)(32 * (lane + 64) + __ffs(w1) - 1);
    w1 &= w1 - 1u;
  }
  __builtin_amdgcn_wave_barrier();
  const float* sb = src + PER * lane;
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  for (int t = 0; t < total; t += 8) {
    float val[8][PER];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = js[min(t + u, total - 1)];
#pragma unroll
      for (int e = 0; e < PER; ++e) val[u][e] = sb[j * D + e];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] += t + u < total ? val[u][e] : 0.f;
  }
#pragma unroll
  for (int e = 0; e < PER; ++e) out[PER * lane + e] = acc[e];
}

// Marginal list of each query block -> a row of the bit matrix (W 32-bit
// words, W even, W <= 128) and zeta_i = sum of z_j over the set bits in
// ascending j (fp32).  One wave per row; entries outside [0, nkb) are dropped
// and a repeated entry counts once, as it does in the bit row.
template <int D>
__global__ __launch_bounds__(256) void lin_mask_kernel(const int32_t* __restrict__ idx,
                                                       const int32_t* __restrict__ cnt, int kmax,
                                                       int64_t rows, int nqb, int nkb, int W,
                                                       const float* __restrict__ Zs,
                                                       uint32_t* __restrict__ bits,
                                                       float* __restrict__ zeta) {
  __shared__ uint32_t words[4][128];
  __shared__ uint16_t js[4][4096];
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
  bitrow_sum<D>(words[wv], W, js[wv], Zs + (row / nqb) * (int64_t)nkb * D, zeta + row * D, lane);
}

// out[row] = sum of src rows over the set bits of bit row `row` (ascending),
// for bit rows already in memory; src holds nsrc rows per head.
template <int D>
__global__ __launch_bounds__(256) void lin_bitrow_sum_kernel(const uint32_t* __restrict__ bits,
                                                             int W, int64_t rows, int per_head,
                                                             int nsrc, const float* __restrict__ src,
                                                             float* __restrict__ out) {
  __shared__ uint32_t words[4][128];
  __shared__ uint16_t js[4][4096];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * 4 + wv;
  if (row >= rows) return;
  for (int x = lane; x < W; x += 64) words[wv][x] = bits[row * W + x];
  __builtin_amdgcn_wave_barrier();
  bitrow_sum<D>(words[wv], W, js[wv], src + (row / per_head) * (int64_t)nsrc * D, out + row * D,
                lane);
}

// 8 mask bits -> 8 bf16 values 1.0 / 0.0 (the B operand of the gather GEMM).
__device__ __forceinline__ u32x4 bits_to_bf16(uint32_t b8) {
  u32x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    r[e] = (((b8 >> (2 * e)) & 1u) * 0x3f80u) | (((b8 >> (2 * e + 1)) & 1u) * 0x3f800000u);
  return r;
}

// Gather GEMM: C^T = Ht^T M^T.  One workgroup per (64 * WAVES query blocks)
// x 128 state columns tile; each wave owns 64 query blocks (two MFMA row
// groups) and all 128 columns, so every Ht^T operand read from LDS feeds two
// MFMAs.  K = key tiles in chunks of 64 streamed through double-buffered LDS
// by asynchronous LDS-direct loads; a column slice of Ht is streamed once per
// row tile, so taller row tiles cut the Ht traffic.  Each lane's mask words
// for the next chunk are loaded into registers while the current one is
// multiplied, and become the bf16 1.0 / 0.0 operand.
// HILO: the states come as a hi + lo bf16 pair (Ht, Ht_lo); both parts are
// multiplied into the same fp32 accumulators (the 0/1 operand is exact), and
// the sum is stored as a hi + lo pair too (C, C_lo): S_i to about 16
// significant bits, for the backward's cancelling dQ terms.
template <int D, int WAVES, bool HILO>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void lin_gather_kernel(
    const uint16_t* __restrict__ Ht, const uint16_t* __restrict__ Ht_lo,
    const uint32_t* __restrict__ bits, int nqb, int nkb, int W, int rowtiles, int coltiles,
    int per_xcd, int64_t tiles, uint16_t* __restrict__ C, uint16_t* __restrict__ C_lo) {
  constexpr int DD = D * D;
  constexpr int CHUNK = 64, COLS = 128, BUFB = CHUNK * COLS * 2;  // 16 KB
  constexpr int ROWS = 64 * WAVES, NI = (16 + WAVES - 1) / WAVES;  // 1 KB DMA blocks per wave
  constexpr int LOB = HILO ? BUFB : 1024;
  __shared__ __attribute__((aligned(1024))) char B0[BUFB];
  __shared__ __attribute__((aligned(1024))) char B1[BUFB];
  __shared__ __attribute__((aligned(1024))) char L0[LOB];
  __shared__ __attribute__((aligned(1024))) char L1[LOB];

  // XCD-aware order: logical tiles [x * per_xcd, (x+1) * per_xcd) run on XCD x,
  // row tiles fastest, so the row tiles sharing one column slice of Ht meet in
  // one L2.
  const int64_t L = (int64_t)(blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (L >= tiles) return;
  const int rt = (int)(L % rowtiles);
  const int64_t rest = L / rowtiles;
  const int ct = (int)(rest % coltiles);
  const int64_t bh = rest / coltiles;
  const int i0 = rt * ROWS, c0 = ct * COLS;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const __amdgpu_buffer_rsrc_t rh = make_rsrc(Ht + bh * (int64_t)nkb * DD, (uint32_t)nkb * DD * 2);
  const __amdgpu_buffer_rsrc_t rl =
      make_rsrc((HILO ? Ht_lo : Ht) + bh * (int64_t)nkb * DD, (uint32_t)nkb * DD * 2);
  const int wu = __builtin_amdgcn_readfirstlane(w);
  uint32_t voff[8];  // NI <= 8 entries used; a size that depends on WAVES, captured by the
                     // lambda below, makes the host compiler drop the kernel's launch stub
#pragma unroll
  for (int e = 0; e < NI; ++e) {
    const int row = 4 * (wu + WAVES * e) + (lane >> 4);
    voff[e] = (uint32_t)(row * DD + ((lane & 15) ^ trs_swz(row)) * 8) * 2;
  }
  // Rows past nkb fall outside the buffer range and land in LDS as zeros.
  auto issue = [&](int chunk, char* buf, char* lbuf) {
    const int soff = (chunk * CHUNK * DD + c0) * 2;
#pragma unroll
    for (int e = 0; e < NI; ++e)
      if (wu + WAVES * e < 16) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rh, (lds_void_ptr)(buf + (wu + WAVES * e) * 1024),
                                                 16, voff[e], soff, 0, 0);
        if (HILO)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (lds_void_ptr)(lbuf + (wu + WAVES * e) * 1024),
                                                   16, voff[e], soff, 0, 0);
      }
  };

  // this lane's two query blocks (one per MFMA row group); rows past nqb get no bits
  const uint32_t* mrow[2];
  bool mok[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int i = i0 + 64 * w + 32 * rb + l32;
    mok[rb] = i < nqb;
    mrow[rb] = bits + ((int64_t)bh * nqb + (mok[rb] ? i : 0)) * W;
  }
  u32x2 mb[2];
  auto load_bits = [&](int chunk) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
      mb[rb] = mok[rb] ? *(const u32x2*)(mrow[rb] + 2 * chunk) : u32x2{0u, 0u};
  };

  f32x16 acc[4][2];  // [column block][row group]
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) acc[cb][0] = acc[cb][1] = f32x16{};
  const int nchunk = (nkb + CHUNK - 1) / CHUNK;
  auto compute = [&](const char* buf, const char* lbuf, const u32x2 (&m)[2]) {
    // a wave whose 64 query blocks mark none of the chunk's 64 key tiles adds
    // only exact zeros: skip its MFMAs (wave-uniform; the loads are unaffected)
    if (__ballot((m[0][0] | m[0][1] | m[1][0] | m[1][1]) != 0u) == 0) return;
#pragma unroll
    for (int ks2 = 0; ks2 < 4; ++ks2) {
      const int sh = 16 * ks2 + 8 * hf;
      u32x4 b[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
        b[rb] = bits_to_bf16((sh < 32 ? m[rb][0] >> sh : m[rb][1] >> (sh - 32)) & 0xffu);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const u32x4 a = tr_operand(buf, 16 * ks2, 32 * cb, lane);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) acc[cb][rb] = mfma32x32x16(a, b[rb], acc[cb][rb]);
        if (HILO) {
          const u32x4 al = tr_operand(lbuf, 16 * ks2, 32 * cb, lane);
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) acc[cb][rb] = mfma32x32x16(al, b[rb], acc[cb][rb]);
        }
      }
    }
  };

  issue(0, B0, L0);
  load_bits(0);
  for (int ch = 0; ch < nchunk; ch += 2) {
    wait_vmcnt0();
    __syncthreads();  // B0 and mb hold chunk ch; every wave is done with B1
    const u32x2 m0[2] = {mb[0], mb[1]};
    if (ch + 1 < nchunk) {
      issue(ch + 1, B1, L1);
      load_bits(ch + 1);
    }
    compute(B0, L0, m0);
    if (ch + 1 < nchunk) {
      wait_vmcnt0();
      __syncthreads();  // B1 and mb hold chunk ch + 1; every wave is done with B0
      const u32x2 m1[2] = {mb[0], mb[1]};
      if (ch + 2 < nchunk) {
        issue(ch + 2, B0, L0);
        load_bits(ch + 2);
      }
      compute(B1, L1, m1);
    }
  }

  // C[i][c0 + col] (bf16): a lane holds query blocks i0 + 64 w + 32 rb + l32,
  // 4 consecutive columns per register group.
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    if (!mok[rb]) continue;
    const int64_t roff = ((int64_t)bh * nqb + i0 + 64 * w + 32 * rb + l32) * DD + c0;
    uint16_t* crow = C + roff;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = 32 * cb + 8 * g + 4 * hf;
        const f32x16& a = acc[cb][rb];
        *(u32x2*)(crow + col) = u32x2{pack_bf16x2(a[4 * g], a[4 * g + 1]),
                                      pack_bf16x2(a[4 * g + 2], a[4 * g + 3])};
        if (HILO)
          *(u32x2*)(C_lo + roff + col) = u32x2{pack_bf16x2_lo(a[4 * g], a[4 * g + 1]),
                                               pack_bf16x2_lo(a[4 * g + 2], a[4 * g + 3])};
      }
  }
}

// O_lin for one query block per workgroup, BLK / 32 waves of 32 queries.
template <int D, int BLK>
__global__ __launch_bounds__(BLK * 2) void lin_apply_kernel(const uint16_t* __restrict__ q, int N,
                                                            int nqb, const uint16_t* __restrict__ C,
                                                            const float* __restrict__ zeta,
                                                            float* __restrict__ o_lin) {
  const int64_t bh = blockIdx.x / nqb;
  const int qb = blockIdx.x % nqb;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int64_t head_off = bh * (int64_t)N * D;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + head_off, (uint32_t)N * D * 2);
  const int qrow = qb * BLK + 32 * w + l32;
  u32x4 qf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
    qf[ks] = buf_load16(rq, (uint32_t)(qrow * D + 16 * ks + 8 * hf) * 2);
  f32x16 lacc[D / 32];
  const int64_t row = bh * nqb + qb;
  const float inv = linear_apply<D>(C + row * D * D, zeta + row * D, qf, l32, hf, lacc);
  if (qrow < N) {
    float* orow = o_lin + head_off + (int64_t)qrow * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * hf;
        *(f32x4*)(orow + d0) = f32x4{lacc[db][4 * g] * inv, lacc[db][4 * g + 1] * inv,
                                     lacc[db][4 * g + 2] * inv, lacc[db][4 * g + 3] * inv};
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
  w.zeta_bytes = up((size_t)BH * nb * d * 4);
  w.c_bytes = up((size_t)BH * nb * d * d * 2);
  w.total = w.ht_bytes + w.z_bytes + w.bits_bytes + w.zeta_bytes + w.c_bytes;
  return w;
}

LinearPtrs linear_ws_ptrs(void* ws, int64_t BH, int nb, int d) {
  const LinearWs lw = linear_ws_layout(BH, nb, d);
  char* p = static_cast<char*>(ws);
  LinearPtrs r;
  r.Ht = reinterpret_cast<uint16_t*>(p);
  p += lw.ht_bytes;
  r.Zs = reinterpret_cast<float*>(p);
  p += lw.z_bytes;
  r.bits = reinterpret_cast<uint32_t*>(p);
  p += lw.bits_bytes;
  r.zeta = reinterpret_cast<float*>(p);
  p += lw.zeta_bytes;
  r.C = reinterpret_cast<uint16_t*>(p);
  r.words = lw.words;
  return r;
}

template <int D, int BLK>
static hipError_t launch_linear_prepare_t(const uint16_t* k, const uint16_t* v, int64_t BH, int N,
                                          int nb, const int32_t* idx, const int32_t* cnt, int kmax,
                                          void* ws, hipStream_t s) {
  const LinearPtrs lp = linear_ws_ptrs(ws, BH, nb, D);
  if constexpr (D == 128 && BLK == 128) {
    const int npairs = (nb + 1) / 2;
    lstate::lin_state_pipe_kernel<false><<<dim3((unsigned)(BH * npairs)), lstate::NT, 0, s>>>(
        k, v, N, nb, npairs, lp.Ht, lp.Zs);
  } else {
    lin_state_kernel<D, BLK><<<dim3((unsigned)(BH * nb)), 256, 0, s>>>(k, v, N, nb, lp.Ht, lp.Zs);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows = BH * nb;
  lin_mask_kernel<D><<<dim3((unsigned)((rows + 3) / 4)), 256, 0, s>>>(idx, cnt, kmax, rows, nb, nb,
                                                                      lp.words, lp.Zs, lp.bits,
                                                                      lp.zeta);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_gather(lp.Ht, lp.bits, BH, nb, lp.words, D, lp.C, s);
}

template <int D, int WAVES, bool HILO>
static void launch_gather_t(const uint16_t* Ht, const uint16_t* Ht_lo, const uint32_t* bits,
                            int64_t BH, int nb, int W, uint16_t* C, uint16_t* C_lo, hipStream_t s) {
  const int rowtiles = (nb + 64 * WAVES - 1) / (64 * WAVES), coltiles = D * D / 128;
  const int64_t tiles = BH * rowtiles * coltiles;
  const int per_xcd = (int)((tiles + 7) / 8);
  lin_gather_kernel<D, WAVES, HILO><<<dim3((unsigned)(per_xcd * 8)), WAVES * 64, 0, s>>>(
      Ht, Ht_lo, bits, nb, nb, W, rowtiles, coltiles, per_xcd, tiles, C, C_lo);
}

template <bool HILO>
static hipError_t launch_gather_any(const uint16_t* Ht, const uint16_t* Ht_lo, const uint32_t* bits,
                                    int64_t BH, int nb, int W, int d, uint16_t* C, uint16_t* C_lo,
                                    hipStream_t s) {
  // Row tiles of 256 query blocks (4 waves; two workgroups fill a CU's wave
  // slots), or of 128 when there are no more query blocks than that.  At the
  // 245,760-token layer 256-row tiles ran in 6.56 ms against 6.86 ms for 192
  // rows (no padding but 3/4 of the wave slots) and 6.59 ms for 512.
  if (d == 128) {
    if (nb > 128) launch_gather_t<128, 4, HILO>(Ht, Ht_lo, bits, BH, nb, W, C, C_lo, s);
    else launch_gather_t<128, 2, HILO>(Ht, Ht_lo, bits, BH, nb, W, C, C_lo, s);
  } else {
    if (nb > 128) launch_gather_t<64, 4, HILO>(Ht, Ht_lo, bits, BH, nb, W, C, C_lo, s);
    else launch_gather_t<64, 2, HILO>(Ht, Ht_lo, bits, BH, nb, W, C, C_lo, s);
  }
  return hipGetLastError();
}

hipError_t launch_gather(const uint16_t* Ht, const uint32_t* bits, int64_t BH, int nb, int W, int d,
                         uint16_t* C, hipStream_t s) {
  return launch_gather_any<false>(Ht, nullptr, bits, BH, nb, W, d, C, nullptr, s);
}

hipError_t launch_gather_hilo(const uint16_t* Ht, const uint16_t* Ht_lo, const uint32_t* bits,
                              int64_t BH, int nb, int W, int d, uint16_t* C, uint16_t* C_lo,
                              hipStream_t s) {
  return launch_gather_any<true>(Ht, Ht_lo, bits, BH, nb, W, d, C, C_lo, s);
}

template <int D, int BLK>
static void launch_states_lo_t(const uint16_t* k, const uint16_t* v, int64_t BH, int N, int nb,
                               uint16_t* Ht_lo, hipStream_t s) {
  if constexpr (D == 128 && BLK == 128) {
    const int npairs = (nb + 1) / 2;
    lstate::lin_state_pipe_kernel<true><<<dim3((unsigned)(BH * npairs)), lstate::NT, 0, s>>>(
        k, v, N, nb, npairs, Ht_lo, nullptr);
  } else {
    lin_state_kernel<D, BLK, true><<<dim3((unsigned)(BH * nb)), 256, 0, s>>>(k, v, N, nb, Ht_lo,
                                                                             nullptr);
  }
}

hipError_t launch_linear_states_lo(const uint16_t* k, const uint16_t* v, int64_t BH, int N, int d,
                                   int block, int nb, uint16_t* Ht_lo, hipStream_t s) {
  if (d == 128 && block == 128) launch_states_lo_t<128, 128>(k, v, BH, N, nb, Ht_lo, s);
  else if (d == 128 && block == 64) launch_states_lo_t<128, 64>(k, v, BH, N, nb, Ht_lo, s);
  else if (d == 64 && block == 128) launch_states_lo_t<64, 128>(k, v, BH, N, nb, Ht_lo, s);
  else launch_states_lo_t<64, 64>(k, v, BH, N, nb, Ht_lo, s);
  return hipGetLastError();
}

hipError_t launch_bitrow_sums(const uint32_t* bits, int W, int64_t rows, int per_head, int nsrc,
                              const float* src, float* out, int d, hipStream_t s) {
  const dim3 grid((unsigned)((rows + 3) / 4));
  if (d == 128)
    lin_bitrow_sum_kernel<128><<<grid, 256, 0, s>>>(bits, W, rows, per_head, nsrc, src, out);
  else
    lin_bitrow_sum_kernel<64><<<grid, 256, 0, s>>>(bits, W, rows, per_head, nsrc, src, out);
  return hipGetLastError();
}

hipError_t launch_linear_prepare(const uint16_t* k, const uint16_t* v, int64_t BH, int N, int d,
                                 int block, int nb, const int32_t* idx, const int32_t* cnt,
                                 int kmax, void* ws, hipStream_t s) {
  if (d == 128 && block == 128)
    return launch_linear_prepare_t<128, 128>(k, v, BH, N, nb, idx, cnt, kmax, ws, s);
  if (d == 128 && block == 64)
    return launch_linear_prepare_t<128, 64>(k, v, BH, N, nb, idx, cnt, kmax, ws, s);
  if (d == 64 && block == 128)
    return launch_linear_prepare_t<64, 128>(k, v, BH, N, nb, idx, cnt, kmax, ws, s);
  return launch_linear_prepare_t<64, 64>(k, v, BH, N, nb, idx, cnt, kmax, ws, s);
}

template <int D, int BLK>
static hipError_t launch_linear_apply_t(const uint16_t* q, int64_t BH, int N, int nb, void* ws,
                                        float* o_lin, hipStream_t s) {
  const LinearPtrs lp = linear_ws_ptrs(ws, BH, nb, D);
  lin_apply_kernel<D, BLK><<<dim3((unsigned)(BH * nb)), BLK * 2, 0, s>>>(q, N, nb, lp.C, lp.zeta,
                                                                        o_lin);
  return hipGetLastError();
}

hipError_t launch_linear_apply(const uint16_t* q, int64_t BH, int N, int d, int block, int nb,
                               void* ws, float* o_lin, hipStream_t s) {
  if (d == 128 && block == 128) return launch_linear_apply_t<128, 128>(q, BH, N, nb, ws, o_lin, s);
  if (d == 128 && block == 64) return launch_linear_apply_t<128, 64>(q, BH, N, nb, ws, o_lin, s);
  if (d == 64 && block == 128) return launch_linear_apply_t<64, 128>(q, BH, N, nb, ws, o_lin, s);
  return launch_linear_apply_t<64, 64>(q, BH, N, nb, ws, o_lin, s);
}

hipError_t launch_combine(const void* o_s, int o_s_fp32, const float* o_lin, uint16_t* o,
                          int64_t n_elems, hipStream_t s) {
  const int64_t n8 = n_elems / 8;
  if (n8 == 0) return hipSuccess;
  combine_kernel<<<dim3((unsigned)((n8 + 255) / 256)), 256, 0, s>>>(o_s, o_s_fp32, o_lin, o, n8);
  return hipGetLastError();
}

}  // namespace sla
