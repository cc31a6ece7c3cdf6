// Block-sparse softmax attention over each query block's critical key tiles
// (SLA post: critical blocks via FlashAttention; Veda article, "what
// happened": attention only in the selected 128-token key tiles), and the
// dense baseline with the same core.
//
// One workgroup per (batch*head, query block); BLK/32 waves, each owning 32
// query rows.  Per kept tile:
//   K tile -> LDS row-major, 16-byte chunks XOR-swizzled per row,
//   V tile -> LDS transposed (feature rows, token-contiguous, XOR-swizzled),
//   S^T = K Q^T on v_mfma_f32_32x32x16_bf16 with Q resident in registers,
//   fp32 online softmax in the exp2 domain (scale * log2 e folded in),
//   O^T += V^T P^T on the same MFMA, P taken straight from the S^T registers.
// Computing S^T (keys x queries) puts one query per lane, so row max, row sum
// and the O rescale are per-lane values with a single exchange between the two
// 32-lane halves of the wave.
//
// With a prepared linear-branch state, the epilogue also computes the
// linear-attention output of the same queries from the Q registers it already
// holds (linear_apply.h) and stores the sum of the two branches once.
#include "common.h"
#include "launch.h"
#include "linear_apply.h"
#include "lists.h"

namespace sla {

// LIST: key tiles from the per-query-block lists (sparse); otherwise every
// tile in order (the dense baseline, a separate instantiation).  d = 64 fits
// three waves per SIMD without spills (a quarter faster than two); d = 128
// keeps two.
template <int D, int BLK, bool LIST>
__global__ __launch_bounds__(BLK * 2) __attribute__((amdgpu_waves_per_eu(D == 64 ? 3 : 2, D == 64 ? 3 : 2))) void attn_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    int N, int nqb, int nkb, const int32_t* __restrict__ idx, const int32_t* __restrict__ cnt,
    int kmax, float sl2, void* __restrict__ o, int o_fp32, float* __restrict__ lse, int seg,
    const uint16_t* __restrict__ lin_C, const float* __restrict__ lin_zeta,
    const int32_t* __restrict__ order) {
  constexpr int NT = BLK * 2;   // threads
  constexpr int CH = D / 8;     // 16-byte chunks per K row
  __shared__ __attribute__((aligned(16))) uint16_t Ks[BLK * D];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * BLK];

  // Workgroups go round-robin to the 8 XCDs.  XCD x takes positions
  // [x*seg, (x+1)*seg) of every head's query-block sequence (natural order, or
  // a row order that puts blocks with similar tile lists next to each other),
  // heads in order: neighbouring query blocks, which share most of their kept
  // tiles, meet in one XCD's L2, and all XCDs work on the same head at a time.
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

  // Q as the B operand of S^T = K Q^T: lane holds Q[row][16 ks + 8 hf + 0..7].
  const int qrow = qb * BLK + 32 * w + l32;
  u32x4 qf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
    qf[ks] = buf_load16(rq, (uint32_t)(qrow * D + 16 * ks + 8 * hf) * 2);

  const int count = LIST ? min(cnt[bh * nqb + qb], kmax) : nkb;
  const int32_t* list = LIST ? idx + (bh * nqb + qb) * (int64_t)kmax : nullptr;
  const bool canon =
      LIST ? __builtin_amdgcn_readfirstlane(list_is_canonical(list, count, nkb, lane)) : true;

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const int krow = swap_bits_2_3(l32);

  for (int t = 0; t < count; ++t) {
    const int j = LIST ? list[t] : t;
    if (LIST && !list_entry_used(list, t, j, nkb, canon)) continue;  // the list is a set of tiles
    __syncthreads();  // previous tile's LDS reads are done
    // K tile, row-major, swizzled chunks.
    {
      constexpr int PER = BLK * CH / NT;
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        const int c = tid + NT * e;
        const int row = c / CH, ch = c % CH;
        const u32x4 x = buf_load16(rk, (uint32_t)((j * BLK + row) * D + ch * 8) * 2);
        *(u32x4*)((char*)Ks + row_offset<CH>(row, ch)) = x;
      }
    }
    // V tile, transposed to feature rows in 8x8 sub-blocks.
    {
      constexpr int NSUB = (BLK / 8) * (D / 8);
#pragma unroll
      for (int s0 = 0; s0 < NSUB; s0 += NT) {
        const int s = s0 + tid;
        if (NSUB % NT == 0 || s < NSUB) {
          int tc, fc;
          subblock_coords<BLK>(s, tc, fc);
          u32x4 in[8], out[8];
#pragma unroll
          for (int r = 0; r < 8; ++r)
            in[r] = buf_load16(rv, (uint32_t)((j * BLK + 8 * tc + r) * D + 8 * fc) * 2);
          transpose8x8(in, out);
#pragma unroll
          for (int f = 0; f < 8; ++f)
            *(u32x4*)((char*)Vt + tr_offset<BLK>(8 * fc + f, tc)) = out[f];
        }
      }
    }
    __syncthreads();

    // S^T = K Q^T for this wave's 32 queries: BLK/32 blocks of 32 keys.
    f32x16 sacc[BLK / 32];
#pragma unroll
    for (int kb = 0; kb < BLK / 32; ++kb) sacc[kb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
#pragma unroll
      for (int kb = 0; kb < BLK / 32; ++kb) {
        const u32x4 a = *(const u32x4*)((const char*)Ks + row_offset<CH>(32 * kb + krow, 2 * ks + hf));
        sacc[kb] = mfma32x32x16(a, qf[ks], sacc[kb]);
      }
    }
    // Keys past N in a partial last tile.
    if ((j + 1) * BLK > N) {
      // register r of block kb holds key j BLK + 8 hf + (32 kb + r + 8 [r >= 8])
      const int lim = N - j * BLK - 8 * hf;
#pragma unroll
      for (int kb = 0; kb < BLK / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * kb + r + (r >= 8 ? 8 : 0) >= lim) sacc[kb][r] = -INFINITY;
    }
    // Online softmax (exp2 domain).
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < BLK / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) mx = fmaxf(fmaxf(mx, sacc[kb][r]), sacc[kb][r + 1]);
    mx = max_halves(mx);
    // Lazy rescale: the running maximum moves only when some row's tile
    // maximum exceeds it by more than 8 (log2 units).  P = 2^(s - m_run) then
    // stays below 2^8, which bf16 P and the fp32 sums carry as precisely; the
    // final division uses the same m_run, so the result is unchanged.
    const float mt = mx * sl2;
    if (__ballot(mt > m_run + 8.f)) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      m_run = m_new;
    }
    u32x4 pb[BLK / 16];
#pragma unroll
    for (int kb = 0; kb < BLK / 32; ++kb)
#pragma unroll
      for (int hs = 0; hs < 2; ++hs)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const float p0 = fast_exp2(fmaf(sacc[kb][8 * hs + 2 * p], sl2, -m_run));
          const float p1 = fast_exp2(fmaf(sacc[kb][8 * hs + 2 * p + 1], sl2, -m_run));
          const uint32_t pk = pack_bf16x2(p0, p1);
          pb[2 * kb + hs][p] = pk;
          l_run = add_bf16x2(pk, l_run);  // the normaliser sums the same rounded P as P V
        }
    // O^T += V^T P^T.
#pragma unroll
    for (int ks2 = 0; ks2 < BLK / 16; ++ks2) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const u32x4 a = *(const u32x4*)((const char*)Vt + tr_offset<BLK>(32 * db + l32, 2 * ks2 + hf));
        oacc[db] = mfma32x32x16(a, pb[ks2], oacc[db]);
      }
    }
  }

  const float l_tot = sum_halves(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const bool lin = lin_C != nullptr;
  f32x16 lacc[D / 32];
  float linv = 0.f;
  if (lin) {
    const int64_t row = bh * nqb + qb;
    linv = linear_apply<D>(lin_C + row * D * D, lin_zeta + row * D, qf, l32, hf, lacc);
  }
  auto out = [&](int db, int r) {
    const float x = oacc[db][r] * inv;
    return lin ? x + lacc[db][r] * linv : x;
  };
  if (qrow < N) {
    const int64_t obase = head_off + (int64_t)qrow * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * hf;
        const float x0 = out(db, 4 * g), x1 = out(db, 4 * g + 1);
        const float x2 = out(db, 4 * g + 2), x3 = out(db, 4 * g + 3);
        if (o_fp32) {
          *(f32x4*)((float*)o + obase + d0) = f32x4{x0, x1, x2, x3};
        } else {
          *(u32x2*)((uint16_t*)o + obase + d0) = u32x2{pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
        }
      }
    if (lse && hf == 0)
      lse[bh * N + qrow] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// d = 128, 128-token blocks: the same computation, pipelined.  Each kept tile
// is processed as two 64-key halves streamed through double-buffered LDS by
// asynchronous LDS-direct buffer loads: the loads of half u+1 are issued
// before half u is computed, so their latency hides behind its MFMA and
// softmax work, with one barrier per half.  64 KB of LDS and <= 256 VGPRs keep
// two workgroups per CU.  V stays row-major in LDS and reaches the MFMA as
// V^T through ds_read_b64_tr_b16: within each 16-lane group, lane i receives
// element i % 4 of the 8-byte chunks addressed by lanes 4e + i / 4 (e = 0..3),
// so two such reads give a lane 8 consecutive keys of its own feature column.
// ---------------------------------------------------------------------------
namespace pipe {

constexpr int D = 128, BLK = 128, HALF = 64, NT = 256;
constexpr int ROWB = D * 2;              // bytes per K / V row
constexpr int BUFB = HALF * ROWB;        // 16 KB per half tile

struct Ctx {
  __amdgpu_buffer_rsrc_t rk, rv;
  int nkb, wu;                // wu: the wave index, known uniform (readfirstlane)
  uint32_t koff[4], voff[4];  // per-lane byte offsets of the 4 rows a lane loads
};

// Issue the asynchronous loads of half hh of key tile j into (kbuf, vbuf).
// Each wave moves 4 KB of K and 4 KB of V: 4 instructions of 64 lanes x 16 B,
// lane-contiguous in LDS; the global chunk each lane fetches implements the
// swizzle (per-lane offsets, loop invariant).  Rows at or past N lie outside
// the buffer's range and load as zeros (finite; their keys are masked in S).
__device__ __forceinline__ void issue_half(const Ctx& c, int j, int hh, char* kbuf, char* vbuf) {
  const int jj = min(max(j, 0), c.nkb - 1);
  const uint32_t tile = (uint32_t)(jj * BLK + HALF * hh) * D * 2;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int inst = 4 * c.wu + e;                 // 1 KB LDS block, 4 rows
    __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rk, (lds_void_ptr)(kbuf + inst * 1024), 16,
                                             c.koff[e] + tile, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rv, (lds_void_ptr)(vbuf + inst * 1024), 16,
                                             c.voff[e] + tile, 0, 0, 0);
  }
}

// One 64-key half: S^T = K Q^T, masking, online softmax, O^T += V^T P^T.
__device__ __forceinline__ void compute_half(const char* kbuf, const char* vbuf, const u32x4 (&qf)[8],
                                             f32x16 (&oacc)[4], float& m_run, float& l_run,
                                             int key0, int N, float sl2, int hf, int krow, int lane) {
  f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const u32x4 a = *(const u32x4*)(kbuf + row_offset<16>(32 * kb + krow, 2 * ks + hf));
      sacc[kb] = mfma32x32x16(a, qf[ks], sacc[kb]);
    }
  }
  // Scheduling hints (LLVM's interleave strategies): the S^T MFMAs, one key
  // block's chain after the other, with their LDS operand reads, and below the
  // exp2 softmax with the P V MFMAs.  They reorder instructions only; results
  // are bit-identical (~2% faster than no hints, and the chain order with this
  // strategy another 0.5-1% over interleaved chains with the other one).
  __builtin_amdgcn_iglp_opt(0);
  if (key0 + HALF > N) {
    // register r of block kb holds key key0 + 8 hf + (32 kb + r + 8 [r >= 8])
    const int lim = N - key0 - 8 * hf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (32 * kb + r + (r >= 8 ? 8 : 0) >= lim) sacc[kb][r] = -INFINITY;
  }
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; r += 2) mx = fmaxf(fmaxf(mx, sacc[kb][r]), sacc[kb][r + 1]);
  mx = max_halves(mx);
  const float mt = mx * sl2;
  if (__ballot(mt > m_run + 8.f)) {  // lazy rescale, as in the generic kernel
    const float m_new = fmaxf(m_run, mt);
    const float alpha = fast_exp2(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    m_run = m_new;
  }
  u32x4 pb[4];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int hs = 0; hs < 2; ++hs)
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float p0 = fast_exp2(fmaf(sacc[kb][8 * hs + 2 * p], sl2, -m_run));
        const float p1 = fast_exp2(fmaf(sacc[kb][8 * hs + 2 * p + 1], sl2, -m_run));
        const uint32_t pk = pack_bf16x2(p0, p1);
        pb[2 * kb + hs][p] = pk;
        l_run = add_bf16x2(pk, l_run);
      }
#pragma unroll
  for (int ks2 = 0; ks2 < 4; ++ks2) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
      oacc[db] = mfma32x32x16(tr_operand(vbuf, 16 * ks2, 32 * db, lane), pb[ks2], oacc[db]);
  }
  __builtin_amdgcn_iglp_opt(2);
}

template <bool LIST>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_fwd_pipe_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    int N, int nqb, int nkb, const int32_t* __restrict__ idx, const int32_t* __restrict__ cnt,
    int kmax, float sl2, void* __restrict__ o, int o_fp32, float* __restrict__ lse, int seg,
    const uint16_t* __restrict__ lin_C, const float* __restrict__ lin_zeta,
    const int32_t* __restrict__ order) {
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
  Ctx c;
  c.rk = make_rsrc(k + head_off, head_bytes);
  c.rv = make_rsrc(v + head_off, head_bytes);
  c.nkb = nkb;
  c.wu = __builtin_amdgcn_readfirstlane(w);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int row = 4 * (4 * w + e) + (lane >> 4);  // row within the half tile
    c.koff[e] = (uint32_t)(row * D + ((lane & 15) ^ row_swz<16>(row)) * 8) * 2;
    c.voff[e] = (uint32_t)(row * D + ((lane & 15) ^ trs_swz(row)) * 8) * 2;
  }
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + head_off, head_bytes);

  const int count = LIST ? min(cnt[bh * nqb + qb], kmax) : nkb;
  const int32_t* list = LIST ? idx + (bh * nqb + qb) * (int64_t)kmax : nullptr;

  int j_cur = count > 0 ? (LIST ? list[0] : 0) : 0;
  if (count > 0) issue_half(c, j_cur, 0, K0, V0);

  const int qrow = qb * BLK + 32 * w + l32;
  u32x4 qf[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
    qf[ks] = buf_load16(rq, (uint32_t)(qrow * D + 16 * ks + 8 * hf) * 2);

  f32x16 oacc[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
  float m_run = -INFINITY, l_run = 0.f;
  const int krow = swap_bits_2_3(l32);
  // the list is a set of tiles: checked once, after the first loads are issued
  const bool canon =
      LIST ? __builtin_amdgcn_readfirstlane(list_is_canonical(list, count, nkb, lane)) : true;

  for (int t = 0; t < count; ++t) {
    const bool ok = LIST ? list_entry_used(list, t, j_cur, nkb, canon) : true;
    // next tile index: loaded before the wait below, which drains it together
    // with the loads of buffer 0
    const int j_next = (t + 1 < count) ? (LIST ? list[t + 1] : t + 1) : 0;
    // first half of tile j_cur, in buffer 0
    wait_vmcnt0();
    __syncthreads();  // buffer 0 complete; every wave is done with buffer 1
    issue_half(c, j_cur, 1, K1, V1);
    if (ok) compute_half(K0, V0, qf, oacc, m_run, l_run, j_cur * BLK, N, sl2, hf, krow, lane);
    // second half, in buffer 1
    wait_vmcnt0();
    __syncthreads();  // buffer 1 complete; every wave is done with buffer 0
    if (t + 1 < count) issue_half(c, j_next, 0, K0, V0);
    if (ok && j_cur * BLK + HALF < N)
      compute_half(K1, V1, qf, oacc, m_run, l_run, j_cur * BLK + HALF, N, sl2, hf, krow, lane);
    j_cur = j_next;
  }

  const float l_tot = sum_halves(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const bool lin = lin_C != nullptr;
  f32x16 lacc[4];
  float linv = 0.f;
  if (lin) {
    const int64_t row = bh * nqb + qb;
    linv = linear_apply<D>(lin_C + row * D * D, lin_zeta + row * D, qf, l32, hf, lacc);
  }
  auto out = [&](int db, int r) {
    const float x = oacc[db][r] * inv;
    return lin ? x + lacc[db][r] * linv : x;
  };
  if (qrow < N) {
    const int64_t obase = head_off + (int64_t)qrow * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * hf;
        const float x0 = out(db, 4 * g), x1 = out(db, 4 * g + 1);
        const float x2 = out(db, 4 * g + 2), x3 = out(db, 4 * g + 3);
        if (o_fp32) {
          *(f32x4*)((float*)o + obase + d0) = f32x4{x0, x1, x2, x3};
        } else {
          *(u32x2*)((uint16_t*)o + obase + d0) = u32x2{pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
        }
      }
    if (lse && hf == 0)
      lse[bh * N + qrow] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

}  // namespace pipe

template <int D, int BLK>
static hipError_t launch_attn_t(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t BH,
                                int N, int nb, const int32_t* idx, const int32_t* cnt, int kmax,
                                float scale, void* o, int o_fp32, float* lse,
                                const uint16_t* lin_C, const float* lin_zeta, const int32_t* order,
                                hipStream_t s) {
  const int seg = (nb + 7) / 8;
  dim3 grid((unsigned)(BH * seg * 8));
  if (idx)
    attn_fwd_kernel<D, BLK, true><<<grid, BLK * 2, 0, s>>>(q, k, v, N, nb, nb, idx, cnt, kmax,
                                                          scale * kLog2e, o, o_fp32, lse, seg,
                                                          lin_C, lin_zeta, order);
  else
    attn_fwd_kernel<D, BLK, false><<<grid, BLK * 2, 0, s>>>(q, k, v, N, nb, nb, idx, cnt, kmax,
                                                           scale * kLog2e, o, o_fp32, lse, seg,
                                                           lin_C, lin_zeta, nullptr);
  return hipGetLastError();
}

hipError_t launch_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t BH, int N,
                       int d, int block, int nb, const int32_t* idx, const int32_t* cnt, int kmax,
                       float scale, void* o, int o_fp32, float* lse, const void* lin_ws,
                       const int32_t* order, hipStream_t s) {
  const uint16_t* lin_C = nullptr;
  const float* lin_zeta = nullptr;
  if (lin_ws) {
    const LinearPtrs lp = linear_ws_ptrs(const_cast<void*>(lin_ws), BH, nb, d);
    lin_C = lp.C;
    lin_zeta = lp.zeta;
  }
  if (d == 128 && block == 128) {
    const int seg = (nb + 7) / 8;
    const dim3 grid((unsigned)(BH * seg * 8));
    if (idx)
      pipe::attn_fwd_pipe_kernel<true><<<grid, pipe::NT, 0, s>>>(
          q, k, v, N, nb, nb, idx, cnt, kmax, scale * kLog2e, o, o_fp32, lse, seg, lin_C, lin_zeta,
          order);
    else
      pipe::attn_fwd_pipe_kernel<false><<<grid, pipe::NT, 0, s>>>(
          q, k, v, N, nb, nb, idx, cnt, kmax, scale * kLog2e, o, o_fp32, lse, seg, lin_C, lin_zeta,
          nullptr);
    return hipGetLastError();
  }
  if (d == 128 && block == 64)
    return launch_attn_t<128, 64>(q, k, v, BH, N, nb, idx, cnt, kmax, scale, o, o_fp32, lse, lin_C,
                                  lin_zeta, order, s);
  if (d == 64 && block == 128)
    return launch_attn_t<64, 128>(q, k, v, BH, N, nb, idx, cnt, kmax, scale, o, o_fp32, lse, lin_C,
                                  lin_zeta, order, s);
  return launch_attn_t<64, 64>(q, k, v, BH, N, nb, idx, cnt, kmax, scale, o, o_fp32, lse, lin_C,
                               lin_zeta, order, s);
}

}  // namespace sla
