// Internal launchers (one per kernel family); the C ABI in api.cpp validates
// arguments and calls these.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace sla {

hipError_t launch_pool(const uint16_t* q, const uint16_t* k, float* qp, float* kp, int64_t BH,
                       int N, int d, int block, int nb, hipStream_t s);
hipError_t launch_scores(const float* qp, const float* kp, float* S, int64_t BH, int d, int nb,
                         float scale, hipStream_t s);
hipError_t launch_select(const float* S, uint8_t* cls, int64_t rows, int nb, int mode, int kc,
                         int km, float thr, hipStream_t s);
hipError_t launch_block_mask(const uint8_t* cls, int64_t rows, int nkb, int32_t* crit_idx,
                             int32_t* crit_cnt, int kc_max, int32_t* marg_idx, int32_t* marg_cnt,
                             int km_max, int32_t* err_flag, hipStream_t s);
// lin_ws: a linear-branch workspace after launch_linear_prepare, or NULL.
// When given, each query's linear-branch output is added before the store.
// order: a row order (per head, a permutation of its nb query blocks) or NULL
hipError_t launch_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t BH, int N,
                       int d, int block, int nb, const int32_t* idx, const int32_t* cnt, int kmax,
                       float scale, void* o, int o_fp32, float* lse, const void* lin_ws,
                       const int32_t* order, hipStream_t s);
// Linear-branch workspace: per-tile states H_j^T (bf16) and z_j (fp32), the
// marginal bit matrix (words 32-bit words per query block), zeta_i (fp32) and
// the gathered S_i^T (bf16), each piece 256-byte aligned.
struct LinearWs {
  int words;
  size_t ht_bytes, z_bytes, bits_bytes, zeta_bytes, c_bytes, total;
};
struct LinearPtrs {
  uint16_t* Ht;
  float* Zs;
  uint32_t* bits;
  float* zeta;
  uint16_t* C;
  int words;
};
LinearWs linear_ws_layout(int64_t BH, int nb, int d);
LinearPtrs linear_ws_ptrs(void* ws, int64_t BH, int nb, int d);
// state, mask and gather: leaves S_i^T and zeta_i of every query block in ws
hipError_t launch_linear_prepare(const uint16_t* k, const uint16_t* v, int64_t BH, int N, int d,
                                 int block, int nb, const int32_t* idx, const int32_t* cnt,
                                 int kmax, void* ws, hipStream_t s);
// C[row] = sum over the set bits k of bit row `row` of Ht[k] (rows of d*d bf16),
// per head: the masked-GEMM gather (nb bit rows of W words, nb source rows)
hipError_t launch_gather(const uint16_t* Ht, const uint32_t* bits, int64_t BH, int nb, int W, int d,
                         uint16_t* C, hipStream_t s);
// The same product with the states as a hi + lo bf16 pair (Ht, Ht_lo), both
// parts accumulated in fp32, the result stored as a hi + lo pair (C, C_lo)
hipError_t launch_gather_hilo(const uint16_t* Ht, const uint16_t* Ht_lo, const uint32_t* bits,
                              int64_t BH, int nb, int W, int d, uint16_t* C, uint16_t* C_lo,
                              hipStream_t s);
// The low parts H_j - bf16(H_j) of the per-tile states that
// launch_linear_prepare stores rounded (same layout as its Ht)
hipError_t launch_linear_states_lo(const uint16_t* k, const uint16_t* v, int64_t BH, int N, int d,
                                   int block, int nb, uint16_t* Ht_lo, hipStream_t s);
// out[row] = sum of src rows (fp32 [nsrc, d] per head) over the set bits of
// bit row `row`, in ascending order; per_head bit rows per head
hipError_t launch_bitrow_sums(const uint32_t* bits, int W, int64_t rows, int per_head, int nsrc,
                              const float* src, float* out, int d, hipStream_t s);
// Column bit matrix of per-row index lists: bit (j, i) for every entry j of
// row i (entries outside [0, ncols) dropped); clears the matrix first
hipError_t launch_col_bits(const int32_t* idx, const int32_t* cnt, int kmax, int64_t BH, int nrows,
                           int ncols, int WC, uint32_t* bitsT, hipStream_t s);
// O_lin (fp32) from a prepared workspace
hipError_t launch_linear_apply(const uint16_t* q, int64_t BH, int N, int d, int block, int nb,
                               void* ws, float* o_lin, hipStream_t s);
// Softmax-branch backward workspace: D (fp32 [BH, N]), the column bit matrix
// (wc words per key tile), column counts and column lists (uint16, width nb),
// each piece 256-byte aligned.
struct AttnBwdWs {
  int wc;
  size_t d_bytes, bits_bytes, cnt_bytes, idx_bytes, total;
};
AttnBwdWs attn_bwd_ws_layout(int64_t BH, int N, int nb);
// d in {64, 128}, block in {64, 128}; dq, dk, dv fp32, overwritten
hipError_t launch_attn_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t BH,
                           int N, int d, int block, int nb, const int32_t* idx, const int32_t* cnt,
                           int kmax, float scale, const void* o_s, int o_fp32, const float* lse,
                           const uint16_t* d_o, float* dq, float* dk, float* dv, void* ws,
                           const int32_t* order, hipStream_t s);
// the two gradient kernels for the shapes other than d = 128 with 128-token
// blocks, given D and the column lists built by launch_attn_bwd
hipError_t launch_attn_bwd_generic(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                   int64_t BH, int N, int d, int block, int nb,
                                   const int32_t* idx, const int32_t* cnt, int kmax, float scale,
                                   const void* o_s, int o_fp32, const float* lse,
                                   const uint16_t* d_o, float* dq, float* dk, float* dv,
                                   float* Dbuf, const uint16_t* col_idx, const int32_t* col_cnt,
                                   const int32_t* order, hipStream_t s);
// Linear-branch backward workspace: dS_i (bf16, laid out like the states),
// dzeta_i (fp32), the transposed marginal bit matrix, dH_j (bf16), dz_j (fp32),
// then three arrays laid out like the states (lo_bytes each): the states' low
// parts and S_i as a hi + lo pair.
struct LinearBwdWs {
  int words;
  size_t ds_bytes, dzeta_bytes, bits_bytes, dh_bytes, dz_bytes, lo_bytes, total;
};
LinearBwdWs linear_bwd_ws_layout(int64_t BH, int nb, int d);
// d in {64, 128}, block in {64, 128}; lin_ws prepared by launch_linear_prepare
// for the same inputs; dq, dk, dv fp32, accumulated into
hipError_t launch_linear_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t BH,
                             int N, int d, int block, int nb, const int32_t* idx, const int32_t* cnt,
                             int kmax, const uint16_t* d_o, const void* lin_ws, float* dq,
                             float* dk, float* dv, void* ws, hipStream_t s);
// the query-side and key-side kernels of the linear-branch backward for the
// shapes other than d = 128 with 128-token blocks
hipError_t launch_linear_bwd_query_generic(const uint16_t* q, const uint16_t* d_o, int64_t BH,
                                           int N, int d, int block, int nb, const uint16_t* C,
                                           const uint16_t* C_lo, const float* zeta, float* dq,
                                           uint16_t* dS, float* dzeta, hipStream_t s);
hipError_t launch_linear_bwd_key_generic(const uint16_t* k, const uint16_t* v, int64_t BH, int N,
                                         int d, int block, int nb, const uint16_t* dH,
                                         const float* dz, float* dk, float* dv, hipStream_t s);
// Mask recall workspace: a scratch O (bf16) and the two LSEs (fp32).
struct RecallWs {
  size_t o_bytes, lse_bytes, total;
};
RecallWs recall_ws_layout(int64_t BH, int N, int d);
hipError_t launch_recall(const uint16_t* q, const uint16_t* k, int64_t BH, int N, int d, int block,
                         int nb, const int32_t* idx, const int32_t* cnt, int kmax, float scale,
                         float* recall, void* ws, hipStream_t s);
// Per-head tile shapes as log2 of (bt, by, bx), passed by value in the kernel
// arguments.
constexpr int kMaxTileHeads = 256;
struct TileShapes {
  int16_t s[kMaxTileHeads][3];
};
hipError_t launch_tile_permute(const uint16_t* x, uint16_t* y, int64_t BH, int H, int T, int Y,
                               int X, int d, const TileShapes& ts, int inverse, hipStream_t s);
hipError_t launch_combine(const void* o_s, int o_s_fp32, const float* o_lin, uint16_t* o,
                          int64_t n_elems, hipStream_t s);
// Row order of each head's query blocks: sorted by the median entry of their
// lists (entry min(cnt, width) / 2; empty rows last), ties by index
hipError_t launch_clock_probe(int64_t* out, uint64_t ticks, uint32_t max_iter, hipStream_t s);
hipError_t launch_check_order(const int32_t* order, int64_t BH, int nqb, int32_t* err_flag,
                              hipStream_t s);
hipError_t launch_row_order(const int32_t* idx, const int32_t* cnt, int64_t BH, int nqb, int width,
                            int32_t* order, hipStream_t s);
// ORs SLA_FLAG_LIST_* bits into *err_flag for rows of `width`-wide lists
// whose first cnt entries leave [0, nkb), repeat, descend, or whose count
// lies outside [0, width]
hipError_t launch_check_lists(const int32_t* idx, const int32_t* cnt, int64_t rows, int width,
                              int nkb, int32_t* err_flag, hipStream_t s);
// Device address of the debug flag word on the current device
hipError_t debug_flag_ptr(int32_t** ptr);
// Bytes of the static device scratch behind sla_pool_classify_noalloc: one
// head's pooled Q and K and fp32 scores at the largest block count (4096
// blocks, d = 128) fit, so every supported shape runs, a chunk of heads at a
// time.
constexpr size_t kNoallocScratchBytes = size_t(80) << 20;
// Device address of that scratch on the current device (looked up once per
// device, then cached).
hipError_t noalloc_scratch(void** ptr);

}  // namespace sla
