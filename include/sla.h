/*
 * sla.h - C ABI of a gfx950 (MI355X) library for block-sparse attention with
 * mean-pooled block selection.
 *
 * The method (as the pages state it):
 *   - SLA post ("what the idea is"): attention is split into critical,
 *     negligible and intermediate block pairs; critical pairs get softmax
 *     attention (FlashAttention-style), negligible pairs are skipped and
 *     intermediate (marginal) pairs get linear attention; a fast mean-pooling
 *     step marks the blocks beforehand.
 *   - NABLA post (points 2-4): Q and K are compressed; blocks are ranked by
 *     the cumulative distribution of the softmax of the compressed scores and
 *     the blocks whose summed mass reaches 1 - thr are computed.
 *   - Veda article ("what happened"): attention is computed only over the
 *     128-token key tiles each query needs, instead of all O(N^2) pairs.
 *
 * Conventions for every call:
 *   - Tensor pointers are DEVICE pointers owned by the caller, contiguous,
 *     row-major, 16-byte aligned.  bf16 tensors are passed as uint16_t bit
 *     patterns.  Q, K, V, O have shape [B, H, N, d].
 *   - Shapes are int64; byte offsets may exceed 2^31.
 *   - Supported: d in {64, 128}; block in {64, 128}; N >= 1; B, H >= 1;
 *     nb = ceil(N / block) <= 4096.  Block j covers tokens
 *     [j*block, min((j+1)*block, N)); a partial last block is handled
 *     exactly (its missing tokens never enter a sum or a softmax).
 *   - Every call validates its arguments on the host first.  On an error it
 *     launches nothing, touches no output and returns a status < 0.
 *   - All work is enqueued asynchronously on `stream` (0 = the null stream).
 *     The library never allocates, frees or synchronises and may be called
 *     from several host threads.  It keeps no state, except the static device
 *     scratch of sla_pool_classify_noalloc (see there).
 *   - A HIP launch error is returned as SLA_ERR_HIP.  No C++ exception
 *     crosses this interface.
 *
 * Class codes in a class map: 0 = skipped, 1 = marginal, 2 = critical.
 */
#ifndef SLA_H
#define SLA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t sla_status;

#define SLA_OK               0
#define SLA_ERR_INVALID_ARG (-1) /* null pointer, bad size, k or thr out of range */
#define SLA_ERR_UNSUPPORTED (-2) /* d, block or nb outside the supported set     */
#define SLA_ERR_ALIGNMENT   (-3) /* a tensor pointer is not 16-byte aligned      */
#define SLA_ERR_WORKSPACE   (-4) /* workspace missing or smaller than required    */
#define SLA_ERR_HIP         (-5) /* a HIP launch failed                           */

#define SLA_SEL_TOPK 0 /* keep the k_crit highest-scoring key blocks per row           */
#define SLA_SEL_CDF  1 /* keep the smallest prefix whose pooled-softmax mass >= 1 - thr */
#define SLA_SEL_SLA3 2 /* first k_crit critical, next k_marg marginal, rest skipped     */

#define SLA_CLS_SKIP     0
#define SLA_CLS_MARGINAL 1
#define SLA_CLS_CRITICAL 2

/* Bits set in the device error flag of sla_block_mask. */
#define SLA_FLAG_BAD_CLASS 1 /* a class value > 2 was found (treated as skipped)   */
#define SLA_FLAG_OVERFLOW  2 /* a row held more blocks than its list width         */
/* Bits set by sla_check_lists (and by builds with SLA_DEBUG_CHECKS). */
#define SLA_FLAG_LIST_RANGE  4  /* an entry outside [0, nkb)                       */
#define SLA_FLAG_LIST_REPEAT 8  /* an entry equal to an earlier one of its row     */
#define SLA_FLAG_LIST_ORDER  16 /* an entry smaller than the one before it         */
#define SLA_FLAG_LIST_COUNT  32 /* a count outside [0, width]                      */
/* Bit set by sla_check_row_order (and by builds with SLA_DEBUG_CHECKS). */
#define SLA_FLAG_ORDER_PERM  64 /* a head's row order is not a permutation of its
                                   query blocks (an entry out of range or repeated) */

/*
 * Tile lists (crit_idx/crit_cnt, marg_idx/marg_cnt) are read as SETS of key
 * tiles by every call that takes them: the first min(count, width) entries of
 * a row are read; an entry outside [0, nkb) is ignored, and an entry equal to
 * an earlier one of its row is ignored (the tile is used once, at its first
 * position).  sla_block_mask writes strictly ascending lists, which need none
 * of this; the softmax branch visits a row's tiles in list order, so a list
 * in another order gives the same set with a different (equally valid)
 * summation order.
 */

/*
 * Mean-pool Q and K over blocks, score every (query block, key block) pair
 * and classify it.  (SLA post: the mean-pooling step that marks blocks;
 * NABLA post points 2-3: compressed Q/K and the 1 - thr softmax-CDF cut;
 * Veda article: top-k over key tiles.)
 *
 *   qbar_i = mean of the valid Q rows of block i (fp32), kbar_j likewise;
 *   s_ij   = scale * (qbar_i . kbar_j) (fp32; scale is normally 1/sqrt(d));
 *   each row i orders its key blocks by descending s_ij, equal scores taking
 *   the lower j first, and then:
 *     SLA_SEL_TOPK: the first k_crit are critical, the rest skipped;
 *     SLA_SEL_CDF:  with p = softmax_j(s_ij), the smallest prefix whose mass
 *                   is >= 1 - thr is critical (at least one block);
 *     SLA_SEL_SLA3: the first k_crit are critical, the next k_marg marginal.
 *
 * q, k     bf16 [B, H, N, d]                                   (in)
 * mode     SLA_SEL_*; k_crit in [1, nb] for TOPK/SLA3; k_marg in
 *          [0, nb - k_crit] for SLA3 (ignored otherwise); thr in (0, 1) for
 *          CDF (ignored otherwise)
 * q_pool, k_pool  fp32 [B, H, nb, d] (out) or NULL (then kept in workspace)
 * cls      uint8 [B, H, nb, nb] class map                       (out)
 * ws       device workspace of at least sla_pool_classify_ws_bytes() bytes
 */
sla_status sla_pool_classify(const uint16_t* q, const uint16_t* k, int64_t B, int64_t H, int64_t N,
                             int64_t d, int32_t block, int32_t mode, int32_t k_crit, int32_t k_marg,
                             float thr, float scale, float* q_pool, float* k_pool, uint8_t* cls,
                             void* ws, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes for sla_pool_classify (pooled Q/K when not given, plus the
 * fp32 score matrix [B, H, nb, nb]).  Returns 0 for unsupported arguments. */
size_t sla_pool_classify_ws_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int32_t block,
                                  int32_t pooled_given);

/*
 * sla_pool_classify for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, rules and outputs as sla_pool_classify (the
 * same kernels; bit-identical results), without the workspace: the pooled
 * Q/K (unless q_pool/k_pool are given) and the scores live in a static
 * device array of sla_pool_classify_noalloc_scratch_bytes() bytes (80 MiB)
 * that the library holds on each GPU it runs on until the process ends.
 * Heads are processed in chunks that fit that array; a shape whose single
 * head does not fit is rejected with SLA_ERR_WORKSPACE (no supported shape
 * is: one head at nb = 4096, d = 128 needs 71.3 MB).  The call allocates
 * nothing and enqueues no memset.  On its first use on a device it looks the
 * array's device address up once (with that device current).  Every call on
 * one GPU shares the array: calls that overlap on one GPU (different
 * streams, or host threads without ordering) race and must be serialised by
 * the caller; calls in one stream are ordered.
 */
sla_status sla_pool_classify_noalloc(const uint16_t* q, const uint16_t* k, int64_t B, int64_t H,
                                     int64_t N, int64_t d, int32_t block, int32_t mode,
                                     int32_t k_crit, int32_t k_marg, float thr, float scale,
                                     float* q_pool, float* k_pool, uint8_t* cls,
                                     hipStream_t stream);

/* Size in bytes of the static device array behind sla_pool_classify_noalloc. */
size_t sla_pool_classify_noalloc_scratch_bytes(void);

/*
 * Turn a class map into compact, ascending per-row lists of key blocks: the
 * per-query-block set of tiles each query needs (Veda article).  Works on a
 * map from sla_pool_classify or on a caller-supplied map (mask-in).
 *
 * cls       uint8 [B, H, nqb, nkb]                              (in)
 * crit_idx  int32 [B, H, nqb, kc_max]: critical key blocks in ascending
 *           order, padded with -1                               (out)
 * crit_cnt  int32 [B, H, nqb]                                   (out)
 * marg_idx, marg_cnt  the same for marginal blocks, width km_max; both NULL
 *           (and km_max 0) when no linear branch is wanted      (out)
 * err_flag  device int32 or NULL.  A class value > 2 ORs SLA_FLAG_BAD_CLASS
 *           into it and the pair is treated as skipped; a row with more
 *           blocks than its width ORs SLA_FLAG_OVERFLOW, keeps its first
 *           `width` blocks and stores count = width.  The flag is never
 *           cleared by the library.
 */
sla_status sla_block_mask(const uint8_t* cls, int64_t B, int64_t H, int64_t nqb, int64_t nkb,
                          int32_t* crit_idx, int32_t* crit_cnt, int32_t kc_max, int32_t* marg_idx,
                          int32_t* marg_cnt, int32_t km_max, int32_t* err_flag, hipStream_t stream);

/*
 * Softmax attention over each query block's critical key blocks only (SLA
 * post: critical blocks via FlashAttention; Veda article: attention only in
 * the selected blocks).  For a query row n of block i:
 *   O_s[n] = sum_m softmax_m(scale * q_n . k_m) v_m over the tokens m of the
 *   blocks in crit_idx[i][0 .. crit_cnt[i]), renormalised over those tokens;
 *   LSE[n] = log sum_m exp(scale * q_n . k_m) (natural log).
 * A row with crit_cnt = 0 gets O_s = 0 and LSE = -inf.  bf16 MFMA products,
 * fp32 online softmax and accumulation.
 *
 * crit_idx/crit_cnt  as written by sla_block_mask (read as sets, see above)
 * row_order int32 [B, H, nb] from sla_row_order, or NULL: the order in which
 *           the query blocks run (a scheduling hint; results are identical).
 *           Each head's nb entries must be a permutation of 0 .. nb-1: a block
 *           missing from it is never computed (its outputs are left as they
 *           were) and a repeated one is computed twice; sla_check_row_order
 *           tells whether an order qualifies.
 * o_s       [B, H, N, d]; fp32 when o_is_fp32 != 0, else bf16 (RNE) (out)
 * lse       fp32 [B, H, N] or NULL                              (out)
 */
sla_status sla_sparse_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t B,
                               int64_t H, int64_t N, int64_t d, int32_t block,
                               const int32_t* crit_idx, const int32_t* crit_cnt, int32_t kc_max,
                               const int32_t* row_order, float scale, void* o_s, int32_t o_is_fp32,
                               float* lse, hipStream_t stream);

/*
 * Linear attention over each query block's marginal key blocks (SLA post:
 * intermediate blocks via linear attention), with phi(x) = elu(x) + 1:
 *   per key tile j: H_j = sum_t phi(k_t) v_t^T (d x d), z_j = sum_t phi(k_t);
 *   per query block i: S_i = sum_{j in marg_i} H_j, zeta_i = sum z_j;
 *   O_lin[n] = phi(q_n)^T S_i / (phi(q_n) . zeta_i).
 * A row with marg_cnt = 0 gets O_lin = 0.  phi(q), phi(k) and S_i enter bf16
 * MFMA products; sums are fp32.  Entries outside [0, nb) are ignored and a
 * repeated entry counts once.
 *
 * o_lin     fp32 [B, H, N, d]                                   (out)
 * ws        device workspace of at least sla_linear_branch_ws_bytes() bytes
 */
sla_status sla_linear_branch_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t B,
                                 int64_t H, int64_t N, int64_t d, int32_t block,
                                 const int32_t* marg_idx, const int32_t* marg_cnt, int32_t km_max,
                                 float* o_lin, void* ws, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes for sla_linear_branch_fwd and sla_linear_branch_prepare:
 * the per-tile states H_j (bf16) and z_j (fp32), the marginal bit matrix, and
 * the per-query-block S_i (bf16) and zeta_i (fp32).  0 for unsupported
 * arguments. */
size_t sla_linear_branch_ws_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int32_t block);

/*
 * The query-independent half of the linear branch (SLA post: intermediate
 * blocks via linear attention): the per-tile states H_j, z_j and, for every
 * query block i, S_i = sum_{j in marg_i} H_j and zeta_i = sum z_j, left in
 * `ws` for sla_sparse_linear_attn_fwd.  Same arguments and rules as
 * sla_linear_branch_fwd; entries outside [0, nb) are ignored and a repeated
 * entry counts once.  The workspace contents are opaque and stay valid until
 * the caller reuses the buffer.
 */
sla_status sla_linear_branch_prepare(const uint16_t* k, const uint16_t* v, int64_t B, int64_t H,
                                     int64_t N, int64_t d, int32_t block, const int32_t* marg_idx,
                                     const int32_t* marg_cnt, int32_t km_max, void* ws,
                                     size_t ws_bytes, hipStream_t stream);

/*
 * Both branches of one SLA layer in one pass (SLA post: critical blocks via
 * FlashAttention, intermediate blocks via linear attention, the results
 * added): O = O_s + O_lin, with O_s as in sla_sparse_attn_fwd and O_lin as in
 * sla_linear_branch_fwd, taken from a workspace that sla_linear_branch_prepare
 * filled for the same K, V, shapes and marginal lists.  Each query's two
 * outputs are summed in fp32 and stored once; this replaces the separate
 * linear apply, the fp32 O_s / O_lin buffers and sla_combine.
 *
 * row_order as in sla_sparse_attn_fwd, or NULL
 * lin_ws    prepared linear-branch workspace (in), at least
 *           sla_linear_branch_ws_bytes() bytes
 * o         [B, H, N, d]; fp32 when o_is_fp32 != 0, else bf16 (RNE) (out)
 * lse       fp32 [B, H, N] of the softmax branch, or NULL         (out)
 */
sla_status sla_sparse_linear_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                      int64_t B, int64_t H, int64_t N, int64_t d, int32_t block,
                                      const int32_t* crit_idx, const int32_t* crit_cnt,
                                      int32_t kc_max, const int32_t* row_order, float scale,
                                      const void* lin_ws,
                                      size_t lin_ws_bytes, void* o, int32_t o_is_fp32, float* lse,
                                      hipStream_t stream);

/*
 * Sum the branches and round to bf16: O = bf16_rne(O_s + O_lin).  The pages
 * only say the intermediate part goes through linear attention; the two
 * outputs are added without weights.
 *
 * o_s   [n_elems], fp32 when o_s_is_fp32 != 0 else bf16         (in)
 * o_lin fp32 [n_elems] or NULL (then O = bf16_rne(O_s))         (in)
 * o     bf16 [n_elems]                                          (out)
 * n_elems must be a multiple of 8.
 */
sla_status sla_combine(const void* o_s, int32_t o_s_is_fp32, const float* o_lin, uint16_t* o,
                       int64_t n_elems, hipStream_t stream);

/*
 * Gradients of the softmax branch with the class map held fixed (SLA post,
 * results: the method is trained with a short fine-tuning).  For the loss
 * gradient dO of O_s (bf16), with P = softmax over each query block's
 * critical keys recomputed from `lse`:
 *   D_n = dO_n . O_s_n,  dS = P * (dO V^T - D),
 *   dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO,
 * each key and value summing over every query block whose list holds its tile.
 * bf16 MFMA products (P and dS rounded to bf16), fp32 accumulation.
 *
 * q, k, v, crit_idx, crit_cnt, kc_max, row_order, scale  as given to
 *           sla_sparse_attn_fwd (the lists read as sets, as there; the row
 *           order is the dQ pass's order and may be NULL)
 * o_s, lse  that call's outputs (o_s fp32 when o_s_is_fp32 != 0, else bf16)
 * d_o       bf16 [B, H, N, d]                                   (in)
 * dq, dk, dv  fp32 [B, H, N, d], overwritten                    (out)
 * ws        device workspace of at least sla_sparse_attn_bwd_ws_bytes() bytes
 * Every shape the forward takes (d = 64 or 128, blocks of 64 or 128 tokens);
 * d = 128 with 128-token blocks runs the pipelined kernels.
 */
sla_status sla_sparse_attn_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t B,
                               int64_t H, int64_t N, int64_t d, int32_t block,
                               const int32_t* crit_idx, const int32_t* crit_cnt, int32_t kc_max,
                               const int32_t* row_order, float scale, const void* o_s,
                               int32_t o_s_is_fp32, const float* lse,
                               const uint16_t* d_o, float* dq, float* dk, float* dv, void* ws,
                               size_t ws_bytes, hipStream_t stream);

/* Workspace bytes for sla_sparse_attn_bwd: D and LSE log2 e (fp32 [B, H, N]
 * each) and the per-key-tile query-block lists.  0 for unsupported
 * arguments. */
size_t sla_sparse_attn_bwd_ws_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int32_t block);

/*
 * Gradients of the linear branch with the class map held fixed (SLA post:
 * intermediate blocks via linear attention; results: trainable).  With
 * a = phi(q), w_n = a_n . zeta_i and O_lin_n = a_n^T S_i / w_n, for the loss
 * gradient dO of O_lin (bf16):
 *   g_n = dO_n / w_n,  h_n = -(dO_n . O_lin_n) / w_n,
 *   dQ_n += (S_i g_n + zeta_i h_n) * phi'(q_n),
 *   dS_i = sum_n a_n g_n^T,  dzeta_i = sum_n a_n h_n,
 *   dH_j = sum of dS_i over the query blocks i whose marginal list holds j,
 *   dz_j likewise,
 *   dK_m += (dH_j v_m + dz_j) * phi'(k_m),  dV_m += dH_j^T phi(k_m),
 * with phi'(x) = 1 for x > 0 and exp(x) otherwise.  phi(q), phi(k), g and
 * the states enter bf16 MFMA products; sums are fp32.
 *
 * q, k, v, marg_idx, marg_cnt, km_max  as given to the forward
 * d_o       bf16 [B, H, N, d]                                   (in)
 * lin_ws    the workspace that sla_linear_branch_prepare (or
 *           sla_linear_branch_fwd) filled for the same q, k, v and lists (in)
 * dq, dk, dv  fp32 [B, H, N, d]: the gradients are ADDED to their contents,
 *           so a call after sla_sparse_attn_bwd yields both branches' sum
 * ws        device workspace of at least sla_linear_branch_bwd_ws_bytes() bytes
 * Every shape the forward takes (d = 64 or 128, blocks of 64 or 128 tokens).
 */
sla_status sla_linear_branch_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t B,
                                 int64_t H, int64_t N, int64_t d, int32_t block,
                                 const int32_t* marg_idx, const int32_t* marg_cnt, int32_t km_max,
                                 const uint16_t* d_o, const void* lin_ws, size_t lin_ws_bytes,
                                 float* dq, float* dk, float* dv, void* ws, size_t ws_bytes,
                                 hipStream_t stream);

/* Workspace bytes for sla_linear_branch_bwd.  0 for unsupported arguments. */
size_t sla_linear_branch_bwd_ws_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int32_t block);

/*
 * Mask quality (Veda article: fidelity to the structure of dense attention,
 * reported as recall).  For each query token n of query block i:
 *   recall[n] = sum over the keys m of the tiles in crit_idx[i] of
 *               softmax over ALL keys of (scale * q_n . k_m),
 * the share of its dense attention mass that the kept tiles hold, computed as
 * exp(LSE over the kept keys - LSE over all keys) from one masked and one
 * dense pass of the attention kernel (bf16 MFMA; each LSE within about 2^-8
 * of its exact value, so recall is within about 2 * 2^-8 relative; it is not
 * clamped to 1).  A row with no kept tile gets 0.  A diagnostic: it costs a
 * dense attention pass.
 *
 * recall    fp32 [B, H, N]                                      (out)
 * ws        device workspace of at least sla_mask_recall_ws_bytes() bytes
 */
sla_status sla_mask_recall(const uint16_t* q, const uint16_t* k, int64_t B, int64_t H, int64_t N,
                           int64_t d, int32_t block, const int32_t* crit_idx,
                           const int32_t* crit_cnt, int32_t kc_max, float scale, float* recall,
                           void* ws, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes for sla_mask_recall (a scratch O and two LSE arrays). */
size_t sla_mask_recall_ws_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int32_t block);

/*
 * Per-head 3D token tiles (Veda article, context: heads get their own tile
 * shapes).  x holds the tokens of a (T, Y, X) latent grid in raster order
 * n = (t Y + y) X + x.  Head h's tile shape (bt, by, bx) = tiles[3h .. 3h+2]
 * cuts the grid into boxes; the tile order lists the boxes in raster order of
 * their box index and, inside a box, its tokens in raster order, so that each
 * block of `block` = bt*by*bx consecutive tokens is one box.  With
 * inverse = 0, y = x rearranged into tile order (run on Q, K, V before the
 * path); with inverse != 0, y = x rearranged from tile order back to raster
 * order (run on O).  Rows are copied bit for bit.
 *
 * x, y      bf16 [B, H, T*Y*X, d], distinct buffers        (in / out)
 * tiles     HOST int32 [H][3]; each shape must divide (T, Y, X) and have
 *           volume `block` (otherwise SLA_ERR_INVALID_ARG)
 * Supported: d in {64, 128}, H <= 256.
 */
sla_status sla_tile_permute(const uint16_t* x, uint16_t* y, int64_t B, int64_t H, int64_t T,
                            int64_t Y, int64_t X, int64_t d, int32_t block, const int32_t* tiles,
                            int32_t inverse, hipStream_t stream);

/*
 * Dense softmax attention with the same kernel core: every key block is kept
 * for every query block.  A baseline for timing the sparse path against.
 */
sla_status sla_dense_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t B,
                              int64_t H, int64_t N, int64_t d, int32_t block, float scale, void* o,
                              int32_t o_is_fp32, float* lse, hipStream_t stream);

/*
 * A locality-aware order in which to run each head's query blocks (Veda
 * article: every query block attends its own set of key tiles).  Query blocks
 * whose lists sit around the same tiles share them in one XCD's L2 when they
 * run together, so the softmax kernels take an optional order: this call sorts
 * each head's query blocks by the median entry of their lists (entry
 * min(count, width) / 2; rows with no entry last; equal medians in index
 * order) and writes the permutation.  It changes only the schedule: every
 * output is the same bit for bit.  On the 75k- and 245k-token layers it cuts
 * the attention kernel's L2-to-fabric traffic by 29% and 39%.
 *
 * idx, cnt  int32 [B, H, nqb, width], [B, H, nqb] (in)
 * order     int32 [B, H, nqb]: per head, a permutation of 0 .. nqb-1 (out)
 */
sla_status sla_row_order(const int32_t* idx, const int32_t* cnt, int64_t B, int64_t H,
                         int64_t nqb, int32_t width, int32_t* order, hipStream_t stream);

/*
 * Validate tile lists supplied by a caller (the Veda article's per-query sets
 * of key tiles; the form sla_block_mask writes): for each of `rows` rows of
 * `width` entries, the first cnt entries must lie in [0, nkb), be strictly
 * ascending and so hold no repeat, and cnt must lie in [0, width].  Each
 * violation ORs its SLA_FLAG_LIST_* bit into *err_flag (device int32, never
 * cleared by the library).  Lists that fail still have a defined meaning (the
 * set rule above); the check tells the caller they were not canonical.
 *
 * idx   int32 [rows, width] (in);  cnt  int32 [rows] (in)
 */
sla_status sla_check_lists(const int32_t* idx, const int32_t* cnt, int64_t rows, int32_t width,
                           int64_t nkb, int32_t* err_flag, hipStream_t stream);

/*
 * Validate a row order supplied by a caller: each of the B*H heads' nqb
 * entries must lie in [0, nqb) and none may repeat, i.e. the head's entries
 * form a permutation of its query blocks (what sla_row_order writes).  A head
 * that fails ORs SLA_FLAG_ORDER_PERM into *err_flag (device int32, never
 * cleared by the library).  The softmax calls do not check this themselves.
 *
 * order  int32 [B, H, nqb] (in);  nqb <= 4096
 */
sla_status sla_check_row_order(const int32_t* order, int64_t B, int64_t H, int64_t nqb,
                               int32_t* err_flag, hipStream_t stream);

/*
 * Shader-clock probe, a measurement aid: one wavefront that reads the shader
 * clock counter and the fixed-rate counter, sleeps until the fixed-rate counter
 * has advanced by span_us microseconds, and reads both again.  Launched on a
 * second stream beside other work (it holds a few registers and no LDS), it
 * measures the clock that work runs at, which the chip lowers under a heavy
 * load:  clock = (out[1] - out[0]) / (out[3] - out[2]) * (*fixed_hz).
 *
 * out       device int64 [4]: shader counter at start and end, fixed-rate
 *           counter at start and end (out; 8-byte aligned)
 * span_us   in [1, 10^6]; the wait also ends after a bounded number of steps
 * fixed_hz  host int64: the fixed-rate counter's frequency (out)
 */
sla_status sla_clock_probe(int64_t* out, int32_t span_us, int64_t* fixed_hz, hipStream_t stream);

/*
 * Builds compiled with SLA_DEBUG_CHECKS validate every list argument as
 * sla_check_lists does, and every row order given to a softmax call as
 * sla_check_row_order does, before each call that reads them, into a flag word
 * the library keeps on each device; this returns that word's device address
 * on the current device (read it and clear it with ordinary copies).  NULL in
 * builds without SLA_DEBUG_CHECKS.
 */
int32_t* sla_debug_flag(void);

/* Human-readable text for a status code (static storage). */
const char* sla_status_string(sla_status status);

/* Library version as major*10000 + minor*100 + patch. */
int32_t sla_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SLA_H */
