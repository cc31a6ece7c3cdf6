// C ABI: host-side validation, workspace layout and kernel launches.
// Every entry point checks all arguments before enqueueing anything.
#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "../../include/sla.h"
#include "launch.h"

namespace {

constexpr int64_t kMaxBlocks = 4096;
constexpr int64_t kMaxHeads = 65535;  // B*H: grid y/z extent of the pooling and score launches

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Shapes shared by every call.  On success *nb is ceil(N / block).
sla_status check_shape(int64_t B, int64_t H, int64_t N, int64_t d, int32_t block, int64_t* nb) {
  if (B < 1 || H < 1 || N < 1) return SLA_ERR_INVALID_ARG;
  if ((d != 64 && d != 128) || (block != 64 && block != 128)) return SLA_ERR_UNSUPPORTED;
  if (B * H > kMaxHeads) return SLA_ERR_UNSUPPORTED;
  const int64_t n = (N + block - 1) / block;
  if (n > kMaxBlocks) return SLA_ERR_UNSUPPORTED;
  // one head's tensor must fit the 31-bit range of a buffer resource, with a
  // block of slack for the rows of a partial last block
  if ((N + block) * d * 2 > INT32_MAX) return SLA_ERR_UNSUPPORTED;
  if (B * H * (n + 8) > UINT32_MAX) return SLA_ERR_UNSUPPORTED;  // grid incl. XCD padding
  *nb = n;
  return SLA_OK;
}

sla_status from_hip(hipError_t e) { return e == hipSuccess ? SLA_OK : SLA_ERR_HIP; }

size_t pooled_bytes(int64_t BH, int64_t nb, int64_t d) {
  return round_up((size_t)(BH * nb * d) * sizeof(float), 256);
}
size_t score_bytes(int64_t BH, int64_t nb) {
  return round_up((size_t)(BH * nb * nb) * sizeof(float), 256);
}

// Checks shared by sla_pool_classify and its allocation-free variant.
sla_status check_pool_classify(const uint16_t* q, const uint16_t* k, int64_t nb, int32_t mode,
                               int32_t k_crit, int32_t k_marg, float thr, float scale,
                               const float* q_pool, const float* k_pool, const uint8_t* cls) {
  if (!q || !k || !cls) return SLA_ERR_INVALID_ARG;
  if ((q_pool == nullptr) != (k_pool == nullptr)) return SLA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(q_pool) || !aligned16(k_pool))
    return SLA_ERR_ALIGNMENT;
  if (mode == SLA_SEL_TOPK || mode == SLA_SEL_SLA3) {
    if (k_crit < 1 || k_crit > nb) return SLA_ERR_INVALID_ARG;
    if (mode == SLA_SEL_SLA3 && (k_marg < 0 || k_marg > nb - k_crit)) return SLA_ERR_INVALID_ARG;
  } else if (mode == SLA_SEL_CDF) {
    if (!(thr > 0.f && thr < 1.f)) return SLA_ERR_INVALID_ARG;
  } else {
    return SLA_ERR_INVALID_ARG;
  }
  if (!(scale > 0.f) || scale == INFINITY) return SLA_ERR_INVALID_ARG;
  return SLA_OK;
}

// Pool, score and select BH heads whose scratch (pooled Q/K unless given, then
// the scores) starts at `scratch`.
sla_status run_pool_classify(const uint16_t* q, const uint16_t* k, int64_t BH, int64_t N,
                             int64_t d, int32_t block, int64_t nb, int32_t mode, int32_t k_crit,
                             int32_t k_marg, float thr, float scale, float* q_pool, float* k_pool,
                             uint8_t* cls, char* scratch, hipStream_t stream) {
  char* p = scratch;
  float* qp = q_pool;
  float* kp = k_pool;
  if (!qp) {
    qp = reinterpret_cast<float*>(p);
    kp = reinterpret_cast<float*>(p + pooled_bytes(BH, nb, d));
    p += 2 * pooled_bytes(BH, nb, d);
  }
  float* S = reinterpret_cast<float*>(p);
  const int kc = mode == SLA_SEL_CDF ? 0 : k_crit;
  const int km = mode == SLA_SEL_SLA3 ? k_marg : 0;
  sla_status st =
      from_hip(sla::launch_pool(q, k, qp, kp, BH, (int)N, (int)d, block, (int)nb, stream));
  if (st != SLA_OK) return st;
  st = from_hip(sla::launch_scores(qp, kp, S, BH, (int)d, (int)nb, scale, stream));
  if (st != SLA_OK) return st;
  return from_hip(sla::launch_select(S, cls, BH * nb, (int)nb, mode, kc, km, thr, stream));
}

// Builds with SLA_DEBUG_CHECKS validate every list argument before the call
// that reads it, into the library's per-device debug flag (sla_debug_flag).
#ifdef SLA_DEBUG_CHECKS
sla_status debug_check_lists(const int32_t* idx, const int32_t* cnt, int64_t rows, int width,
                             int64_t nkb, hipStream_t stream) {
  int32_t* flag = nullptr;
  sla_status st = from_hip(sla::debug_flag_ptr(&flag));
  if (st != SLA_OK) return st;
  return from_hip(sla::launch_check_lists(idx, cnt, rows, width, (int)nkb, flag, stream));
}
#define SLA_DEBUG_LISTS(idx, cnt, rows, width, nkb, stream)                         \
  do {                                                                              \
    const sla_status dbg_ = debug_check_lists(idx, cnt, rows, width, nkb, stream); \
    if (dbg_ != SLA_OK) return dbg_;                                                \
  } while (0)
sla_status debug_check_order(const int32_t* order, int64_t BH, int64_t nqb, hipStream_t stream) {
  if (!order) return SLA_OK;
  int32_t* flag = nullptr;
  sla_status st = from_hip(sla::debug_flag_ptr(&flag));
  if (st != SLA_OK) return st;
  return from_hip(sla::launch_check_order(order, BH, (int)nqb, flag, stream));
}
#define SLA_DEBUG_ORDER(order, BH, nqb, stream)                         \
  do {                                                                 \
    const sla_status dbg_ = debug_check_order(order, BH, nqb, stream); \
    if (dbg_ != SLA_OK) return dbg_;                                   \
  } while (0)
#else
#define SLA_DEBUG_ORDER(order, BH, nqb, stream) \
  do {                                          \
  } while (0)
#define SLA_DEBUG_LISTS(idx, cnt, rows, width, nkb, stream) \
  do {                                                      \
  } while (0)
#endif

}  // namespace

extern "C" {

sla_status sla_row_order(const int32_t* idx, const int32_t* cnt, int64_t B, int64_t H,
                         int64_t nqb, int32_t width, int32_t* order, hipStream_t stream) {
  if (!idx || !cnt || !order) return SLA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || nqb < 1 || nqb > kMaxBlocks || width < 1) return SLA_ERR_INVALID_ARG;
  if (B * H > UINT32_MAX) return SLA_ERR_UNSUPPORTED;
  if (!aligned4(idx) || !aligned4(cnt) || !aligned4(order)) return SLA_ERR_ALIGNMENT;
  return from_hip(sla::launch_row_order(idx, cnt, B * H, (int)nqb, width, order, stream));
}

sla_status sla_clock_probe(int64_t* out, int32_t span_us, int64_t* fixed_hz, hipStream_t stream) {
  if (!out || !fixed_hz || span_us < 1 || span_us > 1000000) return SLA_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(out) & 7u) return SLA_ERR_ALIGNMENT;
  int dev = -1, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0)
    return SLA_ERR_HIP;
  *fixed_hz = (int64_t)khz * 1000;
  const uint64_t ticks = (uint64_t)khz * (uint64_t)span_us / 1000u;
  // each iteration sleeps about 4 x 64 shader cycles (~0.1 us near 2.5 GHz), so 40 per
  // requested microsecond is well above what the span needs; the cap only ends the wait of
  // a counter that does not advance (the readings stay consistent: the ratio uses both
  // counters' actual differences)
  const uint32_t max_iter = (uint32_t)span_us * 40u + 1000u;
  return from_hip(sla::launch_clock_probe(out, ticks > 0 ? ticks : 1, max_iter, stream));
}

sla_status sla_check_row_order(const int32_t* order, int64_t B, int64_t H, int64_t nqb,
                               int32_t* err_flag, hipStream_t stream) {
  if (!order || !err_flag) return SLA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || nqb < 1 || nqb > kMaxBlocks) return SLA_ERR_INVALID_ARG;
  if (B * H > UINT32_MAX) return SLA_ERR_UNSUPPORTED;
  if (!aligned4(order) || !aligned4(err_flag)) return SLA_ERR_ALIGNMENT;
  return from_hip(sla::launch_check_order(order, B * H, (int)nqb, err_flag, stream));
}

sla_status sla_check_lists(const int32_t* idx, const int32_t* cnt, int64_t rows, int32_t width,
                           int64_t nkb, int32_t* err_flag, hipStream_t stream) {
  if (!idx || !cnt || !err_flag) return SLA_ERR_INVALID_ARG;
  if (rows < 1 || width < 1 || nkb < 1 || nkb > kMaxBlocks) return SLA_ERR_INVALID_ARG;
  if ((rows + 3) / 4 > UINT32_MAX) return SLA_ERR_UNSUPPORTED;
  if (reinterpret_cast<uintptr_t>(idx) & 3u || reinterpret_cast<uintptr_t>(cnt) & 3u ||
      reinterpret_cast<uintptr_t>(err_flag) & 3u)
    return SLA_ERR_ALIGNMENT;
  return from_hip(sla::launch_check_lists(idx, cnt, rows, width, (int)nkb, err_flag, stream));
}

int32_t* sla_debug_flag(void) {
#ifdef SLA_DEBUG_CHECKS
  int32_t* flag = nullptr;
  return sla::debug_flag_ptr(&flag) == hipSuccess ? flag : nullptr;
#else
  return nullptr;
#endif
}

size_t sla_pool_classify_ws_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int32_t block,
                                  int32_t pooled_given) {
  int64_t nb = 0;
  if (check_shape(B, H, N, d, block, &nb) != SLA_OK) return 0;
  const int64_t BH = B * H;
  return (pooled_given ? 0 : 2 * pooled_bytes(BH, nb, d)) + score_bytes(BH, nb);
}

sla_status sla_pool_classify(const uint16_t* q, const uint16_t* k, int64_t B, int64_t H, int64_t N,
                             int64_t d, int32_t block, int32_t mode, int32_t k_crit, int32_t k_marg,
                             float thr, float scale, float* q_pool, float* k_pool, uint8_t* cls,
                             void* ws, size_t ws_bytes, hipStream_t stream) {
  int64_t nb = 0;
  sla_status st = check_shape(B, H, N, d, block, &nb);
  if (st != SLA_OK) return st;
  st = check_pool_classify(q, k, nb, mode, k_crit, k_marg, thr, scale, q_pool, k_pool, cls);
  if (st != SLA_OK) return st;
  const size_t need = sla_pool_classify_ws_bytes(B, H, N, d, block, q_pool != nullptr);
  if (!ws || ws_bytes < need || !aligned16(ws)) return SLA_ERR_WORKSPACE;
  return run_pool_classify(q, k, B * H, N, d, block, nb, mode, k_crit, k_marg, thr, scale, q_pool,
                           k_pool, cls, static_cast<char*>(ws), stream);
}

size_t sla_pool_classify_noalloc_scratch_bytes(void) { return sla::kNoallocScratchBytes; }

sla_status sla_pool_classify_noalloc(const uint16_t* q, const uint16_t* k, int64_t B, int64_t H,
                                     int64_t N, int64_t d, int32_t block, int32_t mode,
                                     int32_t k_crit, int32_t k_marg, float thr, float scale,
                                     float* q_pool, float* k_pool, uint8_t* cls,
                                     hipStream_t stream) {
  int64_t nb = 0;
  sla_status st = check_shape(B, H, N, d, block, &nb);
  if (st != SLA_OK) return st;
  st = check_pool_classify(q, k, nb, mode, k_crit, k_marg, thr, scale, q_pool, k_pool, cls);
  if (st != SLA_OK) return st;
  // heads per pass: as many as the static scratch holds
  const bool given = q_pool != nullptr;
  auto need = [&](int64_t heads) {
    return (given ? 0 : 2 * pooled_bytes(heads, nb, d)) + score_bytes(heads, nb);
  };
  if (need(1) > sla::kNoallocScratchBytes) return SLA_ERR_WORKSPACE;
  const int64_t BH = B * H;
  int64_t per = sla::kNoallocScratchBytes / need(1);
  while (per > 1 && need(per) > sla::kNoallocScratchBytes) --per;
  void* scratch = nullptr;
  st = from_hip(sla::noalloc_scratch(&scratch));
  if (st != SLA_OK) return st;
  for (int64_t h0 = 0; h0 < BH; h0 += per) {
    const int64_t c = per < BH - h0 ? per : BH - h0;
    st = run_pool_classify(q + h0 * N * d, k + h0 * N * d, c, N, d, block, nb, mode, k_crit,
                           k_marg, thr, scale, given ? q_pool + h0 * nb * d : nullptr,
                           given ? k_pool + h0 * nb * d : nullptr, cls + h0 * nb * nb,
                           static_cast<char*>(scratch), stream);
    if (st != SLA_OK) return st;
  }
  return SLA_OK;
}

sla_status sla_block_mask(const uint8_t* cls, int64_t B, int64_t H, int64_t nqb, int64_t nkb,
                          int32_t* crit_idx, int32_t* crit_cnt, int32_t kc_max, int32_t* marg_idx,
                          int32_t* marg_cnt, int32_t km_max, int32_t* err_flag,
                          hipStream_t stream) {
  if (!cls || !crit_idx || !crit_cnt) return SLA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || nqb < 1 || nkb < 1 || nkb > kMaxBlocks) return SLA_ERR_INVALID_ARG;
  if (kc_max < 1 || kc_max > nkb) return SLA_ERR_INVALID_ARG;
  if ((marg_idx == nullptr) != (marg_cnt == nullptr)) return SLA_ERR_INVALID_ARG;
  if (marg_idx && (km_max < 1 || km_max > nkb)) return SLA_ERR_INVALID_ARG;
  if (!marg_idx) km_max = 0;
  const int64_t rows = B * H * nqb;
  if ((rows + 3) / 4 > UINT32_MAX) return SLA_ERR_UNSUPPORTED;
  return from_hip(sla::launch_block_mask(cls, rows, (int)nkb, crit_idx, crit_cnt, kc_max, marg_idx,
                                         marg_cnt, km_max, err_flag, stream));
}

sla_status sla_sparse_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t B,
                               int64_t H, int64_t N, int64_t d, int32_t block,
                               const int32_t* crit_idx, const int32_t* crit_cnt, int32_t kc_max,
                               const int32_t* row_order, float scale, void* o_s, int32_t o_is_fp32,
                               float* lse, hipStream_t stream) {
  int64_t nb = 0;
  sla_status st = check_shape(B, H, N, d, block, &nb);
  if (st != SLA_OK) return st;
  if (!q || !k || !v || !o_s || !crit_idx || !crit_cnt) return SLA_ERR_INVALID_ARG;
  if (kc_max < 1 || kc_max > nb) return SLA_ERR_INVALID_ARG;
  if (!(scale > 0.f) || scale == INFINITY) return SLA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o_s)) return SLA_ERR_ALIGNMENT;
  if (!aligned4(row_order)) return SLA_ERR_ALIGNMENT;
  SLA_DEBUG_LISTS(crit_idx, crit_cnt, B * H * nb, kc_max, nb, stream);
  SLA_DEBUG_ORDER(row_order, B * H, nb, stream);
  return from_hip(sla::launch_attn(q, k, v, B * H, (int)N, (int)d, block, (int)nb, crit_idx,
                                   crit_cnt, kc_max, scale, o_s, o_is_fp32 != 0, lse, nullptr,
                                   row_order, stream));
}

sla_status sla_dense_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t B,
                              int64_t H, int64_t N, int64_t d, int32_t block, float scale, void* o,
                              int32_t o_is_fp32, float* lse, hipStream_t stream) {
  int64_t nb = 0;
  sla_status st = check_shape(B, H, N, d, block, &nb);
  if (st != SLA_OK) return st;
  if (!q || !k || !v || !o) return SLA_ERR_INVALID_ARG;
  if (!(scale > 0.f) || scale == INFINITY) return SLA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return SLA_ERR_ALIGNMENT;
  return from_hip(sla::launch_attn(q, k, v, B * H, (int)N, (int)d, block, (int)nb, nullptr, nullptr,
                                   (int)nb, scale, o, o_is_fp32 != 0, lse, nullptr, nullptr,
                                   stream));
}

size_t sla_linear_branch_ws_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int32_t block) {
  int64_t nb = 0;
  if (check_shape(B, H, N, d, block, &nb) != SLA_OK) return 0;
  return sla::linear_ws_layout(B * H, (int)nb, (int)d).total;
}

sla_status sla_linear_branch_prepare(const uint16_t* k, const uint16_t* v, int64_t B, int64_t H,
                                     int64_t N, int64_t d, int32_t block, const int32_t* marg_idx,
                                     const int32_t* marg_cnt, int32_t km_max, void* ws,
                                     size_t ws_bytes, hipStream_t stream) {
  int64_t nb = 0;
  sla_status st = check_shape(B, H, N, d, block, &nb);
  if (st != SLA_OK) return st;
  if (!k || !v || !marg_idx || !marg_cnt) return SLA_ERR_INVALID_ARG;
  if (km_max < 1 || km_max > nb) return SLA_ERR_INVALID_ARG;
  if (!aligned16(k) || !aligned16(v)) return SLA_ERR_ALIGNMENT;
  const size_t need = sla_linear_branch_ws_bytes(B, H, N, d, block);
  if (!ws || ws_bytes < need || !aligned16(ws)) return SLA_ERR_WORKSPACE;
  SLA_DEBUG_LISTS(marg_idx, marg_cnt, B * H * nb, km_max, nb, stream);
  return from_hip(sla::launch_linear_prepare(k, v, B * H, (int)N, (int)d, block, (int)nb, marg_idx,
                                             marg_cnt, km_max, ws, stream));
}

sla_status sla_linear_branch_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t B,
                                 int64_t H, int64_t N, int64_t d, int32_t block,
                                 const int32_t* marg_idx, const int32_t* marg_cnt, int32_t km_max,
                                 float* o_lin, void* ws, size_t ws_bytes, hipStream_t stream) {
  int64_t nb = 0;
  sla_status st = check_shape(B, H, N, d, block, &nb);
  if (st != SLA_OK) return st;
  if (!q || !k || !v || !o_lin || !marg_idx || !marg_cnt) return SLA_ERR_INVALID_ARG;
  if (km_max < 1 || km_max > nb) return SLA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o_lin)) return SLA_ERR_ALIGNMENT;
  const size_t need = sla_linear_branch_ws_bytes(B, H, N, d, block);
  if (!ws || ws_bytes < need || !aligned16(ws)) return SLA_ERR_WORKSPACE;
  SLA_DEBUG_LISTS(marg_idx, marg_cnt, B * H * nb, km_max, nb, stream);
  st = from_hip(sla::launch_linear_prepare(k, v, B * H, (int)N, (int)d, block, (int)nb, marg_idx,
                                           marg_cnt, km_max, ws, stream));
  if (st != SLA_OK) return st;
  return from_hip(sla::launch_linear_apply(q, B * H, (int)N, (int)d, block, (int)nb, ws, o_lin,
                                           stream));
}

sla_status sla_sparse_linear_attn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                      int64_t B, int64_t H, int64_t N, int64_t d, int32_t block,
                                      const int32_t* crit_idx, const int32_t* crit_cnt,
                                      int32_t kc_max, const int32_t* row_order, float scale,
                                      const void* lin_ws,
                                      size_t lin_ws_bytes, void* o, int32_t o_is_fp32, float* lse,
                                      hipStream_t stream) {
  int64_t nb = 0;
  sla_status st = check_shape(B, H, N, d, block, &nb);
  if (st != SLA_OK) return st;
  if (!q || !k || !v || !o || !crit_idx || !crit_cnt) return SLA_ERR_INVALID_ARG;
  if (kc_max < 1 || kc_max > nb) return SLA_ERR_INVALID_ARG;
  if (!(scale > 0.f) || scale == INFINITY) return SLA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return SLA_ERR_ALIGNMENT;
  const size_t need = sla_linear_branch_ws_bytes(B, H, N, d, block);
  if (!lin_ws || lin_ws_bytes < need || !aligned16(lin_ws)) return SLA_ERR_WORKSPACE;
  if (!aligned4(row_order)) return SLA_ERR_ALIGNMENT;
  SLA_DEBUG_LISTS(crit_idx, crit_cnt, B * H * nb, kc_max, nb, stream);
  SLA_DEBUG_ORDER(row_order, B * H, nb, stream);
  return from_hip(sla::launch_attn(q, k, v, B * H, (int)N, (int)d, block, (int)nb, crit_idx,
                                   crit_cnt, kc_max, scale, o, o_is_fp32 != 0, lse, lin_ws,
                                   row_order, stream));
}

size_t sla_sparse_attn_bwd_ws_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int32_t block) {
  int64_t nb = 0;
  if (check_shape(B, H, N, d, block, &nb) != SLA_OK) return 0;
  return sla::attn_bwd_ws_layout(B * H, (int)N, (int)nb).total;
}

sla_status sla_sparse_attn_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t B,
                               int64_t H, int64_t N, int64_t d, int32_t block,
                               const int32_t* crit_idx, const int32_t* crit_cnt, int32_t kc_max,
                               const int32_t* row_order, float scale, const void* o_s,
                               int32_t o_s_is_fp32, const float* lse,
                               const uint16_t* d_o, float* dq, float* dk, float* dv, void* ws,
                               size_t ws_bytes, hipStream_t stream) {
  int64_t nb = 0;
  sla_status st = check_shape(B, H, N, d, block, &nb);
  if (st != SLA_OK) return st;
  if (!q || !k || !v || !crit_idx || !crit_cnt || !o_s || !lse || !d_o || !dq || !dk || !dv)
    return SLA_ERR_INVALID_ARG;
  if (kc_max < 1 || kc_max > nb) return SLA_ERR_INVALID_ARG;
  if (!(scale > 0.f) || scale == INFINITY) return SLA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o_s) || !aligned16(d_o) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned4(lse) || !aligned4(row_order))
    return SLA_ERR_ALIGNMENT;
  const int64_t BH = B * H;
  if ((BH * nb * kc_max + 255) / 256 > UINT32_MAX) return SLA_ERR_UNSUPPORTED;
  const size_t need = sla_sparse_attn_bwd_ws_bytes(B, H, N, d, block);
  if (!ws || ws_bytes < need || !aligned16(ws)) return SLA_ERR_WORKSPACE;
  SLA_DEBUG_LISTS(crit_idx, crit_cnt, BH * nb, kc_max, nb, stream);
  SLA_DEBUG_ORDER(row_order, BH, nb, stream);
  return from_hip(sla::launch_attn_bwd(q, k, v, BH, (int)N, (int)d, block, (int)nb, crit_idx,
                                       crit_cnt, kc_max, scale, o_s, o_s_is_fp32 != 0, lse, d_o,
                                       dq, dk, dv, ws, row_order, stream));
}

size_t sla_linear_branch_bwd_ws_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int32_t block) {
  int64_t nb = 0;
  if (check_shape(B, H, N, d, block, &nb) != SLA_OK) return 0;
  return sla::linear_bwd_ws_layout(B * H, (int)nb, (int)d).total;
}

sla_status sla_linear_branch_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t B,
                                 int64_t H, int64_t N, int64_t d, int32_t block,
                                 const int32_t* marg_idx, const int32_t* marg_cnt, int32_t km_max,
                                 const uint16_t* d_o, const void* lin_ws, size_t lin_ws_bytes,
                                 float* dq, float* dk, float* dv, void* ws, size_t ws_bytes,
                                 hipStream_t stream) {
  int64_t nb = 0;
  sla_status st = check_shape(B, H, N, d, block, &nb);
  if (st != SLA_OK) return st;
  if (!q || !k || !v || !marg_idx || !marg_cnt || !d_o || !dq || !dk || !dv)
    return SLA_ERR_INVALID_ARG;
  if (km_max < 1 || km_max > nb) return SLA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(d_o) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv))
    return SLA_ERR_ALIGNMENT;
  const int64_t BH = B * H;
  if ((BH * nb * km_max + 255) / 256 > UINT32_MAX) return SLA_ERR_UNSUPPORTED;
  if (!lin_ws || lin_ws_bytes < sla_linear_branch_ws_bytes(B, H, N, d, block) ||
      !aligned16(lin_ws))
    return SLA_ERR_WORKSPACE;
  const size_t need = sla_linear_branch_bwd_ws_bytes(B, H, N, d, block);
  if (!ws || ws_bytes < need || !aligned16(ws)) return SLA_ERR_WORKSPACE;
  SLA_DEBUG_LISTS(marg_idx, marg_cnt, BH * nb, km_max, nb, stream);
  return from_hip(sla::launch_linear_bwd(q, k, v, BH, (int)N, (int)d, block, (int)nb, marg_idx,
                                         marg_cnt, km_max, d_o, lin_ws, dq, dk, dv, ws, stream));
}

size_t sla_mask_recall_ws_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int32_t block) {
  int64_t nb = 0;
  if (check_shape(B, H, N, d, block, &nb) != SLA_OK) return 0;
  return sla::recall_ws_layout(B * H, (int)N, (int)d).total;
}

sla_status sla_mask_recall(const uint16_t* q, const uint16_t* k, int64_t B, int64_t H, int64_t N,
                           int64_t d, int32_t block, const int32_t* crit_idx,
                           const int32_t* crit_cnt, int32_t kc_max, float scale, float* recall,
                           void* ws, size_t ws_bytes, hipStream_t stream) {
  int64_t nb = 0;
  sla_status st = check_shape(B, H, N, d, block, &nb);
  if (st != SLA_OK) return st;
  if (!q || !k || !crit_idx || !crit_cnt || !recall) return SLA_ERR_INVALID_ARG;
  if (kc_max < 1 || kc_max > nb) return SLA_ERR_INVALID_ARG;
  if (!(scale > 0.f) || scale == INFINITY) return SLA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || (reinterpret_cast<uintptr_t>(recall) & 3u))
    return SLA_ERR_ALIGNMENT;
  if ((B * H * N + 255) / 256 > UINT32_MAX) return SLA_ERR_UNSUPPORTED;
  const size_t need = sla_mask_recall_ws_bytes(B, H, N, d, block);
  if (!ws || ws_bytes < need || !aligned16(ws)) return SLA_ERR_WORKSPACE;
  SLA_DEBUG_LISTS(crit_idx, crit_cnt, B * H * nb, kc_max, nb, stream);
  return from_hip(sla::launch_recall(q, k, B * H, (int)N, (int)d, block, (int)nb, crit_idx,
                                     crit_cnt, kc_max, scale, recall, ws, stream));
}

sla_status sla_tile_permute(const uint16_t* x, uint16_t* y, int64_t B, int64_t H, int64_t T,
                            int64_t Y, int64_t X, int64_t d, int32_t block, const int32_t* tiles,
                            int32_t inverse, hipStream_t stream) {
  if (!x || !y || !tiles || x == y) return SLA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || T < 1 || Y < 1 || X < 1) return SLA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return SLA_ERR_UNSUPPORTED;
  if (H > sla::kMaxTileHeads) return SLA_ERR_UNSUPPORTED;
  if (T > INT32_MAX / Y || T * Y > INT32_MAX / X) return SLA_ERR_UNSUPPORTED;
  const int64_t N = T * Y * X;
  int64_t nb = 0;
  sla_status st = check_shape(B, H, N, d, block, &nb);
  if (st != SLA_OK) return st;
  if (!aligned16(x) || !aligned16(y)) return SLA_ERR_ALIGNMENT;
  if (N * (d / 8) > INT32_MAX) return SLA_ERR_UNSUPPORTED;
  sla::TileShapes ts{};
  for (int64_t h = 0; h < H; ++h) {
    const int32_t bt = tiles[3 * h], by = tiles[3 * h + 1], bx = tiles[3 * h + 2];
    if (bt < 1 || by < 1 || bx < 1) return SLA_ERR_INVALID_ARG;
    if (T % bt || Y % by || X % bx) return SLA_ERR_INVALID_ARG;
    if ((int64_t)bt * by * bx != block) return SLA_ERR_INVALID_ARG;
    // block is 64 or 128, so each side is a power of two: store log2
    ts.s[h][0] = (int16_t)__builtin_ctz((unsigned)bt);
    ts.s[h][1] = (int16_t)__builtin_ctz((unsigned)by);
    ts.s[h][2] = (int16_t)__builtin_ctz((unsigned)bx);
  }
  return from_hip(sla::launch_tile_permute(x, y, B * H, (int)H, (int)T, (int)Y, (int)X, (int)d, ts,
                                           inverse != 0, stream));
}

sla_status sla_combine(const void* o_s, int32_t o_s_is_fp32, const float* o_lin, uint16_t* o,
                       int64_t n_elems, hipStream_t stream) {
  if (!o_s || !o || n_elems < 0 || n_elems % 8 != 0) return SLA_ERR_INVALID_ARG;
  if (!aligned16(o_s) || !aligned16(o_lin) || !aligned16(o)) return SLA_ERR_ALIGNMENT;
  if ((n_elems / 8 + 255) / 256 > UINT32_MAX) return SLA_ERR_UNSUPPORTED;
  return from_hip(sla::launch_combine(o_s, o_s_is_fp32 != 0, o_lin, o, n_elems, stream));
}

const char* sla_status_string(sla_status status) {
  switch (status) {
    case SLA_OK: return "ok";
    case SLA_ERR_INVALID_ARG: return "invalid argument";
    case SLA_ERR_UNSUPPORTED: return "unsupported shape (d and block must be 64 or 128, nb <= 4096)";
    case SLA_ERR_ALIGNMENT: return "tensor pointer not 16-byte aligned";
    case SLA_ERR_WORKSPACE: return "workspace missing or too small";
    case SLA_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int32_t sla_version(void) { return 500; }

}  // extern "C"
