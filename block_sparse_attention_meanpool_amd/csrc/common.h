// Device helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// Round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats to packed bf16 (lo in bits 0-15), round to nearest even: one
// v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// The low halves of a hi + lo bf16 split of two floats: x - bf16_rne(x) for
// each, rounded to bf16 again (packed like pack_bf16x2).  hi + lo carries
// about 16 significant bits of x.
__device__ __forceinline__ uint32_t pack_bf16x2_lo(float lo, float hi) {
  const uint32_t h = pack_bf16x2(lo, hi);
  return pack_bf16x2(lo - __uint_as_float(h << 16), hi - __uint_as_float(h & 0xffff0000u));
}

// Raw buffer resource over [base, base + bytes): loads past the end return 0
// and stores past the end are dropped by the hardware.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

__device__ __forceinline__ f32x16 mfma32x32x16(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Combine a value across the two 32-lane halves of a wave (lanes l and l^32).
// v_permlane32_swap with one register as both operands returns
// {[x_lo, x_lo], [x_hi, x_hi]}: every lane sees both halves' values.
__device__ __forceinline__ float max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// acc + lo + hi of a packed bf16 pair, in one v_dot2 against (1, 1).
__device__ __forceinline__ float add_bf16x2(uint32_t packed, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, packed),
                                         __builtin_bit_cast(bf16x2, 0x3f803f80u), acc, false);
}

// ---------------------------------------------------------------------------
// MFMA 32x32x16 lane layout (gfx950, wave64), used throughout:
//   A (32 x 16, M x K): lane l holds A[l % 32][8 * (l / 32) + 0..7]
//   B (16 x 32, K x N): lane l holds B[8 * (l / 32) + 0..7][l % 32]
//   C (32 x 32):        lane l, register r holds C[8*(r/4) + 4*(l/32) + r%4][l % 32]
// ---------------------------------------------------------------------------

// Row permutation of a 32-row A operand that makes the C registers 0..7 of a
// lane hold 8 consecutive rows: MFMA row m reads source row swap_bits_2_3(m).
// Lane half h then holds source rows 8h + r (r = 0..7) in C registers 0..7 and
// rows 16 + 8h + (r - 8) in registers 8..15.
__device__ __forceinline__ int swap_bits_2_3(int m) {
  return (m & 0x13) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// ---------------------------------------------------------------------------
// LDS bank rules assumed below: a 16-byte-per-lane access is served 8 lanes
// (128 bytes) at a time, or 16 lanes (256 bytes) at a time; the swizzles
// keep every aligned group of 8 and of 16 lanes on distinct 16-byte bank
// groups, for both the staging writes and the MFMA operand reads.
// ---------------------------------------------------------------------------

// Row-major tile with CH 16-byte chunks per row: chunk ch of row r lives at
// physical chunk ch ^ row_swz(r).  MFMA operand reads take rows
// swap_bits_2_3(l % 32) + 32 kb, one chunk, so lanes 0..7 read rows
// {0,1,2,3,8,9,10,11}; swapping bits 2 and 3 back makes their swizzle 0..7.
template <int CH>
__device__ __forceinline__ int row_swz(int r) {
  return swap_bits_2_3(r & 15) & (CH - 1);
}
template <int CH>
__device__ __forceinline__ uint32_t row_offset(int r, int chunk) {  // bytes
  return (uint32_t)(r * (CH * 16) + 16 * (chunk ^ row_swz<CH>(r)));
}

// Transposed tile: element (row = feature f, col = token t) of a tile with T
// tokens per row, stored token-contiguous in 16-byte chunks of 8 tokens.
// Chunk c of row f lives at physical chunk c ^ (f % (T/8)).
template <int T>
__device__ __forceinline__ uint32_t tr_offset(int f, int chunk) {  // bytes
  return (uint32_t)(f * (T * 2) + 16 * (chunk ^ (f & (T / 8 - 1))));
}

// Transpose an 8 (tokens) x 8 (features) bf16 block held as 8 rows of 16 bytes
// into 8 feature rows of 8 tokens each (one v_perm_b32 per output dword).
__device__ __forceinline__ void transpose8x8(const u32x4 in[8], u32x4 out[8]) {
#pragma unroll
  for (int f = 0; f < 8; ++f) {
    const int w = f >> 1;
    const uint32_t sel = (f & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
    for (int p = 0; p < 4; ++p)
      out[f][p] = __builtin_amdgcn_perm(in[2 * p + 1][w], in[2 * p][w], sel);
  }
}

// Sub-block s of a tile of T tokens (by any feature width) -> (token chunk tc,
// feature chunk fc).  Within each 8-lane group the token chunks differ and the feature
// chunk is shared, so each global load instruction reads 128 contiguous bytes
// of 8 rows and the transposed LDS writes (row 8 fc + i, chunk tc) land on 8
// (and, with the neighbouring group, 16) distinct bank groups.
template <int T>
__device__ __forceinline__ void subblock_coords(int s, int& tc, int& fc) {
  constexpr int TH = T / 64;  // groups of 8 token chunks
  const int lane = s & 63, w = s >> 6;
  tc = 8 * (w % TH) + (lane & 7);
  fc = 8 * (w / TH) + (lane >> 3);
}


// ---------------------------------------------------------------------------
// Row-major bf16 tiles of 256-byte rows (128 elements) read as transposed MFMA
// operands with ds_read_b64_tr_b16.  Within each 16-lane group, lane i of the
// instruction receives element i % 4 of the 8-byte chunks addressed by lanes
// 4e + i / 4 (e = 0..3).  Pointing lane s of group g at row 4a + s / 4 and
// columns c0 + 16 (g & 1) + 4 (s & 3) .. +3 therefore hands lane g*16 + s the
// four values of column c0 + 16 (g & 1) + s in rows 4a .. 4a+3; two reads give
// 8 consecutive rows of one column, i.e. one K-contiguous MFMA operand.
// Chunk c of row r is stored at physical chunk c ^ trs_swz(r): a transpose
// read touches rows 4a..4a+3 and two (16 lanes) or four (32 lanes) adjacent
// chunks, and the table keeps those on distinct bank groups in both cases.
// ---------------------------------------------------------------------------
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;

__device__ __forceinline__ int trs_swz(int r) { return (0xAC60 >> (4 * (r & 3))) & 15; }

// A swizzle that serves both access kinds of a 256-byte-row tile: the
// transpose reads above (rows 4a..4a+3 must differ in bits 2-3 of the
// swizzle) and MFMA operand row reads (16 consecutive rows, one chunk: the
// swizzle must be a bijection on r % 16).  Swapping the two 2-bit halves of
// r % 16 does both.  Used by tiles that are read both ways.
__device__ __forceinline__ int dual_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

struct TrSwz {
  __device__ static int f(int r) { return trs_swz(r); }
};
struct DualSwz {
  __device__ static int f(int r) { return dual_swz(r); }
};

template <class SW = TrSwz>
__device__ __forceinline__ u32x2 tr_read256(const char* base, int row, int col) {
  const int chunk = col >> 3;
  const uint32_t off = (uint32_t)(row * 256 + 16 * (chunk ^ SW::f(row)) + 8 * ((col >> 2) & 1));
  typedef __attribute__((address_space(3))) s16x4* lptr;
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lptr)(base + off)));
}

// K-contiguous MFMA A operand for MFMA row (lane % 32) of the 32-column block
// starting at col0, rows k0 + 8 (lane / 32) + 0..7 of a swizzled 256-byte-row
// tile (see tr_read256).
template <class SW = TrSwz>
__device__ __forceinline__ u32x4 tr_operand(const char* base, int k0, int col0, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const int row = k0 + 8 * (g >> 1) + (s >> 2);
  const int col = col0 + 16 * (g & 1) + 4 * (s & 3);
  const u32x2 lo = tr_read256<SW>(base, row, col);
  const u32x2 hi = tr_read256<SW>(base, row + 4, col);
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// 16-byte chunk `chunk` of row `row` of a dual-swizzled 256-byte-row tile.
__device__ __forceinline__ u32x4 dual_row_read(const char* base, int row, int chunk) {
  return *(const u32x4*)(base + row * 256 + 16 * (chunk ^ dual_swz(row)));
}

__device__ __forceinline__ void wait_vmcnt0() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0); expcnt and lgkmcnt untouched
}

}  // namespace sla
