// Per-head 3D token tiles (Veda article, context: heads and layers get their
// own tile shapes).  Tokens of a (T, Y, X) grid arrive in raster order
// n = (t Y + y) X + x; a head's tile shape (bt, by, bx) orders them box by box
// (boxes in raster order of their box index, raster order inside a box), so
// that each block of bt*by*bx consecutive tokens is one box.  The kernel
// gathers rows into that order, or scatters them back (inverse).  Each group
// of d/8 lanes moves one row in 16-byte chunks, so a load instruction covers
// whole rows; the position -> raster index map is plain integer arithmetic.
#include "common.h"
#include "launch.h"

namespace sla {

// Grid: x over the 16-byte chunks of one head, y over (batch, head).  Tile
// sides are powers of two (their product is the 64- or 128-token block), so
// the in-tile coordinates are shifts and masks; only the box index needs two
// divisions.
template <int D>
__global__ __launch_bounds__(256) void tile_permute_kernel(const uint16_t* __restrict__ x,
                                                           uint16_t* __restrict__ y, int H, int T,
                                                           int Y, int X, TileShapes ts,
                                                           int inverse) {
  constexpr int CH = D / 8, LCH = D == 128 ? 4 : 3;  // 16-byte chunks per row
  const int N = T * Y * X;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= N * CH) return;
  const int64_t bh = blockIdx.y;
  const int h = (int)(bh % H);
  const int p = i >> LCH, ch = i & (CH - 1);  // position in tile order, chunk
  const int lt = ts.s[h][0], ly = ts.s[h][1], lx = ts.s[h][2];  // log2 of the sides
  const int lvol = lt + ly + lx;
  const int tile = p >> lvol, within = p & ((1 << lvol) - 1);
  const int nY = Y >> ly, nX = X >> lx;
  const int tyx = tile / nX;
  const int xi = tile - tyx * nX, ti = tyx / nY, yi = tyx - ti * nY;
  const int dt = within >> (ly + lx), dy = (within >> lx) & ((1 << ly) - 1),
            dx = within & ((1 << lx) - 1);
  const int n = (((ti << lt) + dt) * Y + (yi << ly) + dy) * X + (xi << lx) + dx;
  const int64_t base = bh * (int64_t)N;
  const int64_t src = base + (inverse ? p : n), dst = base + (inverse ? n : p);
  ((u32x4*)y)[dst * CH + ch] = ((const u32x4*)x)[src * CH + ch];
}

hipError_t launch_tile_permute(const uint16_t* x, uint16_t* y, int64_t BH, int H, int T, int Y,
                               int X, int d, const TileShapes& ts, int inverse, hipStream_t s) {
  const int64_t n = (int64_t)T * Y * X * (d / 8);
  const dim3 grid((unsigned)((n + 255) / 256), (unsigned)BH);
  if (d == 128)
    tile_permute_kernel<128><<<grid, 256, 0, s>>>(x, y, H, T, Y, X, ts, inverse);
  else
    tile_permute_kernel<64><<<grid, 256, 0, s>>>(x, y, H, T, Y, X, ts, inverse);
  return hipGetLastError();
}

}  // namespace sla
