// Cube tiling of a latent video grid (Wan2.2 production-values dataset card,
// "Shapes"): a T x Hh x W grid of tokens is cut into 4 x 4 x 4 cubes of 64
// slots, numbered row-major over the cube grid; inside a cube the real tokens
// keep their row-major (t, h, w) order and fill the first vbs[c] slots, the
// rest being padding.  Rows are whole token rows of num_heads * head_dim bf16
// values, so both directions are row gathers: the tile kernel writes every
// padded row (zeros for padding), the untile kernel every natural row.
//
// Both kernels are bound by HBM bandwidth: one workgroup per destination row,
// 16-byte vector loads and stores across the row.
#include "vsa_internal.h"

namespace vsa {
namespace {

typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

constexpr int kCube = 4;
constexpr int kLayoutThreads = 256;

struct Grid {
  int T, Hh, W;      // latent extents
  int ct, ch, cw;    // cube-grid extents
};

__device__ inline int extent(int full, int cube_index) { return min(kCube, full - kCube * cube_index); }

__device__ inline void copy_row(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                int64_t row_bytes) {
  for (int64_t o = (int64_t)threadIdx.x * 16; o < row_bytes; o += kLayoutThreads * 16)
    *(u32x4*)(dst + o) = *(const u32x4*)(src + o);
}

// One workgroup per padded row: find the natural token it holds, if any.
__global__ __launch_bounds__(kLayoutThreads) void tile_kernel(const uint8_t* __restrict__ x,
                                                              uint8_t* __restrict__ xt, Grid g,
                                                              int64_t rows_nat, int64_t rows_pad,
                                                              int64_t row_bytes) {
  const int64_t id = blockIdx.x;
  const int64_t b = id / rows_pad;
  const int slot = (int)(id % rows_pad);
  const int cube = slot / kBlock, r = slot % kBlock;
  const int a = cube / (g.ch * g.cw), bb = (cube / g.cw) % g.ch, c = cube % g.cw;
  const int et = extent(g.T, a), eh = extent(g.Hh, bb), ew = extent(g.W, c);
  uint8_t* dst = xt + (b * rows_pad + slot) * row_bytes;
  if (r >= et * eh * ew) {
    for (int64_t o = (int64_t)threadIdx.x * 16; o < row_bytes; o += kLayoutThreads * 16)
      *(u32x4*)(dst + o) = (u32x4){0u, 0u, 0u, 0u};
    return;
  }
  const int t = kCube * a + r / (eh * ew);
  const int h = kCube * bb + (r / ew) % eh;
  const int w = kCube * c + r % ew;
  const int64_t n = ((int64_t)t * g.Hh + h) * g.W + w;
  copy_row(x + (b * rows_nat + n) * row_bytes, dst, row_bytes);
}

// One workgroup per natural row: find its padded slot.
__global__ __launch_bounds__(kLayoutThreads) void untile_kernel(const uint8_t* __restrict__ xt,
                                                                uint8_t* __restrict__ x, Grid g,
                                                                int64_t rows_nat, int64_t rows_pad,
                                                                int64_t row_bytes) {
  const int64_t id = blockIdx.x;
  const int64_t b = id / rows_nat;
  const int64_t n = id % rows_nat;
  const int w = (int)(n % g.W);
  const int h = (int)((n / g.W) % g.Hh);
  const int t = (int)(n / ((int64_t)g.W * g.Hh));
  const int a = t / kCube, bb = h / kCube, c = w / kCube;
  const int eh = extent(g.Hh, bb), ew = extent(g.W, c);
  const int cube = (a * g.ch + bb) * g.cw + c;
  const int r = ((t % kCube) * eh + (h % kCube)) * ew + (w % kCube);
  copy_row(xt + (b * rows_pad + (int64_t)kBlock * cube + r) * row_bytes,
           x + (b * rows_nat + n) * row_bytes, row_bytes);
}

Grid make_grid(int T, int Hh, int W) {
  Grid g;
  g.T = T;
  g.Hh = Hh;
  g.W = W;
  g.ct = (T + kCube - 1) / kCube;
  g.ch = (Hh + kCube - 1) / kCube;
  g.cw = (W + kCube - 1) / kCube;
  return g;
}

}  // namespace

hipError_t launch_tile(const void* src, void* dst, int batch, int T, int Hh, int W, int64_t row_bytes,
                       bool untile, hipStream_t stream) {
  const Grid g = make_grid(T, Hh, W);
  const int64_t rows_nat = (int64_t)T * Hh * W;
  const int64_t rows_pad = (int64_t)kBlock * g.ct * g.ch * g.cw;
  const int64_t blocks = (int64_t)batch * (untile ? rows_nat : rows_pad);
  if (blocks == 0) return hipSuccess;
  if (!launch_fits(blocks, kLayoutThreads)) return hipErrorInvalidValue;
  if (untile)
    hipLaunchKernelGGL(untile_kernel, dim3((unsigned)blocks), dim3(kLayoutThreads), 0, stream,
                       (const uint8_t*)src, (uint8_t*)dst, g, rows_nat, rows_pad, row_bytes);
  else
    hipLaunchKernelGGL(tile_kernel, dim3((unsigned)blocks), dim3(kLayoutThreads), 0, stream,
                       (const uint8_t*)src, (uint8_t*)dst, g, rows_nat, rows_pad, row_bytes);
  return hipGetLastError();
}

}  // namespace vsa
