// Memory-bound helper kernels of the VSA forward on gfx950:
//   * pack_vt   -- rewrites each (batch, head, 64-row tile) of V (or of the
//                  per-block value totals) as a key-major 16-bit tile laid out
//                  exactly as the attention kernel's LDS wants it;
//   * kc_stats   -- per (batch, head, channel) mean and variance of the block
//                  key means (the Runner's KC statistics);
//   * preprocess -- per-block key means and value totals (TensorRT-Edge-LLM
//                  "Video Sparse Attention Runner", preprocess entry: BF16
//                  [numBlocks, numHeads, 128] block means of K and block sums of V;
//                  TensorRT-LLM VisualGen VSA review snippet: the mean is the block
//                  sum divided by the valid count, cast to the input dtype).
#include "vsa_internal.h"

namespace vsa {
namespace {

typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

// bf16 bits -> fp16 bits (exact for |x| in [2^-14, 65504]; the caller only
// uses fp16 tiles whose magnitudes fit, see pack_vt_kernel).
__device__ inline unsigned bf16_to_f16_bits(unsigned x) {
  _Float16 h = (_Float16)__uint_as_float(x << 16);
  return (unsigned)__builtin_bit_cast(unsigned short, h);
}

// One workgroup (256 threads) packs one 64 x 128 tile.
//
// Output layout (16 KB): key half kh (keys 0-31 / 32-63) at kh * 8192, its
// 16-key group g at + g * 4096; inside a group, row d (0..127) at d * 32 holds
// two 16-byte chunks, chunk s (the MFMA operand's lane half) at physical slot
// s ^ vt_swizzle(d).  Its eight elements are keys
//   32 kh + 16 g + 8*(j/4) + 4*s + (j%4),  j = 0..7,
// the k-slot order in which the 32x32 MFMA output leaves the probabilities.
// Padding keys (rows >= the tile's valid count) are written as zeros, so a
// zero probability never meets a NaN or Inf pad value.
//
// A tile is written as fp16 when its largest valid magnitude lies in
// [2^-10, 65280] (then every value converts exactly, or with an absolute error
// below 2^-25 for values under 2^-14) and as bf16 otherwise; flags[] records it.
__global__ __launch_bounds__(256) void pack_vt_kernel(PackParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[kBlock][kHeadDim + 8];
  __shared__ unsigned smax;
  const int tid = threadIdx.x;
  const int id = blockIdx.x;
  const int t = id % p.tiles;
  const int bh = id / p.tiles;
  const int h = bh % p.heads;
  const int b = bh / p.heads;
  int nvalid;
  if (p.vbs != nullptr) {
    nvalid = min(max(p.vbs[t], 0), kBlock);
  } else {
    nvalid = min(max(p.valid_rows - kBlock * t, 0), kBlock);
  }
  if (tid == 0) smax = 0u;
  __syncthreads();
  unsigned mymax = 0u;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int idx = tid + 256 * it;
    const int r = idx >> 4;
    const int ch = idx & 15;
    u32x4 x = {0u, 0u, 0u, 0u};
    if (r < nvalid) {
      const int64_t row = (int64_t)b * p.src_rows + p.row_offset + (int64_t)kBlock * t + r;
      x = *(const u32x4*)(p.src + (row * p.heads + h) * kHeadDim + ch * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        mymax = max(mymax, x[e] & 0x7FFFu);
        mymax = max(mymax, (x[e] >> 16) & 0x7FFFu);
      }
    }
    *(u32x4*)(&tile[r][ch * 8]) = x;
  }
  atomicMax(&smax, mymax);
  __syncthreads();
  const unsigned m = smax;
  const bool as_bf16 = (m > 0x477Fu) || (m != 0u && m < 0x3A80u);

  uint8_t* dst = p.dst + (int64_t)id * kTileBytes;
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int o = tid + 256 * it;   // 16-byte chunk o of the output tile
    const int kh = o >> 9;
    const int g = (o >> 8) & 1;
    const int d = (o >> 1) & 127;
    const int s = (o & 1) ^ vt_swizzle(d);
    unsigned e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int key = kh * 32 + g * 16 + 8 * (j >> 2) + 4 * s + (j & 3);
      const unsigned x = tile[key][d];
      e[j] = as_bf16 ? x : bf16_to_f16_bits(x);
    }
    u32x4 out;
#pragma unroll
    for (int q = 0; q < 4; ++q) out[q] = e[2 * q] | (e[2 * q + 1] << 16);
    *(u32x4*)(dst + (int64_t)o * 16) = out;
  }
  if (tid == 0) p.flags[id] = as_bf16 ? 1 : 0;
}

// float64 -> bf16 bits, one rounding to nearest-even.
__device__ inline unsigned short f64_to_bf16_rne(double x) {
  if (x == 0.0) return (unsigned short)(__double_as_longlong(x) >> 48) & 0x8000;
  if (!isfinite(x)) return isnan(x) ? 0x7FC0 : ((x < 0) ? 0xFF80 : 0x7F80);
  const int e = ilogb(x);                        // |x| = m * 2^e, 1 <= m < 2
  const double q = ldexp(1.0, max(e - 7, -133)); // bf16 quantum at this binade
  const double r = rint(x / q) * q;              // exact scaling, RNE
  if (fabs(r) >= 0x1p128) return (r < 0) ? 0xFF80 : 0x7F80;
  return (unsigned short)(__float_as_uint((float)r) >> 16);
}

// One workgroup handles one (batch, block) and eight heads.  Threads 0-127
// reduce K, threads 128-255 reduce V; each thread owns 8 head-dim values of one
// head and walks the block's valid rows with 16-byte loads.
__global__ __launch_bounds__(256) void preprocess_kernel(const uint16_t* __restrict__ k,
                                                         const uint16_t* __restrict__ v,
                                                         const int32_t* __restrict__ vbs,
                                                         uint16_t* __restrict__ kmean,
                                                         uint16_t* __restrict__ vsum,
                                                         int seq, int heads) {
  const int nblk = seq / kBlock;
  const int groups = (heads + 7) / 8;
  const int tid = threadIdx.x;
  const int g = blockIdx.x % groups;
  const int blk = (blockIdx.x / groups) % nblk;
  const int b = blockIdx.x / (groups * nblk);
  const bool is_v = tid >= 128;
  const int vec = tid & 127;
  const int h = g * 8 + (vec >> 4);
  const int d0 = (vec & 15) * 8;
  if (h >= heads) return;
  const int n = min(max(vbs[blk], 0), kBlock);
  const uint16_t* src = is_v ? v : k;
  const int64_t row_stride = (int64_t)heads * kHeadDim;
  const uint16_t* base = src + ((int64_t)b * seq + (int64_t)blk * kBlock) * row_stride +
                         (int64_t)h * kHeadDim + d0;
  double acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.0;
  int r = 0;
  for (; r + 4 <= n; r += 4) {
    u32x4 x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) x[u] = *(const u32x4*)(base + (int64_t)(r + u) * row_stride);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += (double)__uint_as_float(x[u][e] << 16);
        acc[2 * e + 1] += (double)__uint_as_float(x[u][e] & 0xFFFF0000u);
      }
  }
  for (; r < n; ++r) {
    u32x4 x = *(const u32x4*)(base + (int64_t)r * row_stride);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += (double)__uint_as_float(x[e] << 16);
      acc[2 * e + 1] += (double)__uint_as_float(x[e] & 0xFFFF0000u);
    }
  }
  u32x4 out;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    double lo = acc[2 * e], hi = acc[2 * e + 1];
    if (!is_v && n > 0) { lo = lo / (double)n; hi = hi / (double)n; }
    out[e] = (unsigned)f64_to_bf16_rne(lo) | ((unsigned)f64_to_bf16_rne(hi) << 16);
  }
  uint16_t* dst = (is_v ? vsum : kmean) +
                  (((int64_t)b * nblk + blk) * heads + h) * kHeadDim + d0;
  *(u32x4*)dst = out;
}

// Statistics of the block key means (Runner preprocess entry: FP32
// [numHeads, 128] mean and diagonal variance of KC, with KC in its BF16
// rounding).  One workgroup per (batch, head): thread t owns channel t % 128
// and every second eligible block starting at first + t / 128; two passes
// (mean, then the mean squared deviation) in float64, the halves combined in
// LDS, each result rounded once from float64 to float32.
__global__ __launch_bounds__(256) void kc_stats_kernel(const uint16_t* __restrict__ kc,
                                                       const int32_t* __restrict__ vbs,
                                                       float* __restrict__ mean_out,
                                                       float* __restrict__ var_out, int nblk,
                                                       int heads, int first, int count) {
  __shared__ double part[2][kHeadDim];
  __shared__ int npart[2];
  const int tid = threadIdx.x;
  const int d = tid & (kHeadDim - 1);
  const int half = tid >> 7;
  const int bh = blockIdx.x;
  const int h = bh % heads;
  const int b = bh / heads;
  const uint16_t* col = kc + ((int64_t)b * nblk * heads + h) * kHeadDim + d;
  const int64_t stride = (int64_t)heads * kHeadDim;
  auto value = [&](int c) { return (double)__uint_as_float((unsigned)col[c * stride] << 16); };
  double s = 0.0;
  int n = 0;
  for (int c = first + half; c < first + count; c += 2) {
    if (vbs[c] <= 0) continue;
    s += value(c);
    ++n;
  }
  part[half][d] = s;
  if (d == 0) npart[half] = n;
  __syncthreads();
  const int ntot = npart[0] + npart[1];
  const double mean = ntot > 0 ? (part[0][d] + part[1][d]) / (double)ntot : 0.0;
  __syncthreads();
  double q = 0.0;
  for (int c = first + half; c < first + count; c += 2) {
    if (vbs[c] <= 0) continue;
    const double e = value(c) - mean;
    q += e * e;
  }
  part[half][d] = q;
  __syncthreads();
  if (half == 0) {
    const double var = ntot > 0 ? (part[0][d] + part[1][d]) / (double)ntot : 0.0;
    mean_out[(int64_t)bh * kHeadDim + d] = (float)mean;
    var_out[(int64_t)bh * kHeadDim + d] = (float)var;
  }
}

}  // namespace

hipError_t launch_kc_stats(const uint16_t* kc, const int32_t* vbs, float* mean, float* var,
                           int batch, int nblk, int heads, int first, int count,
                           hipStream_t stream) {
  const int64_t n = (int64_t)batch * heads;
  if (n <= 0) return hipSuccess;
  if (!launch_fits(n, 256)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kc_stats_kernel, dim3((unsigned)n), dim3(256), 0, stream, kc, vbs, mean,
                     var, nblk, heads, first, count);
  return hipGetLastError();
}

hipError_t launch_pack(const PackParams& p, int batch, hipStream_t stream) {
  const int64_t n = (int64_t)batch * p.heads * p.tiles;
  if (n <= 0) return hipSuccess;
  if (!launch_fits(n, 256)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pack_vt_kernel, dim3((unsigned)n), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_preprocess(const uint16_t* k, const uint16_t* v, const int32_t* vbs,
                             uint16_t* kmean, uint16_t* vsum, int batch, int seq, int heads,
                             hipStream_t stream) {
  const int64_t n = (int64_t)batch * (seq / kBlock) * ((heads + 7) / 8);
  if (n <= 0) return hipSuccess;
  if (!launch_fits(n, 256)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(preprocess_kernel, dim3((unsigned)n), dim3(256), 0, stream, k, v, vbs,
                     kmean, vsum, seq, heads);
  return hipGetLastError();
}

}  // namespace vsa
