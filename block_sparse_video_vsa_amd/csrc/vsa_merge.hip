// Merge of two partial attention results over disjoint key sets (the row
// statistics the forward can return let separately computed parts of a row be
// combined): with lse_k = log sum over set k of exp(s) and o_k the softmax
// average over set k, the union has lse = log(exp(lse1) + exp(lse2)) and
// o = exp(lse1 - lse) o1 + exp(lse2 - lse) o2.  Rows where both parts are
// empty (lse = -inf) get o = 0 and lse = -inf.
//
// Elementwise and bound by HBM bandwidth: one thread per 8-element (16-byte)
// piece of an output row, fp32 arithmetic, one round to bf16 (nearest even).
#include "vsa_internal.h"

#include <math.h>

namespace vsa {
namespace {

typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;

__device__ inline float bf16_lo(unsigned u) { return __uint_as_float(u << 16); }
__device__ inline float bf16_hi(unsigned u) { return __uint_as_float(u & 0xFFFF0000u); }
__device__ inline unsigned rne16(float f) {
  const unsigned u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u) return (u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u);   // inf / nan
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__global__ __launch_bounds__(256) void merge_kernel(const uint16_t* __restrict__ o1,
                                                    const float* __restrict__ lse1,
                                                    const uint16_t* __restrict__ o2,
                                                    const float* __restrict__ lse2,
                                                    uint16_t* __restrict__ out,
                                                    float* __restrict__ lse_out, int64_t pieces,
                                                    int seq, int heads, int pieces_per_row) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < pieces;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = i / pieces_per_row;        // (b * seq + s) * heads + h
    const int piece = (int)(i % pieces_per_row);
    const int h = (int)(row % heads);
    const int64_t bs = row / heads;
    const int s = (int)(bs % seq);
    const int64_t b = bs / seq;
    const int64_t li = (b * heads + h) * seq + s;  // [B, H, S]
    const float l1 = lse1[li], l2 = lse2[li];
    const float m = fmaxf(l1, l2);
    u32x4 res = {0u, 0u, 0u, 0u};
    float lse = -INFINITY;
    if (m != -INFINITY) {
      const float w1 = l1 == -INFINITY ? 0.0f : expf(l1 - m);
      const float w2 = l2 == -INFINITY ? 0.0f : expf(l2 - m);
      const float tot = w1 + w2;
      lse = m + logf(tot);
      const float a1 = w1 / tot, a2 = w2 / tot;
      const u32x4 x1 = *(const u32x4*)(o1 + i * 8);
      const u32x4 x2 = *(const u32x4*)(o2 + i * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = a1 * bf16_lo(x1[e]) + a2 * bf16_lo(x2[e]);
        const float hi = a1 * bf16_hi(x1[e]) + a2 * bf16_hi(x2[e]);
        res[e] = rne16(lo) | (rne16(hi) << 16);
      }
    }
    *(u32x4*)(out + i * 8) = res;
    if (piece == 0) lse_out[li] = lse;
  }
}

// Prefix query blocks of the proxy forward are split over psplit ranges of
// key blocks; each range leaves O/l (fp32) and its row log-sum-exp.  Their
// union is the same identity over psplit parts: weights exp(lse_s - max), the
// fp32 combination divided by the weights' sum, one round to bf16.  Rows past
// vbs of their block, and rows with every part empty, are written as 0.
// One workgroup per (batch, head, prefix block): four threads per query row,
// each combining 32 of its 128 values.
__global__ __launch_bounds__(256) void prefix_merge_kernel(const float* __restrict__ part_o,
                                                           const float* __restrict__ part_lse,
                                                           const int32_t* __restrict__ vbs,
                                                           uint16_t* __restrict__ out, int seq,
                                                           int heads, int nprefix, int psplit) {
  const int qb = blockIdx.x % nprefix;
  const int bh = blockIdx.x / nprefix;
  const int h = bh % heads;
  const int b = bh / heads;
  const int row = threadIdx.x >> 2;            // query row in the block
  const int quarter = threadIdx.x & 3;         // values 32*quarter .. +31
  const int vq = min(max(vbs[qb], 0), 64);
  uint16_t* orow = out + (((int64_t)b * seq + (int64_t)qb * 64 + row) * heads + h) * 128 + 32 * quarter;
  const int64_t base = (int64_t)(bh * nprefix + qb) * psplit;   // sub-item (bh, qb, 0)
  float m = -INFINITY;
  if (row < vq)
    for (int s = 0; s < psplit; ++s) m = fmaxf(m, part_lse[(base + s) * 64 + row]);
  u32x4 res[4] = {};
  if (m != -INFINITY) {
    float acc[32] = {};
    float tot = 0.0f;
    for (int s = 0; s < psplit; ++s) {
      const float l = part_lse[(base + s) * 64 + row];
      if (l == -INFINITY) continue;
      const float wgt = expf(l - m);
      tot += wgt;
      const float* src = part_o + ((base + s) * 64 + row) * 128 + 32 * quarter;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const f32x4 v = *(const f32x4*)(src + 4 * j);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[4 * j + e] = fmaf(wgt, v[e], acc[4 * j + e]);
      }
    }
    const float inv = 1.0f / tot;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float lo = acc[2 * j] * inv, hi = acc[2 * j + 1] * inv;
      res[j / 4][j % 4] = rne16(isfinite(lo) ? lo : 0.0f) | (rne16(isfinite(hi) ? hi : 0.0f) << 16);
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) *(u32x4*)(orow + 8 * j) = res[j];
}

}  // namespace

hipError_t launch_prefix_merge(const float* part_o, const float* part_lse, const int32_t* vbs,
                               uint16_t* out, int batch, int seq, int heads, int nprefix,
                               int psplit, hipStream_t stream) {
  const int64_t blocks = (int64_t)batch * heads * nprefix;
  if (!launch_fits(blocks, 256)) return hipErrorInvalidValue;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(prefix_merge_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, part_o,
                     part_lse, vbs, out, seq, heads, nprefix, psplit);
  return hipGetLastError();
}

hipError_t launch_merge(const uint16_t* o1, const float* lse1, const uint16_t* o2, const float* lse2,
                        uint16_t* out, float* lse_out, int batch, int seq, int heads, int head_dim,
                        hipStream_t stream) {
  const int per_row = head_dim / 8;
  const int64_t pieces = (int64_t)batch * seq * heads * per_row;
  if (pieces == 0) return hipSuccess;
  const int64_t want = (pieces + 255) / 256;
  const unsigned grid = (unsigned)(want < 65536 * 16 ? want : 65536 * 16);
  hipLaunchKernelGGL(merge_kernel, dim3(grid), dim3(256), 0, stream, o1, lse1, o2, lse2, out,
                     lse_out, pieces, seq, heads, per_row);
  return hipGetLastError();
}

}  // namespace vsa
