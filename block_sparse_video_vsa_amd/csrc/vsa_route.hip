// Routing by block-mean scores: for each (batch, head, query block) the topk
// key blocks whose mean key has the largest dot product with the block's mean
// query.  The TensorRT-Edge-LLM runner (class description and preprocess
// entry) makes a video query block exact on the key blocks whose centroid
// score passes a per-block routing threshold whose formula it does not give;
// a fixed count of the highest centroid scores is the plainest form of that
// rule that can be checked exactly.  Blocks with vbs = 0 hold no keys and are
// never chosen; ties go to the lower block index; a row lists its blocks by
// descending score and is padded with -1 when fewer than topk are eligible.
//
// Each score adds the 128 products of the bf16 means in order d = 0..127 with
// one fused multiply-add per term in float64.  A bf16 x bf16 product is exact
// in float64, so this is the same sequence of roundings as summing the exact
// products in that order: scores (and therefore the chosen indices) are
// reproducible to the last bit.
//
// Two kernels per chunk of (batch, head) pairs, through a workspace of fp64
// scores:
//   route_score_kernel: one workgroup per 128 x 128 tile of (query block, key
//     block) scores.  The bf16 means are staged 32 values of d at a time in
//     LDS as fp32 (exact), d-major; each of the 16 x 16 threads keeps an 8 x 8
//     tile of fp64 sums in registers and adds d = 0..127 in order, so every
//     score is the same sequence of roundings as one running sum.  Empty key
//     blocks (vbs = 0) are stored as -inf.
//   route_select_kernel: one wavefront per query block, over its score row:
//     0. a bound from a sample: each lane takes one block of the row, the 64
//        sampled scores are sorted across lanes, and the value a few places
//        past the expected position of the k-th largest is a bound T.  When
//        between k and 256 blocks reach it, step 2 runs on them directly;
//        otherwise:
//     1. radix select over order-preserving 64-bit codes of the scores, 8 bits
//        at a time from the top, until the bin holding the k-th largest score
//        has at most a few more entries than still needed; the bin's lower
//        edge is a bound T at or below the k-th largest score;
//     2. every block with a score at or above T is a candidate.  A block that
//        outranks a candidate is a candidate too, so a candidate's exact rank
//        in (score descending, index ascending) order is its position among
//        the candidates alone: up to 256 of them are listed in LDS and sorted
//        by a bitonic network in registers, and the first topk are written.
//        Every block of rank below topk is a candidate, so each output slot
//        is written once.  When the candidates do not fit the list (massive
//        ties, very large topk) ranks are counted over the whole row instead.
#include "vsa_internal.h"

#include <math.h>

#include <algorithm>

namespace vsa {
namespace {

constexpr int kRouteThreads = 256;
constexpr int kRouteWaves = kRouteThreads / 64;
constexpr int kHistBins = 256;
constexpr int kCandList = 256;         // per-wavefront candidate list (scores and block ids)
constexpr int kExtraCandidates = 32;   // stop refining the bound once this close
constexpr int kSampleSlack = 4;        // sample places added below the expected k-th

typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) double f64x2;

__device__ inline float bf16f(uint16_t b) { return __uint_as_float((unsigned)b << 16); }

// Orders doubles as unsigned integers (no NaN here; zeros are +0).
__device__ inline uint64_t order_code(double s) {
  const uint64_t u = (uint64_t)__double_as_longlong(s);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// LDS accesses of one wavefront complete in program order; this keeps the
// compiler from moving them across the point.
__device__ inline void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

__device__ inline int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((unsigned)(mask >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)mask, 0));
}

__device__ inline int wave_inclusive_sum(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

// (score, block id) order of the output: a higher score first, equal scores
// by the lower block id.
__device__ inline bool before(double sa, int ia, double sb, int ib) {
  return sa > sb || (sa == sb && ia < ib);
}

// Number of entries of list[0, n) that come before (se, position pe): a higher
// score, or an equal score at a lower position (positions follow block ids).
__device__ __attribute__((always_inline)) inline int rank_in(const double* __restrict__ list, int n,
                                                             double se, int pe) {
  int rank = 0;
#pragma unroll 8
  for (int f = 0; f < n; ++f) {
    const double sf = list[f];
    rank += (sf > se) | ((sf == se) & (f < pe));
  }
  return rank;
}

// Sorts the listed candidates of one row into (score descending, index
// ascending) order with a bitonic network over 64 * E positions, E per lane
// (position E * lane + s in register s; positions past the list are padding
// that sorts last), and writes the first topk block ids.  A candidate's sorted
// position is its rank in the whole row, since every block that outranks a
// candidate is a candidate.
template <int E>
__device__ __attribute__((always_inline)) inline void sort_candidates(
    const double* __restrict__ cs, const int* __restrict__ ci, int listed, int topk,
    int32_t* __restrict__ orow, int lane) {
  double sv[E];
  int iv[E];
#pragma unroll
  for (int s = 0; s < E; ++s) {
    const int p = E * lane + s;
    sv[s] = p < listed ? cs[p] : -INFINITY;
    iv[s] = p < listed ? ci[p] : 0x7FFFFFFF - p;   // distinct, after every block id
  }
  constexpr int N = 64 * E;
#pragma unroll
  for (int k = 2; k <= N; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j < E) {   // both positions in this lane's registers
#pragma unroll
        for (int s = 0; s < E; ++s) {
          if (s & j) continue;
          const int t = s | j;
          const bool asc = ((E * lane + s) & k) == 0;   // the lower position takes the first
          const bool swap = asc ? before(sv[t], iv[t], sv[s], iv[s]) : before(sv[s], iv[s], sv[t], iv[t]);
          if (swap) {
            const double ts = sv[s];
            const int ti = iv[s];
            sv[s] = sv[t];
            iv[s] = iv[t];
            sv[t] = ts;
            iv[t] = ti;
          }
        }
      } else {       // partner position in lane ^ (j / E), same register
        const int lm = j / E;
        const bool lower = (lane & lm) == 0;
#pragma unroll
        for (int s = 0; s < E; ++s) {
          const double os = xor_lane_f64(sv[s], lm, lane);
          const int oi = (int)xor_lane((unsigned)iv[s], lm, lane);
          const bool asc = ((E * lane + s) & k) == 0;
          const bool keep_first = lower == asc;
          const bool mine_first = before(sv[s], iv[s], os, oi);
          if (keep_first != mine_first) {
            sv[s] = os;
            iv[s] = oi;
          }
        }
      }
    }
  }
#pragma unroll
  for (int s = 0; s < E; ++s) {
    const int p = E * lane + s;
    if (p < listed && p < topk) orow[p] = iv[s];
  }
}

// The 64 lanes' values in descending order (bitonic network across lanes):
// lane p ends with the p-th largest.
__device__ __attribute__((always_inline)) inline uint64_t wave_sort_desc(uint64_t v, int lane) {
#pragma unroll
  for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const uint64_t o = xor_lane64(v, j, lane);
      const bool lower = (lane & j) == 0;
      const bool desc = (lane & k) == 0;     // this block of the network puts the largest first
      const bool keep_larger = lower == desc;
      v = keep_larger ? (v > o ? v : o) : (v < o ? v : o);
    }
  }
  return v;
}

// Top-k of one row of scores (in memory) by one wavefront.
__device__ __attribute__((always_inline)) inline void select_row(
    const double* __restrict__ row, int n, int topk, int* __restrict__ hist,
    double* __restrict__ cs, int* __restrict__ ci, int32_t* __restrict__ orow, int lane) {
  const int nchunks = (n + 63) >> 6;
  // value of this lane's block in chunk c (-inf past the row)
  auto val = [&](int c) -> double {
    const int e = c * 64 + lane;
    return e < n ? row[e] : -INFINITY;
  };
  auto chunks = [&](auto f) {
    for (int c = 0; c < nchunks; ++c) f(c);
  };
  // candidates (finite, code >= t) listed in index order; returns their count
  auto list_from = [&](uint64_t t) {
    int listed = 0;
    chunks([&](int c) {
      const double v = val(c);
      const bool is_cand = v != -INFINITY && order_code(v) >= t;
      const uint64_t m = __ballot(is_cand);
      const int at = listed + lanes_below(m);
      if (is_cand && at < kCandList) {
        cs[at] = v;
        ci[at] = c * 64 + lane;
      }
      listed += __popcll(m);
    });
    wave_sync();
    return listed;
  };
  auto sort_listed = [&](int listed) {
    if (listed <= 64) sort_candidates<1>(cs, ci, listed, topk, orow, lane);
    else if (listed <= 128) sort_candidates<2>(cs, ci, listed, topk, orow, lane);
    else sort_candidates<4>(cs, ci, listed, topk, orow, lane);
    wave_sync();   // the lists are refilled by this wavefront's next row
  };

  // eligible blocks (finite score) rank before every empty one
  int local = 0;
  chunks([&](int c) { local += val(c) != -INFINITY; });
  int eligible = local;   // butterfly sum: every lane ends with the total
#pragma unroll
  for (int j = 1; j < 64; j <<= 1) eligible += (int)xor_lane((unsigned)eligible, j, lane);
  for (int t = eligible + lane; t < topk; t += 64) orow[t] = -1;
  int need = min(topk, eligible);
  if (need == 0) return;

  // 0. fast path: a threshold from a sample.  Lane l samples block l*n/64;
  // the sorted sample's value a few places past the expected position of the
  // need-th largest is a bound T; if between need and kCandList blocks reach
  // it, they hold every block of rank below need and are sorted directly.
  {
    const double s = row[(int)(((int64_t)lane * n) >> 6)];
    const uint64_t sc = wave_sort_desc(s != -INFINITY ? order_code(s) : 0ull, lane);
    const int q = min(63, (int)(((int64_t)need * 64 + eligible - 1) / eligible) + kSampleSlack);
    const unsigned tlo = __shfl((unsigned)sc, q, 64), thi = __shfl((unsigned)(sc >> 32), q, 64);
    const uint64_t t = ((uint64_t)thi << 32) | tlo;
    if (t != 0ull) {
      const int listed = list_from(t);
      if (listed >= need && listed <= kCandList) {
        sort_listed(listed);
        return;
      }
    }
  }

  // 1. lower bound on the need-th largest code
  uint64_t prefix = 0, pmask = 0;
  for (int shift = 56; shift >= 0; shift -= 8) {
#pragma unroll
    for (int i = 0; i < kHistBins / 64; ++i) hist[lane * (kHistBins / 64) + i] = 0;
    wave_sync();
    chunks([&](int c) {
      const double s = val(c);
      const uint64_t code = order_code(s);
      if (s != -INFINITY && (code & pmask) == prefix) atomicAdd(&hist[(int)((code >> shift) & 0xFF)], 1);
    });
    wave_sync();
    // lane L owns bins 255 - 4L .. 252 - 4L, highest first
    int cnt[kHistBins / 64];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < kHistBins / 64; ++i) {
      cnt[i] = hist[kHistBins - 1 - (lane * (kHistBins / 64) + i)];
      sum += cnt[i];
    }
    const int incl = wave_inclusive_sum(sum, lane);
    const int excl = incl - sum;
    const uint64_t owner = __ballot(excl < need && need <= incl);
    int bin = 0, above = 0, in_bin = 0;
    if (excl < need && need <= incl) {
      int cum = excl;
#pragma unroll
      for (int i = 0; i < kHistBins / 64; ++i) {
        if (in_bin == 0 && cum + cnt[i] >= need) {
          bin = kHistBins - 1 - (lane * (kHistBins / 64) + i);
          above = cum;
          in_bin = cnt[i];
        }
        cum += cnt[i];
      }
    }
    const int src = (int)__builtin_ctzll(owner);
    bin = __shfl(bin, src, 64);
    above = __shfl(above, src, 64);
    in_bin = __shfl(in_bin, src, 64);
    need -= above;
    prefix |= (uint64_t)bin << shift;
    pmask |= 0xFFull << shift;
    wave_sync();   // hist is cleared again by the next pass
    if (in_bin - need <= kExtraCandidates) break;
  }

  // 2. candidates (code >= prefix) listed in index order and sorted; past
  // kCandList of them, ranks are counted over the whole row
  const int listed = list_from(prefix);
  if (listed <= kCandList) {
    sort_listed(listed);
    return;
  }
  chunks([&](int c) {
    const double s = val(c);
    if (s != -INFINITY && order_code(s) >= prefix) {
      const int e = c * 64 + lane;
      const int rank = rank_in(row, n, s, e);
      if (rank < topk) orow[rank] = e;
    }
  });
  wave_sync();
}

constexpr int kScoreTile = 128;   // query and key blocks per score tile
constexpr int kDChunk = 32;       // values of d staged per step

__global__ __launch_bounds__(kRouteThreads) void route_score_kernel(const uint16_t* __restrict__ qmean,
                                                                    const uint16_t* __restrict__ kmean,
                                                                    const int32_t* __restrict__ vbs,
                                                                    double* __restrict__ scores, int bh0,
                                                                    int nblk, int heads, int tiles) {
  __shared__ __attribute__((aligned(16))) float sQ[kDChunk][kScoreTile];
  __shared__ __attribute__((aligned(16))) float sK[kDChunk][kScoreTile];
  const int per_pair = tiles * tiles;
  const int g = blockIdx.x / per_pair;
  const int t = blockIdx.x - g * per_pair;
  const int i0 = (t / tiles) * kScoreTile, j0 = (t % tiles) * kScoreTile;
  const int bh = bh0 + g;
  const int h = bh % heads, b = bh / heads;
  const int tid = threadIdx.x;
  const int ty = tid >> 4, tx = tid & 15;   // rows i0 + 8ty .., columns j0 + 8tx ..

  double acc[8][8];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[a][c] = 0.0;

  // 128 rows x 32 values = 512 pieces of 16 bytes per operand and chunk; four
  // consecutive threads read one row's 64 contiguous bytes.  The next chunk's
  // pieces are loaded into registers while the current one is used.
  constexpr int kPieces = kScoreTile * (kDChunk / 8) / kRouteThreads;   // 2 per thread
  u32x4 nq[kPieces], nk[kPieces];
  auto fetch = [&](int d0) {
#pragma unroll
    for (int s = 0; s < kPieces; ++s) {
      const int pc = tid + s * kRouteThreads;
      const int r = pc >> 2, part = pc & 3;
      nq[s] = (u32x4){0u, 0u, 0u, 0u};
      nk[s] = (u32x4){0u, 0u, 0u, 0u};
      if (i0 + r < nblk)
        nq[s] = *(const u32x4*)(qmean + (((int64_t)b * nblk + i0 + r) * heads + h) * kHeadDim + d0 + 8 * part);
      if (j0 + r < nblk)
        nk[s] = *(const u32x4*)(kmean + (((int64_t)b * nblk + j0 + r) * heads + h) * kHeadDim + d0 + 8 * part);
    }
  };
  fetch(0);
  for (int d0 = 0; d0 < kHeadDim; d0 += kDChunk) {
    __syncthreads();   // the previous chunk is consumed
#pragma unroll
    for (int s = 0; s < kPieces; ++s) {
      const int pc = tid + s * kRouteThreads;
      const int r = pc >> 2, part = pc & 3;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sQ[8 * part + e][r] = bf16f((uint16_t)(nq[s][e / 2] >> (16 * (e % 2))));
        sK[8 * part + e][r] = bf16f((uint16_t)(nk[s][e / 2] >> (16 * (e % 2))));
      }
    }
    __syncthreads();
    if (d0 + kDChunk < kHeadDim) fetch(d0 + kDChunk);
#pragma unroll 2
    for (int d = 0; d < kDChunk; ++d) {
      const f32x4 q0 = *(const f32x4*)&sQ[d][8 * ty], q1 = *(const f32x4*)&sQ[d][8 * ty + 4];
      const f32x4 k0 = *(const f32x4*)&sK[d][8 * tx], k1 = *(const f32x4*)&sK[d][8 * tx + 4];
      double qd[8], kd[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qd[e] = (double)q0[e];
        qd[4 + e] = (double)q1[e];
        kd[e] = (double)k0[e];
        kd[4 + e] = (double)k1[e];
      }
#pragma unroll
      for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[a][c] = fma(qd[a], kd[c], acc[a][c]);
    }
  }

  double* srow = scores + (size_t)g * nblk * nblk;
  const int jb = j0 + 8 * tx;
  bool live[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) live[c] = jb + c < nblk && vbs[jb + c] > 0;
#pragma unroll
  for (int a = 0; a < 8; ++a) {
    const int i = i0 + 8 * ty + a;
    if (i >= nblk) continue;
    double* dst = srow + (size_t)i * nblk + jb;
    // paired 16-byte stores where the absolute element index is even
    if (jb + 8 <= nblk && ((((size_t)g * nblk + i) * nblk + jb) & 1) == 0) {
#pragma unroll
      for (int c = 0; c < 8; c += 2)
        *(f64x2*)(dst + c) = (f64x2){live[c] ? acc[a][c] + 0.0 : -INFINITY,
                                     live[c + 1] ? acc[a][c + 1] + 0.0 : -INFINITY};
    } else {
#pragma unroll
      for (int c = 0; c < 8; ++c)
        if (jb + c < nblk) dst[c] = live[c] ? acc[a][c] + 0.0 : -INFINITY;
    }
  }
}

__global__ __launch_bounds__(kRouteThreads) void route_select_kernel(const double* __restrict__ scores,
                                                                     int32_t* __restrict__ out, int bh0,
                                                                     int rows, int nblk, int topk) {
  __shared__ int hist[kRouteWaves][kHistBins];
  __shared__ double cs[kRouteWaves][kCandList];
  __shared__ int ci[kRouteWaves][kCandList];
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int r = blockIdx.x * kRouteWaves + wave;   // row of the chunk: g * nblk + i
  if (r >= rows) return;                          // per wavefront: no workgroup barriers below
  const double* row = scores + (size_t)r * nblk;
  int32_t* orow = out + ((int64_t)bh0 * nblk + r) * topk;
  select_row(row, nblk, topk, hist[wave], cs[wave], ci[wave], orow, lane);
}

}  // namespace

int route_pairs_per_chunk(int batch, int heads, int nblk) {
  const size_t per_pair = (size_t)nblk * nblk * 8;
  const size_t cap = (size_t)256 << 20;   // score workspace target: 256 MB
  size_t g = cap / per_pair;
  // launch sizes: score tiles^2 x 256 and selection nblk x 64 work-items per pair
  const size_t tiles = (size_t)(nblk + kScoreTile - 1) / kScoreTile;
  g = std::min(g, (size_t)kMaxLaunchThreads / (tiles * tiles * kRouteThreads));
  g = std::min(g, (size_t)kMaxLaunchThreads / ((size_t)nblk * 64));
  if (g < 1) g = 1;
  const size_t pairs = (size_t)batch * heads;
  return (int)(g < pairs ? g : pairs);
}

size_t route_workspace_bytes(int batch, int heads, int nblk) {
  return (size_t)route_pairs_per_chunk(batch, heads, nblk) * nblk * nblk * 8;
}

hipError_t launch_route(const uint16_t* qmean, const uint16_t* kmean, const int32_t* vbs,
                        int32_t* out, int batch, int nblk, int heads, int topk, double* scores,
                        hipStream_t stream) {
  const int pairs = batch * heads;
  const int chunk = route_pairs_per_chunk(batch, heads, nblk);
  const int tiles = (nblk + kScoreTile - 1) / kScoreTile;
  for (int bh0 = 0; bh0 < pairs; bh0 += chunk) {
    const int g = pairs - bh0 < chunk ? pairs - bh0 : chunk;
    if (!launch_fits((int64_t)g * tiles * tiles, kRouteThreads) || !launch_fits((int64_t)g * nblk, 64))
      return hipErrorInvalidValue;
    hipLaunchKernelGGL(route_score_kernel, dim3((unsigned)(g * tiles * tiles)), dim3(kRouteThreads), 0,
                       stream, qmean, kmean, vbs, scores, bh0, nblk, heads, tiles);
    const int rows = g * nblk;
    const dim3 sgrid((unsigned)((rows + kRouteWaves - 1) / kRouteWaves));
    hipLaunchKernelGGL(route_select_kernel, sgrid, dim3(kRouteThreads), 0, stream, scores, out, bh0,
                       rows, nblk, topk);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace vsa
