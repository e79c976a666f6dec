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
// One workgroup of 256 threads handles QB query blocks of one (batch, head).
// Scores: thread t streams KPT mean key rows (t, t + 256, ...) through
// registers and runs QB x KPT independent multiply-add chains; the QB mean
// query values of one d are read from LDS once (the same address in every
// lane) and feed KPT chains each, which keeps the LDS return path below the
// float64 FMA rate.  Selection, one wavefront per query block, no workgroup
// barriers:
//   1. radix select over order-preserving 64-bit codes of the scores, 8 bits
//      at a time from the top, until the bin holding the k-th largest score
//      has at most a few more entries than still needed; the bin's lower edge
//      is a bound T at or below the k-th largest score;
//   2. every block with a score at or above T is a candidate.  A block that
//      outranks a candidate is a candidate too, so a candidate's exact rank in
//      (score descending, index ascending) order is counted over the
//      candidates alone, kept in LDS in index order; it is written out when
//      the rank is below topk.  Every block of rank below topk is a
//      candidate, so each output slot is written once.  When the candidates
//      do not fit the list (massive ties, very large topk) ranks are counted
//      over the whole row instead.
#include "vsa_internal.h"

#include <math.h>

namespace vsa {
namespace {

constexpr int kRouteThreads = 256;
constexpr int kRouteWaves = kRouteThreads / 64;
constexpr int kHistBins = 256;
constexpr int kCandList = 256;         // per-wavefront candidate list (scores and block ids)
constexpr int kExtraCandidates = 32;   // stop refining the bound once this close
constexpr int kBufferWord3 = 0x00020000;   // buffer resource flags for raw (untyped) loads

typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

__device__ inline float bf16f(uint16_t b) { return __uint_as_float((unsigned)b << 16); }

// Buffer loads are calls the compiler keeps where they stand (a plain load's
// prefetch into a register ring gets folded back into a load at the point of
// use), and the hardware returns zeros past num_records.
__device__ inline u32x4 load_piece(__amdgpu_buffer_rsrc_t rsrc, unsigned voff, int piece) {
  return __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)(voff + 16u * piece), 0, 0);
}

// Adds 4 products (d = d0 .. d0 + 3, values w[half*2], w[half*2 + 1] of each
// key's piece) to each of the QB x KPT chains.
template <int QB, int KPT>
__device__ __attribute__((always_inline)) inline void score_quarter(double (&acc)[QB][KPT],
                                                                    const u32x4 (&w)[KPT], int half,
                                                                    const double* qi) {
  double qv[4 * QB];
#pragma unroll
  for (int t = 0; t < 4 * QB; ++t) qv[t] = qi[t];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
#pragma unroll
    for (int c = 0; c < KPT; ++c) {
      const unsigned word = w[c][2 * half + e / 2];
      const double kv = (double)bf16f((uint16_t)(word >> (16 * (e % 2))));
#pragma unroll
      for (int r = 0; r < QB; ++r) acc[r][c] = fma(qv[e * QB + r], kv, acc[r][c]);
    }
  }
}

template <int QB, int KPT>
__device__ __attribute__((always_inline)) inline void score_piece(double (&acc)[QB][KPT],
                                                                  const u32x4 (&w)[KPT],
                                                                  const double* qi) {
  score_quarter<QB, KPT>(acc, w, 0, qi);
  __builtin_amdgcn_sched_barrier(0);   // half a piece's query values live at a time
  score_quarter<QB, KPT>(acc, w, 1, qi + 4 * QB);
}

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

// Top-k of one row of scores by one wavefront.
__device__ __attribute__((always_inline)) inline void select_row(
    const double* __restrict__ row, int n, int topk, int* __restrict__ hist,
    double* __restrict__ cs, int* __restrict__ ci, int32_t* __restrict__ orow, int lane) {
  // eligible blocks (finite score) rank before every empty one
  int local = 0;
  for (int e = lane; e < n; e += 64) local += row[e] != -INFINITY;
  int eligible = wave_inclusive_sum(local, lane);
  eligible = __shfl(eligible, 63, 64);
  for (int t = eligible + lane; t < topk; t += 64) orow[t] = -1;
  int need = min(topk, eligible);
  if (need == 0) return;

  // 1. lower bound on the need-th largest code
  uint64_t prefix = 0, pmask = 0;
  for (int shift = 56; shift >= 0; shift -= 8) {
#pragma unroll
    for (int i = 0; i < kHistBins / 64; ++i) hist[lane * (kHistBins / 64) + i] = 0;
    wave_sync();
    for (int e = lane; e < n; e += 64) {
      const double s = row[e];
      const uint64_t c = order_code(s);
      if (s != -INFINITY && (c & pmask) == prefix) atomicAdd(&hist[(int)((c >> shift) & 0xFF)], 1);
    }
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

  // 2. candidates (code >= prefix) listed in index order
  int listed = 0;
  for (int e0 = 0; e0 < n; e0 += 64) {
    const int e = e0 + lane;
    double s = -INFINITY;
    bool is_cand = false;
    if (e < n) {
      s = row[e];
      is_cand = s != -INFINITY && order_code(s) >= prefix;
    }
    const uint64_t m = __ballot(is_cand);
    const int at = listed + lanes_below(m);
    if (is_cand && at < kCandList) {
      cs[at] = s;
      ci[at] = e;
    }
    listed += __popcll(m);
  }
  wave_sync();
  if (listed <= kCandList) {
    for (int c = lane; c < listed; c += 64) {
      const int rank = rank_in(cs, listed, cs[c], c);
      if (rank < topk) orow[rank] = ci[c];
    }
  } else {
    for (int e0 = 0; e0 < n; e0 += 64) {
      const int e = e0 + lane;
      if (e < n) {
        const double s = row[e];
        if (s != -INFINITY && order_code(s) >= prefix) {
          const int rank = rank_in(row, n, s, e);
          if (rank < topk) orow[rank] = e;
        }
      }
    }
  }
  wave_sync();   // the lists are refilled by this wavefront's next row
}

// LDS allows two workgroups per CU at most (two waves per SIMD), so the
// compiler may spend registers on loads in flight instead of occupancy.
template <int QB, int KPT>
__global__ __launch_bounds__(kRouteThreads) __attribute__((amdgpu_waves_per_eu(1, 2))) void route_kernel(
    const uint16_t* __restrict__ qmean, const uint16_t* kmean, const int32_t* __restrict__ vbs,
    int32_t* __restrict__ out, int nblk, int heads, int topk) {
  extern __shared__ double sRoute[];
  double* score = sRoute;                                     // [QB][nblk]
  double* qd = score + (size_t)QB * nblk;                     // [128][QB] mean query, d-major
  double* cs = qd + kHeadDim * QB;                            // [waves][kCandList]
  int* ci = (int*)(cs + kRouteWaves * kCandList);             // [waves][kCandList]
  int* hist = ci + kRouteWaves * kCandList;                   // [waves][256]
  const int groups = (nblk + QB - 1) / QB;
  const int g = blockIdx.x % groups;
  const int bh = blockIdx.x / groups;
  const int h = bh % heads;
  const int b = bh / heads;
  const int q0 = g * QB;
  const int nq = min(QB, nblk - q0);
  const int tid = threadIdx.x;

  for (int i = tid; i < QB * kHeadDim; i += kRouteThreads) {
    const int r = i / kHeadDim, d = i % kHeadDim;
    qd[d * QB + r] =
        r < nq ? (double)bf16f(qmean[(((int64_t)b * nblk + q0 + r) * heads + h) * kHeadDim + d]) : 0.0;
  }
  __syncthreads();

  // ---- scores -----------------------------------------------------------
  const int64_t row_stride = (int64_t)heads * kHeadDim * 2;              // bytes between key rows
  const unsigned voff = (unsigned)((int64_t)tid * row_stride);           // < 2^32 for heads <= 65536
  for (int j0 = 0; j0 < nblk; j0 += kRouteThreads * KPT) {
    __amdgpu_buffer_rsrc_t rsrc[KPT];
#pragma unroll
    for (int c = 0; c < KPT; ++c) {
      const int first = min(j0 + c * kRouteThreads, nblk);               // rows first .. first+rows-1
      const int rows = min(kRouteThreads, nblk - first);
      const int64_t span = rows > 0 ? (int64_t)(rows - 1) * row_stride + kHeadDim * 2 : 0;
      rsrc[c] = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(kmean + (((int64_t)b * nblk + first) * heads + h) * kHeadDim), (short)0,
          (int)(unsigned)min(span, (int64_t)0xFFFFFFFF), kBufferWord3);
    }
    double acc[QB][KPT];
#pragma unroll
    for (int r = 0; r < QB; ++r)
#pragma unroll
      for (int c = 0; c < KPT; ++c) acc[r][c] = 0.0;
    // 16-byte pieces of 8 values in a ring of two per key: each slot is used,
    // then refilled with the piece two ahead (rows past the end read zeros)
    u32x4 pa[KPT], pb[KPT];
#pragma unroll
    for (int c = 0; c < KPT; ++c) {
      pa[c] = load_piece(rsrc[c], voff, 0);
      pb[c] = load_piece(rsrc[c], voff, 1);
    }
#pragma unroll 1
    for (int i = 0; i < kHeadDim / 8; i += 2) {
      const int last = kHeadDim / 8 - 1;   // the final round refills in-row, unused
      score_piece<QB, KPT>(acc, pa, qd + 8 * i * QB);
#pragma unroll
      for (int c = 0; c < KPT; ++c) pa[c] = load_piece(rsrc[c], voff, min(i + 2, last));
      __builtin_amdgcn_sched_barrier(0);
      score_piece<QB, KPT>(acc, pb, qd + 8 * (i + 1) * QB);
#pragma unroll
      for (int c = 0; c < KPT; ++c) pb[c] = load_piece(rsrc[c], voff, min(i + 3, last));
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int c = 0; c < KPT; ++c) {
      const int j = j0 + c * kRouteThreads + tid;
      if (j < nblk) {
        const bool live = vbs[j] > 0;
#pragma unroll
        for (int r = 0; r < QB; ++r)
          if (r < nq) score[(size_t)r * nblk + j] = live ? acc[r][c] + 0.0 : -INFINITY;
      }
    }
  }
  __syncthreads();

  // ---- selection: one wavefront per query block ---------------------------
  const int wave = tid / 64, lane = tid % 64;
  for (int r = wave; r < nq; r += kRouteWaves)
    select_row(score + (size_t)r * nblk, nblk, topk, hist + wave * kHistBins,
               cs + wave * kCandList, ci + wave * kCandList,
               out + ((int64_t)bh * nblk + q0 + r) * topk, lane);
}

int pick_qb(int nblk) {
  // score rows of 8 bytes per block, at most 48 KB of them, at most 8 rows
  const int fit = (int)(49152 / ((size_t)nblk * 8));
  return fit >= 8 ? 8 : fit >= 4 ? 4 : fit >= 2 ? 2 : 1;
}

// key rows per thread: enough to cover the row in one pass, at most 4
int pick_kpt(int nblk) {
  const int k = (nblk + kRouteThreads - 1) / kRouteThreads;
  return k > 4 ? 4 : k;
}

}  // namespace

int route_blocks_per_wg(int nblk) { return pick_qb(nblk); }

size_t route_lds_bytes(int nblk) {
  const int qb = pick_qb(nblk);
  return (size_t)qb * nblk * 8 + (size_t)kHeadDim * qb * 8 +
         (size_t)kRouteWaves * (kCandList * 12 + kHistBins * 4);
}

template <int QB, int KPT>
static void launch_one(dim3 grid, size_t lds, hipStream_t stream, const uint16_t* qmean,
                       const uint16_t* kmean, const int32_t* vbs, int32_t* out, int nblk, int heads,
                       int topk) {
  hipLaunchKernelGGL((route_kernel<QB, KPT>), grid, dim3(kRouteThreads), lds, stream, qmean, kmean,
                     vbs, out, nblk, heads, topk);
}

hipError_t launch_route(const uint16_t* qmean, const uint16_t* kmean, const int32_t* vbs,
                        int32_t* out, int batch, int nblk, int heads, int topk,
                        hipStream_t stream) {
  const int qb = pick_qb(nblk);
  const int kpt = pick_kpt(nblk);
  const int groups = (nblk + qb - 1) / qb;
  const int64_t blocks = (int64_t)batch * heads * groups;
  if (blocks == 0) return hipSuccess;
  const size_t lds = route_lds_bytes(nblk);
  const dim3 grid((unsigned)blocks);
  // qb = 8 only for nblk <= 768 (kpt <= 3); smaller qb means nblk > 768 (kpt = 4)
  if (qb == 8) {
    if (kpt == 1) launch_one<8, 1>(grid, lds, stream, qmean, kmean, vbs, out, nblk, heads, topk);
    else if (kpt == 2) launch_one<8, 2>(grid, lds, stream, qmean, kmean, vbs, out, nblk, heads, topk);
    else launch_one<8, 3>(grid, lds, stream, qmean, kmean, vbs, out, nblk, heads, topk);
  } else if (qb == 4) {
    launch_one<4, 4>(grid, lds, stream, qmean, kmean, vbs, out, nblk, heads, topk);
  } else if (qb == 2) {
    launch_one<2, 4>(grid, lds, stream, qmean, kmean, vbs, out, nblk, heads, topk);
  } else {
    launch_one<1, 4>(grid, lds, stream, qmean, kmean, vbs, out, nblk, heads, topk);
  }
  return hipGetLastError();
}

}  // namespace vsa
