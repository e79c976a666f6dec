// Fine block-sparse attention forward of Video Sparse Attention on gfx950.
//
// Operation (Wan2.2 production-values dataset card, "Operator contract"): for
// each (batch, head, 64-row query cube) softmax attention over the valid rows of
// the KV cubes its index row selects, vbs[c] being the number of valid rows of
// cube c.  The proxy variant (TensorRT-Edge-LLM "Video Sparse Attention Runner"
// class description; FlashInfer proxy-compensation description on the
// TensorRT-LLM VisualGen VSA PR page) adds, for every unselected video block,
// one key (the block's mean key) whose probability is weighted by the block's
// valid-row count and whose value is the block's value total.
//
// Work decomposition: one workgroup of two wave64s per (batch, head, query
// block); wave w owns query rows 32w..32w+31.  For each selected KV tile:
//
//   S^T (64 keys x 32 queries) = K . Q^T   bf16 MFMA 32x32x16, fp32 accumulate
//   online softmax in exp2, fp32, one query per lane column
//   O^T (128 d x 32 queries) += V^T . P^T  fp16 MFMA 32x32x16 (bf16 for tiles
//                                          whose values do not fit fp16)
//
// Computing S transposed puts one query in each lane column: the row max and
// row sum are in-lane reductions plus a single exchange with the lane 32 apart
// (v_permlane32_swap), and the probabilities are already in the B-operand
// layout of the PV MFMA, so they never leave registers.
//
// K tiles are copied straight from the BSHD input into LDS with
// global_load_lds_dwordx4 (no VGPR staging); each 256-byte K row is stored with
// its sixteen 16-byte chunks XOR-swizzled by the row index, so the MFMA A-operand
// reads (32 rows, one chunk each) spread over all LDS banks.  V tiles are read
// from the packed key-major copy written by pack_vt_kernel, which already has
// the LDS layout, so their copy is linear.  Tiles whose vbs is <= 32 load and
// multiply only their first 32 keys.
#include "vsa_internal.h"

#include <math.h>

namespace vsa {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(2))) short s16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;

#define LDS_AS __attribute__((address_space(3)))

constexpr int kThreads = 128;
// Between two rescales the running maximum may lag the true one by up to this
// many log2 units, so probabilities stay below 2^8 (exact in fp16's range) while
// most tiles skip the accumulator rescale.
constexpr float kRescaleSlack = 8.0f;

// Tile-table entry: block/tile id (bits 0-19), valid rows (20-26), bf16 V (27),
// proxy tile (28).
constexpr int kEntNvShift = 20;
constexpr int kEntBf16 = 1 << 27;
constexpr int kEntProxy = 1 << 28;

__device__ inline int ent_id(int e) { return e & 0xFFFFF; }
__device__ inline int ent_nv(int e) { return (e >> kEntNvShift) & 127; }

// s_waitcnt vmcnt(n) leaving the other counters alone (gfx9 encoding).
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N < 64, "vmcnt field is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier that does not drain outstanding global->LDS copies (a
// __syncthreads() release fence would wait for every vector memory operation).
__device__ inline void wg_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// One global->LDS copy instruction (global_load_lds_dwordx4): every lane
// fetches 16 bytes from base + voff and the hardware writes lane l's bytes to
// LDS address lds + 16 l.  base and lds are wave-uniform.  The instruction is
// issued through inline assembly so that the compiler does not treat later LDS
// reads as possibly aliasing it (it would then drain every copy in flight
// before each read); completion is tracked explicitly with wait_vmcnt.
__device__ inline void dma16(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(base), "s"(lds)
               : "memory");
}

__device__ inline uint32_t lds_addr(const unsigned char* p) {
  return (uint32_t)(uintptr_t)(LDS_AS const unsigned char*)p;
}

// Returns x unchanged but hides its origin from the optimiser, so values
// derived from it are recomputed where they are used instead of being hoisted
// out of the tile loop (where they would occupy registers for its whole length).
__device__ inline uint32_t opaque_v(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}
__device__ inline uint32_t opaque_s(uint32_t x) {
  asm volatile("" : "+s"(x));
  return x;
}

__device__ inline float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline unsigned bf16_rne_bits(float f) {
  const unsigned u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Probabilities p0, p1 (fp32, >= 0) -> packed fp16 pair (round toward zero);
// the row sum gets exactly the values the MFMA will multiply.
__device__ inline unsigned pack_f16(float p0, float p1, float& lsum) {
  const f16x2 h = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(p0, p1));
  lsum = __builtin_amdgcn_fdot2(h, (f16x2){(_Float16)1.0f, (_Float16)1.0f}, lsum, false);
  return __builtin_bit_cast(unsigned, h);
}
// Same for bf16 tiles (round to nearest even).
__device__ inline unsigned pack_bf16(float p0, float p1, float& lsum) {
  const unsigned a = bf16_rne_bits(p0), b = bf16_rne_bits(p1);
  lsum += __uint_as_float(a << 16) + __uint_as_float(b << 16);
  return a | (b << 16);
}

struct Smem {
  unsigned char* k;     // 16 KB K tile
  unsigned char* v;     // 16 KB packed V tile
  int* tab;             // tile table
  int* cnt;             // counters
  int* key;             // sort keys
  float* off;           // proxy logit offsets (log2 weight or -inf)
  float* wt;            // proxy denominator weights (valid rows, 0 = no key)
  unsigned* bits;       // proxy selected-block bitmask
};

// Issue the global->LDS copies of one tile's K rows: N instructions of four
// rows each starting at row r0 (full tiles: wave w copies rows 32w..32w+31 with
// N = 8; half tiles: rows 16w..16w+15 with N = 4).  Lane l brings row
// r0 + 4i + l/16, physical chunk l%16, which holds logical chunk
// (l%16) ^ (row%16) = (l%16) ^ (l/16) ^ ((r0 + 4i) % 16).  The row part of the
// address is folded into the wave-uniform base; the lane part is
// klane ^ (((r0 + 4i) % 16) << 4) with klane = (l/16) * row_bytes +
// (((l%16) ^ (l/16)) << 4).  Rows past rmax (proxy tiles beyond the last video
// block) re-read row rmax.
template <int N, bool kMayClamp>
__device__ inline void issue_k(const uint16_t* kbase, uint32_t row_bytes, int rmax, int r0,
                               uint32_t klane, int lane, unsigned char* sk) {
  const char* kb = (const char*)kbase;
  const uint32_t l0 = opaque_s(lds_addr(sk));
  if (!kMayClamp || r0 + 4 * N - 1 <= rmax) {
    const uint32_t kl = opaque_v(klane);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int rb = r0 + 4 * i;
      dma16(kb + (size_t)rb * row_bytes, kl ^ (uint32_t)((rb & 15) << 4), l0 + rb * 256);
    }
  } else {
    const int pcx = (lane & 15) ^ (lane >> 4);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int rb = r0 + 4 * i;
      const int row = min(rb + (lane >> 4), rmax);
      const uint32_t off = (uint32_t)row * row_bytes + (uint32_t)((pcx ^ (rb & 15)) << 4);
      dma16(kb, off, l0 + rb * 256);
    }
  }
}

// Issue the linear copy of N KB of one packed V tile starting at byte base;
// vlane = 16 * lane.
template <int N>
__device__ inline void issue_v(const uint8_t* vtile, int base, uint32_t vlane, unsigned char* sv) {
  const uint32_t l0 = opaque_s(lds_addr(sv));
  const uint32_t vl = opaque_v(vlane);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int off = base + 1024 * i;
    dma16(vtile + off, vl, l0 + off);
  }
}

constexpr int kModeFull = 0;     // every key of the loaded halves is valid
constexpr int kModePartial = 1;  // keys >= nv are padding
constexpr int kModeProxy = 2;    // per-key log2 weights (-inf = no key)

// S^T (NKB x 32 keys, 32 queries) = K . Q^T.  Register i of s[kb] in lane
// (ln, hh) is key 32kb + 8(i/4) + 4hh + (i%4) against query ln.
template <int NKB>
__device__ inline void s_tile(const unsigned char* sk, const bf16x8 (&qop)[8], int ln, int hh,
                              f32x16 (&s)[2]) {
  const int sw = ln & 15;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
#pragma unroll
  for (int st = 0; st < 8; ++st) {
    const int co = ((2 * st + hh) ^ sw) << 4;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const bf16x8 a = *(const bf16x8*)(sk + (kb * 32 + ln) * 256 + co);
      s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qop[st], s[kb], 0, 0, 0);
    }
  }
}

// Running-max update for one tile: the tile's largest logit (scaled, log2
// units), and a rescale of O and the row sum when it exceeds the running max
// by more than kRescaleSlack.  Returns false when the tile has no live key.
template <int NKB>
__device__ inline bool tile_max(const f32x16 (&s)[2], int mode, int nv, const float* offs,
                                float c, int hh, float& mc, float& lsum, f32x16& o0, f32x16& o1,
                                f32x16& o2, f32x16& o3) {
  float t = -INFINITY;
  if (mode == kModeProxy) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 32 * kb + 8 * (i >> 2) + 4 * hh + (i & 3);
        t = fmaxf(t, fmaf(s[kb][i], c, offs[key]));
      }
    t = pair_max(t);
    if (__ballot(t > -INFINITY) == 0ull) return false;
  } else if (mode == kModePartial) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = 32 * kb + 8 * (i >> 2) + 4 * hh + (i & 3);
        t = fmaxf(t, key < nv ? s[kb][i] : -INFINITY);
      }
    t = pair_max(t) * c;
  } else {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) t = fmaxf(t, s[kb][i]);
    t = pair_max(t) * c;
  }
  const bool trig = t > mc + kRescaleSlack;
  if (__ballot(trig) != 0ull) {
    const float mnew = trig ? t : mc;
    const float alpha = __builtin_amdgcn_exp2f(mc - mnew);
    mc = mnew;
    lsum *= alpha;
    o0 *= alpha;
    o1 *= alpha;
    o2 *= alpha;
    o3 *= alpha;
  }
  return true;
}

// Probabilities of one 32-key half (register i = key 32kb + 8(i/4) + 4hh + i%4)
// packed straight into the PV B operand; the row sum takes exactly the rounded
// values the MFMA multiplies.  A proxy key stands for a whole block: its value
// operand is the block's value total, so the numerator takes its probability
// as is and only the denominator multiplies it by the block's valid-row count.
__device__ inline void half_probs(const f32x16& sk, int kb, int mode, int nv, const float* offs,
                                  const float* wts, bool bf16, float c, float nmc, int hh,
                                  float& lsum, unsigned (&pk)[8]) {
  auto emit = [&](auto prob) {
    if (bf16) {
#pragma unroll
      for (int i = 0; i < 16; i += 2) pk[i / 2] = pack_bf16(prob(i), prob(i + 1), lsum);
    } else {
#pragma unroll
      for (int i = 0; i < 16; i += 2) pk[i / 2] = pack_f16(prob(i), prob(i + 1), lsum);
    }
  };
  if (mode == kModeProxy) {
    auto keyw = [&](int i) { return wts[32 * kb + 8 * (i >> 2) + 4 * hh + (i & 3)]; };
    auto prob = [&](int i) {
      const float e = __builtin_amdgcn_exp2f(fmaf(sk[i], c, nmc));
      return keyw(i) > 0.0f ? e : 0.0f;
    };
    if (bf16) {
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const unsigned a = bf16_rne_bits(prob(i)), b = bf16_rne_bits(prob(i + 1));
        lsum = fmaf(__uint_as_float(a << 16), keyw(i), lsum);
        lsum = fmaf(__uint_as_float(b << 16), keyw(i + 1), lsum);
        pk[i / 2] = a | (b << 16);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const f16x2 h = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(prob(i), prob(i + 1)));
        const f16x2 wv = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(keyw(i), keyw(i + 1)));
        lsum = __builtin_amdgcn_fdot2(h, wv, lsum, false);   // weights <= 64: exact in fp16
        pk[i / 2] = __builtin_bit_cast(unsigned, h);
      }
    }
  } else if (mode == kModePartial) {
    emit([&](int i) {
      const int key = 32 * kb + 8 * (i >> 2) + 4 * hh + (i & 3);
      const float e = __builtin_amdgcn_exp2f(fmaf(sk[i], c, nmc));
      return key < nv ? e : 0.0f;
    });
  } else {
    emit([&](int i) { return __builtin_amdgcn_exp2f(fmaf(sk[i], c, nmc)); });
  }
}

// O^T (128 d x 32 queries) += V^T . P^T for one 32-key half kb: 16-key steps
// ks = 2kb, 2kb+1 with B operand pk[4(ks%2)..+3] (keys 16ks + 8(j/4) + 4hh + j%4);
// the A operand is row d = 32db + ln of the packed V tile, chunk 2(ks%2) + hh.
__device__ inline void pv_half(const unsigned char* sv, int kb, const unsigned (&pk)[8], bool bf16,
                               int ln, int hh, f32x16& o0, f32x16& o1, f32x16& o2, f32x16& o3) {
  const int sw = ((ln >> 1) ^ (ln >> 3)) & 3;
  if (bf16) {
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      const unsigned char* vb = sv + kb * 8192 + ln * 64 + (((k2 * 2 + hh) ^ sw) << 4);
      const bf16x8 bb = __builtin_bit_cast(bf16x8, (u32x4){pk[4 * k2], pk[4 * k2 + 1], pk[4 * k2 + 2], pk[4 * k2 + 3]});
      o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(vb + 0 * 2048), bb, o0, 0, 0, 0);
      o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(vb + 1 * 2048), bb, o1, 0, 0, 0);
      o2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(vb + 2 * 2048), bb, o2, 0, 0, 0);
      o3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(vb + 3 * 2048), bb, o3, 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      const unsigned char* vb = sv + kb * 8192 + ln * 64 + (((k2 * 2 + hh) ^ sw) << 4);
      const f16x8 bb = __builtin_bit_cast(f16x8, (u32x4){pk[4 * k2], pk[4 * k2 + 1], pk[4 * k2 + 2], pk[4 * k2 + 3]});
      o0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(*(const f16x8*)(vb + 0 * 2048), bb, o0, 0, 0, 0);
      o1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(*(const f16x8*)(vb + 1 * 2048), bb, o1, 0, 0, 0);
      o2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(*(const f16x8*)(vb + 2 * 2048), bb, o2, 0, 0, 0);
      o3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(*(const f16x8*)(vb + 3 * 2048), bb, o3, 0, 0, 0);
    }
  }
}

template <bool kProxy>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void attn_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(1024))) unsigned char sK[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char sV[kTileBytes];
  extern __shared__ int sDyn[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform)
  const int hh = lane >> 5;        // lane half
  const int ln = lane & 31;        // lane column (query / key / d)

  // XCD-aware item order: consecutive workgroup ids go round-robin to the 8
  // XCDs, so XCD x gets a contiguous run of items (whole heads) and its L2
  // serves one head's K/V at a time.
  const int item = (int)(blockIdx.x & 7) * p.items_per_xcd + (int)(blockIdx.x >> 3);
  if (item >= p.n_items) return;
  const int qb = item % p.nblk;
  const int bh = item / p.nblk;
  const int h = bh % p.heads;
  const int b = bh / p.heads;
  const int vq = min(max(p.vbs[qb], 0), kBlock);
  const int64_t row_stride = (int64_t)p.heads * kHeadDim;
  const uint32_t row_bytes = (uint32_t)(row_stride * 2);
  const uint32_t klane = (uint32_t)(lane >> 4) * row_bytes + (uint32_t)((((lane & 15) ^ (lane >> 4))) << 4);
  const uint32_t vlane = (uint32_t)lane * 16u;
  uint16_t* out_rows = p.out + (((int64_t)b * p.seq + (int64_t)qb * kBlock) * p.heads + h) * kHeadDim;

  if (vq == 0) {   // no valid query row: the whole block is padding
    for (int i = tid; i < kBlock * 16; i += kThreads) {
      const int r = i >> 4, c = i & 15;
      *(u32x4*)(out_rows + (int64_t)r * row_stride + c * 8) = (u32x4){0u, 0u, 0u, 0u};
    }
    return;
  }

  // ---------------- tile table ------------------------------------------
  Smem sm;
  sm.k = sK;
  sm.v = sV;
  sm.tab = sDyn;
  sm.cnt = sm.tab + p.table_cap;
  sm.key = sm.cnt + 4;
  const int key_cap = kProxy ? (p.nprefix + p.idx_width) : p.idx_width;
  sm.off = (float*)(sm.key + ((key_cap + 3) & ~3));
  sm.wt = sm.off + (kProxy ? p.nproxy * kBlock : 0);
  sm.bits = (unsigned*)(sm.wt + (kProxy ? p.nproxy * kBlock : 0));

  const int64_t bh_tiles = (int64_t)bh * p.nblk;
  const bool prefix_item = kProxy && qb < p.nprefix;
  int nexact;
  if (prefix_item) {
    // every block with valid rows, in order (wave 0 compacts with ballots)
    if (w == 0) {
      int base = 0;
      for (int c0 = 0; c0 < p.nblk; c0 += 64) {
        const int c = c0 + lane;
        const int nv = c < p.nblk ? min(max(p.vbs[c], 0), kBlock) : 0;
        const unsigned long long m = __ballot(nv > 0);
        if (nv > 0) {
          const int pos = base + __popcll(m & ((1ull << lane) - 1ull));
          sm.tab[pos] = c | (nv << kEntNvShift) | (p.vt_flags[bh_tiles + c] ? kEntBf16 : 0);
        }
        base += __popcll(m);
      }
      if (lane == 0) sm.cnt[0] = base;
    }
    wg_barrier();
    nexact = sm.cnt[0];
  } else {
    // selected blocks, sorted ascending (the result does not depend on the
    // order; a fixed order makes it reproducible bit for bit)
    const int32_t* row = p.idx + (int64_t)((int64_t)bh * (kProxy ? p.nvideo : p.nblk) +
                                           (qb - (kProxy ? p.nprefix : 0))) * p.idx_width;
    for (int t = tid; t < key_cap; t += kThreads) {
      int blk;
      if (kProxy) {
        if (t < p.nprefix) blk = t;
        else {
          const int s = row[t - p.nprefix];
          blk = (s >= 0 && s < p.nvideo) ? p.nprefix + s : -1;
        }
      } else {
        blk = row[t];
      }
      const int nv = (blk >= 0 && blk < p.nblk) ? min(max(p.vbs[blk], 0), kBlock) : 0;
      sm.key[t] = nv > 0 ? blk : 0x7FFFFFFF;
    }
    if (tid == 0) sm.cnt[0] = 0;
    wg_barrier();
    for (int t = tid; t < key_cap; t += kThreads) {
      const int key = sm.key[t];
      if (key != 0x7FFFFFFF) {
        int rank = 0;
        for (int u = 0; u < key_cap; ++u) {
          const int ku = sm.key[u];
          rank += (ku < key) | ((ku == key) & (u < t));
        }
        const int nv = min(max(p.vbs[key], 0), kBlock);
        sm.tab[rank] = key | (nv << kEntNvShift) | (p.vt_flags[bh_tiles + key] ? kEntBf16 : 0);
        atomicAdd(&sm.cnt[0], 1);
      }
    }
    wg_barrier();
    nexact = sm.cnt[0];
  }
  // Phase-aligned sweep: the exact tiles are processed in ascending block order
  // starting at block `start` and wrapping around.  Workgroups run on an XCD in
  // dispatch-slot order and take about the same time, so giving slot n the start
  // n * nblk / phase_slots (phase_slots = workgroups resident per XCD) keeps all
  // resident workgroups of a head near the same blocks at the same moment: the
  // XCD's L2 then serves a narrow window of that head's K/V instead of all of it.
  // The order does not change the result beyond rounding.
  int rot = 0;
  {
    const int start = (int)(((int64_t)(blockIdx.x >> 3) * p.nblk / p.phase_slots) % p.nblk);
    for (int c0 = 0; c0 < nexact; c0 += 64) {
      const int t = c0 + lane;
      const bool before = t < nexact && ent_id(sm.tab[t]) < start;
      rot += __popcll(__ballot(before));
    }
  }
  int ntiles = nexact;
  if (kProxy && !prefix_item) {
    // proxy tiles; per proxy key (one per video block) the denominator weight
    // vbs (0 for selected, empty or out-of-range blocks) and its log2, which
    // enters the running maximum so that the weighted terms cannot overflow
    const int nbits = (p.nproxy * kBlock) / 32;
    for (int t = tid; t < nbits; t += kThreads) sm.bits[t] = 0u;
    for (int t = tid; t < p.nproxy; t += kThreads) {
      const int rows = min(p.nvideo - kBlock * t, kBlock);
      sm.tab[nexact + t] = t | (rows << kEntNvShift) | kEntProxy |
                           (p.pt_flags[(int64_t)bh * p.nproxy + t] ? kEntBf16 : 0);
    }
    wg_barrier();
    const int32_t* row = p.idx + ((int64_t)bh * p.nvideo + (qb - p.nprefix)) * p.idx_width;
    for (int t = tid; t < p.idx_width; t += kThreads) {
      const int s = row[t];
      if (s >= 0 && s < p.nvideo) atomicOr(&sm.bits[s >> 5], 1u << (s & 31));
    }
    wg_barrier();
    for (int vblk = tid; vblk < p.nproxy * kBlock; vblk += kThreads) {
      float o = -INFINITY, wv = 0.0f;
      if (vblk < p.nvideo) {
        const int nv = min(max(p.vbs[p.nprefix + vblk], 0), kBlock);
        if (nv > 0 && !((sm.bits[vblk >> 5] >> (vblk & 31)) & 1u)) {
          o = __log2f((float)nv);
          wv = (float)nv;
        }
      }
      sm.off[vblk] = o;
      sm.wt[vblk] = wv;
    }
    ntiles += p.nproxy;
    wg_barrier();
  }

  // ---------------- per-wave state ---------------------------------------
  const bool active = 32 * w < vq;      // wave has at least one valid query row
  const int qrow = 32 * w + ln;         // query row inside the block
  bf16x8 qop[8];
  {
    const uint16_t* qp = p.q + (((int64_t)b * p.seq + (int64_t)qb * kBlock + qrow) * p.heads + h) *
                                   kHeadDim + 8 * hh;
    const bool qvalid = qrow < vq;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (qvalid) x = *(const u32x4*)(qp + 16 * s);
      qop[s] = __builtin_bit_cast(bf16x8, x);
    }
  }
  // Let the Q loads finish here, so that inside the loop the only outstanding
  // vector-memory operations are the tile copies counted by wait_vmcnt_rt.
  wait_vmcnt<0>();
  f32x16 o0 = {}, o1 = {}, o2 = {}, o3 = {};
  float mc = -INFINITY;   // running max of the scaled logits (log2 units)
  float lsum = 0.0f;      // this lane's share of the softmax denominator
  const float c = p.c;

  auto k_src = [&](int e, int& rmax) -> const uint16_t* {
    if (kProxy && (e & kEntProxy)) {
      const int t = ent_id(e);
      rmax = min(kBlock - 1, p.nvideo - 1 - kBlock * t);
      return p.kmean + (((int64_t)b * p.nblk + p.nprefix + (int64_t)kBlock * t) * p.heads + h) *
                           kHeadDim;
    }
    rmax = kBlock - 1;
    return p.k + (((int64_t)b * p.seq + (int64_t)ent_id(e) * kBlock) * p.heads + h) * kHeadDim;
  };
  auto v_src = [&](int e) -> const uint8_t* {
    if (kProxy && (e & kEntProxy))
      return p.pt + ((int64_t)bh * p.nproxy + ent_id(e)) * kTileBytes;
    return p.vt + (bh_tiles + ent_id(e)) * kTileBytes;
  };
  auto issue_tile_k = [&](int e) {
    int rmax;
    const uint16_t* ks = k_src(e, rmax);
    if (ent_nv(e) <= 32) issue_k<4, kProxy>(ks, row_bytes, rmax, 16 * w, klane, lane, sK);
    else issue_k<8, kProxy>(ks, row_bytes, rmax, 32 * w, klane, lane, sK);
  };
  auto issue_tile_v = [&](int e) {
    if (ent_nv(e) <= 32) issue_v<4>(v_src(e), 4096 * w, vlane, sV);
    else issue_v<8>(v_src(e), 8192 * w, vlane, sV);
  };

  auto tab_at = [&](int j) -> int {
    int jj = j;
    if (j < nexact) {
      jj = j + rot;
      if (jj >= nexact) jj -= nexact;
    }
    return __builtin_amdgcn_readfirstlane(sm.tab[jj]);
  };

  if (ntiles > 0) {
    const int e0 = tab_at(0);
    issue_tile_k(e0);
    issue_tile_v(e0);
  }

  for (int j = 0; j < ntiles; ++j) {
    const int e = tab_at(j);
    const int en = (j + 1 < ntiles) ? tab_at(j + 1) : 0;
    const int nv = ent_nv(e);
    const bool half = nv <= 32;
    const int mode = (kProxy && (e & kEntProxy)) ? kModeProxy : ((nv & 31) ? kModePartial : kModeFull);
    const bool is_bf16 = (e & kEntBf16) != 0;

    // K(j) has landed once only V(j)'s copies may still be in flight.
    if (half) wait_vmcnt<4>(); else wait_vmcnt<8>();
    wg_barrier();
    f32x16 s[2];
    if (active) {
      if (half) s_tile<1>(sK, qop, ln, hh, s);
      else s_tile<2>(sK, qop, ln, hh, s);
    }
    wg_barrier();   // both waves are done with sK
    if (j + 1 < ntiles) issue_tile_k(en);

    bool live = false;
    const float* offs = kProxy ? sm.off + kBlock * ent_id(e) : nullptr;
    const float* wts = kProxy ? sm.wt + kBlock * ent_id(e) : nullptr;
    if (active) {
      if (half) live = tile_max<1>(s, mode, nv, offs, c, hh, mc, lsum, o0, o1, o2, o3);
      else live = tile_max<2>(s, mode, nv, offs, c, hh, mc, lsum, o0, o1, o2, o3);
    }

    // V(j) has landed once only K(j+1)'s copies may still be in flight.
    if (j + 1 < ntiles) {
      if (ent_nv(en) <= 32) wait_vmcnt<4>(); else wait_vmcnt<8>();
    } else {
      wait_vmcnt<0>();
    }
    wg_barrier();
    if (live) {
      const float nmc = -mc;
      {
        unsigned pk[8];
        half_probs(s[0], 0, mode, nv, offs, wts, is_bf16, c, nmc, hh, lsum, pk);
        pv_half(sV, 0, pk, is_bf16, ln, hh, o0, o1, o2, o3);
      }
      if (!half) {
        unsigned pk[8];
        half_probs(s[1], 1, mode, nv, offs, wts, is_bf16, c, nmc, hh, lsum, pk);
        pv_half(sV, 1, pk, is_bf16, ln, hh, o0, o1, o2, o3);
      }
    }
    wg_barrier();   // both waves are done with sV
    if (j + 1 < ntiles) issue_tile_v(en);
  }

  // ---------------- epilogue ---------------------------------------------
  // o = O / l for valid rows; padding rows, empty rows and non-finite results
  // are written as 0.  Lane (ln, hh) holds query row 32w+ln and, in register
  // 4a+r of accumulator db, head-dim index 32db + 8a + 4hh + r.
  const float l_tot = pair_sum(lsum);
  const bool row_ok = active && qrow < vq && l_tot > 0.0f;
  const float inv = row_ok ? 1.0f / l_tot : 0.0f;
  uint16_t* orow = out_rows + (int64_t)qrow * row_stride + 4 * hh;
  auto store4 = [&](const f32x16& acc, int db) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      unsigned u[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float x = acc[4 * a + r] * inv;
        if (!row_ok || !isfinite(x)) x = 0.0f;
        u[r] = bf16_rne_bits(x);
      }
      *(u32x2*)(orow + 32 * db + 8 * a) = (u32x2){u[0] | (u[1] << 16), u[2] | (u[3] << 16)};
    }
  };
  store4(o0, 0);
  store4(o1, 1);
  store4(o2, 2);
  store4(o3, 3);
}

}  // namespace

hipError_t launch_attn(const AttnParams& p, bool proxy, hipStream_t stream) {
  if (p.n_items <= 0) return hipSuccess;
  const int key_cap = proxy ? (p.nprefix + p.idx_width) : p.idx_width;
  size_t dyn = (size_t)p.table_cap * 4 + 16 + (size_t)((key_cap + 3) & ~3) * 4;
  if (proxy) dyn += (size_t)p.nproxy * kBlock * 8 + (size_t)p.nproxy * 2 * 4;
  const unsigned grid = (unsigned)p.items_per_xcd * 8u;
  if (proxy)
    hipLaunchKernelGGL(attn_kernel<true>, dim3(grid), dim3(kThreads), dyn, stream, p);
  else
    hipLaunchKernelGGL(attn_kernel<false>, dim3(grid), dim3(kThreads), dyn, stream, p);
  return hipGetLastError();
}

}  // namespace vsa
