// Fine block-sparse attention forward of Video Sparse Attention on gfx950.
//
// Operation (Wan2.2 production-values dataset card, "Operator contract"): for
// each (batch, head, 64-row query cube) softmax attention over the valid rows of
// the KV cubes its index row selects, vbs[c] being the number of valid rows of
// cube c.  The proxy variant (TensorRT-Edge-LLM "Video Sparse Attention Runner"
// class description; FlashInfer proxy-compensation description on the
// TensorRT-LLM VisualGen VSA PR page) adds, for every unselected video block,
// one key (the block's mean key) whose value is the block's value total and
// whose probability counts vbs times in the softmax denominator.
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
//
// Tile order (it changes results only by rounding): the exact fp16 tiles of an
// item are swept in ascending block order from a start block, in nseg segments
// of the block range; inside a segment they go kind by kind (full, full with
// padding keys, half, half with padding keys), each kind through a straight-line
// specialisation of the tile step, so the accumulators never cross
// data-dependent control flow except the rescale.  Proxy and bf16 tiles follow.
// The start block is the average sweep position of the workgroups running on
// the same XCD (per-XCD progress counters that every workgroup advances by a
// segment's width as the segment begins), so the resident workgroups of a head
// move through its blocks together and the XCD's L2 holds a narrow window of
// that head's K/V tiles instead of all of them.  In deterministic mode the
// start depends only on the workgroup index, so the order, and with it the
// rounding, is reproducible.
#include "vsa_internal.h"

#include <math.h>

#include <algorithm>
#include <mutex>
#include <vector>

namespace vsa {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;

#define LDS_AS __attribute__((address_space(3)))

constexpr int kThreads = 128;
// Between two rescales the running maximum may lag the true one by up to this
// many log2 units, so probabilities stay below 2^8 (well inside fp16's range)
// while tiles whose maximum grew only a little skip the accumulator rescale.
constexpr float kRescaleSlack = 8.0f;

// Tile-table entry: block/tile id (bits 0-19), valid rows (20-26), bf16 V (27),
// proxy tile (28).
constexpr int kEntNvShift = 20;
constexpr int kEntBf16 = 1 << 27;
constexpr int kEntProxy = 1 << 28;
__device__ inline int ent_id(int e) { return e & 0xFFFFF; }
__device__ inline int ent_nv(int e) { return (e >> kEntNvShift) & 127; }
// Half tiles (exact fp16 tiles with vbs <= 32) load and multiply 32 keys only.
__device__ inline bool ent_half(int e) { return !(e & (kEntBf16 | kEntProxy)) && ent_nv(e) <= 32; }

// Tile kinds, processed in this order.
enum : int { kGFull = 0, kGFullPad, kGHalf, kGHalfPad, kGProxy, kGBf16, kGroups };
__device__ inline int ent_group(int e) {
  if (e & kEntBf16) return kGBf16;
  if (e & kEntProxy) return kGProxy;
  const int nv = ent_nv(e);
  if (nv == 64) return kGFull;
  if (nv > 32) return kGFullPad;
  if (nv == 32) return kGHalf;
  return kGHalfPad;
}

// Sweep progress per XCD, in blocks swept by all workgroups of all launches
// (wraps modulo 2^64).  Divided by the number of resident workgroups it is a
// virtual clock that advances at their average sweep rate; a starting workgroup
// begins its sweep at that position.  Only the tile order depends on it.  The
// counters of XCD x are touched only by workgroups running there, which share
// that XCD's L2, so workgroup-scope atomics and loads (served by the L2) are
// enough; device scope would send every access past the L2.
// Each XCD's progress is split over kSweepSub counters kSweepStride elements
// (4352 bytes) apart, so that they fall in different L2 channels: a workgroup
// adds to the counter of its dispatch slot and a reader sums all of them.  With
// one counter per XCD the atomics of its 128 resident workgroups serialise in
// one channel and hold up every other access mapped to it.
constexpr int kSweepSub = 4;
constexpr int kSweepStride = 4352 / 8;
__device__ unsigned long long g_sweep_progress[8 * kSweepSub * kSweepStride];

__device__ inline unsigned long long* sweep_counter(int xcd, int sub) {
  return &g_sweep_progress[(xcd * kSweepSub + sub) * kSweepStride];
}

// Softmax variants of a tile step.
enum : int { kModeFull = 0, kModePad = 1, kModeProxy = 2, kModeAny = 3 };

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
    // The row addresses advance from the first one; row_bytes and the LDS
    // start go through opaque values so that the per-copy products are not
    // hoisted out of the tile loop, where they would hold about 40 SGPRs and
    // be spilled to VGPR lanes and reloaded on every tile.
    const uint32_t rs = opaque_s(row_bytes);
    const char* kr = kb + (size_t)r0 * rs;
    const uint32_t m0 = opaque_s(l0 + (uint32_t)r0 * 256u);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      dma16(kr, kl ^ (uint32_t)(((r0 + 4 * i) & 15) << 4), m0 + 1024u * i);
      kr += 4 * rs;
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
  const uint32_t ob = opaque_s((uint32_t)base);   // not hoisted, as in issue_k
  const uint32_t m0 = opaque_s(lds_addr(sv) + ob);
  const uint8_t* vb = vtile + ob;
  const uint32_t vl = opaque_v(vlane);
#pragma unroll
  for (int i = 0; i < N; ++i) dma16(vb + 1024 * i, vl, m0 + 1024u * i);
}

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
  // operand reads run half the chain ahead of the MFMAs
  constexpr int kReads = 8 * NKB, kAhead = kReads / 2;
  __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
  for (int i = 0; i < kReads - kAhead; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, kAhead, 0);
}

__device__ inline int key_of(int kb, int i, int hh) { return 32 * kb + 8 * (i >> 2) + 4 * hh + (i & 3); }

// Per-wave running state of one item.
struct State {
  f32x16 o0, o1, o2, o3;   // O^T accumulators, d blocks 0..3
  float mc;                // running max of the scaled logits (log2 units)
  float lsum;              // this lane's share of the softmax denominator
};

// Proxy weight of key register i of half kb: the block's valid-row count
// (0 = no key), stored as bytes; keys 4j .. 4j+3 share one 32-bit word.
__device__ inline float proxy_weight(const uint8_t* wts, int kb, int i, int hh) {
  const unsigned wd = *(const unsigned*)(wts + key_of(kb, i & ~3, hh));
  return (float)((wd >> (8 * (i & 3))) & 0xFFu);
}

// Running-max update for one tile: the tile's largest logit (scaled, log2
// units), and a rescale of O and the row sum when it exceeds the running max
// by more than kRescaleSlack.
template <int NKB, int MODE>
__device__ inline void tile_max(const f32x16 (&s)[2], int nv, const uint8_t* wts, float c, int hh,
                                State& st) {
  float t = -INFINITY;
  if (MODE == kModeProxy) {
    // a proxy logit is offset by log2 of its weight (-inf for weight 0)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        t = fmaxf(t, fmaf(s[kb][i], c, __log2f(proxy_weight(wts, kb, i, hh))));
    t = pair_max(t);
  } else if (MODE == kModePad) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) t = fmaxf(t, key_of(kb, i, hh) < nv ? s[kb][i] : -INFINITY);
    t = pair_max(t) * c;
  } else {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) t = fmaxf(t, s[kb][i]);
    t = pair_max(t) * c;
  }
  const bool trig = t > st.mc + kRescaleSlack;
  if (__ballot(trig) != 0ull) {
    const float mnew = trig ? t : st.mc;
    const float alpha = __builtin_amdgcn_exp2f(st.mc - mnew);
    st.mc = mnew;
    st.lsum *= alpha;
    st.o0 *= alpha;
    st.o1 *= alpha;
    st.o2 *= alpha;
    st.o3 *= alpha;
  }
}

// Probabilities of one 32-key half (register i = key 32kb + 8(i/4) + 4hh + i%4)
// packed straight into the PV B operand; the row sum takes exactly the rounded
// values the MFMA multiplies.  A proxy key stands for a whole block: its value
// operand is the block's value total, so the numerator takes its probability
// as is and only the denominator multiplies it by the block's valid-row count.
template <int MODE, bool BF16>
__device__ inline void half_probs(const f32x16& sk, int kb, int nv, const uint8_t* wts, float c,
                                  float nmc, int hh, float& lsum, unsigned (&pk)[8]) {
  if (MODE == kModeProxy) {
    auto keyw = [&](int i) { return proxy_weight(wts, kb, i, hh); };
    auto prob = [&](int i) {
      const float e = __builtin_amdgcn_exp2f(fmaf(sk[i], c, nmc));
      return keyw(i) > 0.0f ? e : 0.0f;
    };
    if (BF16) {
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
    return;
  }
  auto prob = [&](int i) {
    const float e = __builtin_amdgcn_exp2f(fmaf(sk[i], c, nmc));
    return (MODE == kModePad && key_of(kb, i, hh) >= nv) ? 0.0f : e;
  };
  if (BF16) {
#pragma unroll
    for (int i = 0; i < 16; i += 2) pk[i / 2] = pack_bf16(prob(i), prob(i + 1), lsum);
  } else {
#pragma unroll
    for (int i = 0; i < 16; i += 2) pk[i / 2] = pack_f16(prob(i), prob(i + 1), lsum);
  }
}

// O^T (128 d x 32 queries) += V^T . P^T for one 32-key half kb: 16-key steps
// ks = 2kb, 2kb+1 with B operand pk[4(ks%2)..+3] (keys 16ks + 8(j/4) + 4hh + j%4);
// the A operand is row d = 32db + ln of the packed V tile, chunk 2(ks%2) + hh.
template <bool BF16>
__device__ inline void pv_half(const unsigned char* sv, int kb, const unsigned (&pk)[8], int ln,
                               int hh, State& st) {
  const int sw = ((ln >> 1) ^ (ln >> 3)) & 3;
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2) {
    const unsigned char* vb = sv + kb * 8192 + ln * 64 + (((k2 * 2 + hh) ^ sw) << 4);
    const u32x4 pb = {pk[4 * k2], pk[4 * k2 + 1], pk[4 * k2 + 2], pk[4 * k2 + 3]};
    if (BF16) {
      const bf16x8 bb = __builtin_bit_cast(bf16x8, pb);
      st.o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(vb + 0 * 2048), bb, st.o0, 0, 0, 0);
      st.o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(vb + 1 * 2048), bb, st.o1, 0, 0, 0);
      st.o2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(vb + 2 * 2048), bb, st.o2, 0, 0, 0);
      st.o3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(vb + 3 * 2048), bb, st.o3, 0, 0, 0);
    } else {
      const f16x8 bb = __builtin_bit_cast(f16x8, pb);
      st.o0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(*(const f16x8*)(vb + 0 * 2048), bb, st.o0, 0, 0, 0);
      st.o1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(*(const f16x8*)(vb + 1 * 2048), bb, st.o1, 0, 0, 0);
      st.o2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(*(const f16x8*)(vb + 2 * 2048), bb, st.o2, 0, 0, 0);
      st.o3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(*(const f16x8*)(vb + 3 * 2048), bb, st.o3, 0, 0, 0);
    }
  }
}

// Everything a tile step needs besides the running state.
struct Ctx {
  const AttnParams* p;
  unsigned char* sk;
  unsigned char* sv;
  const uint8_t* wt;       // proxy denominator weights (valid rows, 0 = no key), per video block
  int b, h;
  int64_t bh_tiles;        // (b * heads + h) * nblk
  int64_t bh_proxy;        // (b * heads + h) * nproxy
  uint32_t row_bytes, klane, vlane;
  int w, lane, ln, hh, tid, xcd;
  float c;
};

template <bool kProxy>
__device__ inline void issue_tile_k(const Ctx& x, int e) {
  const AttnParams& p = *x.p;
  const uint16_t* base;
  int rmax = kBlock - 1;
  if (kProxy && (e & kEntProxy)) {
    const int t = ent_id(e);
    rmax = min(kBlock - 1, p.nvideo - 1 - kBlock * t);
    base = p.kmean + (((int64_t)x.b * p.nblk + p.nprefix + (int64_t)kBlock * t) * p.heads + x.h) *
                         kHeadDim;
  } else {
    base = p.k + (((int64_t)x.b * p.seq + (int64_t)ent_id(e) * kBlock) * p.heads + x.h) * kHeadDim;
  }
  if (ent_half(e)) issue_k<4, kProxy>(base, x.row_bytes, rmax, 16 * x.w, x.klane, x.lane, x.sk);
  else issue_k<8, kProxy>(base, x.row_bytes, rmax, 32 * x.w, x.klane, x.lane, x.sk);
}

template <bool kProxy>
__device__ inline void issue_tile_v(const Ctx& x, int e) {
  const AttnParams& p = *x.p;
  const uint8_t* base = (kProxy && (e & kEntProxy))
                            ? p.pt + (x.bh_proxy + ent_id(e)) * kTileBytes
                            : p.vt + (x.bh_tiles + ent_id(e)) * kTileBytes;
  if (ent_half(e)) issue_v<4>(base, 4096 * x.w, x.vlane, x.sv);
  else issue_v<8>(base, 8192 * x.w, x.vlane, x.sv);
}

// One tile: wait for its K rows, S = K Q^T, release K and prefetch the next
// tile's K rows, running max, wait for its V, probabilities and O += P V,
// release V and prefetch the next tile's V.  NKB / MODE / BF16 are fixed per
// tile kind (MODE kModeAny: bf16 tiles, exact or proxy, decided per tile).
template <bool kProxy, bool kCompute, int NKB, int MODE, bool BF16>
__device__ inline void tile_step(const Ctx& x, const bf16x8 (&qop)[8], State& st, int e, int en,
                                 bool has_next) {
  // K(j) has landed once only V(j)'s copies (4 or 8 instructions per wave) are
  // still in flight.
  if (NKB == 1) wait_vmcnt<4>(); else wait_vmcnt<8>();
  wg_barrier();
  f32x16 s[2];
  if (kCompute) s_tile<NKB>(x.sk, qop, x.ln, x.hh, s);
  wg_barrier();   // both waves are done with sK
  if (has_next) issue_tile_k<kProxy>(x, en);

  const int nv = ent_nv(e);
  const bool px = kProxy && (MODE == kModeProxy || (MODE == kModeAny && (e & kEntProxy)));
  const uint8_t* wts = kProxy ? x.wt + kBlock * ent_id(e) : nullptr;
  // The running max, the probabilities and O += P V run at raised wave
  // priority: where both waves of a SIMD can issue, this phase goes first.
  __builtin_amdgcn_s_setprio(2);
  if (kCompute) {
    if (MODE == kModeAny) {
      if (px) tile_max<NKB, kModeProxy>(s, nv, wts, x.c, x.hh, st);
      else tile_max<NKB, kModePad>(s, nv, wts, x.c, x.hh, st);
    } else {
      tile_max<NKB, MODE>(s, nv, wts, x.c, x.hh, st);
    }
  }

  // V(j) has landed once only K(j+1)'s copies may still be in flight.
  if (has_next) {
    if (ent_half(en)) wait_vmcnt<4>(); else wait_vmcnt<8>();
  } else {
    wait_vmcnt<0>();
  }
  wg_barrier();
  if (kCompute) {
    const float nmc = -st.mc;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      unsigned pk[8];
      if (MODE == kModeAny) {
        if (px) half_probs<kModeProxy, BF16>(s[kb], kb, nv, wts, x.c, nmc, x.hh, st.lsum, pk);
        else half_probs<kModePad, BF16>(s[kb], kb, nv, wts, x.c, nmc, x.hh, st.lsum, pk);
      } else {
        half_probs<MODE, BF16>(s[kb], kb, nv, wts, x.c, nmc, x.hh, st.lsum, pk);
      }
      pv_half<BF16>(x.sv, kb, pk, x.ln, x.hh, st);
    }
  }
  __builtin_amdgcn_s_setprio(0);
  wg_barrier();   // both waves are done with sV
  if (has_next) issue_tile_v<kProxy>(x, en);
}

// Table cells: segment s, exact fp16 kind g -> 4 s + g; then proxy, bf16.
__device__ inline int cell_proxy(int nseg) { return 4 * nseg; }
__device__ inline int cell_bf16(int nseg) { return 4 * nseg + 1; }
__device__ inline int seg_first(int s, int nblk, int nseg) { return (s * nblk + nseg - 1) / nseg; }

// All tiles of one item in the order of `ord`; cbeg[c] is the first position of
// cell c (cbeg[4 nseg + 2] = number of tiles).  As each segment begins, the
// sweep progress counter of the XCD advances by the segment's width in blocks.
template <bool kProxy, bool kCompute>
__device__ inline void run_tiles(const Ctx& x, const bf16x8 (&qop)[8], State& st, const int* ord,
                                 const int* cbeg, int nseg, int n) {
  const int e0 = __builtin_amdgcn_readfirstlane(ord[0]);
  issue_tile_k<kProxy>(x, e0);
  issue_tile_v<kProxy>(x, e0);
  auto cell = [&](auto body, int c) {
    const int beg = __builtin_amdgcn_readfirstlane(cbeg[c]);
    const int end = __builtin_amdgcn_readfirstlane(cbeg[c + 1]);
    for (int j = beg; j < end; ++j) {
      const int e = __builtin_amdgcn_readfirstlane(ord[j]);
      const bool has_next = j + 1 < n;
      const int en = has_next ? __builtin_amdgcn_readfirstlane(ord[j + 1]) : 0;
      body(e, en, has_next);
    }
  };
  const int nblk = x.p->nblk;
  for (int s = 0; s < nseg; ++s) {
    if (x.tid == 0 && !x.p->deterministic)
      __hip_atomic_fetch_add(sweep_counter(x.xcd, (int)((blockIdx.x >> 3) & (kSweepSub - 1))),
                             (unsigned long long)(seg_first(s + 1, nblk, nseg) - seg_first(s, nblk, nseg)),
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    cell([&](int e, int en, bool hn) { tile_step<kProxy, kCompute, 2, kModeFull, false>(x, qop, st, e, en, hn); }, 4 * s + kGFull);
    cell([&](int e, int en, bool hn) { tile_step<kProxy, kCompute, 2, kModePad, false>(x, qop, st, e, en, hn); }, 4 * s + kGFullPad);
    cell([&](int e, int en, bool hn) { tile_step<kProxy, kCompute, 1, kModeFull, false>(x, qop, st, e, en, hn); }, 4 * s + kGHalf);
    cell([&](int e, int en, bool hn) { tile_step<kProxy, kCompute, 1, kModePad, false>(x, qop, st, e, en, hn); }, 4 * s + kGHalfPad);
  }
  if (kProxy)
    cell([&](int e, int en, bool hn) { tile_step<kProxy, kCompute, 2, kModeProxy, false>(x, qop, st, e, en, hn); }, cell_proxy(nseg));
  cell([&](int e, int en, bool hn) { tile_step<kProxy, kCompute, 2, kModeAny, true>(x, qop, st, e, en, hn); }, cell_bf16(nseg));
}

template <bool kProxy>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void attn_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(1024))) unsigned char sK[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char sV[kTileBytes];
  __shared__ int sCell[2 * (4 * kMaxSeg + 2) + 1];   // tiles per cell, then first position per cell
  __shared__ int sStart;
  extern __shared__ int sDyn[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform)
  const int hh = lane >> 5;        // lane half
  const int ln = lane & 31;        // lane column (query / key / d)

  // XCD-aware item order: consecutive workgroup ids go round-robin to the 8
  // XCDs, so XCD x gets a contiguous run of items (whole heads) and its L2
  // serves one head's K/V at a time.  A (batch, head) holds items_per_bh
  // items: its query blocks, or in proxy mode psplit sub-items per prefix
  // block (each over one range of pwidth key blocks) followed by the video
  // blocks.
  const int xcd = (int)(blockIdx.x & 7);
  const int item = xcd * p.items_per_xcd + (int)(blockIdx.x >> 3);
  if (item >= p.n_items) return;
  const int bh = kProxy ? item / p.items_per_bh : item / p.nblk;
  const int ir = kProxy ? item - bh * p.items_per_bh : item % p.nblk;
  int qb = ir, split = 0;
  if (kProxy) {
    const int nsub = p.nprefix * p.psplit;
    if (ir < nsub) {
      qb = ir / p.psplit;
      split = ir - qb * p.psplit;
    } else {
      qb = p.nprefix + (ir - nsub);
    }
  }
  const int h = bh % p.heads;
  const int b = bh / p.heads;
  const int vq = min(max(p.vbs[qb], 0), kBlock);
  const int64_t row_stride = (int64_t)p.heads * kHeadDim;
  uint16_t* out_rows = p.out + (((int64_t)b * p.seq + (int64_t)qb * kBlock) * p.heads + h) * kHeadDim;

  if (vq == 0) {   // no valid query row: the whole block is padding
    for (int i = tid; i < kBlock * 16; i += kThreads) {
      const int r = i >> 4, c = i & 15;
      *(u32x4*)(out_rows + (int64_t)r * row_stride + c * 8) = (u32x4){0u, 0u, 0u, 0u};
    }
    if (p.lse != nullptr && tid < kBlock) p.lse[(int64_t)bh * p.seq + (int64_t)qb * kBlock + tid] = -INFINITY;
    return;
  }

  // ---------------- tile table ------------------------------------------
  // Candidates: plain items -> the index row; proxy prefix items -> every
  // block; proxy video items -> prefix blocks, the index row, then the proxy
  // tiles.  Each valid candidate becomes an entry; entries are sorted by
  // (cell, block position in the sweep).
  const bool prefix_item = kProxy && qb < p.nprefix;
  const bool video_item = kProxy && !prefix_item;
  // Dynamic LDS: the tile table (processing order, then sort keys) of `cap`
  // entries; for proxy video items the per-block weights follow a table sized
  // for video items, and a prefix item's longer table overlays them (prefix
  // items take no weights).
  const int vcap = kProxy ? p.nprefix + (p.sel_format == 0 ? p.idx_width : p.nvideo) + p.nproxy : 0;
  const int cap = video_item ? vcap : p.table_cap;
  int* ord = sDyn;                       // [cap] entries, processing order
  int* key = ord + cap;                  // [cap] sort keys
  uint8_t* wt = (uint8_t*)(sDyn + 2 * vcap);              // [nproxy * 64] weight (valid rows)
  unsigned* bits = (unsigned*)(wt + p.nproxy * kBlock);   // [nproxy * 2] selected video blocks
  const int64_t bh_tiles = (int64_t)bh * p.nblk;
  // The index row: plain items and padded proxy rows read it in place; a BSR
  // row is a slice of the index list; a bitmask row is read through per-word
  // counts of its set bits (below).
  const int32_t* row = p.idx + (kProxy ? ((int64_t)bh * p.nvideo + (qb - p.nprefix)) * p.idx_width
                                       : (int64_t)item * p.idx_width);
  int width = p.idx_width;
  // A bitmask row is read through the prefix counts of its words: wpos[wi]
  // is the number of set bits before word wi (kept in the weight region
  // until the weights are written), so its t-th selected block is found by a
  // binary search and a bit select.  Bits past the last video block are
  // ignored.
  const bool bitmask_row = kProxy && video_item && p.sel_format == 1;
  const uint32_t* mrow = nullptr;
  int* wpos = (int*)wt;                  // [sel_words + 1]
  auto word = [&](int wi) -> uint32_t {
    const uint32_t m = mrow[wi];
    const int valid = p.nvideo - 32 * wi;   // bits of this word that name a video block
    return valid >= 32 ? m : (m & ((1u << valid) - 1u));
  };
  if (kProxy && video_item && p.sel_format != 0) {
    const int64_t rid = (int64_t)bh * p.nvideo + (qb - p.nprefix);
    if (p.sel_format == 2) {
      // row pointers are clamped to the index list, so malformed ones read
      // nothing outside it
      const int beg = min(max(p.sel_indptr[rid], 0), p.sel_nnz);
      const int end = min(max(p.sel_indptr[rid + 1], beg), p.sel_nnz);
      width = min(end - beg, p.nvideo);
      row = p.sel_indices + beg;
    } else {
      mrow = p.sel_mask + rid * p.sel_words;
      if (tid == 0) {
        int acc = 0;
        for (int wi = 0; wi < p.sel_words; ++wi) {
          wpos[wi] = acc;
          acc += __builtin_popcount(word(wi));
        }
        wpos[p.sel_words] = acc;
      }
      wg_barrier();
      width = __builtin_amdgcn_readfirstlane(wpos[p.sel_words]);
    }
  }
  auto sel_bit = [&](int tp) -> int {   // 0 <= tp < width
    int lo = 0, hi = p.sel_words - 1;    // last word with wpos <= tp holds it
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (wpos[mid] <= tp) lo = mid;
      else hi = mid - 1;
    }
    uint32_t m = word(lo);
    for (int r = tp - wpos[lo]; r > 0; --r) m &= m - 1u;
    return 32 * lo + __builtin_ctz(m);
  };
  const int pfirst = split * p.pwidth;   // a prefix sub-item's first key block
  const int ncand = !kProxy ? p.idx_width
                            : (prefix_item ? min(p.pwidth, p.nblk - pfirst) : p.nprefix + width + p.nproxy);
  auto candidate = [&](int t) -> int {   // entry of candidate t, or -1
    int blk;
    if (!kProxy) {
      blk = row[t];
    } else if (prefix_item) {
      blk = pfirst + t;
    } else if (t < p.nprefix) {
      blk = t;
    } else if (t < p.nprefix + width) {
      const int s = bitmask_row ? sel_bit(t - p.nprefix) : row[t - p.nprefix];
      blk = (s >= 0 && s < p.nvideo) ? p.nprefix + s : -1;
    } else {
      const int pt = t - p.nprefix - width;
      const int rows = min(p.nvideo - kBlock * pt, kBlock);
      return pt | (rows << kEntNvShift) | kEntProxy |
             (p.pt_flags[(int64_t)bh * p.nproxy + pt] ? kEntBf16 : 0);
    }
    const int nv = (blk >= 0 && blk < p.nblk) ? min(max(p.vbs[blk], 0), kBlock) : 0;
    if (nv == 0) return -1;
    return blk | (nv << kEntNvShift) | (p.vt_flags[bh_tiles + blk] ? kEntBf16 : 0);
  };
  const int nseg = p.nseg;
  const int ncell = 4 * nseg + 2;
  int* ccnt = sCell;                     // [ncell] tiles per cell
  int* cbeg = sCell + ncell;             // [ncell + 1] first position per cell
  if (tid == 0) {
    if (p.deterministic) {
      // Start block from the dispatch slot (a fixed 128 slots per XCD, so the
      // order depends on nothing but the shapes): resident workgroups spread
      // over the blocks.
      sStart = (int)(((int64_t)(blockIdx.x >> 3) * p.nblk / 128) % p.nblk);
    } else {
      // Start block: the average position of the XCD's resident workgroups.
      unsigned long long prog = 0;
      for (int k = 0; k < kSweepSub; ++k)
        prog += __hip_atomic_load(sweep_counter(xcd, k), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      sStart = (int)((prog / (unsigned long long)p.sweep_slots) % (unsigned long long)p.nblk);
    }
  }
  for (int t = tid; t < 2 * ncell + 1; t += kThreads) sCell[t] = 0;
  wg_barrier();
  const int start = sStart;
  for (int t = tid; t < ncand; t += kThreads) {
    const int e = candidate(t);
    int k = 0x7FFFFFFF;
    if (e >= 0) {
      const int g = ent_group(e);
      if (g <= kGHalfPad) {
        const int rel = ent_id(e) - start + (ent_id(e) < start ? p.nblk : 0);
        k = ((4 * (rel * nseg / p.nblk) + g) << 20) | rel;
      } else {
        k = ((g == kGProxy ? cell_proxy(nseg) : cell_bf16(nseg)) << 20) | ent_id(e);
      }
    }
    key[t] = k;
  }
  wg_barrier();
  // rank sort by key, ties (repeated blocks) by candidate index
  for (int t = tid; t < ncand; t += kThreads) {
    const int kt = key[t];
    if (kt == 0x7FFFFFFF) continue;
    int rank = 0;
    for (int u = 0; u < ncand; ++u) {
      const int ku = key[u];
      rank += (ku < kt) | ((ku == kt) & (u < t));
    }
    ord[rank] = candidate(t);   // entries are recomputed rather than kept in LDS
    atomicAdd(&ccnt[kt >> 20], 1);
  }
  wg_barrier();
  if (tid == 0) {
    int acc = 0;
    for (int c = 0; c < ncell; ++c) {
      cbeg[c] = acc;
      acc += ccnt[c];
    }
    cbeg[ncell] = acc;
  }
  if (video_item) {
    // proxy denominator weights vbs (0 for selected, empty or out-of-range
    // blocks) and their log2, which enters the running maximum so that the
    // weighted terms cannot overflow
    const int nbits = (p.nproxy * kBlock) / 32;
    if (bitmask_row) {
      for (int t = tid; t < nbits; t += kThreads) bits[t] = t < p.sel_words ? word(t) : 0u;
    } else {
      for (int t = tid; t < nbits; t += kThreads) bits[t] = 0u;
      wg_barrier();
      for (int t = tid; t < width; t += kThreads) {
        const int s = row[t];
        if (s >= 0 && s < p.nvideo) atomicOr(&bits[s >> 5], 1u << (s & 31));
      }
    }
    wg_barrier();
    for (int vblk = tid; vblk < p.nproxy * kBlock; vblk += kThreads) {
      int wv = 0;
      if (vblk < p.nvideo) {
        const int nv = min(max(p.vbs[p.nprefix + vblk], 0), kBlock);
        if (!((bits[vblk >> 5] >> (vblk & 31)) & 1u)) wv = nv;
      }
      wt[vblk] = (uint8_t)wv;
    }
  }
  wg_barrier();

  // ---------------- per-wave state ---------------------------------------
  const int n = __builtin_amdgcn_readfirstlane(cbeg[ncell]);
  const bool active = 32 * w < vq;      // wave has at least one valid query row
  const int qrow = 32 * w + ln;         // query row inside the block
  bf16x8 qop[8];
  {
    const uint16_t* qp = p.q + (((int64_t)b * p.seq + (int64_t)qb * kBlock + qrow) * p.heads + h) *
                                   kHeadDim + 8 * hh;
    const bool qvalid = qrow < vq;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      u32x4 v4 = {0u, 0u, 0u, 0u};
      if (qvalid) v4 = *(const u32x4*)(qp + 16 * s);
      qop[s] = __builtin_bit_cast(bf16x8, v4);
    }
  }
  // Let the Q loads finish here, so that inside the loop the only outstanding
  // vector-memory operations are the tile copies counted by wait_vmcnt.
  wait_vmcnt<0>();

  Ctx x;
  x.p = &p;
  x.sk = sK;
  x.sv = sV;
  x.wt = wt;
  x.b = b;
  x.h = h;
  x.bh_tiles = bh_tiles;
  x.bh_proxy = (int64_t)bh * p.nproxy;
  x.row_bytes = (uint32_t)(row_stride * 2);
  x.klane = (uint32_t)(lane >> 4) * x.row_bytes + (uint32_t)((((lane & 15) ^ (lane >> 4))) << 4);
  x.vlane = (uint32_t)lane * 16u;
  x.w = w;
  x.lane = lane;
  x.ln = ln;
  x.hh = hh;
  x.tid = tid;
  x.xcd = xcd;
  x.c = p.c;
  State st;
  st.o0 = f32x16{};
  st.o1 = f32x16{};
  st.o2 = f32x16{};
  st.o3 = f32x16{};
  st.mc = -INFINITY;
  st.lsum = 0.0f;
  if (n > 0) {
    if (active) run_tiles<kProxy, true>(x, qop, st, ord, cbeg, nseg, n);
    else run_tiles<kProxy, false>(x, qop, st, ord, cbeg, nseg, n);
  }

  // ---------------- epilogue ---------------------------------------------
  // o = O / l for valid rows; padding rows, empty rows and non-finite results
  // are written as 0.  Lane (ln, hh) holds query row 32w+ln and, in register
  // 4a+r of accumulator db, head-dim index 32db + 8a + 4hh + r.
  const float l_tot = pair_sum(st.lsum);
  const bool row_ok = active && qrow < vq && l_tot > 0.0f;
  const float inv = row_ok ? 1.0f / l_tot : 0.0f;
  if (p.lse != nullptr && hh == 0) {
    // natural log of the softmax normaliser: l sums 2^(s c - mc), so
    // log sum exp(s * sm_scale) = (mc + log2 l) ln 2; -inf without keys.
    p.lse[(int64_t)bh * p.seq + (int64_t)qb * kBlock + qrow] =
        row_ok ? (st.mc + log2f(l_tot)) * 0.693147180559945f : -INFINITY;
  }
  if (prefix_item) {
    // a prefix sub-item's share: O/l in fp32 and its row log-sum-exp, merged
    // over the sub-items by prefix_merge_kernel
    const int64_t prow = ((int64_t)(bh * p.nprefix + qb) * p.psplit + split) * kBlock + qrow;
    if (hh == 0) p.part_lse[prow] = row_ok ? (st.mc + log2f(l_tot)) * 0.693147180559945f : -INFINITY;
    float* orow32 = p.part_o + prow * kHeadDim + 4 * hh;
    auto store_part = [&](const f32x16& acc, int db) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        f32x4 v4;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = acc[4 * a + r] * inv;
          v4[r] = (row_ok && isfinite(v)) ? v : 0.0f;
        }
        *(f32x4*)(orow32 + 32 * db + 8 * a) = v4;
      }
    };
    store_part(st.o0, 0);
    store_part(st.o1, 1);
    store_part(st.o2, 2);
    store_part(st.o3, 3);
    return;
  }
  uint16_t* orow = out_rows + (int64_t)qrow * row_stride + 4 * hh;
  auto store4 = [&](const f32x16& acc, int db) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      unsigned u[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = acc[4 * a + r] * inv;
        if (!row_ok || !isfinite(v)) v = 0.0f;
        u[r] = bf16_rne_bits(v);
      }
      *(u32x2*)(orow + 32 * db + 8 * a) = (u32x2){u[0] | (u[1] << 16), u[2] | (u[3] << 16)};
    }
  };
  store4(st.o0, 0);
  store4(st.o1, 1);
  store4(st.o2, 2);
  store4(st.o3, 3);
}

}  // namespace

size_t attn_dyn_lds(const AttnParams& p, bool proxy) {
  const size_t table = (size_t)p.table_cap * 8;
  if (!proxy) return table;
  const size_t vcap = (size_t)p.nprefix + (p.sel_format == 0 ? p.idx_width : p.nvideo) + p.nproxy;
  const size_t video = vcap * 8 + (size_t)p.nproxy * kBlock + (size_t)p.nproxy * 2 * 4;
  return table > video ? table : video;
}

namespace {

// Attention workgroups resident per XCD at once for this dynamic LDS size,
// cached per (device, variant, LDS size).
int resident_per_xcd(bool proxy, size_t dyn) {
  struct Entry { int dev; bool proxy; size_t dyn; int slots; };
  static std::mutex mu;
  static std::vector<Entry> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 1;
  std::lock_guard<std::mutex> lock(mu);
  for (const Entry& e : cache)
    if (e.dev == dev && e.proxy == proxy && e.dyn == dyn) return e.slots;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 8;
  const hipError_t err = proxy
      ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_kernel<true>, kThreads, dyn)
      : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_kernel<false>, kThreads, dyn);
  if (err != hipSuccess) per_cu = 1;
  const int slots = std::max(1, per_cu * cus / 8);
  cache.push_back({dev, proxy, dyn, slots});
  return slots;
}

}  // namespace

hipError_t launch_attn(const AttnParams& params, bool proxy, hipStream_t stream) {
  if (params.n_items <= 0) return hipSuccess;
  AttnParams p = params;
  const size_t dyn = attn_dyn_lds(p, proxy);
  p.sweep_slots = resident_per_xcd(proxy, dyn);
  // about ten tiles of a typical item per sweep segment
  const int tiles = p.seg_tiles;
  p.nseg = std::min(kMaxSeg, std::max(1, (tiles + 5) / 10));
  if (!launch_fits((int64_t)p.items_per_xcd * 8, kThreads)) return hipErrorInvalidValue;
  const unsigned grid = (unsigned)p.items_per_xcd * 8u;
  if (proxy)
    hipLaunchKernelGGL(attn_kernel<true>, dim3(grid), dim3(kThreads), dyn, stream, p);
  else
    hipLaunchKernelGGL(attn_kernel<false>, dim3(grid), dim3(kThreads), dyn, stream, p);
  return hipGetLastError();
}

}  // namespace vsa
