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
// block); wave w owns query rows 32w..32w+31.  A block with at most 32 valid
// query rows gives both waves rows 0..31 instead, each wave taking one 32-key
// half of every tile with its own running softmax, and the two partial results
// are merged at the end.  For each selected KV tile:
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
// the LDS layout, so their copy is linear.  Tiles whose vbs is <= 32 (<= 16)
// load and multiply only their first 32 (16) keys.
//
// Tile order (it changes results only by rounding): the exact fp16 tiles of an
// item are swept in ascending block order from a start block, in nseg segments
// of the block range; inside a segment they go kind by kind (full, full with
// padding keys, half, half with padding keys, quarter), each kind through a
// straight-line specialisation of the tile step, so the accumulators never
// cross data-dependent control flow except the rescale.  Proxy and bf16 tiles
// follow.  The start block comes from the item's position in its XCD's run
// (the default: every call gives the same bits) or, on request, from the
// real-time counter (a shared sweep with better L2 reuse; see the kernel
// prologue).
#include "vsa_internal.h"

#include <math.h>

#include <algorithm>

namespace vsa {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
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
// Exact tiles of the proxy forward keep single fp16 probabilities when all of
// them are below 2^-kLowPartSkip (log2 units below the running maximum).
constexpr float kLowPartSkip = 10.0f;
// fp16 rounds every probability below 2^-25 to 0; a tile whose logits are all
// more than kZeroTile (log2 units, one unit of margin for the fp32 exp2 and
// the fused multiply-add) below the running maximum contributes nothing.
constexpr float kZeroTile = 26.0f;


// Tile-table entry: block/tile id (bits 0-19), valid rows (20-26), bf16 V (27),
// proxy tile (28), tile size (29-30, below).
constexpr int kEntNvShift = 20;
constexpr int kEntBf16 = 1 << 27;
constexpr int kEntProxy = 1 << 28;
constexpr int kEntSizeShift = 29;
__device__ inline int ent_id(int e) { return e & 0xFFFFF; }
__device__ inline int ent_nv(int e) { return (e >> kEntNvShift) & 127; }
// Tile sizes: exact fp16 tiles load and multiply only the key rows their vbs
// needs, in granules of 16: 64 (full), 32 (half) or 16 (quarter) keys.  bf16
// and proxy tiles are always full.  The size is stored in the entry, so the
// tile loop reads it with one bit-field extract.
enum : int { kTsFull = 0, kTsHalf = 1, kTsQuarter = 2 };
__device__ inline int make_ent(int id, int nv, bool bf16, bool proxy) {
  const int ts = (bf16 || proxy || nv > 32) ? kTsFull : nv > 16 ? kTsHalf : kTsQuarter;
  return id | (nv << kEntNvShift) | (bf16 ? kEntBf16 : 0) | (proxy ? kEntProxy : 0) |
         (ts << kEntSizeShift);
}
__device__ inline int ent_size(int e) { return (e >> kEntSizeShift) & 3; }

// Tile kinds, processed in this order within a sweep segment (the first
// kKinds), then proxy and bf16 tiles.
enum : int { kGFull = 0, kGFullPad, kGHalf, kGHalfPad, kGQuarter, kKinds, kGProxy = kKinds, kGBf16 };
__device__ inline int ent_group(int e) {
  if (e & kEntBf16) return kGBf16;
  if (e & kEntProxy) return kGProxy;
  const int nv = ent_nv(e);
  if (nv == 64) return kGFull;
  if (nv > 32) return kGFullPad;
  if (nv == 32) return kGHalf;
  if (nv > 16) return kGHalfPad;
  return kGQuarter;
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

// Low part of a probability pair in fp16: lo = fp16(p - hi) for the fp16 pair
// hi = fp16(p), each difference formed exactly from the fp16 value and the fp32
// probability by one mixed-precision fma and rounded once.  hi + lo carries p
// to a relative 2^-22 (hi alone: 2^-12).
__device__ inline unsigned f16_low_part(unsigned hi, float p0, float p1) {
  unsigned lo;
  asm("v_fma_mixlo_f16 %0, -%1, 1.0, %2 op_sel_hi:[1,0,0]\n\t"
      "v_fma_mixhi_f16 %0, -%1, 1.0, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
      : "=&v"(lo)
      : "v"(hi), "v"(p0), "v"(p1));
  return lo;
}

// Tiles whose values do not fit fp16 multiply bf16 V by a two-term bf16 split
// of each probability, p = hi + lo with hi = bf16(p), lo = bf16(p - hi): 16
// significant bits, so the pair carries p to a relative 2^-17 (fp16 alone:
// 2^-12).  The row sum takes hi + lo, the values the two MFMAs multiply.
__device__ inline void split_bf16(float p0, float p1, unsigned& hi, unsigned& lo, float& h0,
                                  float& h1, float& l0, float& l1) {
  hi = __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){p0, p1}, bf16x2));
  h0 = __uint_as_float(hi << 16);
  h1 = __uint_as_float(hi & 0xFFFF0000u);
  lo = __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){p0 - h0, p1 - h1}, bf16x2));
  l0 = __uint_as_float(lo << 16);
  l1 = __uint_as_float(lo & 0xFFFF0000u);
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
// Full and half tiles issue their copies in groups of four that share one
// base address and one M0: the instruction's immediate offset (0, 1, 2, 3 KB)
// moves the global address and the LDS destination alike, and each copy's
// lane offset takes its 4j rows and subtracts the immediate again.
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
    if (N >= 4) {
      // r0 is a multiple of 16 here, so copy j of each group uses chunk
      // swizzle 4j (the lane offsets are the same for every tile).
      uint32_t vo[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) vo[j] = (klane ^ (uint32_t)((4 * j) << 4)) + 4u * j * rs - 1024u * j;
#pragma unroll
      for (int g = 0; g < N; g += 4)
        asm volatile("s_mov_b32 m0, %5\n\t"
                     "global_load_lds_dwordx4 %0, %4\n\t"
                     "global_load_lds_dwordx4 %1, %4 offset:1024\n\t"
                     "global_load_lds_dwordx4 %2, %4 offset:2048\n\t"
                     "global_load_lds_dwordx4 %3, %4 offset:3072"
                     :
                     : "v"(vo[0]), "v"(vo[1]), "v"(vo[2]), "v"(vo[3]), "s"(kr + (size_t)g * 4 * rs),
                       "s"(m0 + 1024u * g)
                     : "memory");
    } else {
#pragma unroll
      for (int i = 0; i < N; ++i) {
        dma16(kr, kl ^ (uint32_t)(((r0 + 4 * i) & 15) << 4), m0 + 1024u * i);
        kr += 4 * rs;
      }
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
// vlane = 16 * lane.  Copies go in groups of up to four per base address and
// M0, 1 KB apart through the immediate offset, which moves the global address
// and the LDS destination alike.
template <int N>
__device__ inline void issue_v(const uint8_t* vtile, int base, uint32_t vlane, unsigned char* sv) {
  static_assert(N == 2 || N % 4 == 0, "copies per wave: 2, 4 or 8");
  const uint32_t ob = opaque_s((uint32_t)base);   // not hoisted, as in issue_k
  const uint32_t m0 = opaque_s(lds_addr(sv) + ob);
  const uint8_t* vb = vtile + ob;
  const uint32_t vl = opaque_v(vlane);
  if (N >= 4) {
#pragma unroll
    for (int g = 0; g < N; g += 4)
      asm volatile("s_mov_b32 m0, %2\n\t"
                   "global_load_lds_dwordx4 %0, %1\n\t"
                   "global_load_lds_dwordx4 %0, %1 offset:1024\n\t"
                   "global_load_lds_dwordx4 %0, %1 offset:2048\n\t"
                   "global_load_lds_dwordx4 %0, %1 offset:3072"
                   :
                   : "v"(vl), "s"(vb + 1024 * g), "s"(m0 + 1024u * g)
                   : "memory");
  } else {
    asm volatile("s_mov_b32 m0, %2\n\t"
                 "global_load_lds_dwordx4 %0, %1\n\t"
                 "global_load_lds_dwordx4 %0, %1 offset:1024"
                 :
                 : "v"(vl), "s"(vb), "s"(m0)
                 : "memory");
  }
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
// NI registers of each 32-key half take part: 16, or 8 (keys 0-15) for
// quarter tiles, whose keys 16-31 are not loaded.  s[kb] holds key half
// kb0 + kb.  Returns the lane's tile maximum.
template <int NKB, int NI, int MODE>
__device__ inline float tile_max(const f32x16 (&s)[2], int nv, const uint8_t* wts, float c, int hh,
                                 State& st, int kb0) {
  float t = -INFINITY;
  if (MODE == kModeProxy) {
    // a proxy logit is offset by log2 of its weight (-inf for weight 0)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < NI; ++i)
        t = fmaxf(t, fmaf(s[kb][i], c, __log2f(proxy_weight(wts, kb0 + kb, i, hh))));
    t = pair_max(t);
  } else if (MODE == kModePad) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < NI; ++i) t = fmaxf(t, key_of(kb0 + kb, i, hh) < nv ? s[kb][i] : -INFINITY);
    t = pair_max(t) * c;
  } else {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < NI; ++i) t = fmaxf(t, s[kb][i]);
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
  return t;
}

// Probabilities of one 32-key half (register i = key 32kb + 8(i/4) + 4hh + i%4)
// packed straight into the PV B operand; the row sum takes exactly the rounded
// values the MFMA multiplies.  A proxy key stands for a whole block: its value
// operand is the block's value total, so the numerator takes its probability
// as is and only the denominator multiplies it by the block's valid-row count.
// fp16 tiles fill pk with fp16 probabilities and, with kSplitP, pl with their
// fp16 low parts (hi + lo, see f16_low_part); bf16 tiles always fill pk with the
// high and pl with the low bf16 parts.  The plain forward keeps single fp16
// probabilities (relative 2^-12 each); the proxy forward splits those of its
// exact tiles, because its value totals and long prefix rows leave less margin
// to the bf16 rounding of the outputs, at the cost of twice the O += P V
// products on those tiles (skipped where all of a tile's probabilities are
// tiny, see tile_step).
template <int MODE, bool BF16, bool kSplitP, int NI>
__device__ inline void half_probs(const f32x16& sk, int kb, int nv, const uint8_t* wts, float c,
                                  float nmc, int hh, bool lo, float& lsum, unsigned (&pk)[8],
                                  unsigned (&pl)[8]) {
  auto keyw = [&](int i) { return proxy_weight(wts, kb, i, hh); };
  auto prob = [&](int i) {
    const float e = __builtin_amdgcn_exp2f(fmaf(sk[i], c, nmc));
    if (MODE == kModeProxy) return keyw(i) > 0.0f ? e : 0.0f;
    return (MODE == kModePad && key_of(kb, i, hh) >= nv) ? 0.0f : e;
  };
  if (BF16) {
#pragma unroll
    for (int i = 0; i < NI; i += 2) {
      float h0, h1, l0, l1;
      split_bf16(prob(i), prob(i + 1), pk[i / 2], pl[i / 2], h0, h1, l0, l1);
      if (MODE == kModeProxy) {
        lsum = fmaf(h0 + l0, keyw(i), lsum);
        lsum = fmaf(h1 + l1, keyw(i + 1), lsum);
      } else {
        lsum += (h0 + l0) + (h1 + l1);
      }
    }
  } else {
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    const unsigned lomask = lo ? 0xFFFFFFFFu : 0u;   // low parts zero when they are skipped
#pragma unroll
    for (int i = 0; i < NI; i += 2) {
      const float p0 = prob(i), p1 = prob(i + 1);
      const f16x2 h = __builtin_convertvector((f32x2){p0, p1}, f16x2);
      // proxy weights <= 64 are exact in fp16
      const f16x2 wv = MODE == kModeProxy
                           ? __builtin_convertvector((f32x2){keyw(i), keyw(i + 1)}, f16x2)
                           : one;
      pk[i / 2] = __builtin_bit_cast(unsigned, h);
      lsum = __builtin_amdgcn_fdot2(h, wv, lsum, false);
      if (kSplitP) {
        pl[i / 2] = f16_low_part(pk[i / 2], p0, p1) & lomask;
        lsum = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pl[i / 2]), wv, lsum, false);
      }
    }
  }
}

// O^T (128 d x 32 queries) += V^T . P^T for one 32-key half kb: 16-key steps
// ks = 2kb, 2kb+1 (only the first for quarter tiles, NK2 = 1) with B operand
// pk[4(ks%2)..+3] (keys 16ks + 8(j/4) + 4hh + j%4); the A operand is row
// d = 32db + ln of 16-key group ks of the packed V tile, chunk hh.
// bf16 tiles run each step twice, with the high and the low probability parts.
template <bool BF16, bool kSplitP, int NK2>
__device__ inline void pv_half(const unsigned char* sv, int kb, const unsigned (&pk)[8],
                               const unsigned (&pl)[8], bool lo, int ln, int hh, State& st) {
  const int chunk = (hh ^ vt_swizzle(ln)) << 4;
#pragma unroll
  for (int k2 = 0; k2 < NK2; ++k2) {
    const unsigned char* vb = sv + kb * 8192 + k2 * 4096 + ln * 32 + chunk;
    const u32x4 pb = {pk[4 * k2], pk[4 * k2 + 1], pk[4 * k2 + 2], pk[4 * k2 + 3]};
    if (BF16) {
      const u32x4 lb = {pl[4 * k2], pl[4 * k2 + 1], pl[4 * k2 + 2], pl[4 * k2 + 3]};
      const bf16x8 bh = __builtin_bit_cast(bf16x8, pb), bl = __builtin_bit_cast(bf16x8, lb);
#define VSA_PV_BF16(acc, db)                                                          \
      {                                                                               \
        const bf16x8 a = *(const bf16x8*)(vb + (db) * 1024);                          \
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bh, acc, 0, 0, 0);           \
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bl, acc, 0, 0, 0);           \
      }
      VSA_PV_BF16(st.o0, 0)
      VSA_PV_BF16(st.o1, 1)
      VSA_PV_BF16(st.o2, 2)
      VSA_PV_BF16(st.o3, 3)
#undef VSA_PV_BF16
    } else {
      const f16x8 bb = __builtin_bit_cast(f16x8, pb);
      st.o0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(*(const f16x8*)(vb + 0 * 1024), bb, st.o0, 0, 0, 0);
      st.o1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(*(const f16x8*)(vb + 1 * 1024), bb, st.o1, 0, 0, 0);
      st.o2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(*(const f16x8*)(vb + 2 * 1024), bb, st.o2, 0, 0, 0);
      st.o3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(*(const f16x8*)(vb + 3 * 1024), bb, st.o3, 0, 0, 0);
    }
  }
  if (!BF16 && kSplitP && lo) {
    // the low parts of split fp16 probabilities, with the V operand read again
#pragma unroll
    for (int k2 = 0; k2 < NK2; ++k2) {
      const unsigned char* vb = sv + kb * 8192 + k2 * 4096 + ln * 32 + chunk;
      const f16x8 bl = __builtin_bit_cast(f16x8, (u32x4){pl[4 * k2], pl[4 * k2 + 1], pl[4 * k2 + 2], pl[4 * k2 + 3]});
      st.o0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(*(const f16x8*)(vb + 0 * 1024), bl, st.o0, 0, 0, 0);
      st.o1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(*(const f16x8*)(vb + 1 * 1024), bl, st.o1, 0, 0, 0);
      st.o2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(*(const f16x8*)(vb + 2 * 1024), bl, st.o2, 0, 0, 0);
      st.o3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(*(const f16x8*)(vb + 3 * 1024), bl, st.o3, 0, 0, 0);
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
  const char* k_bh;        // K row 0 of this (batch, head)
  const uint8_t* vt_bh;    // first packed V tile of this (batch, head)
  int64_t bh_proxy;        // (b * heads + h) * nproxy
  uint32_t row_bytes, klane, vlane;
  int w, lane, ln, hh, tid;
  float c;
  bool qv;                 // this lane's query row is a valid token
  bool zs;                 // zero tiles are skipped
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
    base = (const uint16_t*)(x.k_bh + (uint64_t)(uint32_t)(ent_id(e) * kBlock) * x.row_bytes);
  }
  switch (ent_size(e)) {
    case kTsFull: issue_k<8, kProxy>(base, x.row_bytes, rmax, 32 * x.w, x.klane, x.lane, x.sk); break;
    case kTsHalf: issue_k<4, kProxy>(base, x.row_bytes, rmax, 16 * x.w, x.klane, x.lane, x.sk); break;
    default: issue_k<2, kProxy>(base, x.row_bytes, rmax, 8 * x.w, x.klane, x.lane, x.sk); break;
  }
}

template <bool kProxy>
__device__ inline void issue_tile_v(const Ctx& x, int e) {
  const AttnParams& p = *x.p;
  const uint8_t* base = (kProxy && (e & kEntProxy))
                            ? p.pt + (x.bh_proxy + ent_id(e)) * kTileBytes
                            : x.vt_bh + (uint64_t)(uint32_t)ent_id(e) * kTileBytes;
  switch (ent_size(e)) {
    case kTsFull: issue_v<8>(base, 8192 * x.w, x.vlane, x.sv); break;
    case kTsHalf: issue_v<4>(base, 4096 * x.w, x.vlane, x.sv); break;
    default: issue_v<2>(base, 2048 * x.w, x.vlane, x.sv); break;
  }
}

// One tile: wait for its K rows, S = K Q^T, release K and prefetch the next
// tile's K rows, running max, wait for its V, probabilities and O += P V,
// release V and prefetch the next tile's V.  NKB / MODE / BF16 are fixed per
// tile kind (MODE kModeAny: bf16 tiles, exact or proxy, decided per tile).
// Key split (kKS, items with at most 32 valid query rows): both waves hold
// the same 32 query rows; wave w takes key half w of a full tile, and a half
// or quarter tile (all keys in half 0) goes to the wave for which `mine` is
// set.  Each wave then keeps its own running max, row sum and O, merged at
// the end of the item.  Copies and barriers are the same in both modes.
template <bool kProxy, int TS, int MODE, bool BF16, bool kKS>
__device__ inline void tile_step(const Ctx& x, const bf16x8 (&qop)[8], State& st, int e, int en,
                                 bool has_next, bool mine) {
  constexpr int NKB = (TS == kTsFull && !kKS) ? 2 : 1;   // 32-key halves of S
  constexpr int NI = TS == kTsQuarter ? 8 : 16;    // registers per half that hold loaded keys
  constexpr int NK2 = TS == kTsQuarter ? 1 : 2;    // 16-key steps of O += P V per half
  const int kb0 = (kKS && TS == kTsFull) ? x.w : 0;   // first key half this wave takes
  const bool work = !kKS || TS == kTsFull || mine;
  // K(j) has landed once only V(j)'s copies (8, 4 or 2 instructions per wave)
  // are still in flight.
  wait_vmcnt<(8 >> TS)>();
  wg_barrier();
  f32x16 s[2];
  if (work) s_tile<NKB>(x.sk + kb0 * 8192, qop, x.ln, x.hh, s);
  wg_barrier();   // both waves are done with sK
  if (has_next) issue_tile_k<kProxy>(x, en);

  const int nv = ent_nv(e);
  const bool px = kProxy && (MODE == kModeProxy || (MODE == kModeAny && (e & kEntProxy)));
  const uint8_t* wts = kProxy ? x.wt + kBlock * ent_id(e) : nullptr;
  // The running max, the probabilities and O += P V run at raised wave
  // priority: where both waves of a SIMD can issue, this phase goes first.
  __builtin_amdgcn_s_setprio(2);
  // Exact fp16 tiles of the proxy forward split their probabilities; its
  // proxy tiles do not need to (their rounding moves the outputs far less
  // than that of the exact tiles).  An exact tile whose probabilities are
  // all below 2^-kLowPartSkip in every valid query row of the wave keeps
  // single ones: their low parts are below 2^-(kLowPartSkip + 12) of the
  // running maximum's term.
  // An fp16 tile whose logits all lie more than kZeroTile below the running
  // maximum in every valid query row of the wave has only probabilities that
  // round to 0 in fp16: it adds exactly nothing to O and the row sum, and its
  // exponentials and O += P V products are skipped.
  constexpr bool kSP = kProxy && MODE != kModeProxy && !BF16;
  bool split = kSP;
  bool live = work;
  if (work) {
    float tmax;
    if (MODE == kModeAny) {
      if (px) tmax = tile_max<NKB, NI, kModeProxy>(s, nv, wts, x.c, x.hh, st, kb0);
      else tmax = tile_max<NKB, NI, kModePad>(s, nv, wts, x.c, x.hh, st, kb0);
    } else {
      tmax = tile_max<NKB, NI, MODE>(s, nv, wts, x.c, x.hh, st, kb0);
    }
    if (!BF16 && x.zs) live = __ballot(x.qv && tmax >= st.mc - kZeroTile) != 0ull;
    if (kSP) split = __ballot(x.qv && tmax >= st.mc - kLowPartSkip) != 0ull;
  }

  // V(j) has landed once only K(j+1)'s copies may still be in flight.
  if (has_next) {
    switch (ent_size(en)) {
      case kTsFull: wait_vmcnt<8>(); break;
      case kTsHalf: wait_vmcnt<4>(); break;
      default: wait_vmcnt<2>(); break;
    }
  } else {
    wait_vmcnt<0>();
  }
  wg_barrier();
  if (live) {
    const float nmc = -st.mc;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const int kh = kb0 + kb;
      unsigned pk[8], pl[8];
      if (MODE == kModeAny) {
        if (px) half_probs<kModeProxy, BF16, kSP, NI>(s[kb], kh, nv, wts, x.c, nmc, x.hh, split, st.lsum, pk, pl);
        else half_probs<kModePad, BF16, kSP, NI>(s[kb], kh, nv, wts, x.c, nmc, x.hh, split, st.lsum, pk, pl);
      } else {
        half_probs<MODE, BF16, kSP, NI>(s[kb], kh, nv, wts, x.c, nmc, x.hh, split, st.lsum, pk, pl);
      }
      pv_half<BF16, kSP, NK2>(x.sv, kh, pk, pl, split, x.ln, x.hh, st);
    }
    if (!BF16 && !kProxy) {
      // V operand reads run four MFMAs ahead, across both key halves
      constexpr int kR = 4 * NK2 * NKB;
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
#pragma unroll
      for (int i = 0; i < kR - 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 1);
    }
  }
  __builtin_amdgcn_s_setprio(0);
  wg_barrier();   // both waves are done with sV
  if (has_next) issue_tile_v<kProxy>(x, en);
}

// Table cells: segment s, exact fp16 kind g -> kKinds s + g; then proxy, bf16.
__device__ inline int cell_proxy(int nseg) { return kKinds * nseg; }
__device__ inline int cell_bf16(int nseg) { return kKinds * nseg + 1; }

// All tiles of one item in the order of `ord`; cbeg[c] is the first position of
// cell c (cbeg[kKinds nseg + 2] = number of tiles).
template <bool kProxy, bool kKS>
__device__ inline void run_tiles(const Ctx& x, const bf16x8 (&qop)[8], State& st, const int* ord,
                                 const int* cbeg, int nseg, int n) {
  const int e0 = __builtin_amdgcn_readfirstlane(ord[0]);
  issue_tile_k<kProxy>(x, e0);
  issue_tile_v<kProxy>(x, e0);
  // The entry of tile j + 1 is read from LDS one tile ahead (into a vector
  // register), so that its read latency is not paid at the top of tile j.
  int e_cur = e0;
  int e_nxt = n > 1 ? __builtin_amdgcn_readfirstlane(ord[1]) : 0;
  auto cell = [&](auto body, int c) {
    const int beg = __builtin_amdgcn_readfirstlane(cbeg[c]);
    const int end = __builtin_amdgcn_readfirstlane(cbeg[c + 1]);
    for (int j = beg; j < end; ++j) {
      const bool has_next = j + 1 < n;
      const int v_after = j + 2 < n ? ord[j + 2] : 0;
      body(e_cur, e_nxt, has_next, (j & 1) == x.w);   // key split: half tiles alternate between the waves
      e_cur = e_nxt;
      e_nxt = __builtin_amdgcn_readfirstlane(v_after);
    }
  };
  for (int s = 0; s < nseg; ++s) {
    const int c0 = kKinds * s;
    cell([&](int e, int en, bool hn, bool mi) { tile_step<kProxy, kTsFull, kModeFull, false, kKS>(x, qop, st, e, en, hn, mi); }, c0 + kGFull);
    cell([&](int e, int en, bool hn, bool mi) { tile_step<kProxy, kTsFull, kModePad, false, kKS>(x, qop, st, e, en, hn, mi); }, c0 + kGFullPad);
    cell([&](int e, int en, bool hn, bool mi) { tile_step<kProxy, kTsHalf, kModeFull, false, kKS>(x, qop, st, e, en, hn, mi); }, c0 + kGHalf);
    cell([&](int e, int en, bool hn, bool mi) { tile_step<kProxy, kTsHalf, kModePad, false, kKS>(x, qop, st, e, en, hn, mi); }, c0 + kGHalfPad);
    cell([&](int e, int en, bool hn, bool mi) { tile_step<kProxy, kTsQuarter, kModePad, false, kKS>(x, qop, st, e, en, hn, mi); }, c0 + kGQuarter);
  }
  if (kProxy)
    cell([&](int e, int en, bool hn, bool mi) { tile_step<kProxy, kTsFull, kModeProxy, false, kKS>(x, qop, st, e, en, hn, mi); }, cell_proxy(nseg));
  cell([&](int e, int en, bool hn, bool mi) { tile_step<kProxy, kTsFull, kModeAny, true, kKS>(x, qop, st, e, en, hn, mi); }, cell_bf16(nseg));
}

template <bool kProxy>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void attn_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(1024))) unsigned char sK[kTileBytes];
  __shared__ __attribute__((aligned(1024))) unsigned char sV[kTileBytes];
  __shared__ int sCell[2 * (kKinds * kMaxSeg + 2) + 1];   // tiles per cell, then first position per cell
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
  // blocks.  Tail balancing: the last kSchedPool items of each XCD's run are
  // a pool.  The workgroups that reach it (plus kSchedExtra more per XCD)
  // claim pool items through the XCDs' counters, their own XCD's first, so an
  // XCD that runs ahead takes the last items of one that lags; a workgroup
  // that finds every pool empty exits.  The item alone decides its result.
  const int xcd = (int)(blockIdx.x & 7);
  int iseq = (int)(blockIdx.x >> 3);     // position of the item in its XCD's run
  int ixcd = xcd;
  const int pool0 = p.items_per_xcd - kSchedPool;
  if (p.sched != nullptr && pool0 > 0 && iseq >= pool0) {
    __shared__ int s_claim;
    if (tid == 0) {
      int got = -1;
      for (int d = 0; d < 8; ++d) {
        const int y = (xcd + d) & 7;
        const int j = __hip_atomic_fetch_add(p.sched + y * kSchedStride, 1, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
        if (j < kSchedPool) {
          got = y * kSchedPool + j;
          break;
        }
      }
      s_claim = got;
    }
    __syncthreads();
    const int got = s_claim;
    if (got < 0) return;
    ixcd = got / kSchedPool;
    iseq = pool0 + got % kSchedPool;
  } else if (iseq >= p.items_per_xcd) {
    return;
  }
  const int item = ixcd * p.items_per_xcd + iseq;
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
      return make_ent(pt, rows, p.pt_flags[(int64_t)bh * p.nproxy + pt] != 0, true);
    }
    const int nv = (blk >= 0 && blk < p.nblk) ? min(max(p.vbs[blk], 0), kBlock) : 0;
    if (nv == 0) return -1;
    return make_ent(blk, nv, p.vt_flags[bh_tiles + blk] != 0, false);
  };
  const int nseg = p.nseg;
  const int ncell = kKinds * nseg + 2;
  int* ccnt = sCell;                     // [ncell] tiles per cell
  int* cbeg = sCell + ncell;             // [ncell + 1] first position per cell
  // Start block of the sweep.  Reproducible order: from the item's position
  // in its XCD's run, so that the 128 workgroups resident on an XCD at once
  // start spread evenly over the head's blocks (a slot's later items start
  // where its first did), and the order depends on the shapes only.  Shared sweep (sweep_rate > 0):
  // from the real-time counter, at sweep_rate blocks per tick, about the rate
  // at which a workgroup moves through its blocks; the resident workgroups of
  // a head then move through its blocks together, a narrow window of its K/V
  // tiles stays in the XCD's L2, and the order depends on timing.
  int start;
  if (p.sweep_rate > 0.0f) {
    const double pos = (double)__builtin_amdgcn_s_memrealtime() * (double)p.sweep_rate;
    start = (int)fmod(pos, (double)p.nblk);
  } else {
    start = (int)(((int64_t)iseq * p.nblk / 128) % p.nblk);
  }
  for (int t = tid; t < 2 * ncell + 1; t += kThreads) sCell[t] = 0;
  wg_barrier();
  for (int t = tid; t < ncand; t += kThreads) {
    const int e = candidate(t);
    int k = 0x7FFFFFFF;
    if (e >= 0) {
      const int g = ent_group(e);
      if (g < kKinds) {
        const int rel = ent_id(e) - start + (ent_id(e) < start ? p.nblk : 0);
        k = ((kKinds * (rel * nseg / p.nblk) + g) << 20) | rel;
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
  // Blocks with at most 32 valid query rows split the keys of each tile
  // between the two waves instead of leaving the second wave without rows.
  const bool ks = vq <= 32;
  int qrow = ks ? ln : 32 * w + ln;     // query row inside the block
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
  x.k_bh = (const char*)(p.k + ((int64_t)b * p.seq * p.heads + h) * kHeadDim);
  x.vt_bh = p.vt + bh_tiles * kTileBytes;
  x.bh_proxy = (int64_t)bh * p.nproxy;
  x.row_bytes = (uint32_t)(row_stride * 2);
  x.klane = (uint32_t)(lane >> 4) * x.row_bytes + (uint32_t)((((lane & 15) ^ (lane >> 4))) << 4);
  x.vlane = (uint32_t)lane * 16u;
  x.w = w;
  x.lane = lane;
  x.ln = ln;
  x.hh = hh;
  x.tid = tid;
  x.c = p.c;
  x.qv = qrow < vq;
  x.zs = p.zero_skip != 0;
  State st;
  st.o0 = f32x16{};
  st.o1 = f32x16{};
  st.o2 = f32x16{};
  st.o3 = f32x16{};
  st.mc = -INFINITY;
  st.lsum = 0.0f;
  if (n > 0) {
    if (ks) run_tiles<kProxy, true>(x, qop, st, ord, cbeg, nseg, n);
    else run_tiles<kProxy, false>(x, qop, st, ord, cbeg, nseg, n);
  }
  bool active = true;                   // this wave writes the rows it computed
  if (ks) {
    // Merge the two waves' partial results over disjoint keys: wave 1 hands
    // its O, running max and row sum to wave 0 through the tile buffers (no
    // copy is in flight after the last tile, and both waves have passed its
    // final barrier), and then writes the padding rows 32..63.
    float* so = (float*)sK;             // 64 accumulator registers x 64 lanes = 16 KB
    float* sm = (float*)sV;
    if (w == 1) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        so[(0 * 16 + r) * 64 + lane] = st.o0[r];
        so[(1 * 16 + r) * 64 + lane] = st.o1[r];
        so[(2 * 16 + r) * 64 + lane] = st.o2[r];
        so[(3 * 16 + r) * 64 + lane] = st.o3[r];
      }
      sm[lane] = st.mc;
      sm[64 + lane] = st.lsum;
    }
    wg_barrier();
    if (w == 0) {
      const float m1 = sm[lane], l1 = sm[64 + lane];
      const float m = fmaxf(st.mc, m1);
      const float a0 = st.mc == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(st.mc - m);
      const float a1 = m1 == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m1 - m);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        st.o0[r] = st.o0[r] * a0 + so[(0 * 16 + r) * 64 + lane] * a1;
        st.o1[r] = st.o1[r] * a0 + so[(1 * 16 + r) * 64 + lane] * a1;
        st.o2[r] = st.o2[r] * a0 + so[(2 * 16 + r) * 64 + lane] * a1;
        st.o3[r] = st.o3[r] * a0 + so[(3 * 16 + r) * 64 + lane] * a1;
      }
      st.lsum = st.lsum * a0 + l1 * a1;
      st.mc = m;
    } else {
      qrow = 32 + ln;
      active = false;
    }
  }

  // ---------------- epilogue ---------------------------------------------
  // o = O / l for valid rows; padding rows, empty rows and non-finite results
  // are written as 0.  Lane (ln, hh) holds query row qrow and, in register
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
      float f[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = acc[4 * a + r] * inv;
        f[r] = (row_ok && isfinite(v)) ? v : 0.0f;
      }
      const unsigned u01 = __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){f[0], f[1]}, bf16x2));
      const unsigned u23 = __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){f[2], f[3]}, bf16x2));
      *(u32x2*)(orow + 32 * db + 8 * a) = (u32x2){u01, u23};
    }
  };
  store4(st.o0, 0);
  store4(st.o1, 1);
  store4(st.o2, 2);
  store4(st.o3, 3);
}

// Zeroes the tail-pool counters before a launch (a kernel rather than a
// memset node, so that captured graphs replay it like the other launches).
__global__ void sched_reset_kernel(int* sched) {
  if (threadIdx.x < 8) sched[threadIdx.x * kSchedStride] = 0;
}

}  // namespace

size_t attn_dyn_lds(const AttnParams& p, bool proxy) {
  const size_t table = (size_t)p.table_cap * 8;
  if (!proxy) return table;
  const size_t vcap = (size_t)p.nprefix + (p.sel_format == 0 ? p.idx_width : p.nvideo) + p.nproxy;
  const size_t video = vcap * 8 + (size_t)p.nproxy * kBlock + (size_t)p.nproxy * 2 * 4;
  return table > video ? table : video;
}

hipError_t launch_attn(const AttnParams& params, bool proxy, hipStream_t stream) {
  if (params.n_items <= 0) return hipSuccess;
  AttnParams p = params;
  // Shared sweep: a workgroup crosses about one tile per kTicksPerTile ticks of
  // the 100 MHz real-time counter (MI355X, configs 2 and 3b: 2.0-2.2 us per
  // 64-key tile per workgroup), so its blocks pass at nblk / (tiles *
  // kTicksPerTile) per tick.
  constexpr float kTicksPerTile = 200.0f;
  if (p.sweep_rate > 0.0f)
    p.sweep_rate = (float)p.nblk / ((float)std::max(1, p.seg_tiles) * kTicksPerTile);
  const size_t dyn = attn_dyn_lds(p, proxy);
  // Skipping all-zero tiles takes arithmetic out of a workgroup's sweep.  In
  // the reproducible order that arithmetic paces the sweeps of a head whose
  // K/V is many times the XCD's 4 MB L2 (40 heads x 1440 cubes: 46 MB per
  // head, 3% slower with the skip), so there it stays on only with the shared
  // sweep; for heads of at most 32 MB (624 cubes: 20 MB) it saves 5-11%.
  // The outputs are the same either way.
  constexpr int64_t kZeroSkipHeadBytes = (int64_t)32 << 20;
  p.zero_skip = (p.sweep_rate > 0.0f || (int64_t)p.nblk * 2 * kTileBytes <= kZeroSkipHeadBytes) ? 1 : 0;
  // about ten tiles of a typical item per sweep segment
  const int tiles = p.seg_tiles;
  p.nseg = std::min(kMaxSeg, std::max(1, (tiles + 5) / 10));
  const bool balance = p.sched != nullptr && p.items_per_xcd > kSchedPool;
  const int64_t per_xcd = (int64_t)p.items_per_xcd + (balance ? kSchedExtra : 0);
  if (!launch_fits(per_xcd * 8, kThreads)) return hipErrorInvalidValue;
  const unsigned grid = (unsigned)(per_xcd * 8);
  if (balance) {
    hipLaunchKernelGGL(sched_reset_kernel, dim3(1), dim3(64), 0, stream, p.sched);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (proxy)
    hipLaunchKernelGGL(attn_kernel<true>, dim3(grid), dim3(kThreads), dyn, stream, p);
  else
    hipLaunchKernelGGL(attn_kernel<false>, dim3(grid), dim3(kThreads), dyn, stream, p);
  return hipGetLastError();
}

}  // namespace vsa
