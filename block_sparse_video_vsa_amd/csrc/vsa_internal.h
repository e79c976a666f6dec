// Internal declarations shared by the host entry points and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace vsa {

constexpr int kBlock = 64;       // tokens per cube / block
constexpr int kHeadDim = 128;    // head geometry fixed at compile time
constexpr int kTileBytes = kBlock * kHeadDim * 2;   // one 64 x 128 16-bit tile
constexpr int kMaxSeg = 16;     // most sweep segments per item
// Tail balancing of an attention launch: the last kSchedPool items of each
// XCD's range form a pool, claimed through one agent-scope counter per XCD
// (kSchedStride ints apart, one 256-byte line each) in the caller's
// workspace; kSchedExtra more workgroups per XCD let a faster XCD take items
// from the pools of slower ones.
constexpr int kSchedPool = 256;
constexpr int kSchedExtra = 128;
constexpr int kSchedStride = 64;
constexpr size_t kSchedBytes = 8 * kSchedStride * sizeof(int);
// Work-items of one launch: the dispatch packet holds 32 bits; launches stay
// at or below 2^31 so that a grid never truncates or overflows.
constexpr int64_t kMaxLaunchThreads = (int64_t)1 << 31;
inline bool launch_fits(int64_t blocks, int threads) {
  return blocks >= 0 && blocks * threads <= kMaxLaunchThreads;
}

// ---- wavefront lane exchanges --------------------------------------------
// Value of lane ^ j (j = 1, 2, 4, 8, 16 or 32, a constant after unrolling),
// exchanged inside the VALU: DPP quad permutes for 1 and 2, row rotations for
// 4 and 8, the permlane swaps for 16 and 32 (no LDS round trip).
__device__ __attribute__((always_inline)) inline unsigned xor_lane(unsigned v, int j, int lane) {
  switch (j) {
    case 1: return (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);   // quad_perm 1,0,3,2
    case 2: return (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);   // quad_perm 2,3,0,1
    case 4: {
      const unsigned a = (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0x124, 0xF, 0xF, false);   // row_ror:4
      const unsigned b = (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0x12C, 0xF, 0xF, false);   // row_ror:12
      return (lane & 4) ? a : b;
    }
    case 8: return (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false);   // row_ror:8
    case 16: {
      const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
      return (lane & 16) ? r[0] : r[1];
    }
    default: {
      const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
      return (lane & 32) ? r[0] : r[1];
    }
  }
}
__device__ __attribute__((always_inline)) inline uint64_t xor_lane64(uint64_t v, int j, int lane) {
  const unsigned lo = xor_lane((unsigned)v, j, lane);
  const unsigned hi = xor_lane((unsigned)(v >> 32), j, lane);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __attribute__((always_inline)) inline double xor_lane_f64(double v, int j, int lane) {
  return __longlong_as_double((long long)xor_lane64((uint64_t)__double_as_longlong(v), j, lane));
}

// ---- packed V tiles ------------------------------------------------------
// Each (batch, head, tile) V^T tile is 16 KB: two 8 KB key halves (keys 0-31,
// 32-63), each of two 4 KB 16-key groups; inside a group, 128 rows (one per
// head-dim index d) of 16 keys = 32 B, split in two 16 B chunks (the two lane
// halves of the MFMA operand) stored in the order given by vt_swizzle(d);
// inside a chunk the eight keys follow the MFMA k-slot order (see
// vsa_attn.hip).  A tile's first 16, 32 or 64 keys are thus its first 4, 8 or
// 16 KB.  The swizzle puts rows d and d + 8 of a 16-row band in different
// 16-byte bank groups, so the operand reads (16 consecutive rows per group of
// lanes) touch every LDS bank once.
// Elements are fp16 when the tile's values fit fp16 well, else bf16 (flag 1).
__host__ __device__ inline int vt_swizzle(int d) { return (d >> 3) & 1; }

struct PackParams {
  const uint16_t* src;      // bf16 BSHD source rows
  uint8_t* dst;             // packed tiles
  uint8_t* flags;           // one byte per tile: 0 fp16, 1 bf16
  const int32_t* vbs;       // per-block valid rows (block-indexed mode) or nullptr
  int64_t src_rows;         // rows per batch in src
  int heads;
  int tiles;                // tiles per (batch, head)
  int row_offset;           // first source row of tile 0 (in rows)
  int valid_rows;           // proxy mode: rows [0, valid_rows) after row_offset are valid
};

struct AttnParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* kmean;    // proxy mode
  const uint8_t* vt;        // packed V tiles [B][H][nblk]
  const uint8_t* vt_flags;
  const uint8_t* pt;        // packed vsum tiles [B][H][nproxy] (proxy mode)
  const uint8_t* pt_flags;
  const int32_t* idx;       // topk_idx [B,H,Nq,topk] or sel_idx [B,H,Nv,max_sel]
  const int32_t* vbs;
  uint16_t* out;
  float* lse;               // optional [B, H, S] row log-sum-exp (nullptr: none)
  int batch, seq, heads, nblk;
  int idx_width;            // topk or max_sel (padded rows)
  int sel_format;           // proxy: 0 padded rows (idx), 1 bitmask, 2 BSR
  const uint32_t* sel_mask; // bitmask rows [B*H*nvideo][sel_words]
  int sel_words;
  const int32_t* sel_indptr;   // BSR row pointers [B*H*nvideo + 1]
  const int32_t* sel_indices;  // BSR video-relative block ids
  int sel_nnz;              // BSR: entries in sel_indices
  int nprefix;              // prefix blocks (proxy mode)
  int nvideo;               // video blocks (proxy mode)
  int nproxy;               // proxy tiles of 64 video blocks (proxy mode)
  int n_items;              // batch * heads * items_per_bh
  int items_per_xcd;
  int table_cap;            // tile-table capacity (entries)
  int nseg;                 // sweep segments per item (1..kMaxSeg)
  int seg_tiles;            // tiles of a typical item (sizes the segments)
  float sweep_rate;         // > 0: shared sweep, start block from the real-time counter
  float c;                  // sm_scale * log2(e)
  // proxy prefix split (appended: the fields above keep their offsets)
  int items_per_bh;         // nblk, or (proxy) nprefix * psplit + nvideo
  int psplit;               // proxy: sub-items per prefix query block
  int pwidth;               // proxy: key blocks per prefix sub-item
  float* part_o;            // proxy: prefix partial outputs O/l [B*H][nprefix][psplit][64][128]
  float* part_lse;          // proxy: their row log-sum-exp [B*H][nprefix][psplit][64]
  int* sched;               // kSchedBytes of tail-pool counters (workspace), or nullptr
  int zero_skip;            // skip fp16 tiles whose probabilities all round to 0 (set at launch)
};

hipError_t launch_pack(const PackParams& p, int batch, hipStream_t stream);
hipError_t launch_preprocess(const uint16_t* k, const uint16_t* v, const int32_t* vbs,
                             uint16_t* kmean, uint16_t* vsum, int batch, int seq, int heads,
                             hipStream_t stream);
hipError_t launch_attn(const AttnParams& p, bool proxy, hipStream_t stream);
// Mean and population variance of the bf16 block key means over blocks
// [first, first + count) with vbs > 0, per (batch, head, channel), fp32 out.
hipError_t launch_kc_stats(const uint16_t* kc, const int32_t* vbs, float* mean, float* var,
                           int batch, int nblk, int heads, int first, int count,
                           hipStream_t stream);
// Routing: top-k key blocks by block-mean scores, through an fp64 score
// workspace that holds route_pairs_per_chunk (batch, head) pairs at a time.
int route_pairs_per_chunk(int batch, int heads, int nblk);
size_t route_workspace_bytes(int batch, int heads, int nblk);
hipError_t launch_route(const uint16_t* qmean, const uint16_t* kmean, const int32_t* vbs,
                        int32_t* out, int batch, int nblk, int heads, int topk, double* scores,
                        hipStream_t stream);
// Merge of the prefix sub-items' partial results into the bf16 output rows.
hipError_t launch_prefix_merge(const float* part_o, const float* part_lse, const int32_t* vbs,
                               uint16_t* out, int batch, int seq, int heads, int nprefix,
                               int psplit, hipStream_t stream);
// Merge of two partial attention results over disjoint key sets.
hipError_t launch_merge(const uint16_t* o1, const float* lse1, const uint16_t* o2, const float* lse2,
                        uint16_t* out, float* lse_out, int batch, int seq, int heads, int head_dim,
                        hipStream_t stream);
// Cube tiling (src natural rows -> dst cube-major padded rows) or, with untile,
// its inverse (src cube-major -> dst natural); rows are row_bytes long.
hipError_t launch_tile(const void* src, void* dst, int batch, int T, int Hh, int W, int64_t row_bytes,
                       bool untile, hipStream_t stream);
// Dynamic LDS bytes launch_attn requests for these parameters.
size_t attn_dyn_lds(const AttnParams& p, bool proxy);

}  // namespace vsa
