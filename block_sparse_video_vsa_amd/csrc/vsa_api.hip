// C-ABI entry points: host-side argument checks, workspace carving and kernel
// launches on the caller's stream.  No allocation, no synchronisation.
#include "vsa.h"
#include "vsa_internal.h"

#include <algorithm>
#include <mutex>

#include <math.h>

using namespace vsa;

namespace {

constexpr size_t kWsAlign = 256;
constexpr size_t kMaxDynLds = 32 * 1024;   // beside the 32 KB of K/V tile buffers
constexpr int64_t kMaxBlocks = (1 << 20) - 1;
// (batch, head, block) triples: the V packing runs 256 threads on each, and a
// launch stays at or below 2^31 threads.
constexpr int64_t kMaxTriples = kMaxLaunchThreads / 256;
constexpr int32_t kMaxRouteBlocks = 7680;    // one (batch, head) of scores: 472 MB of workspace
constexpr int32_t kMaxHeads = 65536;      // one 64-row K cube of all heads stays below 2^32 bytes

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct WsLayout {
  size_t vt, pt, vf, pf, po, pl, sc, total;
};

// Key blocks per prefix sub-item of the proxy forward: a prefix query block
// attends to every block, so it is split into ranges of about the length of
// a video block's tile list and the parts are merged afterwards.
constexpr int32_t kPrefixSplit = 96;

int prefix_splits(int64_t nblk) { return (int)((nblk + kPrefixSplit - 1) / kPrefixSplit); }

// [V tiles B*H*nblk*16KB][proxy tiles B*H*nproxy*16KB][V flags][proxy flags]
// [prefix partial O/l: B*H*nprefix*psplit*64*128 fp32][their lse: ... *64 fp32]
// [tail-pool counters of the attention launch: kSchedBytes]
WsLayout ws_layout(int64_t batch, int64_t heads, int64_t nblk, int64_t nproxy,
                   int64_t nprefix = 0, int64_t psplit = 0) {
  WsLayout l;
  const size_t bh = (size_t)batch * (size_t)heads;
  const size_t subs = bh * (size_t)nprefix * (size_t)psplit;   // prefix sub-items
  l.vt = 0;
  l.pt = align_up(l.vt + bh * (size_t)nblk * kTileBytes, kWsAlign);
  l.vf = align_up(l.pt + bh * (size_t)nproxy * kTileBytes, kWsAlign);
  l.pf = align_up(l.vf + bh * (size_t)nblk, kWsAlign);
  l.po = align_up(l.pf + bh * (size_t)nproxy, kWsAlign);
  l.pl = align_up(l.po + subs * kBlock * kHeadDim * 4, kWsAlign);
  l.sc = align_up(l.pl + subs * kBlock * 4, kWsAlign);
  l.total = align_up(l.sc + kSchedBytes, kWsAlign);
  return l;
}

bool is_aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

vsa_status check_common(int32_t batch, int32_t seq_len, int32_t num_heads, int32_t head_dim) {
  if (head_dim != kHeadDim) return VSA_ERR_UNSUPPORTED;
  if (batch < 1 || num_heads < 1 || num_heads > kMaxHeads || seq_len < kBlock ||
      seq_len % kBlock != 0)
    return VSA_ERR_SHAPE;
  const int64_t nblk = seq_len / kBlock;
  if (nblk > kMaxBlocks) return VSA_ERR_SHAPE;
  if ((int64_t)batch * num_heads * nblk > kMaxTriples) return VSA_ERR_SHAPE;
  return VSA_OK;
}

AttnParams base_params(int32_t batch, int32_t seq_len, int32_t num_heads, float sm_scale) {
  AttnParams p = {};
  p.batch = batch;
  p.seq = seq_len;
  p.heads = num_heads;
  p.nblk = seq_len / kBlock;
  p.items_per_bh = p.nblk;
  p.n_items = batch * num_heads * p.nblk;
  p.items_per_xcd = (p.n_items + 7) / 8;
  p.c = sm_scale * 1.4426950408889634f;   // log2(e): softmax evaluated with exp2
  return p;
}

}  // namespace

extern "C" const char* vsa_status_string(vsa_status s) {
  switch (s) {
    case VSA_OK: return "VSA_OK";
    case VSA_ERR_NULL: return "VSA_ERR_NULL: a required pointer is NULL";
    case VSA_ERR_SHAPE: return "VSA_ERR_SHAPE: a size argument is out of range or inconsistent";
    case VSA_ERR_ALIGN: return "VSA_ERR_ALIGN: a pointer is not aligned as documented";
    case VSA_ERR_UNSUPPORTED: return "VSA_ERR_UNSUPPORTED: head_dim must be 128";
    case VSA_ERR_LAUNCH: return "VSA_ERR_LAUNCH: the HIP runtime rejected a kernel launch";
    case VSA_ERR_WORKSPACE: return "VSA_ERR_WORKSPACE: workspace missing or too small";
    case VSA_ERR_VALUE: return "VSA_ERR_VALUE: sm_scale not finite and >= 0, or unknown flags";
    case VSA_ERR_SCRATCH:
      return "VSA_ERR_SCRATCH: the shape needs more scratch than the fixed buffer of vsa_fwd_noalloc";
  }
  return "VSA_ERR_UNKNOWN";
}

extern "C" size_t vsa_fwd_workspace_size(int32_t batch, int32_t seq_len, int32_t num_heads,
                                         int32_t head_dim) {
  if (check_common(batch, seq_len, num_heads, head_dim) != VSA_OK) return 0;
  return ws_layout(batch, num_heads, seq_len / kBlock, 0).total;
}

extern "C" size_t vsa_fwd_proxy_workspace_size(int32_t batch, int32_t seq_len, int32_t prefix_len,
                                               int32_t num_heads, int32_t head_dim) {
  if (check_common(batch, seq_len, num_heads, head_dim) != VSA_OK) return 0;
  if (prefix_len <= 0 || prefix_len >= seq_len || prefix_len % kBlock != 0) return 0;
  const int64_t nvideo = (seq_len - prefix_len) / kBlock;
  const int64_t nblk = seq_len / kBlock;
  return ws_layout(batch, num_heads, nblk, (nvideo + kBlock - 1) / kBlock, prefix_len / kBlock,
                   prefix_splits(nblk)).total;
}

namespace {

// Checks shared by vsa_fwd and its two stages.
vsa_status check_fwd(const void* q, const void* k, const void* v, const int32_t* topk_idx,
                     const int32_t* vbs, const void* out, int32_t batch, int32_t seq_len,
                     int32_t num_heads, int32_t head_dim, int32_t topk, float sm_scale,
                     const void* workspace, size_t workspace_bytes, bool need_q, bool need_v) {
  if ((need_q && (!q || !k || !topk_idx || !out)) || (need_v && !v) || !vbs) return VSA_ERR_NULL;
  vsa_status st = check_common(batch, seq_len, num_heads, head_dim);
  if (st != VSA_OK) return st;
  const int nblk = seq_len / kBlock;
  if (need_q) {
    if (topk < 1 || topk > nblk) return VSA_ERR_SHAPE;
    if ((size_t)topk * 8 > kMaxDynLds) return VSA_ERR_SHAPE;   // 8 bytes of tile table per entry
    if (!isfinite(sm_scale) || sm_scale < 0.0f) return VSA_ERR_VALUE;
    if (!is_aligned(q, 16) || !is_aligned(k, 16) || !is_aligned(out, 16) ||
        !is_aligned(topk_idx, 4))
      return VSA_ERR_ALIGN;
  }
  if (need_v && !is_aligned(v, 16)) return VSA_ERR_ALIGN;
  if (!is_aligned(vbs, 4)) return VSA_ERR_ALIGN;
  const WsLayout ws = ws_layout(batch, num_heads, nblk, 0);
  if (!workspace || workspace_bytes < ws.total) return VSA_ERR_WORKSPACE;
  if (!is_aligned(workspace, kWsAlign)) return VSA_ERR_ALIGN;
  return VSA_OK;
}

vsa_status enqueue_pack(const void* v, const int32_t* vbs, int32_t batch, int32_t seq_len,
                        int32_t num_heads, void* workspace, hipStream_t s) {
  const int nblk = seq_len / kBlock;
  const WsLayout ws = ws_layout(batch, num_heads, nblk, 0);
  uint8_t* wsb = (uint8_t*)workspace;
  PackParams pk = {};
  pk.src = (const uint16_t*)v;
  pk.dst = wsb + ws.vt;
  pk.flags = wsb + ws.vf;
  pk.vbs = vbs;
  pk.src_rows = seq_len;
  pk.heads = num_heads;
  pk.tiles = nblk;
  pk.row_offset = 0;
  return launch_pack(pk, batch, s) == hipSuccess ? VSA_OK : VSA_ERR_LAUNCH;
}

vsa_status enqueue_attend(const void* q, const void* k, const int32_t* topk_idx,
                          const int32_t* vbs, void* out, int32_t batch, int32_t seq_len,
                          int32_t num_heads, int32_t topk, float sm_scale, void* workspace,
                          hipStream_t s, float* lse = nullptr, uint32_t flags = 0) {
  const int nblk = seq_len / kBlock;
  const WsLayout ws = ws_layout(batch, num_heads, nblk, 0);
  uint8_t* wsb = (uint8_t*)workspace;
  AttnParams p = base_params(batch, seq_len, num_heads, sm_scale);
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.vt = wsb + ws.vt;
  p.vt_flags = wsb + ws.vf;
  p.sched = (int*)(wsb + ws.sc);
  p.idx = topk_idx;
  p.vbs = vbs;
  p.out = (uint16_t*)out;
  p.idx_width = topk;
  p.seg_tiles = topk;
  p.table_cap = topk;
  p.lse = lse;
  p.sweep_rate = (flags & VSA_FLAG_SHARED_SWEEP) ? 1.0f : 0.0f;   // set from the shape at launch
  return launch_attn(p, false, s) == hipSuccess ? VSA_OK : VSA_ERR_LAUNCH;
}

}  // namespace

extern "C" vsa_status vsa_fwd(const void* q, const void* k, const void* v,
                              const int32_t* topk_idx, const int32_t* vbs, void* out,
                              int32_t batch, int32_t seq_len, int32_t num_heads, int32_t head_dim,
                              int32_t topk, float sm_scale, void* workspace,
                              size_t workspace_bytes, vsa_stream_t stream) {
  vsa_status st = check_fwd(q, k, v, topk_idx, vbs, out, batch, seq_len, num_heads, head_dim,
                            topk, sm_scale, workspace, workspace_bytes, true, true);
  if (st != VSA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  st = enqueue_pack(v, vbs, batch, seq_len, num_heads, workspace, s);
  if (st != VSA_OK) return st;
  return enqueue_attend(q, k, topk_idx, vbs, out, batch, seq_len, num_heads, topk, sm_scale,
                        workspace, s);
}

// ---- forward without allocation ------------------------------------------
// The scratch of vsa_fwd_noalloc: one fixed array per GPU, held by the loaded
// library until the process ends.  Host code reaches it only through the
// device address hipGetSymbolAddress returns for the current device (the
// array's name is a host-side stand-in, not a device address).
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this GPU's scratch array, looked up once per device with
// that device current; nullptr if the lookup fails.
void* scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" size_t vsa_fwd_noalloc_max_bytes(void) { return kScratchBytes; }

extern "C" vsa_status vsa_fwd_noalloc(const void* q, const void* k, const void* v,
                                      const int32_t* topk_idx, const int32_t* vbs, void* out,
                                      int32_t batch, int32_t seq_len, int32_t num_heads,
                                      int32_t head_dim, int32_t topk, float sm_scale,
                                      vsa_stream_t stream) {
  // shape checks first (with a stand-in workspace size), then the scratch limit
  vsa_status st = check_fwd(q, k, v, topk_idx, vbs, out, batch, seq_len, num_heads, head_dim,
                            topk, sm_scale, (void*)kWsAlign, (size_t)-1, true, true);
  if (st != VSA_OK) return st;
  if (ws_layout(batch, num_heads, seq_len / kBlock, 0).total > kScratchBytes) return VSA_ERR_SCRATCH;
  void* ws = scratch_address();
  if (ws == nullptr) return VSA_ERR_LAUNCH;
  hipStream_t s = (hipStream_t)stream;
  st = enqueue_pack(v, vbs, batch, seq_len, num_heads, ws, s);
  if (st != VSA_OK) return st;
  return enqueue_attend(q, k, topk_idx, vbs, out, batch, seq_len, num_heads, topk, sm_scale, ws, s);
}

extern "C" vsa_status vsa_fwd_ex(const void* q, const void* k, const void* v,
                                 const int32_t* topk_idx, const int32_t* vbs, void* out,
                                 int32_t batch, int32_t seq_len, int32_t num_heads,
                                 int32_t head_dim, int32_t topk, float sm_scale, uint32_t flags,
                                 void* workspace, size_t workspace_bytes, vsa_stream_t stream) {
  if (flags & ~(uint32_t)VSA_FLAG_SHARED_SWEEP) return VSA_ERR_VALUE;
  vsa_status st = check_fwd(q, k, v, topk_idx, vbs, out, batch, seq_len, num_heads, head_dim,
                            topk, sm_scale, workspace, workspace_bytes, true, true);
  if (st != VSA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  st = enqueue_pack(v, vbs, batch, seq_len, num_heads, workspace, s);
  if (st != VSA_OK) return st;
  return enqueue_attend(q, k, topk_idx, vbs, out, batch, seq_len, num_heads, topk, sm_scale,
                        workspace, s, nullptr, flags);
}

extern "C" vsa_status vsa_fwd_prepacked_ex(const void* q, const void* k, const int32_t* topk_idx,
                                           const int32_t* vbs, void* out, int32_t batch,
                                           int32_t seq_len, int32_t num_heads, int32_t head_dim,
                                           int32_t topk, float sm_scale, uint32_t flags,
                                           void* workspace, size_t workspace_bytes,
                                           vsa_stream_t stream) {
  if (flags & ~(uint32_t)VSA_FLAG_SHARED_SWEEP) return VSA_ERR_VALUE;
  vsa_status st = check_fwd(q, k, nullptr, topk_idx, vbs, out, batch, seq_len, num_heads,
                            head_dim, topk, sm_scale, workspace, workspace_bytes, true, false);
  if (st != VSA_OK) return st;
  return enqueue_attend(q, k, topk_idx, vbs, out, batch, seq_len, num_heads, topk, sm_scale,
                        workspace, (hipStream_t)stream, nullptr, flags);
}

extern "C" vsa_status vsa_fwd_lse(const void* q, const void* k, const void* v,
                                  const int32_t* topk_idx, const int32_t* vbs, void* out,
                                  float* lse, int32_t batch, int32_t seq_len, int32_t num_heads,
                                  int32_t head_dim, int32_t topk, float sm_scale, void* workspace,
                                  size_t workspace_bytes, vsa_stream_t stream) {
  if (!lse) return VSA_ERR_NULL;
  vsa_status st = check_fwd(q, k, v, topk_idx, vbs, out, batch, seq_len, num_heads, head_dim,
                            topk, sm_scale, workspace, workspace_bytes, true, true);
  if (st != VSA_OK) return st;
  if (!is_aligned(lse, 4)) return VSA_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  st = enqueue_pack(v, vbs, batch, seq_len, num_heads, workspace, s);
  if (st != VSA_OK) return st;
  return enqueue_attend(q, k, topk_idx, vbs, out, batch, seq_len, num_heads, topk, sm_scale,
                        workspace, s, lse);
}

extern "C" vsa_status vsa_merge(const void* o1, const float* lse1, const void* o2,
                                const float* lse2, void* out, float* lse_out, int32_t batch,
                                int32_t seq_len, int32_t num_heads, int32_t head_dim,
                                vsa_stream_t stream) {
  if (!o1 || !lse1 || !o2 || !lse2 || !out || !lse_out) return VSA_ERR_NULL;
  if (batch < 1 || seq_len < 1 || num_heads < 1 || head_dim < 8 || head_dim % 8 != 0)
    return VSA_ERR_SHAPE;
  if ((int64_t)batch * seq_len * num_heads * head_dim >= ((int64_t)1 << 40)) return VSA_ERR_SHAPE;
  if (!is_aligned(o1, 16) || !is_aligned(o2, 16) || !is_aligned(out, 16) || !is_aligned(lse1, 4) ||
      !is_aligned(lse2, 4) || !is_aligned(lse_out, 4))
    return VSA_ERR_ALIGN;
  return launch_merge((const uint16_t*)o1, lse1, (const uint16_t*)o2, lse2, (uint16_t*)out, lse_out,
                      batch, seq_len, num_heads, head_dim, (hipStream_t)stream) == hipSuccess
             ? VSA_OK
             : VSA_ERR_LAUNCH;
}

extern "C" vsa_status vsa_pack_values(const void* v, const int32_t* vbs, int32_t batch,
                                      int32_t seq_len, int32_t num_heads, int32_t head_dim,
                                      void* workspace, size_t workspace_bytes,
                                      vsa_stream_t stream) {
  vsa_status st = check_fwd(nullptr, nullptr, v, nullptr, vbs, nullptr, batch, seq_len, num_heads,
                            head_dim, 1, 0.0f, workspace, workspace_bytes, false, true);
  if (st != VSA_OK) return st;
  return enqueue_pack(v, vbs, batch, seq_len, num_heads, workspace, (hipStream_t)stream);
}

extern "C" vsa_status vsa_fwd_prepacked(const void* q, const void* k, const int32_t* topk_idx,
                                        const int32_t* vbs, void* out, int32_t batch,
                                        int32_t seq_len, int32_t num_heads, int32_t head_dim,
                                        int32_t topk, float sm_scale, void* workspace,
                                        size_t workspace_bytes, vsa_stream_t stream) {
  vsa_status st = check_fwd(q, k, nullptr, topk_idx, vbs, out, batch, seq_len, num_heads,
                            head_dim, topk, sm_scale, workspace, workspace_bytes, true, false);
  if (st != VSA_OK) return st;
  return enqueue_attend(q, k, topk_idx, vbs, out, batch, seq_len, num_heads, topk, sm_scale,
                        workspace, (hipStream_t)stream);
}

extern "C" vsa_status vsa_preprocess(const void* k, const void* v, const int32_t* vbs,
                                     void* kmean, void* vsum, int32_t batch, int32_t seq_len,
                                     int32_t num_heads, int32_t head_dim, vsa_stream_t stream) {
  if (!k || !v || !vbs || !kmean || !vsum) return VSA_ERR_NULL;
  vsa_status st = check_common(batch, seq_len, num_heads, head_dim);
  if (st != VSA_OK) return st;
  if (!is_aligned(k, 16) || !is_aligned(v, 16) || !is_aligned(kmean, 16) ||
      !is_aligned(vsum, 16) || !is_aligned(vbs, 4))
    return VSA_ERR_ALIGN;
  if (launch_preprocess((const uint16_t*)k, (const uint16_t*)v, vbs, (uint16_t*)kmean,
                        (uint16_t*)vsum, batch, seq_len, num_heads,
                        (hipStream_t)stream) != hipSuccess)
    return VSA_ERR_LAUNCH;
  return VSA_OK;
}

extern "C" vsa_status vsa_kc_stats(const void* kmean, const int32_t* vbs, float* kc_mean,
                                   float* kc_var_diag, int32_t batch, int32_t num_blocks,
                                   int32_t num_heads, int32_t head_dim, int32_t first_block,
                                   int32_t block_count, vsa_stream_t stream) {
  if (!kmean || !vbs || !kc_mean || !kc_var_diag) return VSA_ERR_NULL;
  if (head_dim != kHeadDim) return VSA_ERR_UNSUPPORTED;
  if (batch < 1 || num_heads < 1 || num_heads > kMaxHeads || num_blocks < 1 ||
      num_blocks > kMaxBlocks || first_block < 0 || block_count < 0 ||
      (int64_t)first_block + block_count > num_blocks)
    return VSA_ERR_SHAPE;
  if ((int64_t)batch * num_heads * 256 > kMaxLaunchThreads) return VSA_ERR_SHAPE;
  if (!is_aligned(kmean, 2) || !is_aligned(vbs, 4) || !is_aligned(kc_mean, 4) ||
      !is_aligned(kc_var_diag, 4))
    return VSA_ERR_ALIGN;
  return launch_kc_stats((const uint16_t*)kmean, vbs, kc_mean, kc_var_diag, batch, num_blocks,
                         num_heads, first_block, block_count, (hipStream_t)stream) == hipSuccess
             ? VSA_OK
             : VSA_ERR_LAUNCH;
}

namespace {

// How a proxy call names the exactly computed video blocks of each query block.
struct Selection {
  int format;               // 0 padded rows, 1 bitmask, 2 BSR
  const int32_t* idx;       // padded rows [B, H, Nv, max_sel], -1 = empty slot
  const uint32_t* mask;     // bitmask rows [B, H, Nv, ceil(Nv/32)]
  const int32_t* indptr;    // BSR row pointers [B*H*Nv + 1]
  const int32_t* indices;   // BSR video-relative block ids
  int nnz;                  // BSR: entries in indices
  int max_sel;              // padded width, or the expected selection size
};

vsa_status proxy_call(const void* q, const void* k, const void* v, const Selection& sel,
                      const int32_t* vbs, const void* kmean, const void* vsum, void* out,
                      int32_t batch, int32_t seq_len, int32_t prefix_len, int32_t num_heads,
                      int32_t head_dim, float sm_scale, void* workspace, size_t workspace_bytes,
                      vsa_stream_t stream) {
  const bool have_sel = sel.format == 0 ? sel.idx != nullptr
                        : sel.format == 1 ? sel.mask != nullptr
                                          : (sel.indptr != nullptr && sel.indices != nullptr);
  if (!q || !k || !v || !have_sel || !vbs || !kmean || !vsum || !out) return VSA_ERR_NULL;
  vsa_status st = check_common(batch, seq_len, num_heads, head_dim);
  if (st != VSA_OK) return st;
  if (prefix_len <= 0 || prefix_len >= seq_len || prefix_len % kBlock != 0) return VSA_ERR_SHAPE;
  const int nblk = seq_len / kBlock;
  const int nprefix = prefix_len / kBlock;
  const int nvideo = nblk - nprefix;
  const int nproxy = (nvideo + kBlock - 1) / kBlock;
  const int max_sel = sel.max_sel;
  if (max_sel < 1 || max_sel > nvideo) return VSA_ERR_SHAPE;
  if (sel.format == 2 && sel.nnz < 0) return VSA_ERR_SHAPE;
  // rows of a bitmask or BSR selection may hold up to nvideo blocks
  const int row_cap = sel.format == 0 ? max_sel : nvideo;
  const int psplit = prefix_splits(nblk);
  const int pwidth = std::min<int>(kPrefixSplit, nblk);
  const int64_t items_per_bh = (int64_t)nprefix * psplit + nvideo;
  // one 128-thread workgroup per work item, 8 * ceil(items / 8) of them
  if ((int64_t)batch * num_heads * items_per_bh + 8 > kMaxLaunchThreads / 128) return VSA_ERR_SHAPE;
  const int table_cap = std::max(pwidth, nprefix + row_cap + nproxy);
  const int words = (nvideo + 31) / 32;
  // tile table of 8 bytes per entry; video items add a byte of weight per
  // video block and the selected-block bits
  const size_t table = (size_t)table_cap * 8;
  const size_t video = (size_t)(nprefix + row_cap + nproxy) * 8 + (size_t)nproxy * kBlock +
                       (size_t)nproxy * 8;
  const size_t dyn = table > video ? table : video;
  if (dyn > kMaxDynLds) return VSA_ERR_SHAPE;
  if (!isfinite(sm_scale) || sm_scale < 0.0f) return VSA_ERR_VALUE;
  if (!is_aligned(q, 16) || !is_aligned(k, 16) || !is_aligned(v, 16) || !is_aligned(out, 16) ||
      !is_aligned(kmean, 16) || !is_aligned(vsum, 16) || !is_aligned(vbs, 4) ||
      (sel.idx && !is_aligned(sel.idx, 4)) || (sel.mask && !is_aligned(sel.mask, 4)) ||
      (sel.indptr && !is_aligned(sel.indptr, 4)) || (sel.indices && !is_aligned(sel.indices, 4)))
    return VSA_ERR_ALIGN;
  const WsLayout ws = ws_layout(batch, num_heads, nblk, nproxy, nprefix, psplit);
  if (!workspace || workspace_bytes < ws.total) return VSA_ERR_WORKSPACE;
  if (!is_aligned(workspace, kWsAlign)) return VSA_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  uint8_t* wsb = (uint8_t*)workspace;

  PackParams pk = {};
  pk.src = (const uint16_t*)v;
  pk.dst = wsb + ws.vt;
  pk.flags = wsb + ws.vf;
  pk.vbs = vbs;
  pk.src_rows = seq_len;
  pk.heads = num_heads;
  pk.tiles = nblk;
  if (launch_pack(pk, batch, s) != hipSuccess) return VSA_ERR_LAUNCH;
  PackParams pp = {};
  pp.src = (const uint16_t*)vsum;
  pp.dst = wsb + ws.pt;
  pp.flags = wsb + ws.pf;
  pp.vbs = nullptr;
  pp.src_rows = nblk;
  pp.heads = num_heads;
  pp.tiles = nproxy;
  pp.row_offset = nprefix;
  pp.valid_rows = nvideo;
  if (launch_pack(pp, batch, s) != hipSuccess) return VSA_ERR_LAUNCH;

  AttnParams p = base_params(batch, seq_len, num_heads, sm_scale);
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.kmean = (const uint16_t*)kmean;
  p.vt = wsb + ws.vt;
  p.vt_flags = wsb + ws.vf;
  p.sched = (int*)(wsb + ws.sc);
  p.pt = wsb + ws.pt;
  p.pt_flags = wsb + ws.pf;
  p.idx = sel.idx;
  p.sel_format = sel.format;
  p.sel_mask = sel.mask;
  p.sel_words = words;
  p.sel_indptr = sel.indptr;
  p.sel_indices = sel.indices;
  p.sel_nnz = sel.nnz;
  p.vbs = vbs;
  p.out = (uint16_t*)out;
  p.idx_width = max_sel;
  p.seg_tiles = nprefix + max_sel + nproxy;
  p.nprefix = nprefix;
  p.nvideo = nvideo;
  p.nproxy = nproxy;
  p.table_cap = table_cap;
  p.items_per_bh = (int)items_per_bh;
  p.n_items = (int)((int64_t)batch * num_heads * items_per_bh);
  p.items_per_xcd = (p.n_items + 7) / 8;
  p.psplit = psplit;
  p.pwidth = pwidth;
  p.part_o = (float*)(wsb + ws.po);
  p.part_lse = (float*)(wsb + ws.pl);
  if (launch_attn(p, true, s) != hipSuccess) return VSA_ERR_LAUNCH;
  if (launch_prefix_merge(p.part_o, p.part_lse, vbs, (uint16_t*)out, batch, seq_len, num_heads,
                          nprefix, psplit, s) != hipSuccess)
    return VSA_ERR_LAUNCH;
  return VSA_OK;
}

}  // namespace

extern "C" vsa_status vsa_fwd_proxy(const void* q, const void* k, const void* v,
                                    const int32_t* sel_idx, const int32_t* vbs,
                                    const void* kmean, const void* vsum, void* out,
                                    int32_t batch, int32_t seq_len, int32_t prefix_len,
                                    int32_t num_heads, int32_t head_dim, int32_t max_sel,
                                    float sm_scale, void* workspace, size_t workspace_bytes,
                                    vsa_stream_t stream) {
  Selection sel = {};
  sel.format = 0;
  sel.idx = sel_idx;
  sel.max_sel = max_sel;
  return proxy_call(q, k, v, sel, vbs, kmean, vsum, out, batch, seq_len, prefix_len, num_heads,
                    head_dim, sm_scale, workspace, workspace_bytes, stream);
}

extern "C" vsa_status vsa_fwd_proxy_bitmask(const void* q, const void* k, const void* v,
                                            const uint32_t* sel_mask, const int32_t* vbs,
                                            const void* kmean, const void* vsum, void* out,
                                            int32_t batch, int32_t seq_len, int32_t prefix_len,
                                            int32_t num_heads, int32_t head_dim,
                                            int32_t expected_sel, float sm_scale,
                                            void* workspace, size_t workspace_bytes,
                                            vsa_stream_t stream) {
  Selection sel = {};
  sel.format = 1;
  sel.mask = sel_mask;
  sel.max_sel = expected_sel;
  return proxy_call(q, k, v, sel, vbs, kmean, vsum, out, batch, seq_len, prefix_len, num_heads,
                    head_dim, sm_scale, workspace, workspace_bytes, stream);
}

extern "C" vsa_status vsa_fwd_proxy_bsr(const void* q, const void* k, const void* v,
                                        const int32_t* sel_indptr, const int32_t* sel_indices,
                                        int32_t nnz, const int32_t* vbs, const void* kmean,
                                        const void* vsum,
                                        void* out, int32_t batch, int32_t seq_len,
                                        int32_t prefix_len, int32_t num_heads, int32_t head_dim,
                                        int32_t expected_sel, float sm_scale, void* workspace,
                                        size_t workspace_bytes, vsa_stream_t stream) {
  Selection sel = {};
  sel.format = 2;
  sel.indptr = sel_indptr;
  sel.indices = sel_indices;
  sel.nnz = nnz;
  sel.max_sel = expected_sel;
  return proxy_call(q, k, v, sel, vbs, kmean, vsum, out, batch, seq_len, prefix_len, num_heads,
                    head_dim, sm_scale, workspace, workspace_bytes, stream);
}

namespace {

int64_t cube_count(int32_t T, int32_t Hh, int32_t W) {
  if (T < 1 || Hh < 1 || W < 1) return 0;
  const int64_t n = ((int64_t)T + 3) / 4 * (((int64_t)Hh + 3) / 4) * (((int64_t)W + 3) / 4);
  if (n * kBlock >= ((int64_t)1 << 31)) return 0;
  return n;
}

vsa_status check_tile(const void* a, const void* b, int32_t batch, int32_t T, int32_t Hh, int32_t W,
                      int32_t num_heads, int32_t head_dim) {
  if (!a || !b) return VSA_ERR_NULL;
  if (batch < 1 || num_heads < 1 || head_dim < 1 || cube_count(T, Hh, W) == 0) return VSA_ERR_SHAPE;
  if (((int64_t)num_heads * head_dim) % 8 != 0) return VSA_ERR_SHAPE;
  // one 256-thread workgroup per row
  const int64_t rows = (int64_t)batch * kBlock * cube_count(T, Hh, W);
  if (rows > kMaxLaunchThreads / 256) return VSA_ERR_SHAPE;
  if (!is_aligned(a, 16) || !is_aligned(b, 16)) return VSA_ERR_ALIGN;
  return VSA_OK;
}

}  // namespace

extern "C" size_t vsa_cube_count(int32_t T, int32_t Hh, int32_t W) {
  return (size_t)cube_count(T, Hh, W);
}

extern "C" vsa_status vsa_cube_vbs(int32_t T, int32_t Hh, int32_t W, int32_t* vbs_host, size_t n) {
  if (!vbs_host) return VSA_ERR_NULL;
  const int64_t cubes = cube_count(T, Hh, W);
  if (cubes == 0 || (int64_t)n < cubes) return VSA_ERR_SHAPE;
  const int ct = (T + 3) / 4, ch = (Hh + 3) / 4, cw = (W + 3) / 4;
  for (int a = 0; a < ct; ++a)
    for (int b = 0; b < ch; ++b)
      for (int c = 0; c < cw; ++c) {
        const int et = T - 4 * a < 4 ? T - 4 * a : 4;
        const int eh = Hh - 4 * b < 4 ? Hh - 4 * b : 4;
        const int ew = W - 4 * c < 4 ? W - 4 * c : 4;
        vbs_host[(a * ch + b) * cw + c] = et * eh * ew;
      }
  return VSA_OK;
}

extern "C" vsa_status vsa_tile(const void* x, void* x_tiled, int32_t batch, int32_t T, int32_t Hh,
                               int32_t W, int32_t num_heads, int32_t head_dim,
                               vsa_stream_t stream) {
  vsa_status st = check_tile(x, x_tiled, batch, T, Hh, W, num_heads, head_dim);
  if (st != VSA_OK) return st;
  return launch_tile(x, x_tiled, batch, T, Hh, W, (int64_t)num_heads * head_dim * 2, false,
                     (hipStream_t)stream) == hipSuccess
             ? VSA_OK
             : VSA_ERR_LAUNCH;
}

extern "C" vsa_status vsa_untile(const void* x_tiled, void* x, int32_t batch, int32_t T, int32_t Hh,
                                 int32_t W, int32_t num_heads, int32_t head_dim,
                                 vsa_stream_t stream) {
  vsa_status st = check_tile(x_tiled, x, batch, T, Hh, W, num_heads, head_dim);
  if (st != VSA_OK) return st;
  return launch_tile(x_tiled, x, batch, T, Hh, W, (int64_t)num_heads * head_dim * 2, true,
                     (hipStream_t)stream) == hipSuccess
             ? VSA_OK
             : VSA_ERR_LAUNCH;
}

extern "C" size_t vsa_route_workspace_size(int32_t batch, int32_t num_blocks, int32_t num_heads) {
  if (batch < 1 || num_heads < 1 || num_blocks < 1 || num_blocks > kMaxRouteBlocks) return 0;
  if ((int64_t)batch * num_heads * num_blocks >= ((int64_t)1 << 31)) return 0;
  return align_up(route_workspace_bytes(batch, num_heads, num_blocks), kWsAlign);
}

extern "C" vsa_status vsa_route_topk(const void* qmean, const void* kmean, const int32_t* vbs,
                                     int32_t* topk_idx, int32_t batch, int32_t num_blocks,
                                     int32_t num_heads, int32_t head_dim, int32_t topk,
                                     void* workspace, size_t workspace_bytes, vsa_stream_t stream) {
  if (!qmean || !kmean || !vbs || !topk_idx) return VSA_ERR_NULL;
  if (head_dim != kHeadDim) return VSA_ERR_UNSUPPORTED;
  if (batch < 1 || num_heads < 1 || num_blocks < 1 || num_blocks > kMaxRouteBlocks ||
      topk < 1 || topk > num_blocks)
    return VSA_ERR_SHAPE;
  if ((int64_t)batch * num_heads * num_blocks * topk >= ((int64_t)1 << 31)) return VSA_ERR_SHAPE;
  if (!is_aligned(qmean, 16) || !is_aligned(kmean, 16) || !is_aligned(vbs, 4) ||
      !is_aligned(topk_idx, 4))
    return VSA_ERR_ALIGN;
  if (!workspace || workspace_bytes < vsa_route_workspace_size(batch, num_blocks, num_heads))
    return VSA_ERR_WORKSPACE;
  if (!is_aligned(workspace, kWsAlign)) return VSA_ERR_ALIGN;
  return launch_route((const uint16_t*)qmean, (const uint16_t*)kmean, vbs, topk_idx, batch,
                      num_blocks, num_heads, topk, (double*)workspace, (hipStream_t)stream) == hipSuccess
             ? VSA_OK
             : VSA_ERR_LAUNCH;
}
