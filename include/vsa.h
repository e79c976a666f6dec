/*
 * vsa.h -- C ABI of the MI355X (gfx950) Video Sparse Attention forward library.
 *
 * The library computes the fine block-sparse attention stage of Video Sparse
 * Attention (VSA).  Definitions it follows (cited by page title and section):
 *
 *   [OC]  Wan2.2 production-values dataset card, "Operator contract": non-causal
 *         block-sparse attention in BSHD layout, out = softmax(q k_sel^T / sqrt(D)) v_sel;
 *         for each (batch, head, query cube) topk_idx names the selected KV cubes
 *         and vbs[c] keeps only the first vbs[c] of the 64 slots of cube c.
 *   [SH]  same card, "Shapes": 64-token cubes, D = 128, sm_scale = 1/sqrt(128).
 *   [RUN] TensorRT-Edge-LLM "Video Sparse Attention Runner": the preprocess entry
 *         (BF16 [numBlocks, numHeads, 128] block means of K and block sums of V),
 *         the packed [prefix | video] proxy forward, status-by-return calls that
 *         run asynchronously on a caller stream with a caller-owned workspace.
 *   [PX]  FlashInfer proxy-compensation description on the TensorRT-LLM VisualGen
 *         VSA PR page: an omitted block is represented by one averaged key and one
 *         value total; exactly computed blocks get no proxy; each proxy term is
 *         weighted in the softmax denominator by the real tokens it represents.
 *
 * Conventions shared by every entry point
 *   - Tensors are caller-owned DEVICE memory on the current HIP device.  The
 *     library never allocates, frees, synchronises or logs.
 *   - q, k, v, out, kmean, vsum: bf16, BSHD [batch, rows, heads, 128], contiguous,
 *     16-byte aligned.  Index and vbs arrays: int32, contiguous, 4-byte aligned.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream).  A
 *     call returns after enqueueing; results are ready when the stream is.
 *   - Host-side argument checks run before anything is enqueued; on error
 *     nothing is enqueued and the status says why.  Data preconditions (indices
 *     in range and distinct per row, 0 <= vbs <= 64) are NOT checked on the
 *     device: an out-of-range index is skipped, a repeated index is counted twice.
 *   - Calls that share a workspace must not overlap in time (every attention
 *     call writes the workspace's scheduling counters).
 *   - Only head_dim == 128 is supported ([SH]; the head geometry is fixed at
 *     compile time, as in [RUN]).
 *   - Size limits (VSA_ERR_SHAPE otherwise): seq_len a positive multiple of 64
 *     with at most 2^20 - 1 cubes, 1 <= num_heads <= 65536, batch >= 1, and
 *     batch * num_heads * seq_len/64 <= 2^23 (no launch exceeds 2^31 threads;
 *     the V packing runs 256 threads per (batch, head, cube)).  The
 *     per-workgroup tile table takes 8 bytes per entry out of 32 KB of LDS:
 *     topk <= 4096 for vsa_fwd; proxy calls need, for a video row, 8 bytes per
 *     possible tile (prefix blocks + row width + proxy tiles) plus 72 bytes per
 *     64 video blocks within the same 32 KB, and batch * num_heads * (prefix
 *     blocks * ceil(seq_len/64 / 96) + video blocks) <= 2^24 - 8 work items.
 */
#ifndef VSA_H
#define VSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as hipStream_t (HIP declares it as a pointer to this struct). */
struct ihipStream_t;
typedef struct ihipStream_t* vsa_stream_t;

typedef enum vsa_status {
  VSA_OK = 0,
  VSA_ERR_NULL = 1,        /* a required pointer is NULL                           */
  VSA_ERR_SHAPE = 2,       /* a size argument is out of range or inconsistent     */
  VSA_ERR_ALIGN = 3,       /* a pointer is not aligned as documented              */
  VSA_ERR_UNSUPPORTED = 4, /* head_dim != 128                                     */
  VSA_ERR_LAUNCH = 5,      /* the HIP runtime rejected a kernel launch            */
  VSA_ERR_WORKSPACE = 6,   /* workspace missing or smaller than required          */
  VSA_ERR_VALUE = 7,       /* sm_scale negative, NaN or infinite; unknown flags   */
  VSA_ERR_SCRATCH = 8      /* vsa_fwd_noalloc: the shape exceeds its fixed scratch */
} vsa_status;

/* Human-readable name of a status code (static storage, never NULL). */
const char* vsa_status_string(vsa_status s);

/*
 * Accumulation order.  By default the attention kernels visit each query
 * cube's KV tiles in an order that depends only on the shapes: repeated calls
 * with the same inputs give bitwise identical outputs, and the output does not
 * depend on the order of the entries of an index row.  Which workgroup runs
 * a query cube changes from call to call (the last ones are balanced across
 * the XCDs at run time); its result does not.  The library holds no mutable
 * state between calls.
 *
 * VSA_FLAG_SHARED_SWEEP (vsa_fwd_ex, vsa_fwd_prepacked_ex) instead starts each
 * query cube's sweep over its KV cubes at a block taken from the GPU's
 * real-time counter, so that the query cubes of a head in flight at the same
 * time move through its K/V together and the XCD's L2 serves more of them
 * (40 heads x 624 cubes, 78 per row: about 3-5% less attention time, L2 hit
 * rate 0.68 -> 0.77; 40 x 1440 cubes, 180 per row: about 8% less).  The
 * result then depends on timing in the last bits of fp32 rounding, always
 * within the documented accuracy.
 */
#define VSA_FLAG_SHARED_SWEEP 1u

/*
 * Workspace bytes vsa_fwd needs for this shape (0 if the shape is invalid).
 * The workspace holds each (batch, head, cube) V tile transposed to key-major
 * half precision, plus one byte per tile, plus 2 KB of counters through which
 * the attention launch balances its last work items across the XCDs.  The
 * tiles are rewritten by every call that packs V (vsa_fwd, vsa_pack_values),
 * the counters by every call that runs the attention (vsa_fwd_prepacked
 * included), so even calls that only read the packed tiles must not overlap
 * on one workspace.
 */
size_t vsa_fwd_workspace_size(int32_t batch, int32_t seq_len, int32_t num_heads,
                              int32_t head_dim);

/*
 * vsa_fwd -- fine block-sparse attention forward ([OC]).
 *
 *   q, k, v       bf16 [batch, seq_len, num_heads, head_dim], cube-major tiled:
 *                 rows 64c .. 64c+63 form cube c.
 *   topk_idx      int32 [batch, num_heads, seq_len/64, topk]: selected KV cubes
 *                 of each (batch, head, query cube), in any order (the kernel
 *                 sorts each row, so the output is bitwise independent of the
 *                 order).
 *   vbs           int32 [seq_len/64]: valid rows of each cube, shared by all
 *                 batches and heads; rows >= vbs[c] are padding on both the
 *                 query and the key side.
 *   out           bf16 [batch, seq_len, num_heads, head_dim], written in full:
 *                 valid query rows get softmax(q k^T * sm_scale) v over the valid
 *                 rows of the selected cubes (rounded to nearest-even bf16);
 *                 padding rows, rows with no valid key and non-finite results get 0.
 *   sm_scale      finite, >= 0 (the pages use 1/sqrt(128)).
 *   workspace     device memory of at least vsa_fwd_workspace_size(...) bytes,
 *                 256-byte aligned.
 *
 * Returns VSA_OK, or the error that stopped the call before enqueueing.
 */
vsa_status vsa_fwd(const void* q, const void* k, const void* v,
                   const int32_t* topk_idx, const int32_t* vbs, void* out,
                   int32_t batch, int32_t seq_len, int32_t num_heads, int32_t head_dim,
                   int32_t topk, float sm_scale,
                   void* workspace, size_t workspace_bytes, vsa_stream_t stream);

/*
 * vsa_fwd_noalloc -- vsa_fwd for callers that cannot allocate (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).
 *
 * Same arguments, result and errors as vsa_fwd, minus the workspace: the
 * packed V tiles go to a fixed scratch array of vsa_fwd_noalloc_max_bytes()
 * bytes (64 MiB) that the library holds on each GPU it runs on until the
 * process ends.  VSA_ERR_SCRATCH when the shape needs more than that, i.e.
 * when batch * num_heads * seq_len/64 tiles of 16 KB (plus one byte each and
 * 2 KB of counters, 256-byte aligned) exceed it (about 4090 tiles: 8 heads x 84 cubes fit, the
 * 40 x 624 Wan2.2 shape does not).  The call allocates nothing and touches no
 * memory allocator.  Every call on one GPU shares that GPU's array, which is
 * fully rewritten by each call: calls that overlap in time on one GPU (two
 * streams, two threads) race and must be serialised by the caller.
 */
size_t vsa_fwd_noalloc_max_bytes(void);
vsa_status vsa_fwd_noalloc(const void* q, const void* k, const void* v,
                           const int32_t* topk_idx, const int32_t* vbs, void* out,
                           int32_t batch, int32_t seq_len, int32_t num_heads, int32_t head_dim,
                           int32_t topk, float sm_scale, vsa_stream_t stream);

/*
 * vsa_fwd_ex / vsa_fwd_prepacked_ex -- vsa_fwd / vsa_fwd_prepacked with
 * `flags`: 0 or VSA_FLAG_SHARED_SWEEP (see "Accumulation order");
 * VSA_ERR_VALUE for any other bit.  Other arguments as vsa_fwd.
 */
vsa_status vsa_fwd_ex(const void* q, const void* k, const void* v,
                      const int32_t* topk_idx, const int32_t* vbs, void* out,
                      int32_t batch, int32_t seq_len, int32_t num_heads, int32_t head_dim,
                      int32_t topk, float sm_scale, uint32_t flags,
                      void* workspace, size_t workspace_bytes, vsa_stream_t stream);
vsa_status vsa_fwd_prepacked_ex(const void* q, const void* k, const int32_t* topk_idx,
                                const int32_t* vbs, void* out,
                                int32_t batch, int32_t seq_len, int32_t num_heads,
                                int32_t head_dim, int32_t topk, float sm_scale, uint32_t flags,
                                void* workspace, size_t workspace_bytes,
                                vsa_stream_t stream);

/*
 * The two stages of vsa_fwd, for callers that time or schedule them apart.
 *
 * vsa_pack_values writes the packed V tiles of (v, vbs) into the workspace
 * (what vsa_fwd does first); vsa_fwd_prepacked runs the attention on a
 * workspace that vsa_pack_values filled for the same v, vbs and shape (what
 * vsa_fwd does second).  Arguments have the meaning given for vsa_fwd.
 * Running vsa_pack_values then vsa_fwd_prepacked on one stream gives exactly
 * the result of vsa_fwd.
 */
vsa_status vsa_pack_values(const void* v, const int32_t* vbs,
                           int32_t batch, int32_t seq_len, int32_t num_heads, int32_t head_dim,
                           void* workspace, size_t workspace_bytes, vsa_stream_t stream);

vsa_status vsa_fwd_prepacked(const void* q, const void* k, const int32_t* topk_idx,
                             const int32_t* vbs, void* out,
                             int32_t batch, int32_t seq_len, int32_t num_heads, int32_t head_dim,
                             int32_t topk, float sm_scale,
                             void* workspace, size_t workspace_bytes, vsa_stream_t stream);

/*
 * vsa_preprocess -- block summaries ([RUN] preprocess entry; [PX]).
 *
 *   k, v          bf16 [batch, seq_len, num_heads, head_dim].
 *   vbs           int32 [seq_len/64].
 *   kmean, vsum   bf16 [batch, seq_len/64, num_heads, head_dim] outputs:
 *                 kmean[b,c,h,:] = bf16(sum_{t<vbs[c]} k[b,64c+t,h,:] / vbs[c]),
 *                 vsum [b,c,h,:] = bf16(sum_{t<vbs[c]} v[b,64c+t,h,:]);
 *                 sums in float64, one rounding to nearest-even bf16;
 *                 vbs[c] == 0 gives zeros.
 */
vsa_status vsa_preprocess(const void* k, const void* v, const int32_t* vbs,
                          void* kmean, void* vsum,
                          int32_t batch, int32_t seq_len, int32_t num_heads, int32_t head_dim,
                          vsa_stream_t stream);

/*
 * vsa_kc_stats -- statistics of the block key means ([RUN] preprocess entry:
 * FP32 [numHeads, 128] mean and diagonal variance of KC, KC taken in its BF16
 * rounding).
 *
 *   kmean         bf16 [batch, num_blocks, num_heads, head_dim] block key means
 *                 (as written by vsa_preprocess), 2-byte aligned.
 *   vbs           int32 [num_blocks]; a block takes part when vbs > 0.
 *   first_block, block_count
 *                 the blocks c in [first_block, first_block + block_count) are
 *                 the population (for the packed proxy layout: the video blocks,
 *                 first_block = prefix_len / 64).
 *   kc_mean, kc_var_diag
 *                 float32 [batch, num_heads, head_dim] outputs, 4-byte aligned:
 *                 mean = sum(x_c) / n, var = sum((x_c - mean)^2) / n over the n
 *                 taking part (population variance), evaluated in float64 and
 *                 rounded to float32; both 0 when n = 0.
 *
 * VSA_ERR_SHAPE for an empty or out-of-range block range or sizes outside the
 * common limits; device memory, caller-owned, enqueued on `stream`.
 */
vsa_status vsa_kc_stats(const void* kmean, const int32_t* vbs, float* kc_mean,
                        float* kc_var_diag, int32_t batch, int32_t num_blocks, int32_t num_heads,
                        int32_t head_dim, int32_t first_block, int32_t block_count,
                        vsa_stream_t stream);

/* Workspace bytes vsa_fwd_proxy needs for this shape (0 if the shape is invalid):
 * the packed V and vsum tiles, and the partial results of the prefix query
 * blocks.  A prefix block attends to every key block, so it runs as
 * ceil(seq_len/64 / 96) parts over ranges of 96 key blocks; each part leaves
 * O/l in fp32 and its row log-sum-exp (batch * num_heads * prefix blocks *
 * parts * 64 * 129 floats), which a merge pass combines into the output. */
size_t vsa_fwd_proxy_workspace_size(int32_t batch, int32_t seq_len, int32_t prefix_len,
                                    int32_t num_heads, int32_t head_dim);

/*
 * vsa_fwd_proxy -- packed [prefix | video] proxy-compensated forward ([RUN]; [PX]).
 *
 *   q, k, v       bf16 [batch, seq_len, num_heads, head_dim]; rows < prefix_len
 *                 are the dense prefix, the rest are cube-major video rows.
 *   prefix_len    multiple of 64 with 0 < prefix_len < seq_len.
 *   vbs           int32 [seq_len/64] for every block (prefix blocks normally 64).
 *   sel_idx       int32 [batch, num_heads, (seq_len-prefix_len)/64, max_sel]:
 *                 video-relative block ids attended exactly by each video query
 *                 block (normally itself, its face neighbours and the routed
 *                 blocks); -1 marks an empty slot.
 *   kmean, vsum   bf16 [batch, seq_len/64, num_heads, head_dim] block summaries
 *                 (as written by vsa_preprocess).
 *   out           bf16 [batch, seq_len, num_heads, head_dim], written in full.
 *
 * A prefix query row attends exactly to every valid key.  A video query row in
 * video block qv attends exactly to the valid keys of all prefix blocks and of
 * the blocks in sel_idx[b,h,qv,:]; every other video block c with vbs > 0 adds a
 * proxy term: logit t = (q . kmean_c) * sm_scale, exp(t) * vsum_c to the
 * numerator and exp(t) * vbs[c] to the denominator.
 */
vsa_status vsa_fwd_proxy(const void* q, const void* k, const void* v,
                         const int32_t* sel_idx, const int32_t* vbs,
                         const void* kmean, const void* vsum, void* out,
                         int32_t batch, int32_t seq_len, int32_t prefix_len,
                         int32_t num_heads, int32_t head_dim, int32_t max_sel,
                         float sm_scale, void* workspace, size_t workspace_bytes,
                         vsa_stream_t stream);

/*
 * The same proxy forward with the exact blocks named in the two formats of
 * [PX] (FlashInfer description, "Bitmask format"); both give bit-identical
 * results to vsa_fwd_proxy with the same selection.
 *
 *   sel_mask      uint32 [batch, num_heads, nvideo, ceil(nvideo/32)], one row of
 *                 words per (batch, head, video query block): bit (c % 32) of
 *                 word c / 32 selects video block c; bits past the last video
 *                 block in the final word are ignored.
 *   sel_indptr    int32 [batch * num_heads * nvideo + 1], non-decreasing, row
 *                 pointers into sel_indices for the rows in (batch, head, video
 *                 block) order; sel_indices int32 [nnz], video-relative block
 *                 ids (distinct per row; -1 or out-of-range entries are
 *                 skipped).  Row pointers are clamped to [0, nnz] on the device,
 *                 so a malformed list reads nothing outside sel_indices.
 *   expected_sel  the typical number of selected blocks per row, 1..nvideo: it
 *                 only sizes the sweep segments (rows may hold more or fewer);
 *                 pass the max_sel of a padded call to reproduce its order.
 *   other arguments, outputs and errors as vsa_fwd_proxy (a row may select up
 *   to every video block, which these calls size their LDS tables for).
 */
vsa_status vsa_fwd_proxy_bitmask(const void* q, const void* k, const void* v,
                                 const uint32_t* sel_mask, const int32_t* vbs,
                                 const void* kmean, const void* vsum, void* out,
                                 int32_t batch, int32_t seq_len, int32_t prefix_len,
                                 int32_t num_heads, int32_t head_dim, int32_t expected_sel,
                                 float sm_scale, void* workspace, size_t workspace_bytes,
                                 vsa_stream_t stream);
vsa_status vsa_fwd_proxy_bsr(const void* q, const void* k, const void* v,
                             const int32_t* sel_indptr, const int32_t* sel_indices, int32_t nnz,
                             const int32_t* vbs, const void* kmean, const void* vsum, void* out,
                             int32_t batch, int32_t seq_len, int32_t prefix_len,
                             int32_t num_heads, int32_t head_dim, int32_t expected_sel,
                             float sm_scale, void* workspace, size_t workspace_bytes,
                             vsa_stream_t stream);

/*
 * vsa_fwd_lse -- vsa_fwd that also returns the row statistics.
 *
 *   lse           float32 [batch, num_heads, seq_len] output, 4-byte aligned:
 *                 for each valid query row the natural log of its softmax
 *                 normaliser, log sum_j exp(sm_scale * q . k_j) over the row's
 *                 keys; -inf for padding rows and rows with no valid key.
 *   other arguments, outputs and errors as vsa_fwd.
 *
 * With lse, results over disjoint key sets of the same rows can be combined
 * exactly (vsa_merge) -- splitting a long key list, or joining this output
 * with another attention branch over the same queries.
 */
vsa_status vsa_fwd_lse(const void* q, const void* k, const void* v,
                       const int32_t* topk_idx, const int32_t* vbs, void* out, float* lse,
                       int32_t batch, int32_t seq_len, int32_t num_heads, int32_t head_dim,
                       int32_t topk, float sm_scale,
                       void* workspace, size_t workspace_bytes, vsa_stream_t stream);

/*
 * vsa_merge -- attention over the union of two disjoint key sets from the two
 * partial results: lse = log(exp(lse1) + exp(lse2)),
 * out = exp(lse1 - lse) o1 + exp(lse2 - lse) o2 (fp32, rounded once to bf16,
 * nearest even).  Rows where both parts are empty (-inf) get out = 0 and
 * lse_out = -inf.
 *
 *   o1, o2, out   bf16 [batch, seq_len, num_heads, head_dim], 16-byte aligned;
 *                 out may be o1 or o2 (each piece is read before it is written).
 *   lse1, lse2    float32 [batch, num_heads, seq_len], 4-byte aligned.
 *   lse_out       float32 [batch, num_heads, seq_len]; must not overlap lse1 or
 *                 lse2.
 *   head_dim      a positive multiple of 8 (any head geometry: a pure
 *                 elementwise step).
 */
vsa_status vsa_merge(const void* o1, const float* lse1, const void* o2, const float* lse2,
                     void* out, float* lse_out, int32_t batch, int32_t seq_len,
                     int32_t num_heads, int32_t head_dim, vsa_stream_t stream);

/*
 * vsa_route_topk -- exact-block selection by block-mean scores, the routing
 * step before the attention.  [RUN] makes a video query block exact on the key
 * blocks whose centroid score passes a per-block threshold it does not define;
 * this call takes the topk highest scores instead.  For each (batch, head,
 * query block) i the score of key block j is sum_d qmean[i, d] * kmean[j, d],
 * accumulated in float64 in the order d = 0..127 (exact products, one rounding
 * per term, so the result is fixed to the last bit); the topk eligible blocks
 * of highest score are written by descending score, ties to the lower index.
 * Blocks with vbs = 0 are not eligible; a row with fewer than topk eligible
 * blocks is padded with -1.
 *
 *   qmean, kmean  bf16 [batch, num_blocks, num_heads, head_dim] block means
 *                 (vsa_preprocess of q, resp. k, gives them).
 *   vbs           int32 [num_blocks].
 *   topk_idx      int32 [batch, num_heads, num_blocks, topk] output: ready to
 *                 be the topk_idx of vsa_fwd.
 *   num_blocks    1 .. 7680; head_dim must be 128; 1 <= topk <= num_blocks.
 *   workspace     device memory of at least vsa_route_workspace_size(batch,
 *                 num_blocks, num_heads) bytes, 256-byte aligned
 *                 (VSA_ERR_WORKSPACE / VSA_ERR_ALIGN otherwise): the fp64
 *                 scores of as many (batch, head) pairs as fit about 256 MB
 *                 (at least one pair, num_blocks^2 * 8 bytes); larger calls
 *                 run in chunks of pairs.  Its contents on entry are ignored.
 *                 vsa_route_workspace_size returns 0 for a shape the call
 *                 rejects (batch, num_heads or num_blocks out of range, or
 *                 batch * num_heads * num_blocks >= 2^31).
 *
 * Device memory, caller-owned, enqueued on `stream`; qmean and kmean must be
 * 16-byte aligned, vbs and topk_idx 4-byte (VSA_ERR_ALIGN otherwise).
 */
size_t vsa_route_workspace_size(int32_t batch, int32_t num_blocks, int32_t num_heads);
vsa_status vsa_route_topk(const void* qmean, const void* kmean, const int32_t* vbs,
                          int32_t* topk_idx, int32_t batch, int32_t num_blocks,
                          int32_t num_heads, int32_t head_dim, int32_t topk,
                          void* workspace, size_t workspace_bytes, vsa_stream_t stream);

/*
 * Cube tiling of a latent video grid ([SH]: 4 x 4 x 4 cubes of 64 tokens,
 * padded to 64 * cubes rows).  The grid T x Hh x W has ceil(T/4) * ceil(Hh/4) *
 * ceil(W/4) cubes, numbered row-major over the cube grid; inside a cube the real
 * tokens keep their row-major (t, h, w) order and fill the first vbs[c] slots
 * (vbs[c] = product of the cube's valid extents), the rest being padding.
 *
 * vsa_cube_count   number of cubes, or 0 if an extent is < 1 or the padded
 *                  length would reach 2^31 rows.
 * vsa_cube_vbs     fills vbs_host[0 .. cubes-1] (HOST memory, n >= cubes
 *                  entries); VSA_ERR_NULL / VSA_ERR_SHAPE otherwise.
 * vsa_tile         x [batch, T*Hh*W, num_heads, head_dim] (natural order
 *                  n = (t*Hh + h)*W + w) -> x_tiled [batch, 64*cubes, num_heads,
 *                  head_dim]; padding rows are written as zeros.
 * vsa_untile       the inverse gather: x_tiled -> x (padding rows are ignored).
 *
 * Elements are 16-bit (bf16 here, but the copy is bit-exact for any 2-byte
 * type); batch * 64 * cubes <= 2^23 rows (VSA_ERR_SHAPE otherwise; one
 * 256-thread workgroup per row); num_heads * head_dim must be a multiple of 8
 * (16-byte rows pieces) and
 * both pointers 16-byte aligned (VSA_ERR_ALIGN otherwise).  Device memory,
 * caller-owned, enqueued on `stream`; x and x_tiled must not overlap.
 */
size_t vsa_cube_count(int32_t T, int32_t Hh, int32_t W);
vsa_status vsa_cube_vbs(int32_t T, int32_t Hh, int32_t W, int32_t* vbs_host, size_t n);
vsa_status vsa_tile(const void* x, void* x_tiled, int32_t batch, int32_t T, int32_t Hh, int32_t W,
                    int32_t num_heads, int32_t head_dim, vsa_stream_t stream);
vsa_status vsa_untile(const void* x_tiled, void* x, int32_t batch, int32_t T, int32_t Hh, int32_t W,
                      int32_t num_heads, int32_t head_dim, vsa_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* VSA_H */
