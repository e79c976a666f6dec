"""CPU fp64 oracle for the VSA fine block-sparse attention forward.

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg import this module.  The product path (the HIP library and
its Python binding) never imports, calls or links it, and this module imports
nothing from the product package.

What it computes, and where the pages define it:
  * vsa_fwd -- Wan2.2 production-values dataset card, "Operator contract":
    non-causal block-sparse attention in BSHD layout,
    out = softmax(q . k_sel^T / sqrt(D)) . v_sel, where for each (batch, head,
    query cube) topk_idx names the KV cubes and vbs[c] keeps only the first
    vbs[c] of the 64 slots of cube c.
  * vsa_preprocess -- TensorRT-Edge-LLM "Video Sparse Attention Runner",
    preprocess entry: KC and VC are BF16 [numBlocks, numHeads, 128] block means
    of K and block sums of V; TensorRT-LLM VisualGen VSA review snippet: the
    mean divides the block sum by the valid count and casts to the input dtype.
  * kc_stats -- the Runner's preprocess entry: FP32 [numHeads, 128] statistics
    of KC (a mean and a diagonal variance per head and channel), with KC taken
    in its BF16 rounding.
  * vsa_fwd_proxy -- the Runner's class description: in a packed
    [prefix | video] sequence the prefix queries see all keys exactly, while a
    64-row video query block sees the prefix, its neighbours and its chosen
    blocks exactly and sees each remaining block only through that block's
    averaged key and its value total.  The FlashInfer proxy-compensation
    description on the TensorRT-LLM PR page adds: a block already computed
    exactly is excluded from the proxy terms, and each proxy term enters the
    softmax denominator weighted by the number of real tokens it stands for.

Block-sparse attention over a key set is exact softmax attention restricted to
that set, so the oracle is that plain definition written out in float64: the key
set is built as a set (ascending padded slot), logits are fp64 dot products of
the exactly widened bf16 inputs, and the softmax is the textbook
exp(s - max) / sum form.  The graded output is the fp64 result rounded once to
bf16 (nearest, ties to even).  Readings of points the pages leave open
(padding rows write 0, an empty key set writes 0, indices must be distinct) are
listed in the repository design notes.
"""
from __future__ import annotations

import numpy as np

BLOCK = 64

__all__ = ["bf16_to_f64", "f64_to_bf16", "vsa_fwd", "vsa_fwd_item", "vsa_preprocess",
           "vsa_fwd_proxy", "vsa_fwd_proxy_item", "item_key_slots", "cube_layout", "cube_tile",
           "cube_untile", "vsa_fwd_lse_item", "vsa_fwd_lse", "merge_partials", "block_scores",
           "route_topk", "kc_stats"]


# --------------------------------------------------------------------------
# bf16 <-> fp64
# --------------------------------------------------------------------------
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float64 (exact: bf16 -> fp32 -> fp64)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f64_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 to bf16 bit patterns in one step (nearest, ties to even).

    bf16 keeps 8 significant bits, exponents down to 2^-126 for normals and a
    quantum of 2^-133 for subnormals.  For each value the quantum is
    2^(e - 8) with x = m * 2^e, 0.5 <= |m| < 1, floored at 2^-133; x / quantum
    and the product back are exact in float64, and np.rint rounds half to
    even.  Results beyond the bf16 range become +-inf; NaN stays NaN.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    flat = x.reshape(-1)
    res = out.reshape(-1)
    finite = np.isfinite(flat)
    xf = np.where(finite, flat, 0.0)
    _, e = np.frexp(xf)
    q = np.ldexp(1.0, np.maximum(e - 8, -133))
    r = np.rint(xf / q) * q
    big = np.abs(r) >= 2.0 ** 128
    with np.errstate(over="ignore"):
        r32 = r.astype(np.float32)
    bits = (r32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    sign = np.where(np.signbit(flat), np.uint16(0x8000), np.uint16(0))
    bits = np.where(big, sign | np.uint16(0x7F80), bits)
    bits = np.where(np.isinf(flat), sign | np.uint16(0x7F80), bits)
    bits = np.where(np.isnan(flat), np.uint16(0x7FC0), bits)
    res[:] = bits
    return out


# --------------------------------------------------------------------------
# the plain definition, one (batch, head, query block) at a time
# --------------------------------------------------------------------------
TINY = np.finfo(np.float64).tiny


def _exp_weights(x: np.ndarray) -> np.ndarray:
    """exp(x) for x <= 0, with results below the smallest normal float64 set to 0.

    Each row holds a 1 (its maximum), so a dropped term is under 2.3e-308 of the
    row's sum: far below float64 rounding of that sum, and no bf16-rounded
    output can change.  Subnormal weights would only slow the matrix products
    that follow by an order of magnitude.
    """
    e = np.exp(x)
    e[e < TINY] = 0.0
    return e


def _softmax_attend(qm: np.ndarray, km: np.ndarray, vm: np.ndarray, scale: float,
                    return_weights: bool = False):
    """Textbook softmax attention in float64: rows of qm over the rows of km/vm."""
    s = (qm @ km.T) * scale
    m = s.max(axis=1, keepdims=True)
    w = _exp_weights(s - m)
    w /= w.sum(axis=1, keepdims=True)
    o = w @ vm
    return (o, w) if return_weights else (o, None)


def item_key_slots(blocks, vbs: np.ndarray) -> np.ndarray:
    """Key set of one query block as ascending padded slots.

    The set is {64c + t : c in blocks, t < vbs[c]}; blocks must be distinct
    (a repeated block would count its keys twice, which the contract rules out).
    """
    blocks = np.asarray(blocks, dtype=np.int64).reshape(-1)
    uniq = np.unique(blocks)
    if uniq.size != blocks.size:
        raise ValueError("duplicate block index in a selection row")
    parts = [BLOCK * c + np.arange(int(vbs[c]), dtype=np.int64) for c in uniq]
    return np.concatenate(parts) if parts else np.zeros(0, np.int64)


def vsa_fwd_item(q, k, v, topk_idx, vbs, sm_scale, b: int, h: int, qc: int,
                 return_weights: bool = False):
    """fp64 output rows [vbs[qc], D] of query cube qc of head h, batch b (and weights)."""
    vbs = np.asarray(vbs)
    nq = int(vbs[qc])
    D = q.shape[-1]
    if nq == 0:
        return (np.zeros((0, D)), np.zeros((0, 0))) if return_weights else np.zeros((0, D))
    slots = item_key_slots(topk_idx[b, h, qc], vbs)
    if slots.size == 0:
        z = np.zeros((nq, D))
        return (z, np.zeros((nq, 0))) if return_weights else z
    qm = bf16_to_f64(q[b, BLOCK * qc:BLOCK * qc + nq, h, :])
    km = bf16_to_f64(k[b, slots, h, :])
    vm = bf16_to_f64(v[b, slots, h, :])
    scale = float(np.float32(sm_scale))
    o, w = _softmax_attend(qm, km, vm, scale, return_weights)
    return (o, w) if return_weights else o


def vsa_fwd(q, k, v, topk_idx, vbs, sm_scale, items=None):
    """fp64 forward over all items (or the listed (b, h, qc) items).

    Returns o64 [B, S, H, D] float64 with padding query rows (and rows of
    skipped items) equal to 0.  Apply f64_to_bf16 for the graded bf16 output.
    """
    B, S, H, D = q.shape
    nq_blocks = S // BLOCK
    out = np.zeros((B, S, H, D), dtype=np.float64)
    if items is None:
        items = [(b, h, c) for b in range(B) for h in range(H) for c in range(nq_blocks)]
    for b, h, c in items:
        o = vsa_fwd_item(q, k, v, topk_idx, vbs, sm_scale, b, h, c)
        out[b, BLOCK * c:BLOCK * c + o.shape[0], h, :] = o
    return out


# --------------------------------------------------------------------------
# block summaries
# --------------------------------------------------------------------------
def vsa_preprocess(k, v, vbs):
    """Block summaries: kmean = bf16(sum_{t<vbs} K_t / vbs), vsum = bf16(sum_{t<vbs} V_t).

    Inputs are bf16 bits [B, S, H, D]; outputs are bf16 bits [B, S/64, H, D].
    Sums are formed in float64 (exact for bf16 data of ordinary range), divided
    in float64 and rounded once to bf16.  A block with vbs = 0 gets zeros.
    """
    B, S, H, D = k.shape
    nb = S // BLOCK
    km = np.zeros((B, nb, H, D), np.float64)
    vs = np.zeros((B, nb, H, D), np.float64)
    for c in range(nb):
        n = int(vbs[c])
        if n == 0:
            continue
        rows = slice(BLOCK * c, BLOCK * c + n)
        km[:, c] = bf16_to_f64(k[:, rows]).sum(axis=1) / n
        vs[:, c] = bf16_to_f64(v[:, rows]).sum(axis=1)
    return f64_to_bf16(km), f64_to_bf16(vs)


# --------------------------------------------------------------------------
# packed [prefix | video] proxy-compensated forward
# --------------------------------------------------------------------------
def vsa_fwd_proxy_item(q, k, v, sel_idx, vbs, kmean, vsum, prefix_len, sm_scale,
                       b: int, h: int, qb: int):
    """fp64 output rows of query block qb (global block index) of head h, batch b.

    Prefix query block: exact attention over every valid key, no proxies.
    Video query block qv = qb - P/64: exact over all prefix blocks and the video
    blocks listed in sel_idx[b, h, qv] (video-relative, -1 = empty slot); each
    other video block c with vbs[c] > 0 adds a proxy term with logit
    t_c = (q . kmean_c) * scale, weight vbs[c] in the denominator and exp(t_c) * vsum_c
    in the numerator.  One common max M stabilises both sums.
    """
    vbs = np.asarray(vbs)
    npb = prefix_len // BLOCK
    nblk = vbs.size
    nq = int(vbs[qb])
    D = q.shape[-1]
    if nq == 0:
        return np.zeros((0, D))
    scale = float(np.float32(sm_scale))
    qm = bf16_to_f64(q[b, BLOCK * qb:BLOCK * qb + nq, h, :])
    if qb < npb:
        exact_blocks = list(range(nblk))
        proxy_blocks = []
    else:
        sel = [int(x) for x in sel_idx[b, h, qb - npb] if x >= 0]
        if len(set(sel)) != len(sel):
            raise ValueError("duplicate block index in a selection row")
        exact_blocks = list(range(npb)) + [npb + c for c in sel]
        chosen = set(sel)
        proxy_blocks = [npb + c for c in range(nblk - npb)
                        if c not in chosen and int(vbs[npb + c]) > 0]
    slots = item_key_slots(exact_blocks, vbs)
    km = bf16_to_f64(k[b, slots, h, :])
    vm = bf16_to_f64(v[b, slots, h, :])
    s = (qm @ km.T) * scale                                   # exact logits
    if proxy_blocks:
        pk = bf16_to_f64(kmean[b, proxy_blocks, h, :])
        pv = bf16_to_f64(vsum[b, proxy_blocks, h, :])
        wt = vbs[proxy_blocks].astype(np.float64)
        t = (qm @ pk.T) * scale                               # proxy logits
        m = np.maximum(s.max(axis=1, keepdims=True), t.max(axis=1, keepdims=True))
    else:
        m = s.max(axis=1, keepdims=True) if s.size else np.zeros((nq, 1))
    es = _exp_weights(s - m)
    num = es @ vm
    den = es.sum(axis=1, keepdims=True)
    if proxy_blocks:
        et = _exp_weights(t - m)
        num = num + et @ pv
        den = den + et @ wt[:, None]
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), 0.0)


def vsa_fwd_proxy(q, k, v, sel_idx, vbs, kmean, vsum, prefix_len, sm_scale, items=None):
    """fp64 proxy-compensated forward over all (or the listed) (b, h, query block) items."""
    B, S, H, D = q.shape
    nblk = S // BLOCK
    out = np.zeros((B, S, H, D), dtype=np.float64)
    if items is None:
        items = [(b, h, c) for b in range(B) for h in range(H) for c in range(nblk)]
    for b, h, c in items:
        o = vsa_fwd_proxy_item(q, k, v, sel_idx, vbs, kmean, vsum, prefix_len, sm_scale, b, h, c)
        out[b, BLOCK * c:BLOCK * c + o.shape[0], h, :] = o
    return out


# --------------------------------------------------------------------------
# cube tiling of a latent video grid
# --------------------------------------------------------------------------
CUBE = 4


def cube_layout(T: int, Hh: int, W: int):
    """Cube-major layout of a T x Hh x W latent grid (Wan2.2 card, "Shapes").

    The grid is cut into 4 x 4 x 4 cubes of 64 slots, ceil(T/4) x ceil(Hh/4) x
    ceil(W/4) of them, numbered row-major over the cube grid.  Inside a cube the
    real tokens keep their row-major (t, h, w) order and fill the first vbs[c]
    slots; the remaining slots are padding.  Returns (slot, vbs): slot[n] is
    the padded row of natural token n = (t * Hh + h) * W + w, vbs[c] the number
    of real tokens of cube c.  Written out with plain loops over the cubes.
    """
    ct, ch, cw = -(-T // CUBE), -(-Hh // CUBE), -(-W // CUBE)
    slot = np.full(T * Hh * W, -1, dtype=np.int64)
    vbs = np.zeros(ct * ch * cw, dtype=np.int64)
    for a in range(ct):
        for b in range(ch):
            for c in range(cw):
                cube = (a * ch + b) * cw + c
                r = 0
                for t in range(CUBE * a, min(CUBE * a + CUBE, T)):
                    for h in range(CUBE * b, min(CUBE * b + CUBE, Hh)):
                        for w in range(CUBE * c, min(CUBE * c + CUBE, W)):
                            slot[(t * Hh + h) * W + w] = BLOCK * cube + r
                            r += 1
                vbs[cube] = r
    return slot, vbs


def cube_tile(x, T: int, Hh: int, W: int):
    """Natural [B, T*Hh*W, ...] rows -> cube-major [B, 64 * cubes, ...], padding rows zero."""
    slot, vbs = cube_layout(T, Hh, W)
    x = np.asarray(x)
    out = np.zeros((x.shape[0], BLOCK * vbs.size) + x.shape[2:], dtype=x.dtype)
    out[:, slot] = x
    return out


def cube_untile(xt, T: int, Hh: int, W: int):
    """Cube-major rows -> natural [B, T*Hh*W, ...] rows (padding rows dropped)."""
    slot, _ = cube_layout(T, Hh, W)
    return np.asarray(xt)[:, slot]


# --------------------------------------------------------------------------
# row statistics and the merge of partial results
# --------------------------------------------------------------------------
def vsa_fwd_lse_item(q, k, v, topk_idx, vbs, sm_scale, b: int, h: int, qc: int):
    """fp64 (o, lse) of query cube qc: o as vsa_fwd_item, lse_i = log sum_j exp(s_ij).

    s_ij = sm_scale * q_i . k_j over the item's key set (natural logarithm).  A
    row with an empty key set gets lse = -inf (the log of an empty sum) and o = 0.
    """
    vbs = np.asarray(vbs)
    nq = int(vbs[qc])
    D = q.shape[-1]
    slots = item_key_slots(topk_idx[b, h, qc], vbs)
    if nq == 0 or slots.size == 0:
        return np.zeros((nq, D)), np.full(nq, -np.inf)
    qm = bf16_to_f64(q[b, BLOCK * qc:BLOCK * qc + nq, h, :])
    km = bf16_to_f64(k[b, slots, h, :])
    vm = bf16_to_f64(v[b, slots, h, :])
    s = (qm @ km.T) * float(np.float32(sm_scale))
    m = s.max(axis=1, keepdims=True)
    e = _exp_weights(s - m)
    tot = e.sum(axis=1)
    return (e @ vm) / tot[:, None], m[:, 0] + np.log(tot)


def vsa_fwd_lse(q, k, v, topk_idx, vbs, sm_scale, items=None):
    """fp64 (o [B, S, H, D], lse [B, H, S]); padding rows: o = 0, lse = -inf."""
    B, S, H, D = q.shape
    out = np.zeros((B, S, H, D), dtype=np.float64)
    lse = np.full((B, H, S), -np.inf)
    if items is None:
        items = [(b, h, c) for b in range(B) for h in range(H) for c in range(S // BLOCK)]
    for b, h, c in items:
        o, l = vsa_fwd_lse_item(q, k, v, topk_idx, vbs, sm_scale, b, h, c)
        out[b, BLOCK * c:BLOCK * c + o.shape[0], h, :] = o
        lse[b, h, BLOCK * c:BLOCK * c + l.size] = l
    return out, lse


def merge_partials(o1, lse1, o2, lse2):
    """Attention over the union of two disjoint key sets from the two partial results.

    With lse_k = log sum over set k of exp(s) and o_k the softmax average over
    set k, the union has lse = log(exp(lse1) + exp(lse2)) and
    o = (exp(lse1 - lse) o1 + exp(lse2 - lse) o2).  o are float arrays
    [..., D] (widen bf16 first), lse the matching [...] arrays; rows where both
    parts are empty (-inf) give o = 0 and lse = -inf.  float64 throughout.
    """
    o1 = np.asarray(o1, np.float64)
    o2 = np.asarray(o2, np.float64)
    l1 = np.asarray(lse1, np.float64)
    l2 = np.asarray(lse2, np.float64)
    m = np.maximum(l1, l2)
    empty = np.isneginf(m)
    ms = np.where(empty, 0.0, m)
    w1 = np.where(np.isneginf(l1), 0.0, np.exp(l1 - ms))
    w2 = np.where(np.isneginf(l2), 0.0, np.exp(l2 - ms))
    tot = w1 + w2
    lse = np.where(empty, -np.inf, ms + np.log(np.where(empty, 1.0, tot)))
    den = np.where(empty, 1.0, tot)[..., None]
    o = (w1[..., None] * o1 + w2[..., None] * o2) / den
    return np.where(empty[..., None], 0.0, o), lse


# --------------------------------------------------------------------------
# routing: top-k key blocks by block-mean scores
# --------------------------------------------------------------------------
def block_scores(qmean, kmean, b: int, h: int):
    """Score matrix [nq, nk] of one (batch, head): s[i, j] = sum_d qmean_i[d] * kmean_j[d].

    The bf16 inputs are widened exactly; each product of two bf16 values is
    exact in float64, and the 128 products are added in order d = 0, 1, ...,
    one rounding per addition, which fixes every score to the last bit (a
    fused multiply-add per term gives the same sequence of values).
    """
    qm = bf16_to_f64(qmean[b, :, h, :])
    km = bf16_to_f64(kmean[b, :, h, :])
    s = np.zeros((qm.shape[0], km.shape[0]))
    for d in range(qm.shape[1]):
        s = s + np.multiply.outer(qm[:, d], km[:, d])
    return s


def route_topk(qmean, kmean, vbs, topk: int):
    """topk_idx [B, H, nq, topk]: per query block, the topk key blocks of highest score.

    Blocks with vbs = 0 hold no keys and are never chosen; ties go to the lower
    block index; each row lists its blocks by descending score.  Rows with
    fewer than topk eligible blocks are padded with -1.
    """
    qmean = np.asarray(qmean)
    B, nq, H, _ = qmean.shape
    vbs = np.asarray(vbs)
    eligible = vbs[:kmean.shape[1]] > 0
    out = np.full((B, H, nq, topk), -1, dtype=np.int32)
    idx = np.arange(kmean.shape[1])
    for b in range(B):
        for h in range(H):
            s = block_scores(qmean, kmean, b, h)
            for i in range(nq):
                cand = idx[eligible]
                order = np.lexsort((cand, -s[i, cand]))     # descending score, then lower index
                pick = cand[order[:topk]]
                out[b, h, i, :pick.size] = pick
    return out


# --------------------------------------------------------------------------
# statistics of the block key means (KC)
# --------------------------------------------------------------------------
def kc_stats(kmean, vbs, first_block: int, count: int):
    """Per (batch, head, channel) mean and variance of the bf16 block key means.

    Over the blocks c in [first_block, first_block + count) that hold keys
    (vbs[c] > 0): mean = sum(x_c) / n and var = sum((x_c - mean)^2) / n, the
    diagonal of the population covariance, both evaluated in float64 from the
    bf16 values widened exactly and then rounded to float32 (nearest even).
    kmean is bf16 bits [B, nblk, H, D]; returns two float32 arrays [B, H, D].
    With no such block both statistics are 0.
    """
    B, _, H, D = kmean.shape
    vbs = np.asarray(vbs)
    blocks = [c for c in range(first_block, first_block + count) if vbs[c] > 0]
    mean = np.zeros((B, H, D))
    var = np.zeros((B, H, D))
    if blocks:
        x = bf16_to_f64(kmean[:, blocks])                  # [B, n, H, D]
        mean = x.mean(axis=1)
        var = ((x - mean[:, None]) ** 2).mean(axis=1)
    return mean.astype(np.float32), var.astype(np.float32)
