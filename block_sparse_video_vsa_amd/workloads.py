"""Seeded synthetic VSA workloads (inputs only).

This module makes inputs: the cube-major tiling of a latent video grid, seeded
q/k/v activations and the selection indices.  It contains none of the attention
arithmetic, so both the HIP path and the CPU oracle can draw from it.

Sources (the pages' text, cited by page and section):
  * Wan2.2 production-values dataset card, "Shapes": latent grid T x H x W is
    tiled into 4x4x4 cubes of 64 tokens, padded to S_padded = 64 * Nq with
    Nq = ceil(T/4) * ceil(H/4) * ceil(W/4) (21x30x52 -> 624 cubes, 32760 real
    tokens -> 39936 padded rows), D = 128, sm_scale = 1/sqrt(128).
  * same card, "Operator contract": topk_idx names the selected KV cubes per
    (batch, head, query cube); vbs[c] keeps the first vbs[c] of the 64 slots.
  * TensorRT-Edge-LLM "Video Sparse Attention Runner": packed [prefix | video]
    sequence in 64-row blocks, dense prefix first.

Layout conventions (the plainest reading, stated once here):
  * cubes are numbered in row-major (t/4, h/4, w/4) order;
  * inside a cube the valid tokens keep row-major (t%4, h%4, w%4) order and
    occupy the first vbs[c] slots; vbs[c] is the product of the cube's valid
    extents; the remaining slots are padding;
  * padding slots hold N(0, 10^2) garbage so that masking is exercised.

Every array is numpy: q/k/v as uint16 bf16 bit patterns in BSHD order
[B, S, H, D], indices and vbs as int32.
"""
from __future__ import annotations

from dataclasses import dataclass, field
import math

import numpy as np

BLOCK = 64
HEAD_DIM = 128
CUBE_EDGE = 4


# --------------------------------------------------------------------------
# cube-major tiling
# --------------------------------------------------------------------------
def cube_grid(T: int, Hh: int, W: int) -> tuple[int, int, int]:
    """Cube-grid extents: ceil of each latent extent over the cube edge 4."""
    e = CUBE_EDGE
    return (-(-T // e), -(-Hh // e), -(-W // e))


def tile_map(T: int, Hh: int, W: int) -> tuple[np.ndarray, np.ndarray]:
    """Natural token order -> padded cube-major slot, and vbs per cube.

    Returns (slot, vbs): slot[n] is the padded row of natural token n, where
    natural order is row-major (t, h, w); vbs[c] is the valid-token count of
    cube c.  The map is a bijection from the T*H*W real tokens onto the valid
    slots {64c + r : r < vbs[c]}.
    """
    e = CUBE_EDGE
    ct, ch, cw = cube_grid(T, Hh, W)
    t = np.arange(T)[:, None, None]
    h = np.arange(Hh)[None, :, None]
    w = np.arange(W)[None, None, :]
    cube = ((t // e) * ch + (h // e)) * cw + (w // e)
    # valid extents of the cube a token falls in
    et = np.minimum(e, T - (t // e) * e)
    eh = np.minimum(e, Hh - (h // e) * e)
    ew = np.minimum(e, W - (w // e) * e)
    rank = ((t % e) * eh + (h % e)) * ew + (w % e)
    slot = (cube * BLOCK + rank).reshape(-1)
    ext_t = np.minimum(e, T - np.arange(ct) * e)
    ext_h = np.minimum(e, Hh - np.arange(ch) * e)
    ext_w = np.minimum(e, W - np.arange(cw) * e)
    vbs = (ext_t[:, None, None] * ext_h[None, :, None] * ext_w[None, None, :]).reshape(-1)
    return slot.astype(np.int64), vbs.astype(np.int32)


def face_neighbours(cube: int, grid: tuple[int, int, int]) -> list[int]:
    """In-bounds face neighbours of a cube, in the order t-1, t+1, h-1, h+1, w-1, w+1."""
    ct, ch, cw = grid
    a, rem = divmod(cube, ch * cw)
    b, c = divmod(rem, cw)
    out = []
    for da, db, dc in ((-1, 0, 0), (1, 0, 0), (0, -1, 0), (0, 1, 0), (0, 0, -1), (0, 0, 1)):
        x, y, z = a + da, b + db, c + dc
        if 0 <= x < ct and 0 <= y < ch and 0 <= z < cw:
            out.append((x * ch + y) * cw + z)
    return out


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bf16 (nearest, ties to even); uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    out = np.empty(x.shape, dtype=np.uint16)
    flat_u = u.reshape(-1)
    flat_o = out.reshape(-1)
    step = 1 << 24
    for s in range(0, flat_u.size, step):
        c = flat_u[s:s + step]
        flat_o[s:s + step] = ((c + np.uint32(0x7FFF) + ((c >> np.uint32(16)) & np.uint32(1)))
                              >> np.uint32(16)).astype(np.uint16)
    return out


# --------------------------------------------------------------------------
# workload configurations
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class Config:
    name: str
    batch: int
    heads: int
    grid: tuple[int, int, int]      # latent T, H, W of the video part
    topk: int                      # plain mode: selected cubes per query cube
    structured: bool               # self + face neighbours + random, else purely random
    scaled: bool                   # per-head log-uniform scale + 4 hot channels x20
    outlier: bool                  # head-0 outlier tokens, q and k x200
    seed: int
    prefix_len: int = 0            # >0: packed [prefix | video] proxy workload
    n_random: int = 0              # proxy mode: random exact blocks per video query block
    description: str = ""

    @property
    def cubes(self) -> tuple[int, int, int]:
        return cube_grid(*self.grid)

    @property
    def n_video_blocks(self) -> int:
        a, b, c = self.cubes
        return a * b * c

    @property
    def n_prefix_blocks(self) -> int:
        return self.prefix_len // BLOCK

    @property
    def n_blocks(self) -> int:
        return self.n_prefix_blocks + self.n_video_blocks

    @property
    def seq_len(self) -> int:
        return BLOCK * self.n_blocks

    @property
    def proxy(self) -> bool:
        return self.prefix_len > 0

    @property
    def max_sel(self) -> int:
        """Width of sel_idx in proxy mode: self + up to 6 neighbours + n_random."""
        return 1 + 6 + self.n_random


CONFIGS: dict[str, Config] = {
    "0": Config("0", 1, 2, (5, 6, 7), 2, False, False, False, 1000,
                description="tiny: 5x6x7 grid, 8 cubes, H=2, topk=2 random"),
    "1": Config("1", 1, 8, (10, 15, 26), 11, True, True, False, 1001,
                description="medium: 10x15x26 grid, 84 cubes, H=8, topk=11 structured"),
    "2": Config("2", 1, 40, (21, 30, 52), 78, True, True, False, 1002,
                description="Wan2.2-A14B 832x480x81f: 21x30x52 grid, 624 cubes, H=40, topk=78"),
    "3a": Config("3a", 1, 40, (21, 30, 52), 78, True, True, True, 1003,
                 description="21x30x52 grid, 624 cubes, H=40, topk=78, plus a head-0 outlier stress (64 tokens, q and k x200)"),
    "3b": Config("3b", 1, 40, (21, 45, 80), 180, True, True, True, 1013,
                 description="1280x720x81f: 21x45x80 grid, 1440 cubes, H=40, topk=180, with outlier"),
    "4": Config("4", 1, 56, (21, 30, 52), 0, True, True, False, 1004, prefix_len=512, n_random=60,
                description="packed [512-row prefix | 21x30x52 video], H=56, proxy-compensated"),
}


@dataclass
class Workload:
    config: Config
    q: np.ndarray               # uint16 [B, S, H, D]
    k: np.ndarray
    v: np.ndarray
    vbs: np.ndarray             # int32 [S/64]
    sm_scale: np.float32
    topk_idx: np.ndarray | None = None   # int32 [B, H, Nq, topk] (plain mode)
    sel_idx: np.ndarray | None = None    # int32 [B, H, Nv, max_sel] (proxy mode), -1 padded
    valid_slots: np.ndarray | None = None  # int64 padded rows that hold real tokens
    meta: dict = field(default_factory=dict)


def _structured_rows(rng: np.random.Generator, n_rows_per_cube: int, grid, n_cubes: int,
                     total: int, extra_exclude_neighbours: bool) -> np.ndarray:
    """Rows [n_cubes * n_rows_per_cube, total]: self, face neighbours, then random distinct.

    Row r belongs to query cube r % n_cubes (rows are (b, h, cube) in C order, so
    the cube index runs fastest).  Entries past a row's fixed part are distinct
    random cubes not already in the row, drawn independently per row.  With
    extra_exclude_neighbours the row has exactly len(fixed) + total entries and is
    returned ragged-padded with -1 to len(fixed)_max + total (proxy mode).
    """
    fixed = [[c] + face_neighbours(c, grid) for c in range(n_cubes)]
    n_rows = n_rows_per_cube * n_cubes
    keys = rng.random((n_rows, n_cubes), dtype=np.float32)
    rows_cube = np.tile(np.arange(n_cubes), n_rows_per_cube)
    # exclude each row's fixed entries from the random draw
    for c in range(n_cubes):
        sel = np.nonzero(rows_cube == c)[0]
        keys[np.ix_(sel, fixed[c])] = 2.0
    order = np.argsort(keys, axis=1, kind="stable").astype(np.int32)
    if extra_exclude_neighbours:
        width = 7 + total
        out = np.full((n_rows, width), -1, dtype=np.int32)
        for c in range(n_cubes):
            sel = np.nonzero(rows_cube == c)[0]
            f = len(fixed[c])
            out[sel, :f] = fixed[c]
            out[sel, f:f + total] = order[sel, :total]
        return out
    out = np.empty((n_rows, total), dtype=np.int32)
    for c in range(n_cubes):
        sel = np.nonzero(rows_cube == c)[0]
        f = len(fixed[c])
        if f > total:
            raise ValueError("topk smaller than self + neighbours")
        out[sel, :f] = fixed[c]
        out[sel, f:] = order[sel, :total - f]
    return out


def generate(cfg: Config | str, seed: int | None = None) -> Workload:
    """Build the seeded synthetic workload of a configuration.

    Draw recipe (one SeedSequence child stream each, in this order): head
    scales for q, head scales for k, hot channels, valid q/k/v N(0,1) fp32,
    pad garbage N(0,100), index random parts, outlier slots.  Scaling applies
    to valid tokens only, in fp32, before a single round-to-nearest-even cast
    to bf16.
    """
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    seed = cfg.seed if seed is None else seed
    ss = np.random.SeedSequence(seed)
    r_hq, r_hk, r_hot, r_valid, r_pad, r_idx, r_out = (np.random.Generator(np.random.PCG64(s))
                                                       for s in ss.spawn(7))
    B, H, D = cfg.batch, cfg.heads, HEAD_DIM
    T, Hh, W = cfg.grid
    slot_v, vbs_v = tile_map(T, Hh, W)
    npre = cfg.prefix_len
    if npre % BLOCK:
        raise ValueError("prefix length must be a multiple of 64")
    S = cfg.seq_len
    # valid padded rows: prefix rows first (all valid), then the tiled video rows
    valid_slots = np.concatenate([np.arange(npre, dtype=np.int64), npre + slot_v])
    vbs = np.concatenate([np.full(npre // BLOCK, BLOCK, np.int32), vbs_v]).astype(np.int32)
    n_valid = valid_slots.size
    pad_mask = np.ones(S, dtype=bool)
    pad_mask[valid_slots] = False
    pad_slots = np.nonzero(pad_mask)[0]

    if cfg.scaled:
        lo, hi = math.log(0.5), math.log(8.0)
        sq = np.exp(r_hq.uniform(lo, hi, size=H)).astype(np.float32)
        sk = np.exp(r_hk.uniform(lo, hi, size=H)).astype(np.float32)
        hot = np.stack([r_hot.permutation(D)[:4] for _ in range(H)]).astype(np.int64)
    else:
        sq = sk = np.ones(H, np.float32)
        hot = None
    out_tok = None
    if cfg.outlier:
        out_tok = np.sort(r_out.choice(n_valid, size=64, replace=False))

    tensors = []
    for which in range(3):  # q, k, v
        x = np.empty((B, S, H, D), dtype=np.float32)
        val = r_valid.standard_normal((B, n_valid, H, D), dtype=np.float32)
        if which < 2 and cfg.scaled:
            val *= (sq if which == 0 else sk)[None, None, :, None]
            for h in range(H):
                val[:, :, h, hot[h]] *= np.float32(20.0)
        if which < 2 and out_tok is not None:
            val[:, out_tok, 0, :] *= np.float32(200.0)
        x[:, valid_slots] = val
        del val
        if pad_slots.size:
            x[:, pad_slots] = r_pad.standard_normal((B, pad_slots.size, H, D),
                                                    dtype=np.float32) * np.float32(10.0)
        tensors.append(f32_to_bf16_bits(x))
        del x
    q, k, v = tensors

    grid_c = cfg.cubes
    nv = cfg.n_video_blocks
    topk_idx = sel_idx = None
    if cfg.proxy:
        rows = _structured_rows(r_idx, B * H, grid_c, nv, cfg.n_random, True)
        sel_idx = rows.reshape(B, H, nv, cfg.max_sel)
    elif cfg.structured:
        rows = _structured_rows(r_idx, B * H, grid_c, nv, cfg.topk, False)
        topk_idx = rows.reshape(B, H, nv, cfg.topk)
    else:
        keys = r_idx.random((B * H * nv, nv), dtype=np.float32)
        topk_idx = np.argsort(keys, axis=1, kind="stable")[:, :cfg.topk].astype(np.int32)
        topk_idx = topk_idx.reshape(B, H, nv, cfg.topk)

    meta = {"seed": seed, "head_scale_q": sq.tolist(), "head_scale_k": sk.tolist(),
            "hot_channels": None if hot is None else hot.tolist(),
            "outlier_tokens": None if out_tok is None else valid_slots[out_tok].tolist()}
    return Workload(cfg, q, k, v, vbs, np.float32(1.0 / math.sqrt(D)), topk_idx, sel_idx,
                    valid_slots, meta)


def effective_flops(topk_idx: np.ndarray, vbs: np.ndarray, head_dim: int = HEAD_DIM) -> float:
    """4*D per (valid query, valid selected key) pair, summed over (b, h, query cube)."""
    vbs = vbs.astype(np.int64)
    nq = topk_idx.shape[2]
    sel = vbs[topk_idx].sum(axis=-1)                    # [B, H, Nq]
    return float(4 * head_dim * (sel * vbs[None, None, :nq]).sum())


def effective_flops_proxy(sel_idx: np.ndarray, vbs: np.ndarray, n_prefix_blocks: int,
                          head_dim: int = HEAD_DIM) -> tuple[float, float]:
    """Exact-pair FLOPs and proxy FLOPs of the packed [prefix | video] workload.

    Exact pairs: prefix query rows x every valid key; video query rows x valid
    keys of the prefix blocks and of their selected video blocks.  Proxy terms:
    video query rows x unselected video blocks with vbs > 0, 4*D each.
    """
    vbs = vbs.astype(np.int64)
    B, H, nv, _ = sel_idx.shape
    npb = n_prefix_blocks
    vv = vbs[npb:]
    total_keys = vbs.sum()
    pre_keys = vbs[:npb].sum()
    q_pre = vbs[:npb].sum()
    exact = B * H * q_pre * total_keys
    valid = sel_idx >= 0
    selk = np.where(valid, vv[np.clip(sel_idx, 0, None)], 0).sum(axis=-1)  # [B,H,nv]
    exact += ((pre_keys + selk) * vv[None, None, :]).sum()
    n_sel_nonzero = np.where(valid, vv[np.clip(sel_idx, 0, None)] > 0, False).sum(axis=-1)
    n_proxy = (vv > 0).sum() - n_sel_nonzero
    proxy = (n_proxy * vv[None, None, :]).sum()
    return float(4 * head_dim * exact), float(4 * head_dim * proxy)


# --------------------------------------------------------------------------
# selection formats (same selection, other encodings)
# --------------------------------------------------------------------------
def sel_to_bitmask(sel_idx: np.ndarray, nvideo: int) -> np.ndarray:
    """Padded rows [..., width] (-1 = empty) -> packed words [..., ceil(nvideo/32)] (uint32 bits
    in int32 storage): bit c % 32 of word c // 32 is set for each listed video block c."""
    rows = sel_idx.reshape(-1, sel_idx.shape[-1])
    nw = (nvideo + 31) // 32
    out = np.zeros((rows.shape[0], nw), dtype=np.uint32)
    for r in range(rows.shape[0]):
        for c in rows[r]:
            if 0 <= c < nvideo:
                out[r, c // 32] |= np.uint32(1) << np.uint32(c % 32)
    return out.view(np.int32).reshape(sel_idx.shape[:-1] + (nw,))


def sel_to_bsr(sel_idx: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Padded rows -> (indptr [rows + 1], indices) over the rows in C order, -1 entries dropped."""
    rows = sel_idx.reshape(-1, sel_idx.shape[-1])
    keep = rows >= 0
    counts = keep.sum(axis=1)
    indptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return indptr, rows[keep].astype(np.int32)
