"""Helpers shared by the GPU parity tests: moving workloads to the device and
grading GPU outputs against the CPU fp64 oracle.

The grading rule follows the Wan2.2 production-values dataset card,
"Scoring / loss": every element finite; per-head cosine >= 0.9999 (min over
(b, h)); max |o - o_ref| <= 3e-2 and mean |o - o_ref| <= 1e-4.  Readings of
that rule used here:
  * o_ref is the oracle's fp64 result rounded once to bf16 (nearest, even);
  * the cosine and the differences are taken over valid query rows, in fp64;
  * padding rows must be exactly 0 (and are covered by the finiteness check).
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import vsa_oracle as O

TOL_COS = 0.9999
TOL_MAX = 3e-2
TOL_MEAN = 1e-4


def to_dev(a: np.ndarray, dev, bf16: bool = False) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if bf16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(a).to(dev)


def from_dev(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |x| (2^(e-7) for |x| in [2^e, 2^(e+1)))."""
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, np.ldexp(1.0, (np.maximum(e, -126) - 7).astype(np.int64)), 2.0 ** -133)


class Grade:
    """Statistics of GPU rows against oracle rows (arrays [..., D], head axis given)."""

    def __init__(self, gpu_bits: np.ndarray, o64: np.ndarray, head_ids: np.ndarray):
        g = O.bf16_to_f64(gpu_bits)
        ref = O.bf16_to_f64(O.f64_to_bf16(o64))
        self.finite = bool(np.all(np.isfinite(g)))
        gg = np.where(np.isfinite(g), g, 0.0)
        d = np.abs(gg - ref)
        self.max_abs = float(d.max()) if d.size else 0.0
        self.mean_abs = float(d.mean()) if d.size else 0.0
        self.max_abs_unrounded = float(np.abs(gg - o64).max()) if d.size else 0.0
        self.n = int(d.size)
        self.mismatch = int((d > 0).sum())
        # faithful: the GPU value is one of the two bf16 neighbours of the exact value
        ulp = bf16_ulp(o64)
        self.unfaithful = int((np.abs(gg - o64) >= ulp).sum())
        cos = []
        for hid in np.unique(head_ids):
            sel = head_ids == hid
            a, b = gg[sel].reshape(-1), ref[sel].reshape(-1)
            na, nb = np.linalg.norm(a), np.linalg.norm(b)
            cos.append(1.0 if na == 0 and nb == 0 else float(a @ b / (na * nb)) if na * nb > 0 else 0.0)
        self.min_cos = min(cos) if cos else 1.0

    def ok(self) -> bool:
        return (self.finite and self.min_cos >= TOL_COS and self.max_abs <= TOL_MAX
                and self.mean_abs <= TOL_MEAN)

    def __str__(self) -> str:
        return (f"finite={self.finite} min_head_cos={self.min_cos:.8f} max|d|={self.max_abs:.3g} "
                f"mean|d|={self.mean_abs:.3g} mismatched={self.mismatch}/{self.n} "
                f"not-faithful={self.unfaithful} max|d vs fp64|={self.max_abs_unrounded:.3g}")


def gather_rows(arr: np.ndarray, items, vbs) -> tuple[np.ndarray, np.ndarray]:
    """Rows of the listed (b, h, qb) items' valid query rows, and their (b, h) ids."""
    rows, ids = [], []
    for b, h, qb in items:
        n = int(vbs[qb])
        rows.append(arr[b, 64 * qb:64 * qb + n, h, :])
        ids.append(np.full(n, b * 100000 + h))
    if not rows:
        return np.zeros((0, arr.shape[-1])), np.zeros(0)
    return np.concatenate(rows), np.concatenate(ids)


def oracle_rows_fwd(wl_q, wl_k, wl_v, topk, vbs, sm_scale, items) -> np.ndarray:
    parts = [O.vsa_fwd_item(wl_q, wl_k, wl_v, topk, vbs, sm_scale, b, h, qb) for b, h, qb in items]
    return np.concatenate(parts) if parts else np.zeros((0, wl_q.shape[-1]))


def oracle_rows_proxy(q, k, v, sel, vbs, km, vs, prefix_len, sm_scale, items) -> np.ndarray:
    parts = [O.vsa_fwd_proxy_item(q, k, v, sel, vbs, km, vs, prefix_len, sm_scale, b, h, qb)
             for b, h, qb in items]
    return np.concatenate(parts) if parts else np.zeros((0, q.shape[-1]))


def pad_rows_zero(out_bits: np.ndarray, vbs) -> bool:
    """True when every padding query row of the output is exactly +0."""
    S = out_bits.shape[1]
    slot = np.arange(S)
    pad = (slot % 64) >= np.asarray(vbs)[slot // 64]
    return bool(np.all(out_bits[:, pad] == 0))
