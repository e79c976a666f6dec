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


class FullGrade:
    """The same statistics as Grade, accumulated item by item over a whole output.

    Items are graded in worker threads (the oracle's numpy work releases the
    interpreter lock), one (b, h, query block) at a time, so that no full-size
    float64 copy of the output is ever held.  Also counts the elements whose GPU
    value is not the RNE-rounded oracle value ("flips"), and those among them at
    |o| >= 4, where one bf16 step (1/32) exceeds the 3e-2 max bound.
    """

    def __init__(self):
        self.n = 0
        self.sum_abs = 0.0
        self.max_abs = 0.0
        self.max_abs_unrounded = 0.0
        self.mismatch = 0
        self.flips_ge4 = 0
        self.unfaithful = 0
        self.finite = True
        self.heads = {}          # (b, h) -> [g.r, g.g, r.r]
        self.worst = []          # (|d|, key, row, col, o64, gpu) of the largest differences

    def add(self, key, gpu_bits: np.ndarray, o64: np.ndarray, row0: int = 0):
        g = O.bf16_to_f64(gpu_bits)
        ref = O.bf16_to_f64(O.f64_to_bf16(o64))
        fin = np.isfinite(g)
        self.finite &= bool(fin.all())
        gg = np.where(fin, g, 0.0)
        d = np.abs(gg - ref)
        if d.size:
            self.n += d.size
            self.sum_abs += float(d.sum())
            self.max_abs = max(self.max_abs, float(d.max()))
            self.max_abs_unrounded = max(self.max_abs_unrounded, float(np.abs(gg - o64).max()))
            mis = d > 0
            self.mismatch += int(mis.sum())
            self.flips_ge4 += int((mis & (np.abs(ref) >= 4.0)).sum())
            self.unfaithful += int((np.abs(gg - o64) >= bf16_ulp(o64)).sum())
            if float(d.max()) > TOL_MAX / 2:
                for r, col in zip(*np.nonzero(d > TOL_MAX / 2)):
                    self.worst.append((float(d[r, col]), key, row0 + int(r), int(col),
                                       float(o64[r, col]), float(gg[r, col])))
                self.worst = sorted(self.worst, reverse=True)[:8]
        acc = self.heads.setdefault(key, [0.0, 0.0, 0.0])
        acc[0] += float((gg * ref).sum())
        acc[1] += float((gg * gg).sum())
        acc[2] += float((ref * ref).sum())

    @property
    def mean_abs(self) -> float:
        return self.sum_abs / self.n if self.n else 0.0

    @property
    def min_cos(self) -> float:
        cos = []
        for gr, gg, rr in self.heads.values():
            if gg == 0 and rr == 0:
                cos.append(1.0)
            else:
                cos.append(gr / np.sqrt(gg * rr) if gg * rr > 0 else 0.0)
        return min(cos) if cos else 1.0

    def ok(self) -> bool:
        return (self.finite and self.min_cos >= TOL_COS and self.max_abs <= TOL_MAX
                and self.mean_abs <= TOL_MEAN)

    def __str__(self) -> str:
        worst = "; ".join(f"(b,h)={k} row {r} col {c}: o64={o:.9g} gpu={g:.9g}"
                          for _, k, r, c, o, g in self.worst[:4])
        return (f"finite={self.finite} min_head_cos={self.min_cos:.8f} max|d|={self.max_abs:.3g} "
                f"mean|d|={self.mean_abs:.3g} mismatched={self.mismatch}/{self.n} "
                f"flips at |o|>=4: {self.flips_ge4} not-faithful={self.unfaithful} "
                f"max|d vs fp64|={self.max_abs_unrounded:.3g}" + (f"; largest: {worst}" if worst else ""))


def grade_every_item(out_bits: np.ndarray, vbs, item_rows, items=None, workers=None,
                     progress=None) -> FullGrade:
    """Grade every valid query row of out_bits [B, S, H, D] against the oracle.

    item_rows(b, h, qb) returns the oracle's float64 rows [vbs[qb], D] of that
    item.  Items run on a pool of threads (at most 16, and no more than the
    CPUs this process may use), each with a single-threaded BLAS.
    """
    import os
    import threading
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    B, S, H, _ = out_bits.shape
    vbs = np.asarray(vbs)
    if items is None:
        items = [(b, h, c) for b in range(B) for h in range(H) for c in range(S // 64)
                 if vbs[c] > 0]
    nw = workers or max(1, min(16, len(os.sched_getaffinity(0))))
    chunks = [items[i::nw * 8] for i in range(nw * 8)]
    lock = threading.Lock()
    total = FullGrade()
    done = [0]

    def work(chunk):
        part = FullGrade()
        for b, h, qb in chunk:
            n = int(vbs[qb])
            part.add((b, h), out_bits[b, 64 * qb:64 * qb + n, h, :], item_rows(b, h, qb), 64 * qb)
        with lock:
            total.n += part.n
            total.sum_abs += part.sum_abs
            total.max_abs = max(total.max_abs, part.max_abs)
            total.max_abs_unrounded = max(total.max_abs_unrounded, part.max_abs_unrounded)
            total.mismatch += part.mismatch
            total.flips_ge4 += part.flips_ge4
            total.unfaithful += part.unfaithful
            total.finite &= part.finite
            total.worst = sorted(total.worst + part.worst, reverse=True)[:8]
            for key, (a, b_, c) in part.heads.items():
                acc = total.heads.setdefault(key, [0.0, 0.0, 0.0])
                acc[0] += a
                acc[1] += b_
                acc[2] += c
            done[0] += len(chunk)
            if progress is not None:
                progress(done[0], len(items))

    with threadpool_limits(1):
        with ThreadPoolExecutor(nw) as ex:
            list(ex.map(work, chunks))
    return total
