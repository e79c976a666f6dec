"""GPU parity of the HIP path (through the C ABI) against the CPU fp64 oracle.

Small workloads are compared element by element in full; the full-size ones
(the launch configuration the benchmark times) on sampled (batch, head, query
block) items that the oracle evaluates one by one, plus properties checked
over the whole output (finite everywhere, padding rows exactly zero).
"""
import math

import numpy as np
import pytest
import torch

import block_sparse_video_vsa_amd as vsa
from block_sparse_video_vsa_amd import workloads as W
from oracle import vsa_oracle as O
from tests.parity_util import (Grade, from_dev, gather_rows, grade_every_item, oracle_rows_fwd,
                               oracle_rows_proxy, pad_rows_zero, to_dev)

pytestmark = pytest.mark.gpu
D = 128


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    vsa.load_library()
    return torch.device("cuda:0")


def run_fwd(dev, q, k, v, topk, vbs, scale):
    out = vsa.vsa_fwd(to_dev(q, dev, True), to_dev(k, dev, True), to_dev(v, dev, True),
                      to_dev(topk, dev), to_dev(vbs, dev), float(scale))
    torch.cuda.synchronize()
    return from_dev(out)


def grade_full(out, o64, vbs):
    B, S, H, _ = out.shape
    items = [(b, h, c) for b in range(B) for h in range(H) for c in range(S // 64)]
    g_rows, ids = gather_rows(out, items, vbs)
    r_rows, _ = gather_rows(o64, items, vbs)
    return Grade(g_rows, r_rows, ids)


def sample_items(wl, n, seed):
    """Deterministic sample of (b, h, qb): every vbs class, first/last blocks, outlier rows."""
    rng = np.random.default_rng(seed)
    B, S, H, _ = wl.q.shape
    nblk = S // 64
    items = {(0, 0, 0), (B - 1, H - 1, nblk - 1)}
    for val in np.unique(wl.vbs):
        cubes = np.nonzero(wl.vbs == val)[0]
        for c in rng.choice(cubes, size=min(3, cubes.size), replace=False):
            items.add((int(rng.integers(B)), int(rng.integers(H)), int(c)))
    if wl.meta.get("outlier_tokens"):
        for s in wl.meta["outlier_tokens"][:6]:
            items.add((0, 0, int(s) // 64))
    while len(items) < n:
        items.add((int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(nblk))))
    return sorted(items)


# ------------------------------------------------------------------ small, in full
@pytest.mark.parametrize("name", ["0", "1"])
def test_small_configs_full(dev, name):
    wl = W.generate(name)
    out = run_fwd(dev, wl.q, wl.k, wl.v, wl.topk_idx, wl.vbs, wl.sm_scale)
    o64 = O.vsa_fwd(wl.q, wl.k, wl.v, wl.topk_idx, wl.vbs, wl.sm_scale)
    g = grade_full(out, o64, wl.vbs)
    print(f"config {name}: {g}")
    assert pad_rows_zero(out, wl.vbs)
    assert g.ok(), str(g)


# ------------------------------------------------------------------ full size, every row
# Workloads and GPU outputs of the full-size configurations are made once per
# module and shared by the tests below.
_WL: dict = {}
_OUT: dict = {}


def workload(name):
    if name not in _WL:
        _WL[name] = W.generate(name)
    return _WL[name]


def fwd_output(dev, name):
    if name not in _OUT:
        wl = workload(name)
        _OUT[name] = run_fwd(dev, wl.q, wl.k, wl.v, wl.topk_idx, wl.vbs, wl.sm_scale)
    return _OUT[name]


@pytest.mark.parametrize("name,heads", [("2", None), ("3a", None), ("3b", (0, 20)), ("3b", (20, 40))])
def test_large_configs_every_row(dev, name, heads):
    """Every valid query row of the full-size output against the oracle (the
    card's rule over the whole tensor), in the launch configuration the
    benchmark times; 3b is graded in two halves of its heads."""
    wl = workload(name)
    out = fwd_output(dev, name)
    assert np.all(np.isfinite(O.bf16_to_f64(out))), "non-finite output"
    assert pad_rows_zero(out, wl.vbs)
    B, S, H, _ = out.shape
    h0, h1 = heads or (0, H)
    items = [(b, h, c) for b in range(B) for h in range(h0, h1) for c in range(S // 64)
             if wl.vbs[c] > 0]
    g = grade_every_item(out, wl.vbs, lambda b, h, c: O.vsa_fwd_item(
        wl.q, wl.k, wl.v, wl.topk_idx, wl.vbs, wl.sm_scale, b, h, c), items)
    print(f"config {name} heads {h0}..{h1 - 1}, every valid row ({len(items)} items): {g}")
    assert g.ok(), str(g)


def test_config2_shared_sweep_every_row(dev):
    """The timing-dependent tile order (VSA_FLAG_SHARED_SWEEP) on the full
    config-2 output, every valid row graded; it differs from the default order
    only by rounding."""
    wl = workload("2")
    out = from_dev(vsa.vsa_fwd(to_dev(wl.q, dev, True), to_dev(wl.k, dev, True),
                               to_dev(wl.v, dev, True), to_dev(wl.topk_idx, dev),
                               to_dev(wl.vbs, dev), float(wl.sm_scale), shared_sweep=True))
    torch.cuda.synchronize()
    assert np.all(np.isfinite(O.bf16_to_f64(out))), "non-finite output"
    assert pad_rows_zero(out, wl.vbs)
    g = grade_every_item(out, wl.vbs, lambda b, h, c: O.vsa_fwd_item(
        wl.q, wl.k, wl.v, wl.topk_idx, wl.vbs, wl.sm_scale, b, h, c))
    print(f"config 2, shared sweep, every valid row: {g}")
    assert g.ok(), str(g)
    d = np.abs(O.bf16_to_f64(out) - O.bf16_to_f64(fwd_output(dev, "2")))
    assert d.max() <= 2.0 ** -6 * max(1.0, float(np.abs(O.bf16_to_f64(out)).max()))


def test_small_configs_shared_sweep(dev):
    for name in ("0", "1"):
        wl = W.generate(name)
        out = from_dev(vsa.vsa_fwd(to_dev(wl.q, dev, True), to_dev(wl.k, dev, True),
                                   to_dev(wl.v, dev, True), to_dev(wl.topk_idx, dev),
                                   to_dev(wl.vbs, dev), float(wl.sm_scale), shared_sweep=True))
        torch.cuda.synchronize()
        o64 = O.vsa_fwd(wl.q, wl.k, wl.v, wl.topk_idx, wl.vbs, wl.sm_scale)
        g = grade_full(out, o64, wl.vbs)
        assert pad_rows_zero(out, wl.vbs)
        assert g.ok(), f"config {name}: {g}"


def test_config2_repeats_bitwise(dev):
    """The tile order depends on the shapes only: a repeated call on the
    full-size workload is bitwise identical."""
    wl = workload("2")
    again = run_fwd(dev, wl.q, wl.k, wl.v, wl.topk_idx, wl.vbs, wl.sm_scale)
    assert np.array_equal(fwd_output(dev, "2"), again)


def test_proxy_config4_every_row(dev):
    wl = workload("4")
    cfg = wl.config
    dq, dk, dv = (to_dev(x, dev, True) for x in (wl.q, wl.k, wl.v))
    dvbs = to_dev(wl.vbs, dev)
    km_g, vs_g = vsa.vsa_preprocess(dk, dv, dvbs)
    torch.cuda.synchronize()
    km_o, vs_o = O.vsa_preprocess(wl.k, wl.v, wl.vbs)
    km_gb, vs_gb = from_dev(km_g), from_dev(vs_g)
    # block summaries: bit-identical (both sides sum in float64 and round once)
    assert np.array_equal(km_gb, km_o) and np.array_equal(vs_gb, vs_o)
    out = vsa.vsa_fwd_proxy(dq, dk, dv, to_dev(wl.sel_idx, dev), dvbs, km_g, vs_g, cfg.prefix_len,
                            float(wl.sm_scale))
    torch.cuda.synchronize()
    out = from_dev(out)
    del dq, dk, dv
    assert np.all(np.isfinite(O.bf16_to_f64(out)))
    assert pad_rows_zero(out, wl.vbs)
    g = grade_every_item(out, wl.vbs, lambda b, h, c: O.vsa_fwd_proxy_item(
        wl.q, wl.k, wl.v, wl.sel_idx, wl.vbs, km_o, vs_o, cfg.prefix_len, wl.sm_scale, b, h, c))
    print(f"config 4 proxy, every valid row: {g}")
    assert g.ok(), str(g)


# ------------------------------------------------------------------ edge cases
def _rand_bf16(rng, shape, scale=1.0):
    return W.f32_to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


def test_degenerate_blocks(dev):
    """vbs = 0 cubes (as query and as key), ragged vbs, batch 2 and an odd head count."""
    rng = np.random.default_rng(21)
    B, H, nq = 2, 3, 9
    S = 64 * nq
    q, k, v = (_rand_bf16(rng, (B, S, H, D)) for _ in range(3))
    vbs = np.array([64, 0, 1, 33, 31, 32, 63, 0, 17], np.int32)
    topk = np.argsort(rng.random((B, H, nq, nq)), axis=-1)[..., :4].astype(np.int32)
    topk[0, 1, 2] = [1, 7, 4, 5]          # two of the four selected cubes are empty
    topk[1, 2, 4] = [1, 7, 8, 0]
    out = run_fwd(dev, q, k, v, topk, vbs, 1 / math.sqrt(D))
    o64 = O.vsa_fwd(q, k, v, topk, vbs, np.float32(1 / math.sqrt(D)))
    g = grade_full(out, o64, vbs)
    print(f"degenerate: {g}")
    assert pad_rows_zero(out, vbs)
    assert g.ok(), str(g)


def test_key_split_blocks_against_every_tile_kind(dev):
    """Query blocks with at most 32 valid rows split each tile's keys between
    the two waves, which keep separate running softmax states and merge them
    at the end.  Every such block size (1, 8, 16, 17, 31, 32), next to full
    blocks, attends to every cube: full, padded, half, half-padded and quarter
    tiles, and one bf16 tile (a cube whose values are scaled by 2^-12, below
    the range fp16 keeps exact).  Graded in full, with the row log-sum-exp,
    in the default and in the shared-sweep order."""
    rng = np.random.default_rng(41)
    B, H = 1, 3
    vbs = np.array([1, 8, 16, 17, 31, 32, 64, 40, 33, 20, 16, 5], np.int32)
    nq = vbs.size
    S = 64 * nq
    q, k, v = (_rand_bf16(rng, (B, S, H, D)) for _ in range(3))
    v[:, 64 * 7:64 * 8] = W.f32_to_bf16_bits(
        (O.bf16_to_f64(v[:, 64 * 7:64 * 8]) * 2.0 ** -12).astype(np.float32))
    topk = np.stack([rng.permutation(nq) for _ in range(B * H * nq)]).reshape(B, H, nq, nq)
    topk = topk.astype(np.int32)
    scale = np.float32(1 / math.sqrt(D))
    args = [to_dev(q, dev, True), to_dev(k, dev, True), to_dev(v, dev, True), to_dev(topk, dev),
            to_dev(vbs, dev)]
    out, lse = vsa.vsa_fwd_lse(*args, float(scale))
    shared = vsa.vsa_fwd(*args, float(scale), shared_sweep=True)
    torch.cuda.synchronize()
    o64 = O.vsa_fwd(q, k, v, topk, vbs, scale)
    for name, o in (("default", from_dev(out)), ("shared sweep", from_dev(shared))):
        g = grade_full(o, o64, vbs)
        print(f"key-split blocks, {name}: {g}")
        assert pad_rows_zero(o, vbs)
        assert g.ok(), str(g)
    items = [(0, h, c) for h in range(H) for c in range(nq)]
    worst = _lse_check_items(lse.cpu().numpy(), q, k, topk, vbs, scale, items)
    print(f"key-split blocks: max |d lse| / bound = {worst:.3g}")


def test_all_keys_empty_row_is_zero(dev):
    rng = np.random.default_rng(22)
    B, H, nq = 1, 2, 4
    S = 64 * nq
    q, k, v = (_rand_bf16(rng, (B, S, H, D)) for _ in range(3))
    vbs = np.array([64, 0, 40, 0], np.int32)
    topk = np.tile(np.array([1, 3], np.int32), (B, H, nq, 1))
    topk[0, 1, 2] = [0, 2]
    out = run_fwd(dev, q, k, v, topk, vbs, 1 / math.sqrt(D))
    o64 = O.vsa_fwd(q, k, v, topk, vbs, np.float32(1 / math.sqrt(D)))
    assert np.all(out[0, :, 0] == 0)                       # head 0: every row sees only empty cubes
    assert np.all(out[0, :64, 1] == 0)
    g = grade_full(out, o64, vbs)
    assert g.ok(), str(g)


def test_dense_topk_all_cubes_and_batch(dev):
    rng = np.random.default_rng(23)
    B, H, nq = 2, 3, 6
    S = 64 * nq
    q, k, v = (_rand_bf16(rng, (B, S, H, D)) for _ in range(3))
    vbs = np.array([64, 48, 64, 12, 64, 5], np.int32)
    topk = np.broadcast_to(np.arange(nq, dtype=np.int32), (B, H, nq, nq)).copy()
    out = run_fwd(dev, q, k, v, topk, vbs, 1 / math.sqrt(D))
    o64 = O.vsa_fwd(q, k, v, topk, vbs, np.float32(1 / math.sqrt(D)))
    g = grade_full(out, o64, vbs)
    print(f"dense: {g}")
    assert g.ok(), str(g)


def test_topk_at_the_table_limit(dev):
    """topk = 4096, the most the tile table holds (8 bytes per entry in 32 KB of
    LDS): one head of 4096 cubes in which every row selects every cube, each row
    in its own random order, with ragged and empty cubes mixed in.  Sampled
    items against the oracle; finiteness and zero padding rows everywhere."""
    rng = np.random.default_rng(41)
    B, H, nq = 1, 1, 4096
    S = 64 * nq
    q, k, v = (_rand_bf16(rng, (B, S, H, D)) for _ in range(3))
    vbs = rng.choice(np.array([64, 64, 64, 48, 32, 17, 0], np.int32), size=nq).astype(np.int32)
    topk = np.argsort(rng.random((B, H, nq, nq), dtype=np.float32), axis=-1).astype(np.int32)
    scale = np.float32(1 / math.sqrt(D))
    out = run_fwd(dev, q, k, v, topk, vbs, scale)
    assert np.all(np.isfinite(O.bf16_to_f64(out))), "non-finite output"
    assert pad_rows_zero(out, vbs)
    pick = [0, nq - 1] + [int(np.nonzero(vbs == val)[0][0]) for val in (17, 32, 48)]
    items = [(0, 0, c) for c in pick]
    g_rows, ids = gather_rows(out, items, vbs)
    r_rows = oracle_rows_fwd(q, k, v, topk, vbs, scale, items)
    g = Grade(g_rows, r_rows, ids)
    print(f"topk 4096 ({len(items)} sampled items): {g}")
    assert g.ok(), str(g)


def _offsets_case():
    """B=1, 4096 cubes, H=80 (2.7e9 elements per tensor): only the sampled
    items' query rows and the cubes they select hold data, the rest is zero."""
    rng = np.random.default_rng(43)
    B, H, nq = 1, 80, 4096
    S = 64 * nq
    assert B * S * H * D > 2 ** 31
    vbs = np.full(nq, 64, np.int32)
    vbs[nq - 1] = 40
    vbs[nq - 2] = 0
    base = np.arange(nq, dtype=np.int32)
    topk = np.stack([base, (base + 1) % nq, (base + 3) % nq], axis=-1)
    topk = np.broadcast_to(topk, (B, H, nq, 3)).copy()
    q = np.zeros((B, S, H, D), np.uint16)
    k = np.zeros((B, S, H, D), np.uint16)
    v = np.zeros((B, S, H, D), np.uint16)
    items = [(0, H - 1, nq - 1), (0, H - 1, nq - 3), (0, 0, nq - 1), (0, 41, 2047), (0, H - 1, 0)]
    for _, h, qc in items:
        q[0, 64 * qc:64 * qc + 64, h] = _rand_bf16(rng, (64, D))
        for c in topk[0, h, qc]:
            k[0, 64 * c:64 * c + 64, h] = _rand_bf16(rng, (64, D))
            v[0, 64 * c:64 * c + 64, h] = _rand_bf16(rng, (64, D))
    return q, k, v, topk, vbs, items


def test_element_offsets_beyond_2_31(dev):
    """Tensors of 2.7e9 elements: the last cubes and heads sit past element
    2^31, where 32-bit index arithmetic would wrap.  The sampled items are
    compared with the oracle; the whole output is checked for finiteness and
    zero padding rows."""
    q, k, v, topk, vbs, items = _offsets_case()
    scale = np.float32(1 / math.sqrt(D))
    out = run_fwd(dev, q, k, v, topk, vbs, scale)
    assert not np.any((out & 0x7F80) == 0x7F80), "non-finite output"
    assert pad_rows_zero(out, vbs)
    g_rows, ids = gather_rows(out, items, vbs)
    r_rows = oracle_rows_fwd(q, k, v, topk, vbs, scale, items)
    g = Grade(g_rows, r_rows, ids)
    print(f"2.7e9-element tensors ({len(items)} sampled items): {g}")
    assert g.ok(), str(g)


def test_lse_offsets_beyond_2_31(dev):
    """The row log-sum-exp output at the same 2.7e9-element shape: sampled
    rows against the oracle, -inf on padding rows and on the empty cube."""
    q, k, v, topk, vbs, items = _offsets_case()
    scale = np.float32(1 / math.sqrt(D))
    out, lse = vsa.vsa_fwd_lse(to_dev(q, dev, True), to_dev(k, dev, True), to_dev(v, dev, True),
                               to_dev(topk, dev), to_dev(vbs, dev), float(scale))
    torch.cuda.synchronize()
    del out
    lse = lse.cpu().numpy()
    worst = _lse_check_items(lse, q, k, topk, vbs, scale, items)
    nq = vbs.size
    assert np.all(np.isneginf(lse[0, :, 64 * (nq - 2):64 * (nq - 1)]))   # the empty cube
    print(f"2.7e9-element tensors: max |d lse| / bound = {worst:.3g}")


def test_proxy_offsets_beyond_2_31(dev):
    """Proxy forward on 2.7e9-element tensors (B=1, H=80, one prefix block and
    4095 video blocks, three exact picks per row, every other video block a
    proxy term).  Sampled rows, the last cube and head among them, hold data,
    as do their exact blocks and the last 64-block proxy group; the rest is
    zero.  Block summaries bitwise over the whole tensors, sampled items
    against the oracle, finiteness and zero padding rows everywhere."""
    rng = np.random.default_rng(53)
    H, npb, nb = 80, 1, 4096
    nv = nb - npb
    S = 64 * nb
    assert S * H * D > 2 ** 31
    vbs = np.full(nb, 64, np.int32)
    vbs[nb - 1] = 40
    vbs[nb - 5] = 0
    base = np.arange(nv, dtype=np.int32)
    sel = np.stack([base, (base + 1) % nv, (base + 3) % nv, np.full(nv, -1, np.int32)], axis=-1)
    sel = np.broadcast_to(sel, (1, H, nv, 4)).copy()
    q = np.zeros((1, S, H, D), np.uint16)
    k = np.zeros((1, S, H, D), np.uint16)
    v = np.zeros((1, S, H, D), np.uint16)
    items = [(0, H - 1, nb - 1), (0, H - 1, 0), (0, 0, nb - 2), (0, 41, 2048)]
    for _, h, qb in items:
        q[0, 64 * qb:64 * qb + 64, h] = _rand_bf16(rng, (64, D))
        blocks = list(range(nb - 64, nb)) + [0]
        if qb >= npb:
            blocks += [npb + int(s) for s in sel[0, h, qb - npb] if s >= 0]
        for c in blocks:
            k[0, 64 * c:64 * c + 64, h] = _rand_bf16(rng, (64, D))
            v[0, 64 * c:64 * c + 64, h] = _rand_bf16(rng, (64, D))
    dq, dk, dv, dvbs = (to_dev(q, dev, True), to_dev(k, dev, True), to_dev(v, dev, True),
                        to_dev(vbs, dev))
    km, vs = vsa.vsa_preprocess(dk, dv, dvbs)
    km_o, vs_o = O.vsa_preprocess(k, v, vbs)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(km), km_o) and np.array_equal(from_dev(vs), vs_o)
    del km_o, vs_o
    scale = np.float32(1 / math.sqrt(D))
    out = from_dev(vsa.vsa_fwd_proxy(dq, dk, dv, to_dev(sel, dev), dvbs, km, vs, 64 * npb,
                                     float(scale)))
    km_h, vs_h = from_dev(km), from_dev(vs)
    assert not np.any((out & 0x7F80) == 0x7F80), "non-finite output"
    assert pad_rows_zero(out, vbs)
    g_rows, ids = gather_rows(out, items, vbs)
    r_rows = oracle_rows_proxy(q, k, v, sel, vbs, km_h, vs_h, 64 * npb, scale, items)
    g = Grade(g_rows, r_rows, ids)
    print(f"proxy, 2.7e9-element tensors ({len(items)} sampled items): {g}")
    assert g.ok(), str(g)


def test_topk_order_invariance_bitwise(dev):
    wl = W.generate("1")
    rng = np.random.default_rng(24)
    perm = np.argsort(rng.random(wl.topk_idx.shape), axis=-1)
    shuffled = np.take_along_axis(wl.topk_idx, perm, axis=-1)
    a = run_fwd(dev, wl.q, wl.k, wl.v, wl.topk_idx, wl.vbs, wl.sm_scale)
    b = run_fwd(dev, wl.q, wl.k, wl.v, shuffled, wl.vbs, wl.sm_scale)
    assert np.array_equal(a, b)


def test_repeated_calls_are_bitwise_identical(dev):
    """The tile order depends on the shapes only, so every call gives the same
    bits; each call meets the oracle bar."""
    wl = W.generate("1")
    o64 = O.vsa_fwd(wl.q, wl.k, wl.v, wl.topk_idx, wl.vbs, wl.sm_scale)
    outs = [run_fwd(dev, wl.q, wl.k, wl.v, wl.topk_idx, wl.vbs, wl.sm_scale) for _ in range(3)]
    g = grade_full(outs[0], o64, wl.vbs)
    assert g.ok(), str(g)
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_padding_garbage_nan_and_inf(dev):
    """Non-finite values in padding slots never reach valid outputs."""
    wl = W.generate("0")
    S = wl.q.shape[1]
    pad = np.ones(S, bool)
    pad[wl.valid_slots] = False
    q, k, v = wl.q.copy(), wl.k.copy(), wl.v.copy()
    q[:, pad] = 0x7FC0          # NaN
    k[:, pad] = 0x7F80          # +inf
    v[:, pad] = 0xFFC0          # NaN
    a = run_fwd(dev, wl.q, wl.k, wl.v, wl.topk_idx, wl.vbs, wl.sm_scale)
    b = run_fwd(dev, q, k, v, wl.topk_idx, wl.vbs, wl.sm_scale)
    assert np.array_equal(a, b)


def test_scale_zero_gives_mean(dev):
    wl = W.generate("0")
    out = run_fwd(dev, wl.q, wl.k, wl.v, wl.topk_idx, wl.vbs, 0.0)
    o64 = O.vsa_fwd(wl.q, wl.k, wl.v, wl.topk_idx, wl.vbs, np.float32(0.0))
    g = grade_full(out, o64, wl.vbs)
    assert g.ok(), str(g)


@pytest.mark.parametrize("log2_scale", [16, -12])
def test_values_outside_fp16_range(dev, log2_scale):
    """Tiles whose values do not fit fp16 well (largest |v| above 65280 or below
    2^-10) take the bf16 product path, with each probability split into two
    bf16 parts.  V is scaled by a power of two, so the exact result scales
    exactly; errors are graded after scaling back, to the same bar as every
    other output."""
    wl = W.generate("0")
    s = 2.0 ** log2_scale
    v = W.f32_to_bf16_bits((O.bf16_to_f64(wl.v) * s).astype(np.float32))
    out = run_fwd(dev, wl.q, wl.k, v, wl.topk_idx, wl.vbs, wl.sm_scale)
    o64 = O.vsa_fwd(wl.q, wl.k, wl.v, wl.topk_idx, wl.vbs, wl.sm_scale)
    B, S, H, _ = out.shape
    items = [(b, h, c) for b in range(B) for h in range(H) for c in range(S // 64)]
    g_rows, ids = gather_rows(out, items, wl.vbs)
    r_rows, _ = gather_rows(o64, items, wl.vbs)
    gv = O.bf16_to_f64(g_rows) / s
    rv = O.bf16_to_f64(O.f64_to_bf16(r_rows))
    cos = float(gv.reshape(-1) @ rv.reshape(-1) / (np.linalg.norm(gv) * np.linalg.norm(rv)))
    err = np.abs(gv - rv)
    print(f"v x 2^{log2_scale}: cos={cos:.8f} max|d|={err.max():.3g} mean|d|={err.mean():.3g}")
    assert np.all(np.isfinite(gv))
    assert cos >= 0.9999
    assert err.max() <= 3e-2 and err.mean() <= 1e-4


def test_mixed_fp16_and_bf16_tiles_flat_softmax(dev):
    """One row mixing fp16 tiles and bf16 tiles under a flat softmax (small
    logits, every key carries weight): half of the cubes hold one value of 2^17
    in head-dim column 5, which sends all of that cube's tiles down the bf16
    path.  Every other column has ordinary magnitudes and is graded to the
    usual bar; column 5 must lie within one bf16 step of the rounded oracle."""
    rng = np.random.default_rng(31)
    B, H, nq = 1, 2, 16
    S = 64 * nq
    q = _rand_bf16(rng, (B, S, H, D), 0.25)
    k = _rand_bf16(rng, (B, S, H, D), 0.25)
    v = _rand_bf16(rng, (B, S, H, D))
    vbs = rng.choice(np.array([64, 48, 33, 20], np.int32), size=nq).astype(np.int32)
    big = np.zeros(nq, bool)
    big[::2] = True
    for c in np.nonzero(big)[0]:
        v[:, 64 * c + int(rng.integers(vbs[c])), :, 5] = 0x4800          # 2^17
    topk = np.argsort(rng.random((B, H, nq, nq)), axis=-1)[..., :8].astype(np.int32)
    scale = np.float32(1 / math.sqrt(D))
    out = run_fwd(dev, q, k, v, topk, vbs, scale)
    o64 = O.vsa_fwd(q, k, v, topk, vbs, scale)
    items = [(0, h, c) for h in range(H) for c in range(nq)]
    g_rows, ids = gather_rows(out, items, vbs)
    r_rows, _ = gather_rows(o64, items, vbs)
    cols = np.arange(D) != 5
    g = Grade(g_rows[:, cols], r_rows[:, cols], ids)
    print(f"mixed fp16 / bf16 tiles, ordinary columns: {g}")
    assert g.ok(), str(g)
    gv, rv = O.bf16_to_f64(g_rows[:, 5]), O.bf16_to_f64(O.f64_to_bf16(r_rows[:, 5]))
    assert np.all(np.abs(gv - rv) <= 2.0 ** -7 * np.abs(rv) + 1e-30)


def test_out_of_range_index_is_skipped(dev):
    rng = np.random.default_rng(25)
    B, H, nq = 1, 2, 5
    S = 64 * nq
    q, k, v = (_rand_bf16(rng, (B, S, H, D)) for _ in range(3))
    vbs = np.array([64, 30, 64, 7, 64], np.int32)
    base = np.argsort(rng.random((B, H, nq, nq)), axis=-1)[..., :3].astype(np.int32)
    bad = np.concatenate([base, np.full((B, H, nq, 1), -1, np.int32)], axis=-1)
    bad[0, 1, :, 3] = 1000
    out = run_fwd(dev, q, k, v, bad, vbs, 1 / math.sqrt(D))
    o64 = O.vsa_fwd(q, k, v, base, vbs, np.float32(1 / math.sqrt(D)))
    g = grade_full(out, o64, vbs)
    assert g.ok(), str(g)


def test_stages_equal_fused_call(dev):
    wl = W.generate("1")
    q, k, v = (to_dev(x, dev, True) for x in (wl.q, wl.k, wl.v))
    topk, vbs = to_dev(wl.topk_idx, dev), to_dev(wl.vbs, dev)
    B, S, H, _ = wl.q.shape
    ws = torch.empty(vsa.fwd_workspace_size(B, S, H), dtype=torch.uint8, device=dev)
    a = from_dev(vsa.vsa_fwd(q, k, v, topk, vbs, float(wl.sm_scale)))
    vsa.vsa_pack_values(v, vbs, ws)
    b = from_dev(vsa.vsa_fwd_prepacked(q, k, topk, vbs, ws, float(wl.sm_scale)))
    torch.cuda.synchronize()
    assert np.array_equal(a, b)


def test_proxy_small_cases(dev):
    """Proxy forward on small packed sequences: ragged video blocks, -1 slots,
    every video block selected (then it is exact attention), empty video blocks."""
    rng = np.random.default_rng(26)
    H = 3
    vbs = np.array([64, 64] + [64, 12, 0, 64, 33, 64, 1, 64, 50, 64, 64, 64] * 6, np.int32)
    npb = 2
    nv = vbs.size - npb
    S = 64 * vbs.size
    q, k, v = (_rand_bf16(rng, (1, S, H, D)) for _ in range(3))
    width = 9
    sel = np.full((1, H, nv, width), -1, np.int32)
    for h in range(H):
        for c in range(nv):
            picks = rng.choice(nv, size=int(rng.integers(1, width + 1)), replace=False)
            sel[0, h, c, :picks.size] = picks
    sel[0, 2, 5, :] = -1                                     # a video block with no exact picks
    dq, dk, dv, dvbs = (to_dev(q, dev, True), to_dev(k, dev, True), to_dev(v, dev, True),
                        to_dev(vbs, dev))
    km, vs = vsa.vsa_preprocess(dk, dv, dvbs)
    km_o, vs_o = O.vsa_preprocess(k, v, vbs)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(km), km_o) and np.array_equal(from_dev(vs), vs_o)
    scale = np.float32(1 / math.sqrt(D))
    out = from_dev(vsa.vsa_fwd_proxy(dq, dk, dv, to_dev(sel, dev), dvbs, km, vs, 64 * npb,
                                     float(scale)))
    o64 = O.vsa_fwd_proxy(q, k, v, sel, vbs, km_o, vs_o, 64 * npb, scale)
    g = grade_full(out, o64, vbs)
    print(f"proxy small: {g}")
    assert pad_rows_zero(out, vbs)
    assert g.ok(), str(g)
    # every video block selected -> exact attention over all valid keys
    allsel = np.broadcast_to(np.arange(nv, dtype=np.int32), (1, H, nv, nv)).copy()
    out2 = from_dev(vsa.vsa_fwd_proxy(dq, dk, dv, to_dev(allsel, dev), dvbs, km, vs, 64 * npb,
                                      float(scale)))
    full = np.broadcast_to(np.arange(vbs.size, dtype=np.int32), (1, H, vbs.size, vbs.size)).copy()
    o64b = O.vsa_fwd(q, k, v, full, vbs, scale)
    g2 = grade_full(out2, o64b, vbs)
    assert g2.ok(), str(g2)


def test_proxy_flat_softmax_full_shape(dev):
    """The packed [512 | 21x30x52] geometry with unscaled N(0,1) q and k: a flat
    softmax, so the proxy terms carry a large share of the mass (the scaled
    config-4 recipe is so peaky that they barely move its outputs)."""
    rng = np.random.default_rng(27)
    cfg = W.CONFIGS["4"]
    H = 2
    vbs = np.concatenate([np.full(cfg.n_prefix_blocks, 64, np.int32), W.tile_map(*cfg.grid)[1]])
    S = 64 * vbs.size
    q, k, v = (_rand_bf16(rng, (1, S, H, D)) for _ in range(3))
    sel = W._structured_rows(rng, H, cfg.cubes, cfg.n_video_blocks, cfg.n_random, True)
    sel = sel.reshape(1, H, cfg.n_video_blocks, cfg.max_sel)
    dq, dk, dv, dvbs = (to_dev(q, dev, True), to_dev(k, dev, True), to_dev(v, dev, True),
                        to_dev(vbs, dev))
    km, vs = vsa.vsa_preprocess(dk, dv, dvbs)
    out = from_dev(vsa.vsa_fwd_proxy(dq, dk, dv, to_dev(sel, dev), dvbs, km, vs, cfg.prefix_len,
                                     1 / math.sqrt(D)))
    km_o, vs_o = from_dev(km), from_dev(vs)
    items = sorted({(0, int(rng.integers(H)), int(rng.integers(vbs.size))) for _ in range(60)}
                   | {(0, 0, 0), (0, 1, vbs.size - 1)})
    g_rows, ids = gather_rows(out, items, vbs)
    r_rows = oracle_rows_proxy(q, k, v, sel, vbs, km_o, vs_o, cfg.prefix_len,
                               np.float32(1 / math.sqrt(D)), items)
    g = Grade(g_rows, r_rows, ids)
    print(f"proxy flat softmax ({len(items)} items): {g}")
    assert g.ok(), str(g)


@pytest.mark.parametrize("grid,B,H,D", [((5, 5, 5), 1, 2, 128), ((5, 6, 7), 2, 3, 64),
                                       ((9, 2, 13), 1, 1, 8), ((21, 30, 52), 1, 40, 128)])
def test_cube_tile_untile_bitwise(dev, grid, B, H, D):
    """Tile and untile against the oracle's layout: exact bit patterns, zero padding."""
    rng = np.random.default_rng(50 + H)
    n = int(np.prod(grid))
    x = rng.integers(0, 2 ** 16, size=(B, n, H, D), dtype=np.uint16)
    xd = torch.from_numpy(x.view(np.int16)).to(dev)
    xt = vsa.vsa_tile(xd, grid)
    back = vsa.vsa_untile(xt, grid)
    torch.cuda.synchronize()
    xt_h = xt.cpu().numpy().view(np.uint16)
    assert np.array_equal(xt_h, O.cube_tile(x, *grid))
    assert np.array_equal(back.cpu().numpy().view(np.uint16), x)
    # untile of an arbitrary padded tensor ignores its padding rows
    junk = rng.integers(0, 2 ** 16, size=xt_h.shape, dtype=np.uint16)
    got = vsa.vsa_untile(torch.from_numpy(junk.view(np.int16)).to(dev), grid)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy().view(np.uint16), O.cube_untile(junk, *grid))


def test_cube_tile_offsets_beyond_2_31(dev):
    """Tile and untile of tensors past 2^31 elements (grid 15 x 63 x 254 -> 4096
    cubes, 240 030 real rows, H = 80): the round trip is exact over the whole
    tensor (compared on the GPU), padding rows are zero, and marked rows, the
    last ones past element 2^31, land on the oracle's slots."""
    T, Hh, Wd, H = 15, 63, 254, 80
    slot, vbs = O.cube_layout(T, Hh, Wd)
    n = T * Hh * Wd
    S = 64 * vbs.size
    assert n * H * D > 2 ** 31 and S * H * D > 2 ** 31
    rng = np.random.default_rng(55)
    rows = np.array([0, 1, n // 2, n - 2, n - 1])
    marks = rng.integers(1, 2 ** 15, size=(rows.size, H, D)).astype(np.int16)
    x = torch.zeros((1, n, H, D), dtype=torch.int16, device=dev)
    x[0, torch.from_numpy(rows).to(dev)] = torch.from_numpy(marks).to(dev)
    x[0, n - 300:n - 200] = torch.randint(-2 ** 15, 2 ** 15, (100, H, D), dtype=torch.int16, device=dev)
    xt = vsa.vsa_tile(x, (T, Hh, Wd))
    back = vsa.vsa_untile(xt, (T, Hh, Wd))
    torch.cuda.synchronize()
    assert torch.equal(back, x)
    for r, m in zip(rows, marks):
        assert np.array_equal(xt[0, int(slot[r])].cpu().numpy(), m)
    used = torch.zeros(S, dtype=torch.bool, device=dev)
    used[torch.from_numpy(slot).to(dev)] = True
    assert not torch.any(xt[0, ~used])
    assert int(slot[rows[-1]]) * H * D > 2 ** 31


# --------------------------------------------------------------------------
# row statistics and merge
# --------------------------------------------------------------------------
# Bound on |lse_gpu - lse_64| per row, from the kernel's arithmetic:
#  * l sums the fp16 (round to nearest even) probabilities, each within 2^-11
#    of its value relative, so log l is within 2^-11;
#  * each logit is an fp32 MFMA sum of 128 exact bf16 products: its error is at
#    most 128 * 2^-24 = 2^-17 of sum_d |q_d k_d| (times sm_scale), and the
#    weighted average of the logits' errors bounds their effect on lse;
#  * the final (m + log2 l) ln 2 in fp32 adds a few units of 2^-24 |lse|.
# So |d| <= 2^-11 + 2^-17 * scale * max_j sum_d |q_d k_jd| + 2^-21 |lse|.
def _lse_amax(q, k, topk, vbs, scale, b, h, c):
    """Per valid query row of item (b, h, c): scale * max over its keys of sum_d |q_d k_d|."""
    nq = int(vbs[c])
    slots = O.item_key_slots(topk[b, h, c], vbs)
    if nq == 0 or slots.size == 0:
        return np.zeros(nq)
    qa = np.abs(O.bf16_to_f64(q[b, 64 * c:64 * c + nq, h, :]))
    ka = np.abs(O.bf16_to_f64(k[b, slots, h, :]))
    return float(scale) * (qa @ ka.T).max(axis=1)


def _lse_ok(lse_gpu, lse64, amax):
    fin = np.isfinite(lse64)
    assert np.array_equal(np.isfinite(lse_gpu), fin), "finite pattern differs"
    assert np.all(np.isneginf(lse_gpu[~fin]))
    d = np.abs(lse_gpu[fin] - lse64[fin])
    tol = 2.0 ** -11 + 2.0 ** -17 * amax[fin] + 2.0 ** -21 * np.abs(lse64[fin])
    assert np.all(d <= tol), f"max |d lse| {d.max():.3g}, worst d/tol {(d / tol).max():.3g}"
    return float((d / tol).max()) if d.size else 0.0


def _lse_check_items(lse, q, k, topk, vbs, scale, items):
    """Worst d / bound over the listed items; padding rows must be -inf."""
    worst = 0.0
    for b, h, c in items:
        _, l64 = O.vsa_fwd_lse_item(q, k, k, topk, vbs, scale, b, h, c)   # lse needs no V
        n = l64.size
        worst = max(worst, _lse_ok(lse[b, h, 64 * c:64 * c + n], l64,
                                   _lse_amax(q, k, topk, vbs, scale, b, h, c)))
        assert np.all(np.isneginf(lse[b, h, 64 * c + n:64 * c + 64]))
    return worst


@pytest.mark.parametrize("name", ["0", "1"])
def test_lse_small_configs_full(dev, name):
    wl = W.generate(name)
    args = [to_dev(wl.q, dev, True), to_dev(wl.k, dev, True), to_dev(wl.v, dev, True),
            to_dev(wl.topk_idx, dev), to_dev(wl.vbs, dev)]
    out, lse = vsa.vsa_fwd_lse(*args, float(wl.sm_scale))
    plain = vsa.vsa_fwd(*args, float(wl.sm_scale))
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(out), from_dev(plain))      # same output as vsa_fwd
    o64, _ = O.vsa_fwd_lse(wl.q, wl.k, wl.v, wl.topk_idx, wl.vbs, wl.sm_scale)
    g = grade_full(from_dev(out), o64, wl.vbs)
    assert g.ok(), str(g)
    B, S, H, _ = wl.q.shape
    items = [(b, h, c) for b in range(B) for h in range(H) for c in range(S // 64)]
    worst = _lse_check_items(lse.cpu().numpy(), wl.q, wl.k, wl.topk_idx, wl.vbs, wl.sm_scale, items)
    print(f"config {name}: max |d lse| / bound = {worst:.3g}")


def test_lse_batch_two(dev):
    """Row log-sum-exp with two batch entries of their own data and indices,
    ragged and empty cubes: output equal to vsa_fwd, every row graded."""
    rng = np.random.default_rng(92)
    B, H, nblk, topk = 2, 3, 20, 6
    vbs = rng.choice(np.array([64, 64, 33, 16, 1, 0], np.int32), size=nblk).astype(np.int32)
    S = 64 * nblk
    q, k = (_rand_bf16(rng, (B, S, H, D), 3.0) for _ in range(2))    # large logits, as the recipe
    v = _rand_bf16(rng, (B, S, H, D))
    topk_idx = np.argsort(rng.random((B, H, nblk, nblk)), axis=-1)[..., :topk].astype(np.int32)
    args = [to_dev(q, dev, True), to_dev(k, dev, True), to_dev(v, dev, True), to_dev(topk_idx, dev),
            to_dev(vbs, dev)]
    scale = np.float32(1 / math.sqrt(D))
    out, lse = vsa.vsa_fwd_lse(*args, float(scale))
    plain = vsa.vsa_fwd(*args, float(scale))
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(out), from_dev(plain))
    o64, _ = O.vsa_fwd_lse(q, k, v, topk_idx, vbs, scale)
    g = grade_full(from_dev(out), o64, vbs)
    assert g.ok(), str(g)
    items = [(b, h, c) for b in range(B) for h in range(H) for c in range(nblk)]
    worst = _lse_check_items(lse.cpu().numpy(), q, k, topk_idx, vbs, scale, items)
    print(f"batch two: max |d lse| / bound = {worst:.3g}")


def test_lse_config2_sampled(dev):
    wl = workload("2")
    out, lse = vsa.vsa_fwd_lse(to_dev(wl.q, dev, True), to_dev(wl.k, dev, True),
                               to_dev(wl.v, dev, True), to_dev(wl.topk_idx, dev), to_dev(wl.vbs, dev),
                               float(wl.sm_scale))
    torch.cuda.synchronize()
    lse = lse.cpu().numpy()
    items = sample_items(wl, 24, seed=8)
    worst = _lse_check_items(lse, wl.q, wl.k, wl.topk_idx, wl.vbs, wl.sm_scale, items)
    print(f"config 2 (24 sampled items): max |d lse| / bound = {worst:.3g}")


def test_split_and_merge_equals_the_whole_row(dev):
    """Each index row split in two disjoint parts, attended separately and merged."""
    wl = W.generate("1")
    rng = np.random.default_rng(64)
    T = wl.topk_idx
    Ts = np.take_along_axis(T, np.argsort(rng.random(T.shape), axis=-1), axis=-1)
    cut = T.shape[-1] // 3
    q, k, v = (to_dev(x, dev, True) for x in (wl.q, wl.k, wl.v))
    vbs = to_dev(wl.vbs, dev)
    o1, l1 = vsa.vsa_fwd_lse(q, k, v, to_dev(np.ascontiguousarray(Ts[..., :cut]), dev), vbs,
                             float(wl.sm_scale))
    o2, l2 = vsa.vsa_fwd_lse(q, k, v, to_dev(np.ascontiguousarray(Ts[..., cut:]), dev), vbs,
                             float(wl.sm_scale))
    om, lm = vsa.vsa_merge(o1, l1, o2, l2)
    torch.cuda.synchronize()
    o64, l64 = O.vsa_fwd_lse(wl.q, wl.k, wl.v, T, wl.vbs, wl.sm_scale)
    g = grade_full(from_dev(om), o64, wl.vbs)
    print(f"split + merge: {g}")
    # The merged rows are rounded to bf16 three times (each part, then the
    # merge), so a value near a bf16 step may land one step away from the
    # single rounding of the exact result (0.03125 for |o| in [4, 8)).  The
    # 3e-2 bound is therefore applied against the exact (fp64) values here.
    assert g.finite and g.min_cos >= 0.9999 and g.mean_abs <= 1e-4, str(g)
    assert g.max_abs_unrounded <= 3e-2, str(g)
    # the merge adds fp32 roundings of exp and log on top of each part's bound
    B, S, H, _ = wl.q.shape
    items = [(b, h, c) for b in range(B) for h in range(H) for c in range(S // 64)]
    _lse_check_items(lm.cpu().numpy(), wl.q, wl.k, T, wl.vbs, wl.sm_scale, items)


def test_merge_against_the_oracle(dev):
    """vsa_merge on random parts, with empty parts on one side, the other, or both."""
    rng = np.random.default_rng(65)
    B, S, H, D = 2, 96, 3, 64
    o1 = W.f32_to_bf16_bits(rng.standard_normal((B, S, H, D)).astype(np.float32))
    o2 = W.f32_to_bf16_bits((3 * rng.standard_normal((B, S, H, D))).astype(np.float32))
    l1 = (rng.standard_normal((B, H, S)) * 20).astype(np.float32)
    l2 = (rng.standard_normal((B, H, S)) * 20).astype(np.float32)
    l1[:, :, :10] = -np.inf
    l2[:, :, 5:15] = -np.inf
    out, lo = vsa.vsa_merge(to_dev(o1, dev, True), torch.from_numpy(l1).to(dev),
                            to_dev(o2, dev, True), torch.from_numpy(l2).to(dev))
    torch.cuda.synchronize()
    om, lm = O.merge_partials(np.moveaxis(O.bf16_to_f64(o1), 2, 1), l1.astype(np.float64),
                              np.moveaxis(O.bf16_to_f64(o2), 2, 1), l2.astype(np.float64))
    ref = O.f64_to_bf16(np.moveaxis(om, 1, 2))
    got = from_dev(out)
    # fp32 arithmetic, one rounding: within one bf16 step of the rounded fp64 value
    dg, dr = O.bf16_to_f64(got), O.bf16_to_f64(ref)
    assert np.all(np.abs(dg - dr) <= 2.0 ** -7 * np.abs(dr) + 1e-30)
    assert (got != ref).mean() < 0.01
    lo = lo.cpu().numpy()
    fin = np.isfinite(lm)
    assert np.array_equal(np.isfinite(lo), fin) and np.all(np.isneginf(lo[~fin]))
    assert np.all(np.abs(lo[fin] - lm[fin]) <= 1e-5 * (1 + np.abs(lm[fin])))
    assert not got[:, 5:10].any()                      # both parts empty -> zeros


# --------------------------------------------------------------------------
# bitmask and BSR selections for the proxy forward
# --------------------------------------------------------------------------
def test_proxy_at_the_table_limit(dev):
    """Proxy forward with the largest selection rows its tile table holds: one
    prefix block and 3500 video blocks, rows 3500 wide (8 bytes per possible
    tile plus 72 bytes per 64 video blocks: 32 408 of the 32 768 bytes), each
    row selecting 3000-3500 blocks so that the rest enter as proxy terms.  The
    prefix row is split over 37 key ranges.  Block summaries bitwise, sampled
    items against the oracle, finiteness and zero padding rows everywhere."""
    rng = np.random.default_rng(47)
    H, npb, nv = 1, 1, 3500
    vbs = np.concatenate([[64], rng.choice(np.array([64, 64, 64, 40, 17, 0], np.int32), size=nv)]).astype(np.int32)
    S = 64 * vbs.size
    q, k, v = (_rand_bf16(rng, (1, S, H, D)) for _ in range(3))
    sel = np.full((1, H, nv, nv), -1, np.int32)
    for c in range(nv):
        picks = rng.permutation(nv)[:int(rng.integers(3000, nv + 1))]
        sel[0, 0, c, :picks.size] = picks
    dq, dk, dv, dvbs = (to_dev(q, dev, True), to_dev(k, dev, True), to_dev(v, dev, True),
                        to_dev(vbs, dev))
    km, vs = vsa.vsa_preprocess(dk, dv, dvbs)
    km_o, vs_o = O.vsa_preprocess(k, v, vbs)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(km), km_o) and np.array_equal(from_dev(vs), vs_o)
    scale = np.float32(1 / math.sqrt(D))
    out = from_dev(vsa.vsa_fwd_proxy(dq, dk, dv, to_dev(sel, dev), dvbs, km, vs, 64 * npb,
                                     float(scale)))
    assert np.all(np.isfinite(O.bf16_to_f64(out))), "non-finite output"
    assert pad_rows_zero(out, vbs)
    pick = [0, 1, vbs.size - 1] + [int(np.nonzero(vbs == val)[0][0]) for val in (17, 40)]
    items = [(0, 0, c) for c in pick]
    g_rows, ids = gather_rows(out, items, vbs)
    r_rows = oracle_rows_proxy(q, k, v, sel, vbs, km_o, vs_o, 64 * npb, scale, items)
    g = Grade(g_rows, r_rows, ids)
    print(f"proxy at the table limit ({len(items)} sampled items): {g}")
    assert g.ok(), str(g)


def _proxy_formats(dev, wl_q, wl_k, wl_v, sel, vbs, prefix_len, scale, garbage_bits=False):
    """Outputs of the padded, bitmask and BSR calls."""
    nv = sel.shape[2]
    width = sel.shape[-1]
    dq, dk, dv, dvbs = (to_dev(wl_q, dev, True), to_dev(wl_k, dev, True), to_dev(wl_v, dev, True),
                        to_dev(vbs, dev))
    km, vs = vsa.vsa_preprocess(dk, dv, dvbs)
    mask = W.sel_to_bitmask(sel, nv)
    if garbage_bits and nv % 32:
        mask = mask.view(np.uint32).copy()
        mask[..., -1] |= np.uint32(0xFFFFFFFF) << np.uint32(nv % 32)   # bits past the last block
        mask = mask.view(np.int32)
    indptr, indices = W.sel_to_bsr(sel)
    a = vsa.vsa_fwd_proxy(dq, dk, dv, to_dev(sel, dev), dvbs, km, vs, prefix_len, scale)
    b = vsa.vsa_fwd_proxy_bitmask(dq, dk, dv, to_dev(mask, dev), dvbs, km, vs, prefix_len, width, scale)
    c = vsa.vsa_fwd_proxy_bsr(dq, dk, dv, to_dev(indptr, dev), to_dev(indices, dev), dvbs, km, vs,
                              prefix_len, width, scale)
    torch.cuda.synchronize()
    return from_dev(a), from_dev(b), from_dev(c)


def test_proxy_bitmask_and_bsr_small_bitwise(dev):
    """Same selection in three encodings: bit-identical outputs, and the oracle bar."""
    rng = np.random.default_rng(70)
    H = 3
    vbs = np.array([64, 64] + [64, 12, 0, 64, 33, 64, 1, 64, 50, 64, 64, 64] * 6, np.int32)
    npb = 2
    nv = vbs.size - npb                       # 72 video blocks: the last word is partial
    S = 64 * vbs.size
    q, k, v = (_rand_bf16(rng, (1, S, H, D)) for _ in range(3))
    width = 9
    sel = np.full((1, H, nv, width), -1, np.int32)
    for h in range(H):
        for c in range(nv):
            picks = rng.choice(nv, size=int(rng.integers(0, width + 1)), replace=False)
            sel[0, h, c, :picks.size] = picks
    a, b, c = _proxy_formats(dev, q, k, v, sel, vbs, 64 * npb, float(1 / math.sqrt(D)), True)
    assert np.array_equal(a, b) and np.array_equal(a, c)
    km_o, vs_o = O.vsa_preprocess(k, v, vbs)
    o64 = O.vsa_fwd_proxy(q, k, v, sel, vbs, km_o, vs_o, 64 * npb, np.float32(1 / math.sqrt(D)))
    g = grade_full(b, o64, vbs)
    assert g.ok(), str(g)


def test_proxy_bitmask_and_bsr_config4_bitwise(dev):
    wl = workload("4")
    a, b, c = _proxy_formats(dev, wl.q, wl.k, wl.v, wl.sel_idx, wl.vbs, wl.config.prefix_len,
                             float(wl.sm_scale), True)
    assert np.array_equal(a, b), "bitmask differs from the padded selection"
    assert np.array_equal(a, c), "BSR differs from the padded selection"


# --------------------------------------------------------------------------
# statistics of the block key means
# --------------------------------------------------------------------------
def _kc_stats_check(dev, km_bits, vbs, first, count):
    mean, var = vsa.vsa_kc_stats(to_dev(km_bits, dev, True), to_dev(vbs, dev), first, count)
    torch.cuda.synchronize()
    m_o, v_o = O.kc_stats(km_bits, vbs, first, count)
    m_g, v_g = mean.cpu().numpy(), var.cpu().numpy()
    # float64 sums in another order, one rounding to float32: equal, or one
    # float32 step apart where the float64 values straddle a rounding boundary
    for g, r in ((m_g, m_o), (v_g, v_o)):
        step = np.spacing(np.abs(r).astype(np.float32))
        assert np.all(np.abs(g.astype(np.float64) - r) <= step), np.abs(g - r).max()
        assert (g != r).mean() <= 1e-3
    return m_g, v_g


def test_kc_stats_config4_video_blocks(dev):
    """KC statistics of config 4 over its video blocks, from the GPU's own block
    summaries (which are bitwise the oracle's)."""
    wl = workload("4")
    cfg = wl.config
    dk, dvbs = to_dev(wl.k, dev, True), to_dev(wl.vbs, dev)
    km, _ = vsa.vsa_preprocess(dk, dk, dvbs)
    torch.cuda.synchronize()
    km_bits = from_dev(km)
    del dk, km
    nv = cfg.n_blocks - cfg.n_prefix_blocks
    _kc_stats_check(dev, km_bits, wl.vbs, cfg.n_prefix_blocks, nv)


def test_kc_stats_ragged_and_empty(dev):
    rng = np.random.default_rng(62)
    B, nb, H = 2, 37, 3
    km = _rand_bf16(rng, (B, nb, H, D), 5.0)
    vbs = rng.choice(np.array([64, 33, 0, 1], np.int32), size=nb).astype(np.int32)
    _kc_stats_check(dev, km, vbs, 0, nb)
    _kc_stats_check(dev, km, vbs, 5, 1)
    m, v = _kc_stats_check(dev, km, np.zeros(nb, np.int32), 3, 20)     # no block takes part
    assert not m.any() and not v.any()


# --------------------------------------------------------------------------
# routing
# --------------------------------------------------------------------------
@pytest.mark.parametrize("name,topk,heads", [("0", 3, None), ("1", 11, None), ("2", 78, 3), ("3b", 180, 2)])
def test_route_topk_bitwise(dev, name, topk, heads):
    """Block means from q and k, then the top-k blocks: indices identical to the oracle's."""
    wl = workload(name)
    q, k = wl.q, wl.k
    if heads is not None:            # large grids: a few heads keep the oracle quick
        q, k = np.ascontiguousarray(q[:, :, :heads]), np.ascontiguousarray(k[:, :, :heads])
    dq, dk, dvbs = to_dev(q, dev, True), to_dev(k, dev, True), to_dev(wl.vbs, dev)
    qm, _ = vsa.vsa_preprocess(dq, dq, dvbs)
    km, _ = vsa.vsa_preprocess(dk, dk, dvbs)
    got = vsa.vsa_route_topk(qm, km, dvbs, topk)
    torch.cuda.synchronize()
    qm_o, _ = O.vsa_preprocess(q, q, wl.vbs)
    km_o, _ = O.vsa_preprocess(k, k, wl.vbs)
    assert np.array_equal(from_dev(qm), qm_o) and np.array_equal(from_dev(km), km_o)
    want = O.route_topk(qm_o, km_o, wl.vbs, topk)
    assert np.array_equal(got.cpu().numpy(), want)


@pytest.mark.parametrize("nblk,heads,topks,kind", [
    (200, 2, (1, 50, 200), "ties"),      # ragged last score tile
    (201, 3, (5, 201), "random"),        # odd block count: score rows start at odd offsets
    (200, 1, (7, 200), "zeros"),         # every score equal: pure index order
    (1000, 1, (1, 125), "ties"),
    (2000, 1, (250,), "random"),
    (3200, 1, (3, 400), "random"),
])
def test_route_topk_ties_and_empty_blocks(dev, nblk, heads, topks, kind):
    """Synthetic block means with exact ties and empty blocks (vbs = 0): indices equal the oracle's."""
    rng = np.random.default_rng(nblk * 7 + heads)
    if kind == "zeros":
        qm = np.zeros((1, nblk, heads, 128), np.float32)
        km = np.zeros((1, nblk, heads, 128), np.float32)
    else:
        qm = rng.standard_normal((1, nblk, heads, 128)).astype(np.float32)
        km = rng.standard_normal((1, nblk, heads, 128)).astype(np.float32)
        if kind == "ties":               # key means drawn from 3 distinct rows: many equal scores
            km = km[:, rng.integers(0, 3, nblk)]
    qm_b, km_b = W.f32_to_bf16_bits(qm), W.f32_to_bf16_bits(km)
    vbs = rng.integers(1, 65, nblk).astype(np.int32)
    vbs[rng.random(nblk) < 0.1] = 0
    dq, dk, dvbs = to_dev(qm_b, dev, True), to_dev(km_b, dev, True), to_dev(vbs, dev)
    # a row's top t is the first t entries of its longest list: one oracle call
    want = O.route_topk(qm_b, km_b, vbs, max(topks))
    for topk in topks:
        got = vsa.vsa_route_topk(dq, dk, dvbs, topk)
        torch.cuda.synchronize()
        assert np.array_equal(got.cpu().numpy(), want[..., :topk]), f"topk={topk}"


def test_route_topk_follows_sequential_rounding(dev):
    """Block 0 scores 2^60 + 1 - 2^60: 0 after rounding in d order (exactly it
    would be 1); block 1 scores 0.5.  The kernel ranks by the rounded scores."""
    qm = np.zeros((1, 2, 1, 128), np.float32)
    qm[0, :, 0, :3] = [2.0 ** 60, 1.0, -(2.0 ** 60)]
    km = np.zeros((1, 2, 1, 128), np.float32)
    km[0, 0, 0, :3] = 1.0
    km[0, 1, 0, 1] = 0.5
    qm_b, km_b = W.f32_to_bf16_bits(qm), W.f32_to_bf16_bits(km)
    vbs = np.array([64, 64], np.int32)
    want = O.route_topk(qm_b, km_b, vbs, 2)
    assert want[0, 0, 0].tolist() == [1, 0]
    got = vsa.vsa_route_topk(to_dev(qm_b, dev, True), to_dev(km_b, dev, True), to_dev(vbs, dev), 2)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), want)


def test_proxy_prefix_split_and_merge(dev):
    """200 blocks: each prefix query block runs as three sub-items over key
    blocks [0, 96), [96, 192), [192, 200) and the parts are merged; the last
    range holds only empty blocks (an empty part).  Full comparison with the
    oracle, prefix rows included."""
    rng = np.random.default_rng(27)
    H, npb = 2, 3
    nblk = 200
    vbs = rng.integers(1, 65, nblk).astype(np.int32)
    vbs[:npb] = [64, 40, 64]
    vbs[192:] = 0
    nv = nblk - npb
    S = 64 * nblk
    q, k, v = (_rand_bf16(rng, (1, S, H, D)) for _ in range(3))
    width = 12
    sel = np.full((1, H, nv, width), -1, np.int32)
    for h in range(H):
        for c in range(nv):
            picks = rng.choice(nv, size=int(rng.integers(1, width + 1)), replace=False)
            sel[0, h, c, :picks.size] = picks
    dq, dk, dv, dvbs = (to_dev(q, dev, True), to_dev(k, dev, True), to_dev(v, dev, True),
                        to_dev(vbs, dev))
    km, vs = vsa.vsa_preprocess(dk, dv, dvbs)
    km_o, vs_o = O.vsa_preprocess(k, v, vbs)
    scale = np.float32(1 / math.sqrt(D))
    out = from_dev(vsa.vsa_fwd_proxy(dq, dk, dv, to_dev(sel, dev), dvbs, km, vs, 64 * npb,
                                     float(scale)))
    o64 = O.vsa_fwd_proxy(q, k, v, sel, vbs, km_o, vs_o, 64 * npb, scale)
    g = grade_full(out, o64, vbs)
    print(f"proxy prefix split: {g}")
    assert pad_rows_zero(out, vbs)
    assert g.ok(), str(g)


def test_proxy_batch_two(dev):
    """Two batch entries with their own data and selections: 2 prefix + 110
    video blocks, so each prefix query block runs as two sub-items merged per
    (batch, head).  Block summaries bitwise, the padded call graded in full,
    the bitmask and BSR calls bit-identical to it."""
    rng = np.random.default_rng(91)
    B, H, npb, nv = 2, 2, 2, 110
    vbs = np.concatenate([[64, 48], rng.choice(np.array([64, 64, 64, 40, 17, 9, 0], np.int32),
                                               size=nv)]).astype(np.int32)
    S = 64 * vbs.size
    q, k, v = (_rand_bf16(rng, (B, S, H, D)) for _ in range(3))
    width = 10
    sel = np.full((B, H, nv, width), -1, np.int32)
    for b in range(B):
        for h in range(H):
            for c in range(nv):
                picks = rng.choice(nv, size=int(rng.integers(0, width + 1)), replace=False)
                sel[b, h, c, :picks.size] = picks
    dk, dv, dvbs = to_dev(k, dev, True), to_dev(v, dev, True), to_dev(vbs, dev)
    km, vs = vsa.vsa_preprocess(dk, dv, dvbs)
    km_o, vs_o = O.vsa_preprocess(k, v, vbs)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(km), km_o) and np.array_equal(from_dev(vs), vs_o)
    scale = np.float32(1 / math.sqrt(D))
    a, b_, c = _proxy_formats(dev, q, k, v, sel, vbs, 64 * npb, float(scale), True)
    assert np.array_equal(a, b_), "bitmask differs from the padded selection"
    assert np.array_equal(a, c), "BSR differs from the padded selection"
    o64 = O.vsa_fwd_proxy(q, k, v, sel, vbs, km_o, vs_o, 64 * npb, scale)
    g = grade_full(a, o64, vbs)
    print(f"proxy batch two: {g}")
    assert pad_rows_zero(a, vbs)
    assert g.ok(), str(g)


def test_graph_replays_match_eager(dev):
    """vsa_fwd on config 2 (its last items balanced across the XCDs through
    workspace counters that a kernel zeroes) and vsa_fwd_noalloc on config 1,
    each captured in a HIP graph: every replay, with eager work and
    synchronisations between the replays, is bitwise the eager result."""
    wl = workload("2")
    q, k, v = (to_dev(x, dev, True) for x in (wl.q, wl.k, wl.v))
    t, vbs = to_dev(wl.topk_idx, dev), to_dev(wl.vbs, dev)
    B, S, H, _ = wl.q.shape
    ws = torch.empty(vsa.fwd_workspace_size(B, S, H), dtype=torch.uint8, device=dev)
    scale = float(wl.sm_scale)
    eager = vsa.vsa_fwd(q, k, v, t, vbs, scale, workspace=ws).clone()
    out = torch.empty_like(q)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        vsa.vsa_fwd(q, k, v, t, vbs, scale, out=out, workspace=ws)
    for rep in range(3):
        out.fill_(float("nan"))
        vsa.vsa_fwd(q, k, v, t, vbs, scale, workspace=ws)    # eager use of the same workspace
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"vsa_fwd replay {rep}"
    del q, k, v, ws, out, eager, g
    wl1 = W.generate("1")
    q1, k1, v1 = (to_dev(x, dev, True) for x in (wl1.q, wl1.k, wl1.v))
    t1, vbs1 = to_dev(wl1.topk_idx, dev), to_dev(wl1.vbs, dev)
    eager1 = vsa.vsa_fwd_noalloc(q1, k1, v1, t1, vbs1, torch.empty_like(q1), float(wl1.sm_scale))
    wl0 = W.generate("0")
    q0, k0, v0 = (to_dev(x, dev, True) for x in (wl0.q, wl0.k, wl0.v))
    t0, vbs0 = to_dev(wl0.topk_idx, dev), to_dev(wl0.vbs, dev)
    out0 = torch.empty_like(q0)
    out1 = torch.empty_like(q1)
    torch.cuda.synchronize()
    g1 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g1):
        vsa.vsa_fwd_noalloc(q1, k1, v1, t1, vbs1, out1, float(wl1.sm_scale))
    for rep in range(3):
        out1.fill_(float("nan"))
        vsa.vsa_fwd_noalloc(q0, k0, v0, t0, vbs0, out0, float(wl0.sm_scale))   # rewrites the scratch
        torch.cuda.synchronize()
        g1.replay()
        torch.cuda.synchronize()
        assert torch.equal(out1.view(torch.int16), eager1.view(torch.int16)), f"noalloc replay {rep}"


def test_concurrent_streams_get_their_own_workspace(dev):
    """Two calls enqueued on two streams with no synchronisation between them
    (different inputs, same shapes) each equal their single-stream result bit
    for bit: the binding does not hand one workspace to overlapping calls."""
    wl = W.generate("1")
    rng = np.random.default_rng(51)
    v2 = _rand_bf16(rng, wl.v.shape)
    ref1 = run_fwd(dev, wl.q, wl.k, wl.v, wl.topk_idx, wl.vbs, wl.sm_scale)
    ref2 = run_fwd(dev, wl.q, wl.k, v2, wl.topk_idx, wl.vbs, wl.sm_scale)
    q, k = to_dev(wl.q, dev, True), to_dev(wl.k, dev, True)
    va, vb = to_dev(wl.v, dev, True), to_dev(v2, dev, True)
    idx, vbs = to_dev(wl.topk_idx, dev), to_dev(wl.vbs, dev)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            o1 = vsa.vsa_fwd(q, k, va, idx, vbs, float(wl.sm_scale))
        with torch.cuda.stream(s2):
            o2 = vsa.vsa_fwd(q, k, vb, idx, vbs, float(wl.sm_scale))
        outs.append((o1, o2))
    torch.cuda.synchronize()
    for o1, o2 in outs:
        assert np.array_equal(from_dev(o1), ref1)
        assert np.array_equal(from_dev(o2), ref2)


def test_side_stream_matches_default_stream(dev):
    """The library enqueues on the caller's current stream: a call made under
    a side stream (inputs written on that stream) equals the default-stream
    result bit for bit."""
    wl = W.generate("1")
    ref = None
    ref = run_fwd(dev, wl.q, wl.k, wl.v, wl.topk_idx, wl.vbs, wl.sm_scale)
    side = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(side):
        args = (to_dev(wl.q, dev, True), to_dev(wl.k, dev, True), to_dev(wl.v, dev, True),
                to_dev(wl.topk_idx, dev), to_dev(wl.vbs, dev))
        out = vsa.vsa_fwd(*args, float(wl.sm_scale))
    side.synchronize()
    assert np.array_equal(from_dev(out), ref)


def test_route_topk_across_chunks(dev):
    """1440 blocks: the fp64 score workspace holds 16 (batch, head) pairs, so
    B = 2, H = 10 runs as two chunks (16 + 4 pairs, the boundary inside batch
    1).  Sampled rows of every pair, bitwise against the oracle."""
    rng = np.random.default_rng(29)
    B, H, nblk, topk = 2, 10, 1440, 180
    assert vsa.route_workspace_size(B, nblk, H) == 16 * nblk * nblk * 8
    qm = W.f32_to_bf16_bits(rng.standard_normal((B, nblk, H, 128)).astype(np.float32))
    km = W.f32_to_bf16_bits(rng.standard_normal((B, nblk, H, 128)).astype(np.float32))
    vbs = rng.integers(0, 65, nblk).astype(np.int32)
    got = vsa.vsa_route_topk(to_dev(qm, dev, True), to_dev(km, dev, True), to_dev(vbs, dev), topk)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    rows = np.array([0, 719, 1439])
    want = O.route_topk(np.ascontiguousarray(qm[:, rows]), km, vbs, topk)
    assert np.array_equal(got[:, :, rows], want)


def test_route_topk_at_the_block_limit(dev):
    """7680 blocks (the largest routing shape: one (batch, head) per chunk,
    472 MB of fp64 scores); sampled query rows against the oracle, which
    scores a row from that row's mean and every key mean alone."""
    rng = np.random.default_rng(28)
    nblk, topk = 7680, 40
    qm = W.f32_to_bf16_bits(rng.standard_normal((1, nblk, 1, 128)).astype(np.float32))
    km = W.f32_to_bf16_bits(rng.standard_normal((1, nblk, 1, 128)).astype(np.float32))
    vbs = rng.integers(0, 65, nblk).astype(np.int32)
    got = vsa.vsa_route_topk(to_dev(qm, dev, True), to_dev(km, dev, True), to_dev(vbs, dev), topk)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    rows = np.array([0, 1, 2047, 4096, 7679])
    want = O.route_topk(np.ascontiguousarray(qm[:, rows]), km, vbs, topk)
    assert np.array_equal(got[:, :, rows], want)
