"""C-ABI checks that need no GPU: the library loads, exports every function
include/vsa.h declares, and rejects bad arguments on the host before any
device work (so these calls never reach the HIP runtime)."""
import ctypes
import os
import re

import pytest

from block_sparse_video_vsa_amd import native

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "vsa.h")
OK, NULL, SHAPE, ALIGN, UNSUP, LAUNCH, WS, VALUE = range(8)
FAKE = 0x10000          # a non-null, 256-byte-aligned address that is never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(vsa_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return native.load_library()


def test_every_declared_function_is_exported(lib):
    names = declared_functions()
    assert {"vsa_fwd", "vsa_preprocess", "vsa_fwd_proxy", "vsa_status_string",
            "vsa_fwd_workspace_size", "vsa_fwd_proxy_workspace_size", "vsa_pack_values",
            "vsa_fwd_prepacked",
            "vsa_cube_count", "vsa_cube_vbs", "vsa_tile", "vsa_untile", "vsa_fwd_lse",
            "vsa_merge", "vsa_fwd_proxy_bitmask", "vsa_fwd_proxy_bsr", "vsa_route_topk",
            "vsa_route_workspace_size", "vsa_kc_stats", "vsa_fwd_noalloc",
            "vsa_fwd_noalloc_max_bytes", "vsa_fwd_ex", "vsa_fwd_prepacked_ex"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert set(native._SIGNATURES) == set(names)


def test_status_strings(lib):
    for s in range(9):
        assert native.status_string(s).startswith("VSA_")
    assert native.status_string(99) == "VSA_ERR_UNKNOWN"


def test_workspace_sizes(lib):
    # 16 KB packed V tile + one flag byte per (batch, head, cube), then 2 KB of
    # tail-pool counters (eight, one 256-byte line each), 256-byte aligned regions
    n = native.fwd_workspace_size(1, 39936, 40)
    assert n == 40 * 624 * 16384 + ((40 * 624 + 255) // 256) * 256 + 2048
    assert native.fwd_workspace_size(2, 512, 2) >= 2 * 2 * 8 * 16384 + 32
    assert native.fwd_workspace_size(1, 100, 2) == 0
    assert native.fwd_workspace_size(1, 512, 2, 64) == 0
    assert native.proxy_workspace_size(1, 40448, 512, 56) > native.fwd_workspace_size(1, 40448, 56)
    assert native.proxy_workspace_size(1, 40448, 0, 56) == 0
    assert native.proxy_workspace_size(1, 40448, 100, 56) == 0


def _fwd(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, idx=FAKE, vbs=FAKE, out=FAKE, B=1, S=512, H=2, D=128, topk=2,
             scale=0.088, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return lib.vsa_fwd(a["q"], a["k"], a["v"], a["idx"], a["vbs"], a["out"], a["B"], a["S"], a["H"],
                       a["D"], a["topk"], a["scale"], a["ws"], a["wsb"], None)


def test_fwd_rejects_bad_arguments_on_host(lib):
    assert _fwd(lib, q=None) == NULL
    assert _fwd(lib, vbs=None) == NULL
    assert _fwd(lib, D=64) == UNSUP
    assert _fwd(lib, S=100) == SHAPE
    assert _fwd(lib, S=0) == SHAPE
    assert _fwd(lib, B=0) == SHAPE
    assert _fwd(lib, H=0) == SHAPE
    assert _fwd(lib, topk=0) == SHAPE
    assert _fwd(lib, topk=9) == SHAPE
    assert _fwd(lib, scale=-1.0) == VALUE
    assert _fwd(lib, scale=float("nan")) == VALUE
    assert _fwd(lib, scale=float("inf")) == VALUE
    assert _fwd(lib, q=FAKE + 8) == ALIGN
    assert _fwd(lib, idx=FAKE + 2) == ALIGN
    assert _fwd(lib, ws=None) == WS
    assert _fwd(lib, wsb=1000) == WS
    assert _fwd(lib, ws=FAKE + 16) == ALIGN


def test_stage_and_proxy_entry_points_reject_bad_arguments(lib):
    assert lib.vsa_pack_values(None, FAKE, 1, 512, 2, 128, FAKE, 1 << 30, None) == NULL
    assert lib.vsa_pack_values(FAKE, FAKE, 1, 512, 2, 128, FAKE, 10, None) == WS
    assert lib.vsa_fwd_prepacked(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 512, 2, 128, 0, 0.1, FAKE,
                                 1 << 30, None) == SHAPE
    assert lib.vsa_preprocess(FAKE, FAKE, FAKE, FAKE, None, 1, 512, 2, 128, None) == NULL
    assert lib.vsa_preprocess(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 512, 2, 96, None) == UNSUP
    assert lib.vsa_preprocess(FAKE + 4, FAKE, FAKE, FAKE, FAKE, 1, 512, 2, 128, None) == ALIGN
    px = lambda **kw: lib.vsa_fwd_proxy(  # noqa: E731
        FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, kw.get("S", 1024), kw.get("P", 128),
        2, 128, kw.get("sel", 4), kw.get("scale", 0.1), FAKE, kw.get("wsb", 1 << 30), None)
    assert px(P=0) == SHAPE
    assert px(P=1024) == SHAPE
    assert px(P=100) == SHAPE
    assert px(sel=0) == SHAPE
    assert px(sel=15) == SHAPE
    assert px(scale=-2.0) == VALUE
    assert px(wsb=100) == WS


def test_noalloc_rejects_shapes_beyond_its_scratch_on_host(lib):
    """vsa_fwd_noalloc checks the shape first, then its fixed scratch: the
    Wan2.2 shape (40 x 624 tiles of 16 KB) exceeds the 64 MiB array."""
    assert lib.vsa_fwd_noalloc_max_bytes() == 64 << 20
    call = lambda **kw: lib.vsa_fwd_noalloc(  # noqa: E731
        FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, kw.get("S", 39936), kw.get("H", 40), 128,
        kw.get("topk", 78), 0.088, None)
    assert call() == 8                       # VSA_ERR_SCRATCH
    assert call(topk=0) == SHAPE             # shape errors come first
    assert lib.vsa_fwd_noalloc(None, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 512, 2, 128, 2, 0.1,
                               None) == NULL


def test_fwd_ex_rejects_unknown_flags_on_host(lib):
    ex = lambda flags, topk=2: lib.vsa_fwd_ex(  # noqa: E731
        FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 512, 2, 128, topk, 0.088, flags, FAKE, 1 << 30, None)
    assert ex(2) == VALUE
    assert ex(1 << 31) == VALUE
    assert ex(1, topk=0) == SHAPE
    assert lib.vsa_fwd_prepacked_ex(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 512, 2, 128, 2, 0.088, 4, FAKE,
                                    1 << 30, None) == VALUE


def test_kc_stats_rejects_bad_arguments_on_host(lib):
    kc = lambda **kw: lib.vsa_kc_stats(  # noqa: E731
        kw.get("km", FAKE), FAKE, kw.get("mean", FAKE), FAKE, 1, kw.get("nb", 16), 2,
        kw.get("D", 128), kw.get("first", 4), kw.get("count", 12), None)
    assert kc(km=None) == NULL
    assert kc(mean=None) == NULL
    assert kc(D=64) == UNSUP
    assert kc(first=-1) == SHAPE
    assert kc(count=13) == SHAPE            # 4 + 13 > 16 blocks
    assert kc(nb=0) == SHAPE
    assert kc(km=FAKE + 1) == ALIGN
    assert kc(mean=FAKE + 2) == ALIGN


def test_launch_size_limits_on_host(lib):
    """Every launch stays at or below 2^31 threads: at most 2^23 (batch, head,
    block) triples for the forward family and the block summaries, at most
    2^24 - 8 proxy work items, at most 2^23 tiled rows."""
    nb = (1 << 20) - 1
    assert _fwd(lib, S=64 * nb, H=9) == SHAPE                       # 9 (2^20 - 1) > 2^23
    assert lib.vsa_preprocess(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 64 * nb, 9, 128, None) == SHAPE
    # 50 000 prefix blocks, each split over ceil(100 000 / 96) key ranges: 5.2e7 items
    assert lib.vsa_fwd_proxy(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 64 * 100000,
                             64 * 50000, 1, 128, 4, 0.1, FAKE, 1 << 30, None) == SHAPE
    assert lib.vsa_tile(FAKE, FAKE, 2, 256, 256, 256, 2, 128, None) == SHAPE   # 2 x 64 x 64^3 rows
    assert lib.vsa_untile(FAKE, FAKE, 2, 256, 256, 256, 2, 128, None) == SHAPE


def test_binding_fails_loudly_without_the_library(tmp_path, monkeypatch):
    """No CPU fallback: with the shared library absent, every entry point of the
    binding raises instead of computing anything."""
    import torch
    from block_sparse_video_vsa_amd import native
    monkeypatch.setattr(native, "_lib", None)
    monkeypatch.setattr(native, "LIB_PATH", str(tmp_path / "libvsa.so"))
    with pytest.raises(ImportError):
        native.load_library()
    t = torch.zeros((1, 64, 1, 128), dtype=torch.bfloat16)
    with pytest.raises(ImportError):
        native.vsa_fwd(t, t, t, torch.zeros((1, 1, 1, 1), dtype=torch.int32),
                       torch.full((1,), 64, dtype=torch.int32))


def test_binding_rejects_cpu_tensors():
    import torch
    q = torch.zeros(1, 64, 1, 128, dtype=torch.bfloat16)
    idx = torch.zeros(1, 1, 1, 1, dtype=torch.int32)
    vbs = torch.zeros(1, dtype=torch.int32)
    with pytest.raises((ValueError, TypeError, RuntimeError, AssertionError)):
        native.vsa_fwd(q, q, q, idx, vbs, out=q)


def test_cube_count_and_vbs_match_the_oracle(lib):
    """vsa_cube_vbs runs on the host: compare it with the oracle's layout directly."""
    import numpy as np
    from oracle import vsa_oracle as O
    for grid in [(5, 5, 5), (21, 30, 52), (21, 45, 80), (1, 1, 1), (4, 4, 4), (9, 2, 13)]:
        _, vbs_o = O.cube_layout(*grid)
        assert lib.vsa_cube_count(*grid) == vbs_o.size
        assert np.array_equal(native.cube_vbs(*grid), vbs_o)
    assert lib.vsa_cube_count(0, 4, 4) == 0
    assert lib.vsa_cube_count(4, -1, 4) == 0
    buf = (ctypes.c_int32 * 7)()
    assert lib.vsa_cube_vbs(5, 5, 5, buf, 7) == SHAPE          # 8 cubes do not fit in 7
    assert lib.vsa_cube_vbs(5, 5, 5, None, 8) == NULL


def test_tile_rejects_bad_arguments_on_host(lib):
    t = lambda **kw: lib.vsa_tile(kw.get("x", FAKE), kw.get("xt", FAKE), kw.get("B", 1), kw.get("T", 5),
                                  kw.get("Hh", 5), kw.get("W", 5), kw.get("H", 2), kw.get("D", 128), None)
    assert t(x=None) == NULL
    assert t(xt=None) == NULL
    assert t(B=0) == SHAPE
    assert t(T=0) == SHAPE
    assert t(H=1, D=4) == SHAPE                  # rows of 4 elements are not 16-byte pieces
    assert t(x=FAKE + 8) == ALIGN
    assert lib.vsa_untile(FAKE + 4, FAKE, 1, 5, 5, 5, 2, 128, None) == ALIGN
    assert lib.vsa_untile(FAKE, FAKE, 1, 5, 5, 0, 2, 128, None) == SHAPE


def test_lse_and_merge_reject_bad_arguments_on_host(lib):
    f = lambda lse=FAKE, **kw: lib.vsa_fwd_lse(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, lse, 1, 512, 2, 128,
                                               kw.get("topk", 2), 0.088, FAKE, 1 << 30, None)
    assert f(lse=None) == NULL
    assert f(topk=0) == SHAPE
    assert f(lse=FAKE + 2) == ALIGN
    m = lambda **kw: lib.vsa_merge(kw.get("o1", FAKE), kw.get("l1", FAKE), FAKE, FAKE, FAKE,
                                   kw.get("lo", FAKE), 1, kw.get("S", 64), 2, kw.get("D", 128), None)
    assert m(o1=None) == NULL
    assert m(lo=None) == NULL
    assert m(D=12) == SHAPE
    assert m(S=0) == SHAPE
    assert m(o1=FAKE + 8) == ALIGN
    assert m(l1=FAKE + 2) == ALIGN


def test_bitmask_and_bsr_proxy_reject_bad_arguments_on_host(lib):
    S, P = 64 * 40, 128                        # 38 video blocks
    bm = lambda mask=FAKE, es=5: lib.vsa_fwd_proxy_bitmask(FAKE, FAKE, FAKE, mask, FAKE, FAKE, FAKE, FAKE,
                                                         1, S, P, 2, 128, es, 0.088, FAKE, 1 << 30, None)
    assert bm(mask=None) == NULL
    assert bm(es=0) == SHAPE
    assert bm(es=39) == SHAPE
    assert bm(mask=FAKE + 2) == ALIGN
    bs = lambda ip=FAKE, ix=FAKE, nnz=10: lib.vsa_fwd_proxy_bsr(FAKE, FAKE, FAKE, ip, ix, nnz, FAKE, FAKE,
                                                               FAKE, FAKE, 1, S, P, 2, 128, 5, 0.088,
                                                               FAKE, 1 << 30, None)
    assert bs(ip=None) == NULL
    assert bs(ix=None) == NULL
    assert bs(nnz=-1) == SHAPE
    assert bs(ix=FAKE + 1) == ALIGN


def test_selection_format_helpers():
    import numpy as np
    from block_sparse_video_vsa_amd import workloads as W
    sel = np.array([[[[3, 0, -1, 37], [-1, -1, -1, -1], [5, 31, 32, 33]]]], np.int32)
    m = W.sel_to_bitmask(sel, 38).view(np.uint32)
    assert m.shape == (1, 1, 3, 2)
    assert m[0, 0, 0].tolist() == [(1 << 3) | 1, 1 << 5]
    assert m[0, 0, 1].tolist() == [0, 0]
    assert m[0, 0, 2].tolist() == [(1 << 5) | (1 << 31), 0b11]
    ip, ix = W.sel_to_bsr(sel)
    assert ip.tolist() == [0, 3, 3, 7] and ix.tolist() == [3, 0, 37, 5, 31, 32, 33]


def test_route_rejects_bad_arguments_on_host(lib):
    need = lib.vsa_route_workspace_size(1, 624, 2)
    assert need == 2 * 624 * 624 * 8                       # both pairs fit one chunk
    assert lib.vsa_route_workspace_size(1, 7680, 40) == 7680 * 7680 * 8   # one pair per chunk
    assert lib.vsa_route_workspace_size(1, 7681, 1) == 0
    # one block per row: a chunk is capped at 2^23 pairs, so that the score
    # kernel's launch (one 256-thread workgroup per pair) stays at 2^31 threads
    assert lib.vsa_route_workspace_size(4096, 1, 65536) == (1 << 23) * 8
    r = lambda **kw: lib.vsa_route_topk(kw.get("q", FAKE), FAKE, FAKE, kw.get("o", FAKE), 1,
                                        kw.get("nb", 624), 2, kw.get("D", 128), kw.get("k", 78),
                                        kw.get("ws", FAKE), kw.get("wsb", need), None)
    assert r(q=None) == NULL
    assert r(o=None) == NULL
    assert r(D=64) == UNSUP
    assert r(k=0) == SHAPE
    assert r(k=625) == SHAPE
    assert r(nb=7681, k=5) == SHAPE
    assert r(q=FAKE + 8) == ALIGN                          # means are read 16 bytes at a time
    assert r(ws=None) == WS
    assert r(wsb=need - 1) == WS
    assert r(ws=FAKE + 16) == ALIGN
