"""GPU test of vsa_fwd_noalloc, the forward entry point that allocates nothing
(its scratch is a fixed array the library holds per GPU): through the C ABI, two
calls in a row, the second on a smaller input, each bitwise equal to vsa_fwd,
which runs the same kernels on a caller-provided workspace."""
import numpy as np
import pytest
import torch

import block_sparse_video_vsa_amd as vsa
from block_sparse_video_vsa_amd import workloads as W
from tests.parity_util import from_dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    vsa.load_library()
    return torch.device("cuda:0")


def _both(dev, name):
    wl = W.generate(name)
    q, k, v = (to_dev(x, dev, True) for x in (wl.q, wl.k, wl.v))
    topk, vbs = to_dev(wl.topk_idx, dev), to_dev(wl.vbs, dev)
    out = torch.full_like(q, float("nan"))           # every element must be written
    vsa.vsa_fwd_noalloc(q, k, v, topk, vbs, out, float(wl.sm_scale))
    ref = vsa.vsa_fwd(q, k, v, topk, vbs, float(wl.sm_scale))
    torch.cuda.synchronize()
    return from_dev(out), from_dev(ref)


def test_noalloc_equals_fwd_on_two_calls_the_second_smaller(dev):
    a, ra = _both(dev, "1")          # 8 heads x 84 cubes: 672 tiles of scratch
    assert np.array_equal(a, ra)
    b, rb = _both(dev, "0")          # 2 heads x 8 cubes: the scratch keeps the first call's bytes
    assert np.array_equal(b, rb)
