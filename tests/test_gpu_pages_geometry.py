"""The pages' own block geometry through the C ABI: d = 512, 16 heads of 32,
gate width F = 28,480 (1,780 gate columns per head, not a multiple of the
64-column blocks the kernels walk, so the library pads every head to 1,792
columns internally), window and prefix-sum block 64.

Short sequences against the whole float64 oracle; the full 8,192-token
sequence against sampled oracle rows stored by
tests/golden/make_pages_geometry_golden.py.  Bar: max|err|/rms <= 2e-2 (bf16).
"""
import os

import numpy as np
import pytest
import torch

from cross_token_gated_amd import workload as wl
from tests import helpers as H
from tests.gpu_common import announce, host, run_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from cross_token_gated_amd import _lib
    _lib.load()


@pytest.mark.parametrize("name", ["tango_pages_t8192_r4", "wango_pages_t8192_w64_r4"])
@pytest.mark.parametrize("T,R", [(200, 1), (300, 2)])
def test_pages_geometry_short(name, T, R):
    w = wl.PAGES_WORKLOADS[name].scaled(T=T, repeats=R)
    inp = wl.make_inputs(w)
    announce(f"pages geometry {name} T={T} R={R}")
    out = run_workload(w, inp)
    torch.cuda.synchronize()
    ref = H.oracle_stack(w, inp)
    e = H.err_ratio(host(out), ref)
    print(f"{name} T={T} R={R}: max|err|/rms = {e:.3e}")
    assert e < H.tol(w.dtype)


@pytest.mark.parametrize("name", ["tango_pages_t8192_r4", "wango_pages_t8192_w64_r4"])
def test_pages_geometry_t8192_sampled(name):
    path = os.path.join(os.path.dirname(__file__), "golden", "pages_geometry_t8192_samples.npz")
    gold = np.load(path, allow_pickle=False)
    w = wl.PAGES_WORKLOADS[name].scaled(repeats=1)
    inp = wl.make_inputs(w)
    announce(f"pages geometry {name} T=8192 R=1 (sampled rows)")
    out = run_workload(w, inp)
    torch.cuda.synchronize()
    rows = gold["rows"]
    got = host(out)[0, rows]
    exp = gold[f"{w.mode}_expected"]
    e = float(np.max(np.abs(got - exp))) / float(gold[f"{w.mode}_rms"])
    print(f"{name} T=8192: max|err|/rms over {rows.size} rows = {e:.3e}")
    assert np.isfinite(got).all() and e < H.tol(w.dtype)
