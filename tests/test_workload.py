"""Seeded input generator: determinism, shapes and dtype rounding."""
import numpy as np
import torch

from cross_token_gated_amd import workload as wl


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.standard_normal(100000) * 10.0 ** rng.integers(-8, 8, 100000),
                        [0.0, -0.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 65504.0, 1e-40]])
    ours = wl.round_bf16(a)
    ref = torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(ours, ref)


def test_inputs_are_deterministic_and_quantized():
    w = wl.small_workload(T=33, d_model=64, d_gate=128, head_dim=32)
    a, b = wl.make_inputs(w), wl.make_inputs(w)
    for f in ("h", "w_g", "w_v", "w_q", "w_k", "w_o"):
        x, y = getattr(a, f), getattr(b, f)
        np.testing.assert_array_equal(x, y)
        np.testing.assert_array_equal(wl.round_bf16(x), x)
    assert a.h.shape == (1, 33, 64) and a.w_o.shape == (64, 128)
    assert abs(float(a.w_g.std()) * 8.0 - 1.0) < 0.05


def test_workload_table():
    t = wl.WORKLOADS
    assert [t[k].T for k in wl.WORKLOAD_ORDER] == [256, 2048, 8192, 8192, 65536]
    assert t["wango_bf16_t8192_w256"].n_heads * t["wango_bf16_t8192_w256"].head_dim == 128
    assert t["tango_bf16_t8192_r4"].repeats == 4
    assert t["wango_bf16_b2_t65536_w512_r8"].repeats == 8


def test_layout_packers_roundtrip():
    from tests import helpers as H
    rng = np.random.default_rng(1)
    g = rng.standard_normal((256, 48))
    np.testing.assert_array_equal(H.unpack_gates(H.pack_gates(g), 256, 48), g)
    gp = H.pack_gates(g)
    # element (blk, grp, f, s) is g[32 blk + perm(grp, s), f]
    for blk, grp, f, s in [(0, 0, 0, 0), (1, 3, 47, 7), (5, 2, 10, 4), (7, 1, 3, 3)]:
        t = 32 * blk + (4 * grp + s if s < 4 else 16 + 4 * grp + s - 4)
        assert gp[blk, grp, f, s] == g[t, f]
    f = rng.standard_normal((5, 64))
    np.testing.assert_array_equal(H.unpermute_features(H.permute_features(f)), f)
    assert H.permute_features(f)[2, 32 + 8 * 3 + 5] == f[2, 32 + 16 + 4 * 3 + 1]
    n = rng.standard_normal((64, 32))
    nb = H.block_nold(n)
    np.testing.assert_array_equal(H.unblock_nold(nb, 64, 32), n)
    # lane l of block (ib, fb) holds row 16 ib + l % 16, columns 16 fb + 4 (l // 16) + r
    assert nb[1, 1, 37, 2] == n[16 + 37 % 16, 16 + 4 * (37 // 16) + 2]
