"""The binding refuses, before any C call, tensors the library could not read
correctly: host tensors, strided views, wrong dtypes and wrong shapes (the C
side receives bare device pointers and cannot see any of these).  CPU only:
the checks run before the library is touched."""
import numpy as np
import pytest
import torch

from cross_token_gated_amd import api

CPU = torch.device("cpu")


def _weights(F=128, d=128, H=2, dh=32, dtype=torch.bfloat16):
    return api.BlockWeights(
        w_g=torch.zeros(F, d, dtype=dtype), w_v=torch.zeros(F, d, dtype=dtype),
        w_q=torch.zeros(H * dh, d, dtype=dtype), w_k=torch.zeros(H * dh, d, dtype=dtype),
        w_o=torch.zeros(d, F, dtype=dtype), theta=torch.zeros(H, dtype=torch.float32),
        n_heads=H, head_dim=dh)


def test_check_tensor_accepts_a_good_tensor():
    api.check_tensor(torch.zeros(4, 8), "t", device=CPU, dtype=torch.float32, shape=(4, 8), min_numel=32)
    api.check_tensor(None, "t", device=CPU, optional=True)


@pytest.mark.parametrize("bad, kw, err", [
    (np.zeros(4), {}, TypeError),                                            # not a tensor
    (torch.zeros(8, 4).t(), {}, ValueError),                                 # strided view
    (torch.zeros(8, dtype=torch.float64), {"dtype": torch.float32}, TypeError),
    (torch.zeros(8, dtype=torch.float16), {"dtype": (torch.float32, torch.bfloat16)}, TypeError),
    (torch.zeros(4, 8), {"shape": (8, 4)}, ValueError),
    (torch.zeros(7), {"min_numel": 8}, ValueError),
    (None, {}, ValueError),                                                  # required
])
def test_check_tensor_rejects(bad, kw, err):
    with pytest.raises(err):
        api.check_tensor(bad, "t", device=CPU, **kw)


def test_host_tensor_is_refused_without_a_device():
    with pytest.raises(ValueError, match="GPU memory"):
        api.check_tensor(torch.zeros(4), "x")


@pytest.mark.parametrize("field, value", [
    ("w_o", torch.zeros(128, 128, dtype=torch.bfloat16).t()),        # transposed view
    ("w_o", torch.zeros(64, 128, dtype=torch.bfloat16)),             # [d, F] expected
    ("w_q", torch.zeros(32, 128, dtype=torch.bfloat16)),             # [H*d_h, d] expected
    ("w_v", torch.zeros(128, 128, dtype=torch.float32)),             # dtype differs from w_g
    ("theta", torch.zeros(2, dtype=torch.bfloat16)),                 # float32 expected
    ("theta", torch.zeros(3, dtype=torch.float32)),                  # [H] expected
    ("gain", torch.zeros(128, dtype=torch.float32)),                 # compute dtype expected
    ("null_bias", torch.zeros(2, dtype=torch.bfloat16)),             # float32 expected
])
def test_weight_checks(field, value):
    w = _weights()
    w.check(128, CPU)   # the unmodified set passes
    setattr(w, field, value)
    with pytest.raises((TypeError, ValueError)):
        w.check(128, CPU)


def test_block_call_with_host_tensors_raises_before_the_library():
    w = _weights()
    x = torch.zeros(1, 16, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU memory"):
        api.tango_block_fwd(x, w, out=torch.empty_like(x), ws=torch.empty(16, dtype=torch.uint8))
    with pytest.raises(ValueError, match="GPU memory"):
        api.wango_block_fwd(x, w, 64, 32, 64, out=torch.empty_like(x), ws=torch.empty(16, dtype=torch.uint8))


def test_stage_and_decode_calls_with_host_tensors_raise():
    w = _weights()
    shape = api.make_shape(1, 16, 128, 128, 2, 32, torch.bfloat16)
    t = torch.zeros(128 * 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU memory"):
        api.tango_stage_aggregate(shape, w.theta, None, t, t, t, t, torch.empty(16, dtype=torch.uint8))
    with pytest.raises(ValueError, match="GPU memory"):
        api.wango_stage_scan(shape, 64, 64, t, t, t, torch.zeros(4), torch.zeros(4),
                             torch.empty(16, dtype=torch.uint8))
    dshape = api.decode_shape(2, 8, w, torch.bfloat16, 128)
    with pytest.raises(ValueError, match="GPU memory"):
        api.tango_decode_step(dshape, w, torch.zeros(2, dtype=torch.int32), torch.zeros(2, 128), torch.zeros(2, 128),
                              torch.empty(16, dtype=torch.uint8), torch.empty(16, dtype=torch.uint8))
