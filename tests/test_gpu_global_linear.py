"""GPU parity of the global linear-branch variant (SALAD-style: linear branch
over every key block, projected output scaled by a gate) with the oracle,
forward and backward, the GPU's mask injected into the oracle."""
import numpy as np
import pytest
import torch

import oracle as orc
from helpers import assert_close, decoded, device_inputs, to_np
from sparse_linear_attention_mean_amd.inputs import make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    global SlaProblem, B
    from sparse_linear_attention_mean_amd import _binding as B  # noqa: F811
    from sparse_linear_attention_mean_amd.attention import SlaProblem  # noqa: F811


CASES = [
    # d, grid, valid_len, frac_critical, frac_negligible, gate
    (64, (8, 8, 16), 1000, 0.125, 0.25, 0.6),
    (128, (4, 8, 32), 1024, 0.0625, 0.5, 1.0),
    (64, (8, 8, 16), 1024, 0.25, 0.0, 0.0),
    (128, (4, 8, 32), 990, 0.0, 0.0, 0.3),
]


@pytest.mark.parametrize("d,grid,vl,fc,fn,gate", CASES)
def test_global_linear_forward_backward(d, grid, vl, fc, fn, gate):
    b, h, n = 1, 2, 1024
    inp = make_inputs(b, h, n, d, grid, vl, seed=21, with_grad=True)
    dev = device_inputs(inp)
    prob = SlaProblem.create(b, h, n, d, fc, fn, valid_len=vl,
                             linear_mode=B.SLA_LINEAR_GLOBAL, linear_gate=gate)
    o, mask = prob.forward(dev["q"], dev["k"], dev["v"], dev["w"])
    dq, dk, dv, dw = prob.backward(dev["q"], dev["k"], dev["v"], dev["w"], o, dev["do"], mask)
    torch.cuda.synchronize()
    x = decoded(inp)
    m = mask.cpu().numpy()
    k_c, k_n, _ = orc.block_counts(n // 64, fc, fn)
    assert ((m == 1).sum(-1) == k_c).all() and ((m == -1).sum(-1) == k_n).all()
    ref = orc.forward(x["q"], x["k"], x["v"], x["w"], fc, fn, valid_len=vl, mask=m,
                      linear="global", gate=gate)
    assert_close("o", to_np(o), ref["o"])
    _, _, y = prob.saved_views()
    if np.abs(ref["y"]).max() > 0:
        assert_close("y", to_np(y), ref["y"])
    g = orc.backward(x["q"], x["k"], x["v"], x["w"], x["do"], m, valid_len=vl,
                     linear="global", gate=gate)
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv), ("dw", dw)):
        r = g[name]
        scale = float(np.abs(r).max()) or 1.0
        assert_close(name, to_np(t), r, atol=2e-2 * scale)
