"""Rows at or past valid_len are padding: whatever they hold (here NaN) must
not reach any output.  The GPU runs on inputs whose padded rows are NaN; the
oracle runs on the same inputs with those rows zeroed (they are excluded by
definition); forward output, mask and all gradients must agree, and padded
rows of O, dQ, dK, dV must be zero."""
import numpy as np
import pytest
import torch

import oracle as orc
from helpers import assert_close, decoded, to_np
from sparse_linear_attention_mean_amd.inputs import make_inputs

pytestmark = pytest.mark.gpu

BF16_NAN = np.uint16(0x7FC0)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    global SlaProblem, bf16_from_bits
    from sparse_linear_attention_mean_amd.attention import SlaProblem, bf16_from_bits  # noqa: F811


@pytest.mark.parametrize("d,grid,vl", [(64, (8, 8, 16), 1000), (128, (4, 8, 32), 970)])
def test_nan_in_padded_rows_does_not_leak(d, grid, vl):
    b, h, n, fc, fn = 1, 2, 1024, 0.125, 0.25
    inp = make_inputs(b, h, n, d, grid, vl, seed=31, with_grad=True)
    dirty = {x: inp[x].copy() for x in ("q", "k", "v", "do")}
    for x in dirty.values():
        x[:, :, vl:] = BF16_NAN
    dev = {x: bf16_from_bits(dirty[x], "cuda") for x in dirty}
    dev["w"] = bf16_from_bits(inp["w"], "cuda")
    prob = SlaProblem.create(b, h, n, d, fc, fn, valid_len=vl)
    o, mask = prob.forward(dev["q"], dev["k"], dev["v"], dev["w"])
    dq, dk, dv, dw = prob.backward(dev["q"], dev["k"], dev["v"], dev["w"], o, dev["do"], mask)
    torch.cuda.synchronize()
    x = decoded(inp)   # clean: padded rows are zero in the generator's output
    m = mask.cpu().numpy()
    ref = orc.forward(x["q"], x["k"], x["v"], x["w"], fc, fn, valid_len=vl, mask=m)
    assert_close("o", to_np(o), ref["o"])
    g = orc.backward(x["q"], x["k"], x["v"], x["w"], x["do"], m, valid_len=vl)
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv), ("dw", dw)):
        r = g[name]
        assert_close(name, to_np(t), r, atol=2e-2 * float(np.abs(r).max()))
    for name, t in (("o", o), ("dq", dq), ("dk", dk), ("dv", dv)):
        assert torch.all(t[:, :, vl:] == 0), f"{name}: padded rows not zero"
    # the mask itself is computed from the valid rows only
    ref_mask = orc.forward(x["q"], x["k"], x["v"], x["w"], fc, fn, valid_len=vl)["mask"]
    agree = (m == ref_mask).all(-1).mean()
    assert agree >= 0.9, f"only {agree:.2f} of the mask rows agree with the oracle's"
