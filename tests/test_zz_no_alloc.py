"""The allocation-free forward (``sla_forward_static``) against ``sla_forward``.

The static entry point runs the same kernels on a fixed device array instead
of a caller workspace, in passes over the (batch, head) problems, so its
outputs must be bit-identical to the workspace entry point's.  Both are called
through the C ABI (ctypes) on the same inputs; the static one twice in a row
and with a smaller problem second (the array keeps the last call's contents),
then in the given-mask and global-linear modes."""
import ctypes

import numpy as np
import pytest
import torch

from helpers import device_inputs, log
from sparse_linear_attention_mean_amd.inputs import make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    global SlaProblem, B
    from sparse_linear_attention_mean_amd import _binding as B  # noqa: F811
    from sparse_linear_attention_mean_amd.attention import SlaProblem  # noqa: F811


def _static(prob, dev, o, mask):
    st = B.lib.sla_forward_static(ctypes.byref(prob.cfg), dev["q"].data_ptr(), dev["k"].data_ptr(),
                                  dev["v"].data_ptr(), dev["w"].data_ptr(), o.data_ptr(),
                                  mask.data_ptr(), prob.saved.data_ptr(),
                                  torch.cuda.current_stream().cuda_stream)
    assert st == B.SLA_OK, B.sla_last_error()


def _workspace(prob, dev, o, mask):
    ws = prob.workspace
    st = B.lib.sla_forward(ctypes.byref(prob.cfg), dev["q"].data_ptr(), dev["k"].data_ptr(),
                           dev["v"].data_ptr(), dev["w"].data_ptr(), o.data_ptr(), mask.data_ptr(),
                           prob.saved.data_ptr(), ws.data_ptr(), ws.numel(),
                           torch.cuda.current_stream().cuda_stream)
    assert st == B.SLA_OK, B.sla_last_error()


def _saved(prob, global_linear):
    """lse, den, y and the H / Z slots the forward writes, as host arrays."""
    lse, den, y = prob.saved_views()
    off = B.sla_saved_offsets(prob.cfg)
    c = prob.cfg
    bh, t, d = c.batch * c.heads, c.seq_len // 64, c.head_dim
    hst = prob.saved[off["hst"]:off["hst"] + bh * t * d * d * 2].view(torch.int16).view(bh, t, -1)
    zst = prob.saved[off["zst"]:off["zst"] + bh * t * 2 * d * 4].view(torch.float32).view(bh, t, -1)
    if global_linear:
        hst, zst = hst[:, :1], zst[:, :1]
    return [x.cpu().numpy() for x in (lse, den, y.view(torch.int16), hst, zst)]


def _compare(name, inp, fc, fn, mode=None, mask_in=None, global_linear=False):
    b, h, n, d = inp["q"].shape
    log(f"{name}: B={b} H={h} N={n} d={d} fc={fc} fn={fn}")
    kw = dict(valid_len=inp["valid_len"])
    if mode is not None:
        kw["mask_mode"] = mode
    if global_linear:
        kw.update(linear_mode=B.SLA_LINEAR_GLOBAL, linear_gate=0.7)
    dev = device_inputs(inp)
    outs = []
    for run in (_workspace, _static):
        prob = SlaProblem.create(b, h, n, d, fc, fn, **kw)
        o = torch.full(prob.shape(), float("nan"), dtype=torch.bfloat16, device="cuda")
        mask = prob.new_mask()
        if mask_in is not None:
            mask.copy_(mask_in)
        prob.saved.fill_(0xFF)
        run(prob, dev, o, mask)
        torch.cuda.synchronize()
        outs.append((o.view(torch.int16).cpu().numpy(), mask.cpu().numpy(),
                     _saved(prob, global_linear)))
    (o0, m0, s0), (o1, m1, s1) = outs
    assert np.array_equal(m0, m1), f"{name}: mask"
    assert np.array_equal(o0, o1), f"{name}: O"
    for label, a0, a1 in zip(("lse", "den", "y", "H", "Z"), s0, s1):
        assert np.array_equal(a0, a1), f"{name}: {label}"
    return torch.from_numpy(m0)


def test_static_forward_matches_workspace_forward():
    per_pass = B.SLA_STATIC_SCRATCH_BYTES // 19_696_128   # heads of T = 512, d = 128 per pass
    assert per_pass == 3
    # 6 heads of 32768 tokens: two passes of three (batch, head) problems
    big = make_inputs(2, 3, 32768, 128, (21, 30, 52), 32760, seed=61, with_grad=False)
    _compare("two passes", big, 0.05, 0.10)
    # a smaller problem right after (the array holds the last call's contents)
    small = make_inputs(1, 2, 1024, 64, (8, 8, 16), 1000, seed=62, with_grad=False)
    m = _compare("one pass", small, 0.125, 0.25)
    _compare("given mask", small, 0.0, 0.0, mode=B.SLA_MASK_GIVEN, mask_in=m)
    _compare("global linear", small, 0.125, 0.25, global_linear=True)


def test_static_forward_refuses_oversized_problem():
    buf = torch.empty(16, dtype=torch.uint8, device="cuda")
    p = buf.data_ptr()
    cfg = B.make_config(1, 1, 64 * 1441, 128, 0.05, 0.1)
    st = B.lib.sla_forward_static(ctypes.byref(cfg), *([p] * 7),
                                  torch.cuda.current_stream().cuda_stream)
    assert st == B.SLA_ERR_WORKSPACE
