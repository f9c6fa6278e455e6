"""GPU parity with the CPU oracle for block lists longer than 64 entries.

The three attention kernels keep their block list in one register per lane
(64 entries) and take the next 64 entries when the loop reaches them: the
fused forward over the critical key blocks of a query block, the dQ kernel
over the same list, and the key-block backward over the query blocks for
which a key block is critical (its column).  These cases put more than 64
entries in rows and columns: the flat split with k_c = 77, given masks with
rows and columns of 64, 65, 128, 129 and T critical blocks, the dense mode
(every row and column of length T > 64) and mask reuse in the autograd module
with every block critical.  Critical blocks get exact softmax attention
however many there are ("SLA: Beyond Sparsity in Diffusion Transformers via
Fine-Tunable Sparse-Linear Attention", English abstract)."""
import numpy as np
import pytest
import torch

import oracle as orc
from helpers import assert_close, decoded, device_inputs, log, mask_validity, rel_l2, to_np
from sparse_linear_attention_mean_amd.inputs import make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    global SlaProblem, B
    from sparse_linear_attention_mean_amd import _binding as B  # noqa: F811
    from sparse_linear_attention_mean_amd.attention import SlaProblem  # noqa: F811


def _run(inp, fc, fn, mask=None, backward=True):
    b, h, n, d = inp["q"].shape
    mode = B.SLA_MASK_GIVEN if mask is not None else B.SLA_MASK_COMPUTE
    prob = SlaProblem.create(b, h, n, d, fc, fn, valid_len=inp["valid_len"], mask_mode=mode)
    dev = device_inputs(inp)
    m = prob.new_mask()
    if mask is not None:
        m.copy_(torch.from_numpy(mask))
    o, m = prob.forward(dev["q"], dev["k"], dev["v"], dev["w"], mask=m)
    torch.cuda.synchronize()
    lse, den, y = prob.saved_views()
    out = dict(o=to_np(o), mask=m.cpu().numpy(), lse=lse.cpu().numpy(), den=den.cpu().numpy(),
               y=to_np(y))
    if backward:
        dq, dk, dv, dw = prob.backward(dev["q"], dev["k"], dev["v"], dev["w"], o, dev["do"], m)
        torch.cuda.synchronize()
        out.update(dq=to_np(dq), dk=to_np(dk), dv=to_np(dv), dw=to_np(dw))
    return out


def _check_forward(name, got, ref, vl, rows=None):
    n = got["o"].shape[2]
    valid = np.arange(n) < vl
    sel = np.broadcast_to(valid, got["o"].shape[:3]).copy()
    if rows is not None:
        sel &= np.repeat(rows, 64, axis=-1)[..., :n]
    assert_close(f"{name} O", got["o"][sel], ref["o"][sel])
    assert_close(f"{name} Y", got["y"][sel], ref["y"][sel])
    fin = np.isfinite(ref["lse"]) & sel
    assert np.array_equal(np.isfinite(got["lse"]) & sel, fin), "lse finiteness"
    if fin.any():
        assert np.abs(got["lse"][fin] - ref["lse"][fin]).max() < 1e-3
    dpos = sel & (ref["den"] > 0)
    if dpos.any():
        assert rel_l2(got["den"][dpos], ref["den"][dpos]) < 1e-2
    assert np.all(got["o"][:, :, ~valid] == 0)


def _check_grads(name, got, ref):
    for g in ("dq", "dk", "dv", "dw"):
        scale = float(np.abs(ref[g]).max()) or 1.0
        assert_close(f"{name} {g}", got[g], ref[g], atol=2e-2 * scale)


@pytest.mark.parametrize("d", [64, 128])
def test_forward_77_critical_blocks(d):
    """Flat split with f_c = 0.3 at T = 256: every row has k_c = 77 critical
    blocks (the library classifies, as in the benchmark's mode)."""
    b, h, n, vl, fc, fn = 1, 2, 16384, 16380, 0.3, 0.1
    t = n // 64
    k_c, k_n, _ = orc.block_counts(t, fc, fn)
    assert k_c == 77
    log(f"flat split T={t} k_c={k_c} d={d}")
    inp = make_inputs(b, h, n, d, (16, 32, 32), vl, seed=41, with_grad=False)
    x = decoded(inp)
    ref = orc.forward(x["q"], x["k"], x["v"], x["w"], fc, fn, valid_len=vl)
    got = _run(inp, fc, fn, backward=False)
    tol = 1e-4 * float(np.abs(ref["scores"]).max()) + 1e-6
    same = mask_validity(got["mask"], ref["scores"], k_c, k_n, tol)
    log(f"  mask rows equal to the oracle's: {same.mean():.4f}")
    assert same.mean() > 0.9
    _check_forward(f"kc77_d{d}", got, ref, vl, rows=same)


def _long_mask(rng, h, t):
    """Given masks whose rows and columns hold 64, 65, 128, 129 and about t
    critical blocks, plus random rows with about half of the blocks critical."""
    mask = rng.choice(np.array([1, 0, -1], np.int8), size=(1, h, t, t), p=(0.5, 0.3, 0.2))
    m = mask[0, 0]
    for cix, c in ((7, 65), (8, 129), (9, t), (10, 64)):
        m[:, cix] = rng.choice(np.array([0, -1], np.int8), size=t)
        m[np.sort(rng.choice(t, c, replace=False)), cix] = 1
    m[:, t - 1] = 1                            # the padded last key block critical in every row
    for r, c in ((0, 64), (1, 65), (2, 128), (3, 129), (4, t)):
        m[r] = rng.choice(np.array([0, -1], np.int8), size=t)
        m[r, np.sort(rng.choice(t, c, replace=False))] = 1
    m[5] = 0                                   # no critical block, all marginal
    m[6] = 1
    m[6, 0] = 0                                # t - 1 critical blocks and one marginal
    return mask


@pytest.mark.parametrize("d", [64, 128])
def test_given_mask_long_rows_and_columns(d):
    """Forward and backward with a given mask whose rows and columns hold more
    than 64 and more than 128 critical blocks, element-wise against the oracle."""
    h, n, vl = 2, 160 * 64, 160 * 64 - 7
    t = n // 64
    rng = np.random.default_rng(d)
    mask = _long_mask(rng, h, t)
    rows = (mask == 1).sum(-1)
    cols = (mask == 1).sum(-2)
    log(f"given mask T={t} d={d}: longest row {rows.max()}, longest column {cols.max()}")
    assert rows.max() == t and cols.max() >= t - 7
    inp = make_inputs(1, h, n, d, (10, 16, 64), vl, seed=43)
    x = decoded(inp)
    ref = orc.forward(x["q"], x["k"], x["v"], x["w"], 0.0, 0.0, valid_len=vl, mask=mask)
    got = _run(inp, 0.0, 0.0, mask=mask)
    assert np.array_equal(got["mask"], mask)
    _check_forward(f"long_given_d{d}", got, ref, vl)
    g = orc.backward(x["q"], x["k"], x["v"], x["w"], x["do"], mask, valid_len=vl)
    _check_grads(f"long_given_d{d}", got, g)


@pytest.mark.parametrize("d", [64, 128])
def test_dense_mode_long(d):
    """Every block critical (frac_critical = 1): the dense mode with T = 130,
    so every row of the forward and every row and column of the backward has
    130 entries."""
    n, vl = 130 * 64, 130 * 64 - 20
    log(f"dense T=130 d={d}")
    inp = make_inputs(1, 1, n, d, (13, 8, 80), vl, seed=47)
    x = decoded(inp)
    ones = np.ones((1, 1, 130, 130), np.int8)
    ref = orc.forward(x["q"], x["k"], x["v"], x["w"], 1.0, 0.0, valid_len=vl)
    assert np.array_equal(ref["mask"], ones)
    got = _run(inp, 1.0, 0.0)
    assert np.array_equal(got["mask"], ones)
    _check_forward(f"dense130_d{d}", got, ref, vl)
    g = orc.backward(x["q"], x["k"], x["v"], x["w"], x["do"], ones, valid_len=vl)
    _check_grads(f"dense130_d{d}", got, g)


def test_autograd_reuse_dense_mask_long():
    """The autograd module with f_c = 1 and mask reuse at N = 4224 (T = 66): the
    first call runs the dense mode, the second passes the all-critical mask
    back in the given-mask mode, which walks lists of 66 entries."""
    from sparse_linear_attention_mean_amd.autograd import SparseLinearAttention

    b, h, n, d, vl = 1, 2, 4224, 128, 4224
    inp = make_inputs(b, h, n, d, (6, 8, 88), vl, seed=53)
    dev = device_inputs(inp)
    mod = SparseLinearAttention(d, 1.0, 0.0, valid_len=vl, reuse_mask=True,
                                weight=dev["w"].float())
    x = decoded(inp)
    ones = np.ones((b, h, n // 64, n // 64), np.int8)
    ref = orc.forward(x["q"], x["k"], x["v"], x["w"], 1.0, 0.0, valid_len=vl)
    g = orc.backward(x["q"], x["k"], x["v"], x["w"], x["do"], ones, valid_len=vl)
    for call in range(2):
        q, k, v = (dev[nm].clone().requires_grad_(True) for nm in ("q", "k", "v"))
        mod.weight.grad = None
        o = mod(q, k, v)
        o.backward(dev["do"])
        torch.cuda.synchronize()
        assert np.array_equal(mod.cached_mask.cpu().numpy(), ones)
        log(f"call {call}")
        assert_close(f"call{call} o", to_np(o), ref["o"])
        for name, t in (("dq", q.grad), ("dk", k.grad), ("dv", v.grad)):
            r = g[name]
            assert_close(f"call{call} {name}", to_np(t), r, atol=2e-2 * float(np.abs(r).max()))
