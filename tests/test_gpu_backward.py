"""GPU parity of the SLA backward (HIP library through the C ABI) with the CPU oracle.

The GPU forward runs with the oracle's own mask supplied (fixed-mask mode), so
every gradient element can be compared; classification itself is covered by
the forward tests.  Tolerance per gradient tensor: rel-L2 <= 1e-2 and
max-abs <= 2e-2 * max|reference| (the output tolerance of the method, read
relative to the gradient's scale)."""
import numpy as np
import pytest
import torch

import oracle as orc
from helpers import assert_close, decoded, device_inputs, log, to_np
from sparse_linear_attention_mean_amd.inputs import WORKLOADS, make_inputs, make_workload_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    global SlaProblem, B
    from sparse_linear_attention_mean_amd import _binding as B  # noqa: F811
    from sparse_linear_attention_mean_amd.attention import SlaProblem  # noqa: F811


def _gpu_fwd_bwd(inp, fc, fn, mask, mode=None):
    b, h, n, d = inp["q"].shape
    if mode is None:
        mode = B.SLA_MASK_GIVEN
    prob = SlaProblem.create(b, h, n, d, fc, fn, valid_len=inp["valid_len"], mask_mode=mode)
    dev = device_inputs(inp)
    m = prob.new_mask()
    if mask is not None:
        m.copy_(torch.from_numpy(mask))
    o, m = prob.forward(dev["q"], dev["k"], dev["v"], dev["w"], mask=m)
    dq, dk, dv, dw = prob.backward(dev["q"], dev["k"], dev["v"], dev["w"], o, dev["do"], m)
    torch.cuda.synchronize()
    return dict(o=to_np(o), mask=m.cpu().numpy(), dq=to_np(dq), dk=to_np(dk), dv=to_np(dv),
                dw=to_np(dw))


def _check_grads(name, got, ref, heads=None):
    for g in ("dq", "dk", "dv"):
        a, r = got[g], ref[g]
        if heads is not None:
            a = np.stack([a[bb, hh] for bb, hh in heads])
            r = np.stack([r[bb, hh] for bb, hh in heads]) if r.ndim == a.ndim else r
        scale = float(np.abs(r).max()) or 1.0
        assert_close(f"{name} {g}", a, r, atol=2e-2 * scale)
    if heads is None:
        assert_close(f"{name} dw", got["dw"], ref["dw"], atol=2e-2 * float(np.abs(ref["dw"]).max()))


def _oracle_mask(x, fc, fn, vl):
    b, h, n, d = x["q"].shape
    t = n // 64
    k_c, k_n, _ = orc.block_counts(t, fc, fn)
    scale = orc.default_scale(d)
    return np.stack([np.stack([orc.classify(orc.compressed_scores(x["q"][bb, hh], x["k"][bb, hh],
                                                                  vl, scale), k_c, k_n)
                               for hh in range(h)]) for bb in range(b)])


CASES = [
    # name, B, H, N, d, grid, valid_len, f_c, f_n
    ("tiny_workload", 1, 2, 1024, 64, (8, 8, 16), 1024, 0.125, 0.25),
    ("ragged_d128", 2, 3, 640, 128, (2, 16, 20), 600, 0.3, 0.2),
    ("one_token_tail_d64", 1, 2, 320, 64, (5, 8, 8), 257, 0.4, 0.2),
    ("dense_d128", 1, 2, 512, 128, (2, 16, 16), 500, 1.0, 0.0),
    ("all_marginal_d64", 1, 2, 512, 64, (2, 16, 16), 512, 0.0, 0.0),
    ("no_critical_negligible", 1, 2, 768, 128, (3, 16, 16), 760, 0.0, 0.3),
    ("no_marginal", 1, 2, 640, 128, (10, 8, 8), 640, 0.5, 0.5),
    ("single_block", 1, 1, 64, 128, (4, 4, 4), 60, 0.0, 0.0),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_backward_matches_oracle(case):
    name, b, h, n, d, grid, vl, fc, fn = case
    log(f"case {name}: B={b} H={h} N={n} d={d} L={vl} fc={fc} fn={fn}")
    inp = make_inputs(b, h, n, d, grid, vl, seed=13)
    x = decoded(inp)
    mask = _oracle_mask(x, fc, fn, vl)
    ref = orc.backward(x["q"], x["k"], x["v"], x["w"], x["do"], mask, valid_len=vl)
    # compute mode (the library classifies) must pick the same mask here
    got = _gpu_fwd_bwd(inp, fc, fn, None, mode=B.SLA_MASK_COMPUTE)
    assert np.array_equal(got["mask"], mask)
    _check_grads(name, got, ref)
    for g in ("dq", "dk", "dv"):
        assert np.all(got[g][:, :, vl:] == 0)


@pytest.mark.parametrize("d", [64, 128])
def test_backward_given_mask(d):
    b, h, n, vl = 1, 3, 576, 570
    t = n // 64
    inp = make_inputs(b, h, n, d, (9, 8, 8), vl, seed=17)
    rng = np.random.default_rng(8)
    mask = rng.choice(np.array([1, 0, -1], np.int8), size=(b, h, t, t), p=(0.25, 0.5, 0.25))
    mask[0, 0, 0] = 0
    mask[0, 1, :, 2] = 1          # a column that is critical everywhere
    mask[0, 2, 3] = -1            # a row with nothing
    mask[0, 2, :, 4] = 0          # a column marginal everywhere
    x = decoded(inp)
    ref = orc.backward(x["q"], x["k"], x["v"], x["w"], x["do"], mask, valid_len=vl)
    got = _gpu_fwd_bwd(inp, 0.0, 0.0, mask)
    _check_grads(f"given_d{d}", got, ref)


@pytest.mark.parametrize("case", [(1, 9, 4160, 64, (26, 8, 20), 4150),
                                  (2, 8, 4160, 128, (26, 8, 20), 4100)],
                         ids=["585_blocks_d64", "1040_blocks_d128"])
def test_backward_multi_block_runs(case):
    """More query blocks than dW partials (512): the preparation kernel's
    workgroups run through one to three blocks each, runs that cross head
    (and batch) boundaries and end in the ragged tail; every gradient, dW in
    particular, against the oracle."""
    b, h, n, d, grid, vl = case
    log(f"multi-block runs: B={b} H={h} N={n} d={d} L={vl} ({b * h * (n // 64)} blocks)")
    inp = make_inputs(b, h, n, d, grid, vl, seed=31)
    x = decoded(inp)
    mask = _oracle_mask(x, 0.1, 0.2, vl)
    ref = orc.backward(x["q"], x["k"], x["v"], x["w"], x["do"], mask, valid_len=vl)
    got = _gpu_fwd_bwd(inp, 0.0, 0.0, mask)
    _check_grads(f"runs_d{d}", got, ref)


def test_dw_runs_of_24_query_blocks():
    """dW with 12,288 query blocks, so that each of the preparation kernel's
    512 runs holds 24 blocks, as in the benchmark's layout (B = 2, H = 12,
    T = 512); here B = 1, H = 24 at d = 64 keeps the oracle to seconds.  Runs
    cross head boundaries and the ragged tail of every head; every gradient,
    dW in particular, against the oracle."""
    b, h, n, d, vl = 1, 24, 32768, 64, 32760
    log(f"dW runs of 24 blocks: B={b} H={h} N={n} d={d} L={vl} ({b * h * (n // 64)} blocks)")
    inp = make_inputs(b, h, n, d, (21, 30, 52), vl, seed=37)
    x = decoded(inp)
    mask = _oracle_mask(x, 0.02, 0.9, vl)
    got = _gpu_fwd_bwd(inp, 0.0, 0.0, mask)
    ref = orc.backward(x["q"], x["k"], x["v"], x["w"], x["do"], mask, valid_len=vl)
    _check_grads("runs24_d64", got, ref)


def test_backward_is_deterministic():
    inp = make_inputs(1, 2, 1024, 128, (4, 16, 16), 1000, seed=21)
    x = decoded(inp)
    mask = _oracle_mask(x, 0.1, 0.2, 1000)
    a = _gpu_fwd_bwd(inp, 0.1, 0.2, mask)
    b = _gpu_fwd_bwd(inp, 0.1, 0.2, mask)
    for g in ("dq", "dk", "dv", "dw"):
        assert np.array_equal(a[g], b[g]), g


@pytest.mark.parametrize("name", ["video_bwd_b1_h12_n16384_d128", "video_dit_b2_h12_n32768_d128"])
def test_backward_full_size_sampled(name):
    """Full-size workloads in the benchmark's launch configuration (the library
    classifies): two heads are recomputed by the oracle and compared in full."""
    wl = WORKLOADS[name]
    log(f"workload {name}")
    inp = make_workload_inputs(name, seed=0)
    got = _gpu_fwd_bwd(inp, wl.frac_critical, wl.frac_negligible, None, mode=B.SLA_MASK_COMPUTE)
    t = wl.num_blocks
    k_c, k_n, _ = orc.block_counts(t, wl.frac_critical, wl.frac_negligible)
    scale = orc.default_scale(wl.head_dim)
    w = orc.decode_bf16(inp["w"])
    for bb, hh in [(0, 0), (wl.batch - 1, wl.heads - 1)]:
        q, k, v, do = (orc.decode_bf16(inp[n][bb, hh]) for n in ("q", "k", "v", "do"))
        mask = orc.classify(orc.compressed_scores(q, k, wl.valid_len, scale), k_c, k_n)
        assert np.array_equal(got["mask"][bb, hh], mask)
        r = orc.backward_head(q, k, v, w, do, mask, wl.valid_len, scale)
        for g in ("dq", "dk", "dv"):
            ref = r[g]
            assert_close(f"  head ({bb},{hh}) {g}", got[g][bb, hh], ref,
                         atol=2e-2 * float(np.abs(ref).max()))
    assert np.all(np.isfinite(got["dw"]))
