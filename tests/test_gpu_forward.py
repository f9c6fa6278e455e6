"""GPU parity of the SLA forward (HIP library through the C ABI) with the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle as orc
from helpers import (assert_close, decoded, device_inputs, log, mask_validity, rel_l2, to_np)
from sparse_linear_attention_mean_amd.inputs import (WORKLOADS, make_inputs,
                                                      make_workload_inputs)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    global SlaProblem, classify, B
    from sparse_linear_attention_mean_amd import _binding as B  # noqa: F811
    from sparse_linear_attention_mean_amd.attention import SlaProblem, classify  # noqa: F811


def _gpu_forward(inp, fc, fn, mask=None, zero_w=False):
    b, h, n, d = inp["q"].shape
    mode = B.SLA_MASK_GIVEN if mask is not None else B.SLA_MASK_COMPUTE
    prob = SlaProblem.create(b, h, n, d, fc, fn, valid_len=inp["valid_len"], mask_mode=mode)
    dev = device_inputs(inp)
    w = torch.zeros_like(dev["w"]) if zero_w else dev["w"]
    m = prob.new_mask()
    if mask is not None:
        m.copy_(torch.from_numpy(mask))
    o, m = prob.forward(dev["q"], dev["k"], dev["v"], w, mask=m)
    torch.cuda.synchronize()
    lse, den, y = prob.saved_views()
    return dict(o=to_np(o), mask=m.cpu().numpy(), lse=lse.cpu().numpy(), den=den.cpu().numpy(),
                y=to_np(y))


def _score_tol(scores):
    return 1e-4 * float(np.abs(scores).max()) + 1e-6


def _compare(name, got, ref, rows, valid_len):
    """Compare forward outputs on the tokens of the query blocks in ``rows``
    ([B, H, T] bool), valid rows only; padded rows must be exactly zero."""
    n = got["o"].shape[2]
    tok = np.repeat(rows, 64, axis=-1)[..., :n]
    valid = np.arange(n) < valid_len
    sel = tok & valid
    assert_close(f"{name} O", got["o"][sel], ref["o"][sel])
    assert_close(f"{name} Y", got["y"][sel], ref["y"][sel])
    fin = np.isfinite(ref["lse"]) & sel
    assert np.array_equal(np.isfinite(got["lse"]) & sel, fin), "lse finiteness"
    if fin.any():
        assert np.abs(got["lse"][fin] - ref["lse"][fin]).max() < 1e-3
    dpos = sel & (ref["den"] > 0)
    if dpos.any():
        assert rel_l2(got["den"][dpos], ref["den"][dpos]) < 1e-2
    assert np.all(got["den"][sel & (ref["den"] == 0)] == 0)
    assert np.all(got["o"][:, :, ~valid] == 0)
    assert np.all(got["y"][:, :, ~valid] == 0)


CASES = [
    # name, B, H, N, d, grid, valid_len, f_c, f_n
    ("tiny_workload", 1, 2, 1024, 64, (8, 8, 16), 1024, 0.125, 0.25),
    ("ragged_d128", 2, 3, 640, 128, (2, 16, 20), 600, 0.3, 0.2),
    ("one_token_tail_d64", 1, 2, 320, 64, (5, 8, 8), 257, 0.4, 0.2),
    ("single_block", 1, 2, 64, 128, (4, 4, 4), 64, 0.0, 0.0),
    ("dense_d128", 1, 2, 512, 128, (2, 16, 16), 500, 1.0, 0.0),
    ("dense_d64", 2, 1, 384, 64, (6, 8, 8), 384, 1.0, 0.0),
    ("all_marginal", 1, 2, 512, 128, (2, 16, 16), 512, 0.0, 0.0),
    ("no_critical_negligible", 1, 2, 768, 64, (3, 16, 16), 760, 0.0, 0.3),
    ("no_marginal", 1, 2, 640, 128, (10, 8, 8), 640, 0.5, 0.5),
    ("odd_37_blocks", 1, 1, 64 * 37, 128, (37, 8, 8), 64 * 37 - 5, 0.1, 0.1),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_forward_matches_oracle(case):
    name, b, h, n, d, grid, vl, fc, fn = case
    log(f"case {name}: B={b} H={h} N={n} d={d} L={vl} fc={fc} fn={fn}")
    inp = make_inputs(b, h, n, d, grid, vl, seed=7, with_grad=False)
    x = decoded(inp)
    ref = orc.forward(x["q"], x["k"], x["v"], x["w"], fc, fn, valid_len=vl)
    got = _gpu_forward(inp, fc, fn)
    t = n // 64
    k_c, k_n, _ = orc.block_counts(t, fc, fn)
    same = mask_validity(got["mask"], ref["scores"], k_c, k_n, _score_tol(ref["scores"]))
    log(f"  mask rows equal to the oracle's: {same.mean():.4f}")
    _compare(name, got, ref, same, vl)
    # sparse branch alone (W = 0)
    got0 = _gpu_forward(inp, fc, fn, zero_w=True)
    tok = np.repeat(same, 64, axis=-1)[..., :n] & (np.arange(n) < vl)
    assert_close(f"{name} O_s", got0["o"][tok], ref["o_sparse"][tok])


def test_forward_video_8k_workload():
    wl = WORKLOADS["video_b1_h12_n8192_d128"]
    log(f"workload {wl.name}")
    inp = make_workload_inputs(wl.name, seed=0, with_grad=False)
    x = decoded(inp)
    ref = orc.forward(x["q"], x["k"], x["v"], x["w"], wl.frac_critical, wl.frac_negligible,
                      valid_len=wl.valid_len)
    got = _gpu_forward(inp, wl.frac_critical, wl.frac_negligible)
    k_c, k_n, _ = orc.block_counts(wl.num_blocks, wl.frac_critical, wl.frac_negligible)
    same = mask_validity(got["mask"], ref["scores"], k_c, k_n, _score_tol(ref["scores"]))
    log(f"  mask rows equal to the oracle's: {same.mean():.4f}")
    _compare(wl.name, got, ref, same, wl.valid_len)


@pytest.mark.parametrize("d", [64, 128])
def test_forward_given_mask(d):
    """Fixed (injected) masks that need not follow the top-k rule: rows without
    critical blocks, without marginal blocks, all negligible."""
    b, h, n, vl = 2, 2, 576, 570
    t = n // 64
    inp = make_inputs(b, h, n, d, (9, 8, 8), vl, seed=11, with_grad=False)
    rng = np.random.default_rng(5)
    mask = rng.choice(np.array([1, 0, -1], np.int8), size=(b, h, t, t), p=(0.25, 0.5, 0.25))
    mask[0, 0, 0] = 0
    mask[0, 0, 1] = 1
    mask[0, 1, 2] = -1
    mask[1, 0, 3] = [1, -1] * (t // 2) + [1] * (t % 2)
    x = decoded(inp)
    ref = orc.forward(x["q"], x["k"], x["v"], x["w"], 0.0, 0.0, valid_len=vl, mask=mask)
    got = _gpu_forward(inp, 0.0, 0.0, mask=mask)
    assert np.array_equal(got["mask"], mask), "a given mask must not be modified"
    _compare(f"given_d{d}", got, ref, np.ones((b, h, t), bool), vl)


@pytest.mark.parametrize("t,kind", [(37, "workload"), (37, "integers"), (64, "constant"),
                                    (50, "signed_zeros"), (1, "integers"), (2048, "workload"),
                                    (129, "integers"), (512, "integers"), (513, "signed_zeros")])
def test_classify_bit_exact(t, kind):
    """Identical fp32 score maps must give byte-identical masks."""
    rng = np.random.default_rng(t)
    b, h = 1, 3
    if kind == "workload":
        scores = (rng.standard_normal((b, h, t, t)) * 2).astype(np.float32)
    elif kind == "integers":
        scores = rng.integers(-3, 4, size=(b, h, t, t)).astype(np.float32)
    elif kind == "constant":
        scores = np.full((b, h, t, t), 1.5, np.float32)
    else:
        scores = np.where(rng.random((b, h, t, t)) < 0.5, np.float32(0.0), np.float32(-0.0))
        scores[..., ::5] = 2.0
    for fc, fn in [(0.1, 0.2), (0.0, 0.0), (1.0, 0.0), (0.0, 1.0), (0.5, 0.5), (0.3, 0.05)]:
        cfg = B.make_config(b, h, 64 * t, 64, fc, fn)
        k_c, k_n, _ = orc.block_counts(t, fc, fn)
        assert B.sla_block_counts(cfg)[:2] == (k_c, k_n)
        got = classify(cfg, torch.from_numpy(scores).cuda()).cpu().numpy()
        torch.cuda.synchronize()
        ref = orc.classify(scores, k_c, k_n)
        assert np.array_equal(got, ref), f"mask mismatch T={t} {kind} fc={fc} fn={fn}"


def test_classify_oracle_scores_bit_exact():
    """The oracle's own fp32 score map of a workload, classified on the GPU."""
    wl = WORKLOADS["video_b1_h12_n8192_d128"]
    inp = make_workload_inputs(wl.name, seed=1, with_grad=False)
    x = decoded(inp)
    scores = np.stack([orc.compressed_scores(x["q"][0, h], x["k"][0, h], wl.valid_len,
                                             orc.default_scale(wl.head_dim))
                       for h in range(wl.heads)])[None]
    k_c, k_n, _ = orc.block_counts(wl.num_blocks, wl.frac_critical, wl.frac_negligible)
    cfg = B.make_config(1, wl.heads, wl.seq_len, wl.head_dim, wl.frac_critical, wl.frac_negligible)
    got = classify(cfg, torch.from_numpy(scores).cuda()).cpu().numpy()
    assert np.array_equal(got, orc.classify(scores, k_c, k_n))


@pytest.mark.parametrize("case", [("ragged", 2, 3, 640, 128, (2, 16, 20), 600),
                                  ("d64", 1, 2, 1024, 64, (8, 8, 16), 1000)])
def test_pool_scores_match_oracle(case):
    name, b, h, n, d, grid, vl = case
    inp = make_inputs(b, h, n, d, grid, vl, seed=3, with_grad=False)
    x = decoded(inp)
    prob = SlaProblem.create(b, h, n, d, 0.1, 0.1, valid_len=vl)
    dev = device_inputs(inp)
    got = prob.pool_scores(dev["q"], dev["k"]).cpu().numpy()
    ref = np.stack([np.stack([orc.compressed_scores(x["q"][bb, hh], x["k"][bb, hh], vl,
                                                    orc.default_scale(d))
                              for hh in range(h)]) for bb in range(b)])
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64)).max()
    assert err <= _score_tol(ref), f"{name}: score error {err}"
    # the forward classifies exactly this map
    o, m = prob.forward(dev["q"], dev["k"], dev["v"], dev["w"])
    k_c, k_n, _ = orc.block_counts(n // 64, 0.1, 0.1)
    assert np.array_equal(m.cpu().numpy(), orc.classify(got, k_c, k_n))


def test_forward_is_deterministic():
    inp = make_inputs(1, 4, 2048, 128, (8, 16, 16), 2040, seed=9, with_grad=False)
    a = _gpu_forward(inp, 0.1, 0.2)
    b = _gpu_forward(inp, 0.1, 0.2)
    for k in ("o", "mask", "lse", "den", "y"):
        assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("name", ["video_dit_b2_h12_n32768_d128", "pixel_b1_h8_n65536_d64"])
def test_forward_full_size_sampled(name):
    """Full-size workloads in the benchmark's launch configuration: every mask
    row is checked against the oracle's classification; head (0, 0) is
    compared with the oracle on every query block whose mask row equals the
    oracle's (a whole head), the last head on sampled query blocks."""
    wl = WORKLOADS[name]
    log(f"workload {name}")
    inp = make_workload_inputs(name, seed=0, with_grad=False)
    got = _gpu_forward(inp, wl.frac_critical, wl.frac_negligible)
    t = wl.num_blocks
    k_c, k_n, _ = orc.block_counts(t, wl.frac_critical, wl.frac_negligible)
    scale = orc.default_scale(wl.head_dim)
    rng = np.random.default_rng(0)
    heads = [(0, 0), (wl.batch - 1, wl.heads - 1)]
    w = orc.decode_bf16(inp["w"])
    for b in range(wl.batch):
        for h in range(wl.heads):
            q = orc.decode_bf16(inp["q"][b, h])
            k = orc.decode_bf16(inp["k"][b, h])
            scores = orc.compressed_scores(q, k, wl.valid_len, scale)
            same = mask_validity(got["mask"][b, h], scores, k_c, k_n, _score_tol(scores))
            if (b, h) not in heads:
                continue
            log(f"  head ({b},{h}): mask rows equal {same.mean():.4f}")
            v = orc.decode_bf16(inp["v"][b, h])
            mask = orc.classify(scores, k_c, k_n)
            cand = np.flatnonzero(same)
            if (b, h) == (0, 0):
                blocks = [int(i) for i in cand]
                assert len(blocks) >= 0.95 * t
            else:
                blocks = set(rng.choice(cand, min(6, cand.size), replace=False).tolist())
                if same[t - 1]:
                    blocks.add(t - 1)
                blocks = sorted(blocks)
            ref = orc.forward_head(q, k, v, w, mask, wl.valid_len, scale, blocks=blocks)
            rows = np.zeros(wl.seq_len, bool)
            for i in blocks:
                rows[i * 64:min((i + 1) * 64, wl.valid_len)] = True
            log(f"  head ({b},{h}): {len(blocks)} query blocks compared")
            assert_close(f"  head ({b},{h}) O", got["o"][b, h, rows], ref["o"][rows])
            assert_close(f"  head ({b},{h}) Y", got["y"][b, h, rows], ref["y"][rows])
            assert np.abs(got["lse"][b, h, rows] - ref["lse"][rows]).max() < 1e-3
    assert np.all(got["o"][:, :, wl.valid_len:] == 0)
