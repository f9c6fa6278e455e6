"""GPU parity of the two-level (hierarchical) key-block selection.

Protocol, as for the flat classifier: identical fp32 maps must give
byte-identical masks, checked with ``sla_classify_hier`` on synthetic maps
(ties, signed zeros, a short last group, kept and negligible groups that
overlap).  The forward's mask is checked against the oracle's own coarse and
fine maps: rows equal to the oracle's split are compared element-wise, the
others (near-ties, rounded differently by the two independently computed
maps) must be a valid two-level split within the rounding gap.  Gradients are
compared with the GPU run in fixed-mask mode on the oracle's mask.
"""
import numpy as np
import pytest
import torch

import oracle as orc
from helpers import assert_close, decoded, device_inputs, log, to_np
from sparse_linear_attention_mean_amd.inputs import (WORKLOADS, make_inputs,
                                                      make_workload_inputs)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    global SlaProblem, classify, classify_hier, B
    from sparse_linear_attention_mean_amd import _binding as B  # noqa: F811
    from sparse_linear_attention_mean_amd.attention import (  # noqa: F811
        SlaProblem, classify, classify_hier)


def _maps(kind, b, h, t, tg, seed):
    rng = np.random.default_rng(seed)
    if kind == "random":
        s = rng.standard_normal((b, h, t, t))
        c = rng.standard_normal((b, h, t, tg))
    elif kind == "integers":
        s = rng.integers(-2, 3, size=(b, h, t, t))
        c = rng.integers(-2, 3, size=(b, h, t, tg))
    else:
        s = np.where(rng.random((b, h, t, t)) < 0.5, 0.0, -0.0)
        c = np.where(rng.random((b, h, t, tg)) < 0.5, 0.0, -0.0)
        s[..., ::5] = 1.0
    return c.astype(np.float32), s.astype(np.float32)


HIER_CASES = [
    # T, G, keep, f_c, f_n
    (37, 4, 3, 0.2, 0.3),      # short last group
    (64, 8, 2, 0.2, 0.5),      # 2 kept and 4 negligible of 8 groups
    (40, 8, 4, 0.25, 0.45),    # 4 kept + 2 negligible of 5 groups: overlap
    (33, 1, 33, 0.2, 0.3),     # unit groups, all kept: the flat split
    (129, 16, 5, 0.1, 0.2),
    (1024, 8, 8, 0.02, 0.2),   # the long-sequence workload's split
    (600, 4, 40, 0.05, 0.1),   # 160 candidate blocks (several 64-wide chunks)
    (1500, 16, 20, 0.02, 0.1), # more than 1024 blocks, short last group
    (2048, 2, 1024, 0.05, 0.05),  # every group kept: all 2048 blocks are candidates
]


@pytest.mark.parametrize("kind", ["random", "integers", "signed_zeros"])
@pytest.mark.parametrize("case", HIER_CASES, ids=[f"T{c[0]}_G{c[1]}_keep{c[2]}" for c in HIER_CASES])
def test_classify_hier_bit_exact(kind, case):
    t, g, keep, fc, fn = case
    b, h = 1, 2
    tg = orc.num_groups(t, g)
    coarse, scores = _maps(kind, b, h, t, tg, seed=t + g)
    k_c, k_n, _ = orc.block_counts(t, fc, fn)
    _, n_g = orc.hier_counts(t, g, keep, k_c, k_n)
    cfg = B.make_config(b, h, 64 * t, 64, fc, fn, select_group=g, select_keep=keep)
    got = classify_hier(cfg, torch.from_numpy(coarse).cuda(), torch.from_numpy(scores).cuda())
    got = got.cpu().numpy()
    ref = orc.classify_hier(coarse, scores, k_c, n_g, keep, g)
    assert np.array_equal(got, ref), f"mask mismatch {case} {kind}"
    if g == 1 and keep == t:
        # unit groups have coarse map = fine map: then the split is the flat one
        sc = torch.from_numpy(scores).cuda()
        same = classify_hier(cfg, sc, sc).cpu().numpy()
        flat = classify(B.make_config(b, h, 64 * t, 64, fc, fn), sc).cpu().numpy()
        assert np.array_equal(same, flat)


def test_coarse_scores_match_oracle():
    b, h, n, d, vl, g = 2, 3, 64 * 21, 128, 64 * 21 - 30, 4
    inp = make_inputs(b, h, n, d, (3, 16, 28), vl, seed=4, with_grad=False)
    x = decoded(inp)
    prob = SlaProblem.create(b, h, n, d, 0.1, 0.1, valid_len=vl, select_group=g, select_keep=2)
    dev = device_inputs(inp)
    got = prob.coarse_scores(dev["q"], dev["k"]).cpu().numpy()
    ref = np.stack([np.stack([orc.coarse_scores(x["q"][bb, hh], x["k"][bb, hh], vl,
                                                orc.default_scale(d), g)
                              for hh in range(h)]) for bb in range(b)])
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64)).max()
    assert err <= 1e-4 * float(np.abs(ref).max()) + 1e-6, f"coarse score error {err}"


def _hier_forward(inp, fc, fn, g, keep):
    b, h, n, d = inp["q"].shape
    prob = SlaProblem.create(b, h, n, d, fc, fn, valid_len=inp["valid_len"], select_group=g,
                             select_keep=keep)
    dev = device_inputs(inp)
    o, m = prob.forward(dev["q"], dev["k"], dev["v"], dev["w"])
    # the library's own maps, classified by sla_classify_hier: the forward's
    # internal candidate scores must reproduce them (GPU against GPU)
    coarse = prob.coarse_scores(dev["q"], dev["k"])
    scores = prob.pool_scores(dev["q"], dev["k"])
    again = classify_hier(prob.cfg, coarse, scores)
    torch.cuda.synchronize()
    assert torch.equal(again, m), "forward mask differs from sla_classify_hier on the same maps"
    lse, den, y = prob.saved_views()
    return prob, dev, dict(o=to_np(o), mask=m.cpu().numpy(), lse=lse.cpu().numpy(), y=to_np(y))


def _oracle_maps(x, vl, g, b, h):
    scale = orc.default_scale(x["q"].shape[-1])
    coarse = np.stack([np.stack([orc.coarse_scores(x["q"][bb, hh], x["k"][bb, hh], vl, scale, g)
                                 for hh in range(h)]) for bb in range(b)])
    scores = np.stack([np.stack([orc.compressed_scores(x["q"][bb, hh], x["k"][bb, hh], vl, scale)
                                 for hh in range(h)]) for bb in range(b)])
    return coarse, scores


def _hier_validity(gpu, coarse, scores, k_c, n_g, keep, g):
    """Rows of the GPU mask that differ from the oracle's own split must still
    be a two-level split of the oracle's maps up to the rounding gap between
    independently computed maps.  Returns the [..., T] rows that are equal."""
    ref = orc.classify_hier(coarse, scores, k_c, n_g, keep, g)
    same = (gpu == ref).all(axis=-1)
    t, tg = scores.shape[-1], coarse.shape[-1]
    tol_c = 1e-4 * float(np.abs(coarse).max()) + 1e-6
    tol_s = 1e-4 * float(np.abs(scores).max()) + 1e-6
    gf = gpu.reshape(-1, t)
    cf = coarse.reshape(-1, tg).astype(np.float64)
    sf = scores.reshape(-1, t).astype(np.float64)
    for r in np.flatnonzero(~same.reshape(-1)):
        row, c, s = gf[r], cf[r], sf[r]
        assert (row == 1).sum() == k_c, "critical count"
        grp = np.arange(t) // g
        kth = np.sort(c)[::-1][keep - 1]          # the keep-th largest coarse score
        crit_groups = np.unique(grp[row == 1])
        assert np.all(c[crit_groups] >= kth - tol_c), "critical block outside the kept groups"
        sure = c > kth + tol_c                    # groups kept whatever the rounding
        cand = sure[grp] & (row != 1)
        if cand.any() and k_c:
            assert s[row == 1].min() >= s[cand].max() - tol_s, "critical order beyond rounding"
        negl = np.unique(grp[row == -1])
        if n_g:
            nth = np.sort(c)[n_g - 1]             # the n_g-th smallest coarse score
            assert np.all(c[negl] <= nth + tol_c), "negligible group beyond rounding"
    return same


FWD_CASES = [
    # name, B, H, N, d, grid, valid_len, f_c, f_n, G, keep
    ("d64_short_group", 1, 2, 64 * 21, 64, (3, 16, 28), 64 * 21 - 9, 0.15, 0.3, 4, 3),
    ("d128_overlap", 2, 2, 64 * 16, 128, (4, 16, 16), 64 * 16, 0.2, 0.5, 4, 3),
    ("unit_groups", 1, 2, 64 * 12, 64, (3, 16, 16), 64 * 12 - 1, 0.25, 0.25, 1, 12),
]


@pytest.mark.parametrize("case", FWD_CASES, ids=[c[0] for c in FWD_CASES])
def test_forward_two_level_matches_oracle(case):
    name, b, h, n, d, grid, vl, fc, fn, g, keep = case
    inp = make_inputs(b, h, n, d, grid, vl, seed=12, with_grad=True)
    prob, dev, got = _hier_forward(inp, fc, fn, g, keep)
    t = n // 64
    k_c, k_n, _ = orc.block_counts(t, fc, fn)
    _, n_g = orc.hier_counts(t, g, keep, k_c, k_n)
    x = decoded(inp)
    coarse, scores = _oracle_maps(x, vl, g, b, h)
    same = _hier_validity(got["mask"], coarse, scores, k_c, n_g, keep, g)
    assert same.mean() >= 0.9, f"{name}: only {same.mean():.3f} of the rows equal the oracle's"
    # outputs on the query blocks whose mask rows equal the oracle's own split
    ref_mask = orc.classify_hier(coarse, scores, k_c, n_g, keep, g)
    ref = orc.forward(x["q"], x["k"], x["v"], x["w"], 0.0, 0.0, valid_len=vl, mask=ref_mask)
    sel = np.repeat(same, 64, axis=-1) & (np.arange(n) < vl)
    assert_close(f"{name} O", got["o"][sel], ref["o"][sel])
    assert_close(f"{name} Y", got["y"][sel], ref["y"][sel])
    # the backward, run with the oracle's mask held fixed
    m = torch.from_numpy(ref_mask).cuda()
    gp = SlaProblem.create(b, h, n, d, fc, fn, valid_len=vl, mask_mode=B.SLA_MASK_GIVEN)
    o, m = gp.forward(dev["q"], dev["k"], dev["v"], dev["w"], mask=m)
    dq, dk, dv, dw = gp.backward(dev["q"], dev["k"], dev["v"], dev["w"], o, dev["do"], m)
    torch.cuda.synchronize()
    gref = orc.backward(x["q"], x["k"], x["v"], x["w"], x["do"], ref_mask, valid_len=vl)
    for nm, tt in (("dq", dq), ("dk", dk), ("dv", dv), ("dw", dw)):
        r = gref[nm]
        assert_close(f"{name} {nm}", to_np(tt), r, atol=2e-2 * float(np.abs(r).max()))


def test_two_level_rejects_bad_parameters():
    with pytest.raises(B.SlaError):
        SlaProblem.create(1, 1, 64 * 40, 64, 0.5, 0.0, select_group=8, select_keep=2)  # 16 < 20
    with pytest.raises(B.SlaError):
        SlaProblem.create(1, 1, 64 * 40, 64, 0.1, 0.0, select_group=8, select_keep=6)  # > 5 groups


def test_two_level_full_size_long_sequence():
    """The long-sequence workload (N = 65536, d = 64, 2% critical, 20%
    negligible) with groups of 8 blocks and 8 kept groups, in the benchmark's
    launch configuration: every mask row against the oracle's own maps;
    outputs on sampled query blocks whose rows equal the oracle's split."""
    name, g, keep = "pixel_b1_h8_n65536_d64", 8, 8
    wl = WORKLOADS[name]
    log(f"workload {name}, G={g}, keep={keep}")
    inp = make_workload_inputs(name, seed=0, with_grad=False)
    _, _, got = _hier_forward(inp, wl.frac_critical, wl.frac_negligible, g, keep)
    t = wl.num_blocks
    k_c, k_n, _ = orc.block_counts(t, wl.frac_critical, wl.frac_negligible)
    _, n_g = orc.hier_counts(t, g, keep, k_c, k_n)
    scale = orc.default_scale(wl.head_dim)
    w = orc.decode_bf16(inp["w"])
    rng = np.random.default_rng(1)
    for hh in range(wl.heads):
        q, k = (orc.decode_bf16(inp[x][0, hh]) for x in ("q", "k"))
        coarse = orc.coarse_scores(q, k, wl.valid_len, scale, g)
        scores = orc.compressed_scores(q, k, wl.valid_len, scale)
        same = _hier_validity(got["mask"][0, hh], coarse, scores, k_c, n_g, keep, g)
        log(f"  head {hh}: mask rows equal {same.mean():.4f}")
        assert same.mean() >= 0.9
        if hh not in (0, wl.heads - 1):
            continue
        v = orc.decode_bf16(inp["v"][0, hh])
        ref_mask = orc.classify_hier(coarse, scores, k_c, n_g, keep, g)
        cand = np.flatnonzero(same)
        blocks = set(rng.choice(cand, min(5, cand.size), replace=False).tolist())
        if same[t - 1]:
            blocks.add(t - 1)
        blocks = sorted(blocks)
        ref = orc.forward_head(q, k, v, w, ref_mask, wl.valid_len, scale, blocks=blocks)
        for i in blocks:
            lo, hi = i * 64, min((i + 1) * 64, wl.valid_len)
            assert_close(f"  head {hh} blk {i} O", got["o"][0, hh, lo:hi], ref["o"][lo:hi])
