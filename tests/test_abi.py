"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point that include/sla.h declares, computes block counts like
the oracle, and rejects bad arguments before touching the device."""
import ctypes
import os
import re

import pytest

import oracle as orc
from helpers import ensure_library

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def B():
    ensure_library()
    from sparse_linear_attention_mean_amd import _binding

    return _binding


def test_exports_every_declared_symbol(B):
    header = open(os.path.join(ROOT, "include", "sla.h")).read()
    declared = set(re.findall(r"\b(sla_[a-z_]+)\s*\(", header))
    assert declared, "no declarations found"
    assert declared == set(B.EXPORTED)
    for name in declared:
        assert hasattr(B.lib, name), name


@pytest.mark.parametrize("t", [1, 2, 16, 37, 128, 256, 512, 1024, 2048])
def test_block_counts_match_oracle(B, t):
    for fc, fn in [(0.125, 0.25), (0.05, 0.10), (0.02, 0.20), (0.0, 0.0), (1.0, 0.0),
                   (0.0, 1.0), (0.5, 0.5), (0.3333, 0.3333), (0.07, 0.9)]:
        cfg = B.make_config(1, 1, 64 * t, 128, fc, fn)
        try:
            want = orc.block_counts(t, fc, fn)
        except ValueError:
            with pytest.raises(B.SlaError):
                B.sla_block_counts(cfg)
            continue
        assert B.sla_block_counts(cfg) == want


def _status(B, cfg):
    kc = ctypes.c_int32()
    return B.lib.sla_block_counts(ctypes.byref(cfg), ctypes.byref(kc), None, None)


@pytest.mark.parametrize("field,value,status", [
    ("batch", 0, 1), ("heads", -1, 1), ("seq_len", 100, 1), ("seq_len", 0, 1),
    ("head_dim", 96, 2), ("block", 128, 2), ("valid_len", 64 * 4 - 64, 1),
    ("valid_len", 64 * 4 + 1, 1), ("frac_critical", 1.5, 1), ("frac_negligible", -0.1, 1),
    ("frac_critical", float("nan"), 1), ("mask_mode", 7, 1), ("softmax_scale", float("inf"), 1),
    ("seq_len", 64 * 4096, 2),
])
def test_invalid_configs_rejected(B, field, value, status):
    cfg = B.make_config(1, 2, 64 * 4, 64, 0.25, 0.25)
    assert _status(B, cfg) == 0
    setattr(cfg, field, value)
    assert _status(B, cfg) == status
    assert B.sla_last_error() != ""
    assert B.sla_workspace_size(cfg) == 0 and B.sla_saved_size(cfg) == 0


def test_forward_rejects_bad_pointers_before_any_launch(B):
    cfg = B.make_config(1, 2, 256, 64, 0.25, 0.25)
    ws = B.sla_workspace_size(cfg)
    buf = ctypes.create_string_buffer(64)
    good = (ctypes.addressof(buf) + 15) & ~15
    args = [good] * 8
    # a NULL input
    st = B.lib.sla_forward(ctypes.byref(cfg), None, *args[1:], ws, None)
    assert st == B.SLA_ERR_INVALID_ARGUMENT and "q" in B.sla_last_error()
    # a misaligned pointer
    bad = list(args)
    bad[2] = good + 2
    st = B.lib.sla_forward(ctypes.byref(cfg), *bad, ws, None)
    assert st == B.SLA_ERR_INVALID_ARGUMENT and "aligned" in B.sla_last_error()
    # a short workspace
    st = B.lib.sla_forward(ctypes.byref(cfg), *args, ws - 1, None)
    assert st == B.SLA_ERR_WORKSPACE
    st = B.lib.sla_backward(ctypes.byref(cfg), *([good] * 13), ws - 1, None)
    assert st == B.SLA_ERR_WORKSPACE
    st = B.lib.sla_pool_scores(ctypes.byref(cfg), good, good, None, good, ws, None)
    assert st == B.SLA_ERR_INVALID_ARGUMENT
    st = B.lib.sla_classify(None, good, good, None)
    assert st == B.SLA_ERR_INVALID_ARGUMENT


def test_static_forward_rejects_on_the_host(B):
    """The allocation-free forward validates like sla_forward and refuses a
    problem whose one (batch, head) share of scratch exceeds its static array,
    all before any device call."""
    buf = ctypes.create_string_buffer(64)
    good = (ctypes.addressof(buf) + 15) & ~15
    cfg = B.make_config(1, 2, 256, 64, 0.25, 0.25)
    st = B.lib.sla_forward_static(ctypes.byref(cfg), good, None, *([good] * 6), None)
    assert st == B.SLA_ERR_INVALID_ARGUMENT and "k" in B.sla_last_error()
    st = B.lib.sla_forward_static(ctypes.byref(cfg), *([good] * 6), good + 4, good, None)
    assert st == B.SLA_ERR_INVALID_ARGUMENT and "aligned" in B.sla_last_error()
    bad = B.make_config(0, 2, 256, 64, 0.25, 0.25)
    assert B.lib.sla_forward_static(ctypes.byref(bad), *([good] * 7), None) == \
        B.SLA_ERR_INVALID_ARGUMENT
    # T = 1441 blocks at d = 128: one head needs more than the 64 MiB array
    big = B.make_config(1, 1, 64 * 1441, 128, 0.05, 0.1)
    st = B.lib.sla_forward_static(ctypes.byref(big), *([good] * 7), None)
    assert st == B.SLA_ERR_WORKSPACE and "static scratch" in B.sla_last_error()
    assert B.SLA_STATIC_SCRATCH_BYTES == 64 << 20
    header = open(os.path.join(ROOT, "include", "sla.h")).read()
    assert "#define SLA_STATIC_SCRATCH_BYTES (64ull << 20)" in header


def test_status_strings_and_sizes(B):
    for s in range(5):
        assert B.sla_status_string(s)
    cfg = B.make_config(2, 12, 32768, 128, 0.05, 0.10, 32760)
    assert B.sla_block_counts(cfg) == (26, 51, 435)
    off = B.sla_saved_offsets(cfg)
    n = 2 * 12 * 32768
    assert off["lse"] == 0 and off["den"] >= 4 * n and off["y"] >= off["den"] + 4 * n
    assert all(v % 256 == 0 for v in off.values())
    assert B.sla_saved_size(cfg) >= off["zst"] + 2 * 12 * 512 * 2 * 128 * 4
    assert B.sla_workspace_size(cfg) > 0


def test_linear_mode_and_gate_are_validated_on_the_host():
    from sparse_linear_attention_mean_amd import _binding as B

    ok = B.make_config(1, 2, 1024, 64, 0.1, 0.2, linear_mode=B.SLA_LINEAR_GLOBAL, linear_gate=0.5)
    assert B.sla_block_counts(ok) == (2, 3, 11)
    for mode, gate in ((2, 0.5), (B.SLA_LINEAR_GLOBAL, 1.5), (B.SLA_LINEAR_GLOBAL, -0.1),
                       (B.SLA_LINEAR_GLOBAL, float("nan"))):
        bad = B.make_config(1, 2, 1024, 64, 0.1, 0.2, linear_mode=mode, linear_gate=gate)
        with pytest.raises(B.SlaError):
            B.sla_block_counts(bad)
    # the gate is ignored by the method's own (marginal) linear branch
    plain = B.make_config(1, 2, 1024, 64, 0.1, 0.2, linear_gate=7.0)
    assert B.sla_block_counts(plain) == (2, 3, 11)


def test_two_level_selection_is_validated_on_the_host():
    from sparse_linear_attention_mean_amd import _binding as B
    import oracle as orc

    # T = 40 blocks: groups of 8 -> 5 groups of 8; groups of 6 -> 7 groups, the last of 4
    for g, keep, fc, fn in ((8, 2, 0.25, 0.3), (6, 3, 0.35, 0.5), (1, 40, 0.1, 0.1), (40, 1, 0.9, 0.1)):
        cfg = B.make_config(1, 2, 64 * 40, 64, fc, fn, select_group=g, select_keep=keep)
        k_c, k_n, _ = B.sla_block_counts(cfg)
        orc.hier_counts(40, g, keep, k_c, k_n)   # the oracle accepts it too
        assert B.sla_workspace_size(cfg) > 0
    bad = [
        (8, 0, 0.1, 0.1),     # nothing kept
        (8, 6, 0.1, 0.1),     # more kept than groups
        (8, 2, 0.45, 0.1),    # 18 critical > 16 candidates
        (6, 2, 0.26, 0.1),    # 11 critical > 6 + 4 (the short last group kept)
        (41, 1, 0.1, 0.1),    # group larger than the row
        (-1, 1, 0.1, 0.1),
    ]
    for g, keep, fc, fn in bad:
        cfg = B.make_config(1, 2, 64 * 40, 64, fc, fn, select_group=g, select_keep=keep)
        with pytest.raises(B.SlaError):
            B.sla_block_counts(cfg)
        assert B.sla_workspace_size(cfg) == 0
        if g >= 1:
            k_c, k_n, _ = orc.block_counts(40, fc, fn)
            with pytest.raises(ValueError):
                orc.hier_counts(40, g, keep, k_c, k_n)
