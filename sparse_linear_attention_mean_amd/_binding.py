"""ctypes binding of ``libsla.so`` (C ABI in include/sla.h).

Argument marshalling only: every step of the computation runs in the HIP
library.  The functions take torch tensors (for device memory and the stream)
and call the C entry points of the same name.  If the library is missing the
import of this module fails loudly; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsla.so")

SLA_OK = 0
SLA_ERR_INVALID_ARGUMENT = 1
SLA_ERR_UNSUPPORTED = 2
SLA_ERR_WORKSPACE = 3
SLA_ERR_DEVICE = 4
SLA_MASK_COMPUTE = 0
SLA_MASK_GIVEN = 1
SLA_LINEAR_MARGINAL = 0
SLA_LINEAR_GLOBAL = 1
SLA_NUM_STAGES = 8
STAGES = ("kv_state", "pool_q", "classify", "aggregate", "attention", "bwd_pre", "bwd_kv", "bwd_q")

EXPORTED = (
    "sla_block_counts", "sla_workspace_size", "sla_saved_size", "sla_saved_offsets",
    "sla_forward", "sla_backward", "sla_pool_scores", "sla_classify", "sla_coarse_scores",
    "sla_classify_hier", "sla_status_string", "sla_last_error", "sla_forward_static",
)
SLA_STATIC_SCRATCH_BYTES = 64 << 20


class SlaConfig(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("seq_len", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("valid_len", ctypes.c_int32),
        ("block", ctypes.c_int32),
        ("frac_critical", ctypes.c_float),
        ("frac_negligible", ctypes.c_float),
        ("softmax_scale", ctypes.c_float),
        ("mask_mode", ctypes.c_int32),
        ("stage_events", ctypes.c_void_p),
        ("linear_mode", ctypes.c_int32),
        ("linear_gate", ctypes.c_float),
        ("select_group", ctypes.c_int32),
        ("select_keep", ctypes.c_int32),
    ]


class SlaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"SLA status {status}: {detail}")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run python -m sparse_linear_attention_mean_amd.builder")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, cfgp = ctypes.c_void_p, ctypes.c_size_t, ctypes.POINTER(SlaConfig)
    i32p = ctypes.POINTER(ctypes.c_int32)
    szp = ctypes.POINTER(ctypes.c_size_t)
    sig = {
        "sla_block_counts": (ctypes.c_int, [cfgp, i32p, i32p, i32p]),
        "sla_workspace_size": (sz, [cfgp]),
        "sla_saved_size": (sz, [cfgp]),
        "sla_saved_offsets": (ctypes.c_int, [cfgp, szp, szp, szp, szp, szp]),
        "sla_forward": (ctypes.c_int, [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "sla_forward_static": (ctypes.c_int, [cfgp, vp, vp, vp, vp, vp, vp, vp, vp]),
        "sla_backward": (ctypes.c_int, [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                        sz, vp]),
        "sla_pool_scores": (ctypes.c_int, [cfgp, vp, vp, vp, vp, sz, vp]),
        "sla_classify": (ctypes.c_int, [cfgp, vp, vp, vp]),
        "sla_coarse_scores": (ctypes.c_int, [cfgp, vp, vp, vp, vp, sz, vp]),
        "sla_classify_hier": (ctypes.c_int, [cfgp, vp, vp, vp, vp]),
        "sla_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "sla_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def make_config(batch, heads, seq_len, head_dim, frac_critical, frac_negligible, valid_len=0,
                softmax_scale=0.0, mask_mode=SLA_MASK_COMPUTE, stage_events=None,
                linear_mode=SLA_LINEAR_MARGINAL, linear_gate=1.0, select_group=0,
                select_keep=0) -> SlaConfig:
    return SlaConfig(batch, heads, seq_len, head_dim, valid_len, 64, frac_critical,
                     frac_negligible, softmax_scale, mask_mode, stage_events, linear_mode,
                     linear_gate, select_group, select_keep)


def _check(status: int) -> None:
    if status != SLA_OK:
        raise SlaError(status, lib.sla_last_error().decode())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def sla_block_counts(cfg: SlaConfig):
    kc, kn, km = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(lib.sla_block_counts(ctypes.byref(cfg), ctypes.byref(kc), ctypes.byref(kn),
                                ctypes.byref(km)))
    return kc.value, kn.value, km.value


def sla_workspace_size(cfg: SlaConfig) -> int:
    return lib.sla_workspace_size(ctypes.byref(cfg))


def sla_saved_size(cfg: SlaConfig) -> int:
    return lib.sla_saved_size(ctypes.byref(cfg))


def sla_saved_offsets(cfg: SlaConfig) -> dict:
    vals = [ctypes.c_size_t() for _ in range(5)]
    _check(lib.sla_saved_offsets(ctypes.byref(cfg), *[ctypes.byref(v) for v in vals]))
    return dict(zip(("lse", "den", "y", "hst", "zst"), (v.value for v in vals)))


def sla_forward(cfg, q, k, v, w, o, mask, saved, workspace, stream=None) -> None:
    _check(lib.sla_forward(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(w), _ptr(o),
                           _ptr(mask), _ptr(saved), _ptr(workspace),
                           workspace.numel() * workspace.element_size(), _stream(stream)))


def sla_forward_static(cfg, q, k, v, w, o, mask, saved, stream=None) -> None:
    _check(lib.sla_forward_static(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(w), _ptr(o),
                                  _ptr(mask), _ptr(saved), _stream(stream)))


def sla_backward(cfg, q, k, v, w, o, d_o, mask, saved, dq, dk, dv, dw, workspace,
                 stream=None) -> None:
    _check(lib.sla_backward(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(v), _ptr(w), _ptr(o),
                            _ptr(d_o), _ptr(mask), _ptr(saved), _ptr(dq), _ptr(dk), _ptr(dv),
                            _ptr(dw), _ptr(workspace),
                            workspace.numel() * workspace.element_size(), _stream(stream)))


def sla_pool_scores(cfg, q, k, scores, workspace, stream=None) -> None:
    _check(lib.sla_pool_scores(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(scores), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _stream(stream)))


def sla_classify(cfg, scores, mask, stream=None) -> None:
    _check(lib.sla_classify(ctypes.byref(cfg), _ptr(scores), _ptr(mask), _stream(stream)))


def sla_coarse_scores(cfg, q, k, coarse, workspace, stream=None) -> None:
    _check(lib.sla_coarse_scores(ctypes.byref(cfg), _ptr(q), _ptr(k), _ptr(coarse),
                                 _ptr(workspace), workspace.numel() * workspace.element_size(),
                                 _stream(stream)))


def sla_classify_hier(cfg, coarse, scores, mask, stream=None) -> None:
    _check(lib.sla_classify_hier(ctypes.byref(cfg), _ptr(coarse), _ptr(scores), _ptr(mask),
                                 _stream(stream)))


def sla_status_string(status: int) -> str:
    return lib.sla_status_string(status).decode()


def sla_last_error() -> str:
    return lib.sla_last_error().decode()
