"""Differentiable SLA attention for fine-tuning, over ``sla_forward`` / ``sla_backward``.

"SLA: Beyond Sparsity in Diffusion Transformers via Fine-Tunable Sparse-Linear
Attention" (English abstract): the method is meant to be fine-tuned in place of
full attention, so it needs a forward and a backward that autograd can chain.
The projection weight of the linear branch (O = O_s + Y W^T) is the only
parameter; the block mask is piecewise constant in Q and K and gets no
gradient (the backward runs with the mask held fixed).  ``global_linear=True``
selects the SALAD-style variant: a linear branch over every key block and
O = O_s + gate Y W^T.

Mask reuse across calls (denoising steps): with ``reuse_mask=True`` the module
keeps the mask of its first call and passes it back to the library in the
``SLA_MASK_GIVEN`` mode, which skips block pooling, the score map and the
classifier.  The page on Meta-Cached Sparse Attention (MC-Sparse; its key
facts and "how to apply" sections) describes caching sparse-attention metadata
between denoising steps; ``reset_mask()`` forgets the cache.

Every computation runs in ``libsla.so``; this file only allocates buffers,
checks arguments and wires the two entry points into ``torch.autograd``.
"""
from __future__ import annotations

import math

import torch

from . import _binding as B


def _check_operand(name, t, shape, dtype):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU (got {t.device})")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


class _Buffers:
    """Workspace cache per (config, device): scratch only, shared by calls on
    one stream; the saved state of each forward gets its own buffer."""

    def __init__(self):
        self._ws = {}

    def workspace(self, cfg, device):
        key = (cfg.batch, cfg.heads, cfg.seq_len, cfg.head_dim, cfg.valid_len,
                cfg.frac_critical, cfg.frac_negligible, cfg.mask_mode, cfg.select_group,
                cfg.select_keep, str(device))
        ws = self._ws.get(key)
        if ws is None:
            ws = torch.empty(B.sla_workspace_size(cfg), dtype=torch.uint8, device=device)
            self._ws[key] = ws
        return ws


_BUFFERS = _Buffers()


class SlaFunction(torch.autograd.Function):
    """o, mask = SlaFunction.apply(q, k, v, w, cfg, mask_in)

    q, k, v: bf16 [B, H, N, d] contiguous on the GPU; w: bf16 [d, d].
    cfg: a ``SlaConfig``; with ``SLA_MASK_GIVEN`` ``mask_in`` (int8 [B, H, T, T])
    is used as the block mask, else it is ignored and the mask is computed.
    Returns O (bf16) and the mask (int8, not differentiable).  Gradients come
    back in the dtypes of the inputs (the library computes them in fp32).
    """

    @staticmethod
    def forward(ctx, q, k, v, w, cfg, mask_in):
        shp = (cfg.batch, cfg.heads, cfg.seq_len, cfg.head_dim)
        for name, t in (("q", q), ("k", k), ("v", v)):
            _check_operand(name, t, shp, torch.bfloat16)
        _check_operand("w", w, (cfg.head_dim, cfg.head_dim), torch.bfloat16)
        dev = q.device
        t = cfg.seq_len // 64
        if cfg.mask_mode == B.SLA_MASK_GIVEN:
            _check_operand("mask", mask_in, (cfg.batch, cfg.heads, t, t), torch.int8)
            mask = mask_in
        else:
            mask = torch.empty((cfg.batch, cfg.heads, t, t), dtype=torch.int8, device=dev)
        o = torch.empty(shp, dtype=torch.bfloat16, device=dev)
        saved = torch.empty(B.sla_saved_size(cfg), dtype=torch.uint8, device=dev)
        ws = _BUFFERS.workspace(cfg, dev)
        B.sla_forward(cfg, q, k, v, w, o, mask, saved, ws)
        ctx.cfg = cfg
        ctx.save_for_backward(q, k, v, w, o, mask, saved)
        ctx.mark_non_differentiable(mask)
        return o, mask

    @staticmethod
    def backward(ctx, d_o, _d_mask):
        q, k, v, w, o, mask, saved = ctx.saved_tensors
        cfg = ctx.cfg
        d_o = d_o.to(torch.bfloat16).contiguous()
        shp = tuple(q.shape)
        dev = q.device
        dq, dk, dv = (torch.empty(shp, dtype=torch.float32, device=dev) for _ in range(3))
        dw = torch.empty((cfg.head_dim, cfg.head_dim), dtype=torch.float32, device=dev)
        ws = _BUFFERS.workspace(cfg, dev)
        B.sla_backward(cfg, q, k, v, w, o, d_o, mask, saved, dq, dk, dv, dw, ws)
        return dq.to(q.dtype), dk.to(k.dtype), dv.to(v.dtype), dw.to(w.dtype), None, None


class SparseLinearAttention(torch.nn.Module):
    """Attention module: ``o = module(q, k, v)`` for bf16 [B, H, N, d] inputs.

    frac_critical / frac_negligible: the fractions of key blocks per query
    block that get exact softmax attention / are skipped; the rest take the
    linear branch.  valid_len: tokens at or past it are padding (0 = none).
    The projection weight (d x d, nn.Linear layout, O = O_s + Y W^T) is kept in
    the dtype of ``weight`` (fp32 by default) and cast to bf16 per call.
    select_group / select_keep: two-level key-block selection (groups of
    select_group blocks, select_keep kept per query block); 0 is the flat one.
    """

    def __init__(self, head_dim: int, frac_critical: float, frac_negligible: float,
                 valid_len: int = 0, softmax_scale: float = 0.0, reuse_mask: bool = False,
                 weight: torch.Tensor | None = None, device=None, global_linear: bool = False,
                 gate: float = 1.0, select_group: int = 0, select_keep: int = 0):
        super().__init__()
        if head_dim not in (64, 128):
            raise ValueError("head_dim must be 64 or 128")
        self.head_dim = head_dim
        self.frac_critical = float(frac_critical)
        self.frac_negligible = float(frac_negligible)
        self.valid_len = int(valid_len)
        self.softmax_scale = float(softmax_scale)
        self.reuse_mask = bool(reuse_mask)
        self.global_linear = bool(global_linear)   # SALAD-style linear branch over every block
        self.gate = float(gate)                     # its output scale (global_linear only)
        self.select_group = int(select_group)       # two-level selection: blocks per group (0: flat)
        self.select_keep = int(select_keep)         # two-level selection: groups kept per row
        if weight is None:
            weight = torch.randn(head_dim, head_dim, device=device) / math.sqrt(head_dim)
        self.weight = torch.nn.Parameter(weight.clone())
        self._mask = None
        self._mask_key = None

    def reset_mask(self) -> None:
        self._mask = None
        self._mask_key = None

    @property
    def cached_mask(self):
        return self._mask

    def forward(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor) -> torch.Tensor:
        b, h, n, d = q.shape
        if d != self.head_dim:
            raise ValueError(f"head_dim {d} != {self.head_dim}")
        key = (b, h, n, d, str(q.device))
        given = self.reuse_mask and self._mask is not None and self._mask_key == key
        cfg = B.make_config(b, h, n, d, self.frac_critical, self.frac_negligible, self.valid_len,
                            self.softmax_scale, B.SLA_MASK_GIVEN if given else B.SLA_MASK_COMPUTE,
                            linear_mode=B.SLA_LINEAR_GLOBAL if self.global_linear
                            else B.SLA_LINEAR_MARGINAL, linear_gate=self.gate,
                            select_group=self.select_group, select_keep=self.select_keep)
        B.sla_block_counts(cfg)   # validates the configuration, raises SlaError
        w = self.weight.to(torch.bfloat16)
        o, mask = SlaFunction.apply(q, k, v, w, cfg, self._mask if given else None)
        if self.reuse_mask and not given:
            self._mask, self._mask_key = mask, key
        return o
