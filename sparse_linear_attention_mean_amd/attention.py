"""Torch-facing helpers over the C ABI: buffer allocation and calls.

Memory and streams come from torch; every computation runs in ``libsla.so``.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import _binding as B


def bf16_from_bits(bits, device) -> torch.Tensor:
    """numpy uint16 bf16 bit patterns -> a bf16 torch tensor on ``device``."""
    import numpy as np

    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(device).view(torch.bfloat16)


@dataclass
class SlaProblem:
    """A configuration plus the device buffers one forward/backward needs."""

    cfg: B.SlaConfig
    device: torch.device
    workspace: torch.Tensor
    saved: torch.Tensor

    @classmethod
    def create(cls, batch, heads, seq_len, head_dim, frac_critical, frac_negligible,
               valid_len=0, softmax_scale=0.0, mask_mode=B.SLA_MASK_COMPUTE, device="cuda",
               linear_mode=B.SLA_LINEAR_MARGINAL, linear_gate=1.0, select_group=0,
               select_keep=0):
        cfg = B.make_config(batch, heads, seq_len, head_dim, frac_critical, frac_negligible,
                            valid_len, softmax_scale, mask_mode, linear_mode=linear_mode,
                            linear_gate=linear_gate, select_group=select_group,
                            select_keep=select_keep)
        ws = B.sla_workspace_size(cfg)
        sv = B.sla_saved_size(cfg)
        if ws == 0 or sv == 0:
            B.sla_block_counts(cfg)  # raises with the library's message
        device = torch.device(device)
        workspace = torch.empty(ws, dtype=torch.uint8, device=device)
        saved = torch.empty(sv, dtype=torch.uint8, device=device)
        return cls(cfg, device, workspace, saved)

    @property
    def num_blocks(self) -> int:
        return self.cfg.seq_len // 64

    def shape(self):
        c = self.cfg
        return (c.batch, c.heads, c.seq_len, c.head_dim)

    def new_mask(self) -> torch.Tensor:
        c = self.cfg
        t = self.num_blocks
        return torch.empty((c.batch, c.heads, t, t), dtype=torch.int8, device=self.device)

    def forward(self, q, k, v, w, o=None, mask=None, stream=None):
        if o is None:
            o = torch.empty(self.shape(), dtype=torch.bfloat16, device=self.device)
        if mask is None:
            mask = self.new_mask()
        B.sla_forward(self.cfg, q, k, v, w, o, mask, self.saved, self.workspace, stream)
        return o, mask

    def backward(self, q, k, v, w, o, d_o, mask, grads=None, stream=None):
        if grads is None:
            shp = self.shape()
            d = self.cfg.head_dim
            grads = tuple(torch.empty(shp, dtype=torch.float32, device=self.device) for _ in range(3))
            grads = grads + (torch.empty((d, d), dtype=torch.float32, device=self.device),)
        dq, dk, dv, dw = grads
        B.sla_backward(self.cfg, q, k, v, w, o, d_o, mask, self.saved, dq, dk, dv, dw,
                       self.workspace, stream)
        return dq, dk, dv, dw

    def pool_scores(self, q, k, stream=None):
        t = self.num_blocks
        c = self.cfg
        scores = torch.empty((c.batch, c.heads, t, t), dtype=torch.float32, device=self.device)
        B.sla_pool_scores(self.cfg, q, k, scores, self.workspace, stream)
        return scores

    def num_groups(self) -> int:
        g = self.cfg.select_group
        return -(-self.num_blocks // g) if g > 0 else 0

    def coarse_scores(self, q, k, stream=None):
        """Two-level selection only: the coarse map fp32 [B, H, T, Tg]."""
        c = self.cfg
        coarse = torch.empty((c.batch, c.heads, self.num_blocks, self.num_groups()),
                             dtype=torch.float32, device=self.device)
        B.sla_coarse_scores(self.cfg, q, k, coarse, self.workspace, stream)
        return coarse

    def saved_views(self):
        """Views into the saved buffer: lse, den (fp32 [B,H,N]), y (bf16 [B,H,N,d])."""
        off = B.sla_saved_offsets(self.cfg)
        c = self.cfg
        n = c.batch * c.heads * c.seq_len
        lse = self.saved[off["lse"]:off["lse"] + 4 * n].view(torch.float32)
        den = self.saved[off["den"]:off["den"] + 4 * n].view(torch.float32)
        y = self.saved[off["y"]:off["y"] + 2 * n * c.head_dim].view(torch.bfloat16)
        shp = (c.batch, c.heads, c.seq_len)
        return lse.view(shp), den.view(shp), y.view(shp + (c.head_dim,))


def classify(cfg: B.SlaConfig, scores: torch.Tensor, stream=None) -> torch.Tensor:
    t = cfg.seq_len // 64
    mask = torch.empty((cfg.batch, cfg.heads, t, t), dtype=torch.int8, device=scores.device)
    B.sla_classify(cfg, scores, mask, stream)
    return mask


def classify_hier(cfg: B.SlaConfig, coarse: torch.Tensor, scores: torch.Tensor,
                  stream=None) -> torch.Tensor:
    """Two-level split of given coarse [B, H, T, Tg] and fine [B, H, T, T] maps."""
    t = cfg.seq_len // 64
    mask = torch.empty((cfg.batch, cfg.heads, t, t), dtype=torch.int8, device=scores.device)
    B.sla_classify_hier(cfg, coarse, scores, mask, stream)
    return mask
