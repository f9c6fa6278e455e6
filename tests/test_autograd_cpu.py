"""Host-side checks of the autograd wrapper: argument validation happens on
the host, before any device call, and bad configurations raise the
library's error (no GPU needed)."""
import pytest
import torch

from sparse_linear_attention_mean_amd import _binding as B
from sparse_linear_attention_mean_amd.autograd import SparseLinearAttention


def test_rejects_host_tensors_before_any_device_call():
    mod = SparseLinearAttention(64, 0.125, 0.25)
    x = torch.zeros(1, 2, 1024, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        mod(x, x, x)


def test_rejects_wrong_head_dim():
    with pytest.raises(ValueError):
        SparseLinearAttention(96, 0.1, 0.1)
    mod = SparseLinearAttention(64, 0.125, 0.25)
    x = torch.zeros(1, 2, 1024, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        mod(x, x, x)


def test_rejects_bad_fractions_through_the_library():
    mod = SparseLinearAttention(64, 0.8, 0.5)   # k_c + k_n > T
    x = torch.zeros(1, 2, 1024, 64, dtype=torch.bfloat16)
    with pytest.raises(B.SlaError):
        mod(x, x, x)


def test_rejects_impossible_two_level_selection_through_the_library():
    # 1024 tokens = 16 blocks, groups of 4: keeping 1 group leaves 4 candidates < k_c = 6
    mod = SparseLinearAttention(64, 0.35, 0.0, select_group=4, select_keep=1)
    x = torch.zeros(1, 2, 1024, 64, dtype=torch.bfloat16)
    with pytest.raises(B.SlaError):
        mod(x, x, x)
