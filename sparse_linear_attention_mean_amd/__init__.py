"""Sparse-Linear Attention (SLA) forward and backward for AMD MI355X (gfx950).

The computation lives in the HIP library ``libsla.so`` behind the C ABI of
``include/sla.h``; ``_binding`` marshals torch tensors into it and
``attention`` allocates the buffers a call needs.  ``inputs`` draws the seeded
synthetic operands.  Importing the binding fails loudly if the library has not
been built (``python -m sparse_linear_attention_mean_amd.builder``).
"""
