"""CPU oracle for Sparse-Linear Attention (SLA), forward and backward, in fp64.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import or call this
module: only the tests, the package smoke check and the benchmark's CPU-baseline
leg use it.  It shares no code with the HIP library.

What SLA computes (source: "SLA: Beyond Sparsity in Diffusion Transformers via
Fine-Tunable Sparse-Linear Attention", English abstract and the method section
of the paper card): the attention weights of each query block are sorted into
critical, marginal and negligible parts; critical weights get exact O(N^2)
softmax attention, marginal weights get O(N) linear attention, negligible
weights are skipped, and the two results are fused into one output.  The pages
print no equations; the concrete operators below are the plainest readings
that the rest supports (each marked "reading"):

* blocks of 64 tokens for queries and keys;
* the classifier compresses tokens into block-wise representations (mean
  pooling) and ranks key blocks per query block on the compressed score map --
  the selection family described in the abstract of "Trainable Log-linear
  Sparse Attention for Efficient Diffusion Transformers";
* per row, under the total order (score descending, block index ascending),
  the first k_c blocks are critical, the last k_n negligible, the rest
  marginal;
* linear attention uses the feature map phi(x) = elu(x) + 1 on queries and
  keys; per key block the states h_j = phi(K_j)^T V_j and z_j = sum phi(K_j);
* the linear output phi(q) H_i / phi(q) . Z_i (H_i, Z_i summed over the
  marginal blocks of row i) passes through a d x d projection W (no bias,
  y W^T) and is added to the sparse output;
* tokens at or past ``valid_len`` are padding: excluded from pooling,
  softmax and states; padded rows output zero and get zero gradients.

A variant from the pages on SALAD ("Achieve High-Sparsity Attention via
Efficient Linear Attention Tuning for Video Diffusion Transformer", method:
parallel architecture and the static-dynamic scaling) runs the linear branch
next to the sparse one over every token instead of the marginal blocks only,
and scales the projected linear output by a scalar gate in [0, 1] (reading:
the layer's static projection is W, the input- and timestep-dependent factor
is supplied as the number ``gate``).  ``linear="global"`` selects it; the SLA
default is ``linear="marginal"`` with no gate.

Everything is written out directly: two-pass softmax, direct sums over the
marginal blocks, no online rescaling, no complement tricks.  Inputs are fp64
arrays (decode bf16 bits with ``decode_bf16``).  The one rounding the method
itself fixes is the compressed score map, which is rounded to fp32 before it is
ranked, so that the ranking is taken in the precision a GPU classifier uses.
"""
from __future__ import annotations

import math

import numpy as np

BLOCK = 64


# ----------------------------------------------------------------------------
# input decoding and sizes
# ----------------------------------------------------------------------------
def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def block_counts(num_blocks: int, frac_critical: float, frac_negligible: float):
    """Per-row counts (k_c, k_n, k_m) of critical / negligible / marginal key blocks.

    Reading: the critical count rounds up (the critical share is never below
    the requested fraction) and the negligible count rounds down (the skipped
    share is never above it); a 1e-6 slack absorbs float noise in the
    fractions.  Both are taken in double precision from float32 fractions."""
    fc = float(np.float32(frac_critical))
    fn = float(np.float32(frac_negligible))
    if not (0.0 <= fc <= 1.0 and 0.0 <= fn <= 1.0):
        raise ValueError("fractions must lie in [0, 1]")
    k_c = int(math.ceil(fc * num_blocks - 1e-6))
    k_n = int(math.floor(fn * num_blocks + 1e-6))
    k_c = max(0, min(k_c, num_blocks))
    k_n = max(0, min(k_n, num_blocks))
    if k_c + k_n > num_blocks:
        raise ValueError("critical + negligible blocks exceed the row")
    return k_c, k_n, num_blocks - k_c - k_n


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)


# ----------------------------------------------------------------------------
# feature map of the linear branch (reading: elu + 1)
# ----------------------------------------------------------------------------
def phi(x: np.ndarray) -> np.ndarray:
    """elu(x) + 1: x + 1 for x > 0, exp(x) otherwise (always positive)."""
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def phi_prime(x: np.ndarray) -> np.ndarray:
    """Derivative of elu(x) + 1: 1 for x > 0, exp(x) otherwise."""
    return np.where(x > 0, 1.0, np.exp(np.minimum(x, 0.0)))


# ----------------------------------------------------------------------------
# classifier: block mean-pool, compressed score map, three-way split
# ----------------------------------------------------------------------------
def block_means(x: np.ndarray, valid_len: int, block: int = BLOCK) -> np.ndarray:
    """Mean of the valid tokens of every block.  x: [N, d] -> [T, d]."""
    n, d = x.shape
    t = n // block
    out = np.zeros((t, d))
    for j in range(t):
        lo, hi = j * block, min((j + 1) * block, valid_len)
        out[j] = x[lo:hi].mean(axis=0)
    return out


def compressed_scores(q: np.ndarray, k: np.ndarray, valid_len: int, scale: float,
                      block: int = BLOCK) -> np.ndarray:
    """Compressed score map of one head: scale * qbar_i . kbar_j, computed in
    fp64 and rounded to fp32.  q, k: [N, d] -> [T, T] float32."""
    qb = block_means(q, valid_len, block)
    kb = block_means(k, valid_len, block)
    return (scale * (qb @ kb.T)).astype(np.float32)


def classify_row(scores: np.ndarray, k_c: int, k_n: int) -> np.ndarray:
    """Three-way split of one row of fp32 scores: +1 critical, 0 marginal,
    -1 negligible.  Order: score descending, block index ascending; -0 and +0
    are equal; NaN is an error."""
    s = np.asarray(scores, dtype=np.float32)
    if np.isnan(s).any():
        raise ValueError("NaN in compressed scores")
    t = s.shape[0]
    # +0.0 makes -0 compare equal to +0 in the key below
    order = np.lexsort((np.arange(t), -(s.astype(np.float64) + 0.0)))
    row = np.zeros(t, np.int8)
    row[order[:k_c]] = 1
    if k_n > 0:
        row[order[t - k_n:]] = -1
    return row


def classify(scores: np.ndarray, k_c: int, k_n: int) -> np.ndarray:
    """Classify every row of a [..., T, T] fp32 score map."""
    s = np.asarray(scores, dtype=np.float32)
    flat = s.reshape(-1, s.shape[-1])
    out = np.stack([classify_row(r, k_c, k_n) for r in flat])
    return out.reshape(s.shape)


# ----------------------------------------------------------------------------
# two-level (hierarchical) selection
#
# "Trainable Log-linear Sparse Attention for Efficient Diffusion Transformers"
# (English abstract): top-k selection is done level by level, each level
# selecting sparsely among the indices the coarser level kept, so that the
# selection cost no longer grows with the full T x T compressed map.  The page
# gives no further detail; the readings used here:
#   * two levels: key blocks are grouped G at a time (the last group may hold
#     fewer blocks); a group's coarse key is the mean of its valid tokens, the
#     query side stays at block level;
#   * coarse scores scale * qbar_i . kgbar_g (fp32, as the fine map);
#   * under the total order (coarse score descending, group index ascending)
#     the first `keep` groups are kept and the last n_g = floor(k_n / G)
#     groups are negligible as a whole (the negligible share is never above
#     the requested fraction, as in the flat split);
#   * the candidates are the blocks of the kept groups; under the total order
#     (fine score descending, block index ascending) their first k_c are
#     critical (also when their group is among the negligible ones, which
#     happens only when keep + n_g exceeds the number of groups);
#   * every other block is marginal.
# With G = 1 and keep = T this is exactly the flat split.
# ----------------------------------------------------------------------------
def num_groups(num_blocks: int, group: int) -> int:
    return -(-num_blocks // group)


def group_means(x: np.ndarray, valid_len: int, group: int, block: int = BLOCK) -> np.ndarray:
    """Mean of the valid tokens of every group of `group` consecutive blocks.
    x: [N, d] -> [ceil(T / group), d]."""
    n, d = x.shape
    t = n // block
    tg = num_groups(t, group)
    out = np.zeros((tg, d))
    for g in range(tg):
        lo, hi = g * group * block, min((g + 1) * group * block, valid_len, n)
        out[g] = x[lo:hi].mean(axis=0)
    return out


def coarse_scores(q: np.ndarray, k: np.ndarray, valid_len: int, scale: float, group: int,
                  block: int = BLOCK) -> np.ndarray:
    """Coarse score map of one head: scale * qbar_i . kgbar_g in fp64, rounded
    to fp32.  q, k: [N, d] -> [T, ceil(T / group)] float32."""
    qb = block_means(q, valid_len, block)
    kg = group_means(k, valid_len, group, block)
    return (scale * (qb @ kg.T)).astype(np.float32)


def hier_counts(num_blocks: int, group: int, keep: int, k_c: int, k_n: int):
    """Checked parameters of the two-level split: returns (Tg, n_g).  The
    smallest candidate set (the short last group among the kept ones) must
    still hold k_c blocks; kept and negligible groups may overlap."""
    if not 1 <= group <= num_blocks:
        raise ValueError("group must lie in [1, T]")
    tg = num_groups(num_blocks, group)
    n_g = k_n // group
    last = num_blocks - (tg - 1) * group
    if not 1 <= keep <= tg:
        raise ValueError("keep must lie in [1, number of groups]")
    if k_c > (keep - 1) * group + last:
        raise ValueError("the kept groups hold fewer than k_c blocks")
    return tg, n_g


def _rank_desc(values: np.ndarray) -> np.ndarray:
    """Indices sorted by value descending, index ascending; -0 equals +0; NaN
    is an error."""
    v = np.asarray(values, dtype=np.float32)
    if np.isnan(v).any():
        raise ValueError("NaN in compressed scores")
    return np.lexsort((np.arange(v.size), -(v.astype(np.float64) + 0.0)))


def classify_hier_row(coarse: np.ndarray, scores: np.ndarray, k_c: int, n_g: int, keep: int,
                      group: int) -> np.ndarray:
    """Two-level split of one row: coarse [Tg] and fine [T] fp32 scores ->
    int8 [T] (+1 critical, 0 marginal, -1 negligible).  Only the fine scores
    of the candidate blocks are read."""
    t = np.asarray(scores).shape[0]
    tg = np.asarray(coarse).shape[0]
    order_g = _rank_desc(coarse)
    kept = np.sort(order_g[:keep])
    negl = order_g[tg - n_g:] if n_g > 0 else np.zeros(0, np.int64)
    row = np.zeros(t, np.int8)
    for g in negl:
        row[g * group:min((g + 1) * group, t)] = -1
    cand = np.concatenate([np.arange(g * group, min((g + 1) * group, t)) for g in kept])
    sc = np.asarray(scores, dtype=np.float32)[cand]
    row[cand[_rank_desc(sc)[:k_c]]] = 1
    return row


def classify_hier(coarse: np.ndarray, scores: np.ndarray, k_c: int, n_g: int, keep: int,
                  group: int) -> np.ndarray:
    """Two-level split of every row: coarse [..., T, Tg], fine [..., T, T]."""
    c = np.asarray(coarse, dtype=np.float32)
    s = np.asarray(scores, dtype=np.float32)
    cf = c.reshape(-1, c.shape[-1])
    sf = s.reshape(-1, s.shape[-1])
    out = np.stack([classify_hier_row(a, b, k_c, n_g, keep, group) for a, b in zip(cf, sf)])
    return out.reshape(s.shape)


# ----------------------------------------------------------------------------
# forward, one head
# ----------------------------------------------------------------------------
def key_block_states(k: np.ndarray, v: np.ndarray, valid_len: int, block: int = BLOCK):
    """Per key block j: h_j = sum_t phi(k_t) v_t^T  ([d, d], rows = feature of
    phi(k), columns = value channel) and z_j = sum_t phi(k_t), over valid t."""
    n, d = k.shape
    t = n // block
    h = np.zeros((t, d, d))
    z = np.zeros((t, d))
    for j in range(t):
        lo, hi = j * block, min((j + 1) * block, valid_len)
        pk = phi(k[lo:hi])
        h[j] = pk.T @ v[lo:hi]
        z[j] = pk.sum(axis=0)
    return h, z


def _valid_keys(blocks, valid_len: int, block: int = BLOCK) -> np.ndarray:
    idx = [np.arange(j * block, (j + 1) * block) for j in blocks]
    if not idx:
        return np.zeros(0, np.int64)
    keys = np.concatenate(idx)
    return keys[keys < valid_len]


def _linear_blocks(mask_row, linear: str):
    """Key blocks whose states feed the linear branch of one query block."""
    if linear == "marginal":
        return np.flatnonzero(mask_row == 0)
    if linear == "global":
        return np.arange(mask_row.size)
    raise ValueError(f"unknown linear branch {linear!r}")


def forward_head(q, k, v, w, mask, valid_len, scale, blocks=None, block: int = BLOCK,
                 states=None, linear: str = "marginal", gate: float = 1.0):
    """SLA forward for one (batch, head) with a given three-way block mask.

    q, k, v: [N, d] fp64; w: [d, d]; mask: [T, T] int8.  ``blocks`` limits the
    query blocks computed (default all).  ``linear``: "marginal" (SLA) or
    "global" (every key block, SALAD-style), with O = O_s + gate * Y W^T.
    Returns a dict of [N, ...] arrays (rows of blocks not computed are left
    zero): o, o_sparse, y (ungated), lse, den; and the per-query-block H
    [T, d, d], Z [T, d] that were used."""
    n, d = q.shape
    t = n // block
    if blocks is None:
        blocks = range(t)
    h, z = states if states is not None else key_block_states(k, v, valid_len, block)
    o = np.zeros((n, d))
    o_s = np.zeros((n, d))
    y = np.zeros((n, d))
    lse = np.full(n, -np.inf)
    den = np.zeros(n)
    big_h = np.zeros((t, d, d))
    big_z = np.zeros((t, d))
    for i in blocks:
        lo, hi = i * block, min((i + 1) * block, valid_len)
        if hi <= lo:
            continue
        qi = q[lo:hi]
        # sparse branch: exact softmax over the tokens of the critical blocks
        keys = _valid_keys(np.flatnonzero(mask[i] == 1), valid_len, block)
        if keys.size:
            logits = scale * (qi @ k[keys].T)
            m = logits.max(axis=1, keepdims=True)
            p = np.exp(logits - m)
            l = p.sum(axis=1, keepdims=True)
            o_s[lo:hi] = (p @ v[keys]) / l
            lse[lo:hi] = (m + np.log(l))[:, 0]
        # linear branch: states summed over the marginal (or all) blocks
        marg = _linear_blocks(mask[i], linear)
        hi_state = h[marg].sum(axis=0) if marg.size else np.zeros((d, d))
        zi_state = z[marg].sum(axis=0) if marg.size else np.zeros(d)
        big_h[i], big_z[i] = hi_state, zi_state
        pq = phi(qi)
        num = pq @ hi_state
        dn = pq @ zi_state
        yi = np.zeros_like(num)
        pos = dn > 0
        yi[pos] = num[pos] / dn[pos, None]
        y[lo:hi] = yi
        den[lo:hi] = dn
        # fusion: sparse output plus the (gated) projected linear output
        o[lo:hi] = o_s[lo:hi] + gate * (yi @ w.T)
    return dict(o=o, o_sparse=o_s, y=y, lse=lse, den=den, H=big_h, Z=big_z)


# ----------------------------------------------------------------------------
# backward, one head (mask held fixed: no gradient through the classifier)
# ----------------------------------------------------------------------------
def backward_head(q, k, v, w, do, mask, valid_len, scale, block: int = BLOCK, fwd=None,
                  linear: str = "marginal", gate: float = 1.0):
    """Gradients of sum(dO * O) for one head with a fixed mask.

    Returns dq, dk, dv [N, d] and this head's contribution to dw [d, d]."""
    n, d = q.shape
    t = n // block
    if fwd is None:
        fwd = forward_head(q, k, v, w, mask, valid_len, scale, block=block, linear=linear,
                           gate=gate)
    o_s, y, lse, den = fwd["o_sparse"], fwd["y"], fwd["lse"], fwd["den"]
    big_h, big_z = fwd["H"], fwd["Z"]
    valid = np.arange(n) < valid_len
    dov = np.where(valid[:, None], do, 0.0)
    # projection: O = O_s + gate * Y W^T
    dy = gate * (dov @ w)
    dw = gate * (dov.T @ y)
    dq = np.zeros((n, d))
    dk = np.zeros((n, d))
    dv = np.zeros((n, d))
    # sparse branch
    dsum = (dov * o_s).sum(axis=1)
    for i in range(t):
        lo, hi = i * block, min((i + 1) * block, valid_len)
        if hi <= lo:
            continue
        keys = _valid_keys(np.flatnonzero(mask[i] == 1), valid_len, block)
        if keys.size == 0:
            continue
        qi, doi = q[lo:hi], dov[lo:hi]
        p = np.exp(scale * (qi @ k[keys].T) - lse[lo:hi, None])
        dv[keys] += p.T @ doi
        dp = doi @ v[keys].T
        ds = p * (dp - dsum[lo:hi, None])
        dq[lo:hi] += scale * (ds @ k[keys])
        dk[keys] += scale * (ds.T @ qi)
    # linear branch, query side
    d_big_h = np.zeros((t, d, d))
    d_big_z = np.zeros((t, d))
    for i in range(t):
        lo, hi = i * block, min((i + 1) * block, valid_len)
        if hi <= lo:
            continue
        dn_i = den[lo:hi]
        pos = dn_i > 0
        if not pos.any():
            continue
        qi = q[lo:hi][pos]
        dyi = dy[lo:hi][pos]
        yi = y[lo:hi][pos]
        dni = dn_i[pos]
        d_num = dyi / dni[:, None]
        d_den = -(dyi * yi).sum(axis=1) / dni
        d_phi_q = d_num @ big_h[i].T + d_den[:, None] * big_z[i][None, :]
        rows = np.arange(lo, hi)[pos]
        dq[rows] += d_phi_q * phi_prime(qi)
        pq = phi(qi)
        d_big_h[i] = pq.T @ d_num
        d_big_z[i] = pq.T @ d_den
    # linear branch, key/value side: through H_i = sum over marginal (or all) j of h_j
    for j in range(t):
        lo, hi = j * block, min((j + 1) * block, valid_len)
        if hi <= lo:
            continue
        rows_marg = np.flatnonzero(mask[:, j] == 0) if linear == "marginal" else np.arange(t)
        if rows_marg.size == 0:
            continue
        dh = d_big_h[rows_marg].sum(axis=0)
        dz = d_big_z[rows_marg].sum(axis=0)
        kj, vj = k[lo:hi], v[lo:hi]
        d_phi_k = vj @ dh.T + dz[None, :]
        dk[lo:hi] += d_phi_k * phi_prime(kj)
        dv[lo:hi] += phi(kj) @ dh
    dq[~valid] = 0.0
    dk[~valid] = 0.0
    dv[~valid] = 0.0
    return dict(dq=dq, dk=dk, dv=dv, dw=dw)


# ----------------------------------------------------------------------------
# whole problems [B, H, N, d]
# ----------------------------------------------------------------------------
def forward(q, k, v, w, frac_critical, frac_negligible, valid_len=None, scale=None,
            mask=None, block: int = BLOCK, linear: str = "marginal", gate: float = 1.0,
            select_group: int = 0, select_keep: int = 0):
    """Full SLA forward.  q, k, v: [B, H, N, d] fp64; w: [d, d].

    If ``mask`` ([B, H, T, T] int8) is given it is used as is; otherwise it is
    built by the classifier: the flat split, or with ``select_group`` > 0 the
    two-level split (groups of ``select_group`` key blocks, ``select_keep``
    kept per row).  ``linear`` / ``gate`` as in ``forward_head``.  Returns o,
    o_sparse, y, lse, den, mask, scores and coarse (the maps only when the
    mask was built here)."""
    bsz, nh, n, d = q.shape
    if n % block:
        raise ValueError("sequence length must be a multiple of the block size")
    t = n // block
    valid_len = n if valid_len is None else valid_len
    scale = default_scale(d) if scale is None else scale
    k_c, k_n, _ = block_counts(t, frac_critical, frac_negligible)
    out = {name: np.zeros((bsz, nh, n, d)) for name in ("o", "o_sparse", "y")}
    out["lse"] = np.full((bsz, nh, n), -np.inf)
    out["den"] = np.zeros((bsz, nh, n))
    scores = coarse = None
    if mask is None:
        scores = np.zeros((bsz, nh, t, t), np.float32)
        mask = np.zeros((bsz, nh, t, t), np.int8)
        if select_group > 0:
            tg, n_g = hier_counts(t, select_group, select_keep, k_c, k_n)
            coarse = np.zeros((bsz, nh, t, tg), np.float32)
        for b in range(bsz):
            for h in range(nh):
                scores[b, h] = compressed_scores(q[b, h], k[b, h], valid_len, scale, block)
                if select_group > 0:
                    coarse[b, h] = coarse_scores(q[b, h], k[b, h], valid_len, scale,
                                                 select_group, block)
                    mask[b, h] = classify_hier(coarse[b, h], scores[b, h], k_c, n_g,
                                               select_keep, select_group)
                else:
                    mask[b, h] = classify(scores[b, h], k_c, k_n)
    for b in range(bsz):
        for h in range(nh):
            r = forward_head(q[b, h], k[b, h], v[b, h], w, mask[b, h], valid_len, scale,
                             block=block, linear=linear, gate=gate)
            for name in ("o", "o_sparse", "y", "lse", "den"):
                out[name][b, h] = r[name]
    out["mask"] = mask
    out["scores"] = scores
    out["coarse"] = coarse
    return out


def backward(q, k, v, w, do, mask, valid_len=None, scale=None, block: int = BLOCK,
             linear: str = "marginal", gate: float = 1.0):
    """Full SLA backward with a fixed mask.  Returns dq, dk, dv, dw."""
    bsz, nh, n, d = q.shape
    valid_len = n if valid_len is None else valid_len
    scale = default_scale(d) if scale is None else scale
    out = {name: np.zeros((bsz, nh, n, d)) for name in ("dq", "dk", "dv")}
    out["dw"] = np.zeros((d, d))
    for b in range(bsz):
        for h in range(nh):
            r = backward_head(q[b, h], k[b, h], v[b, h], w, do[b, h], mask[b, h],
                              valid_len, scale, block=block, linear=linear, gate=gate)
            for name in ("dq", "dk", "dv"):
                out[name][b, h] = r[name]
            out["dw"] += r["dw"]
    return out
