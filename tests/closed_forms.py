"""Closed-form attention results for inputs with special structure, used to
check the HIP path on every row at full size, where the float64 oracle can
only afford seeded row subsets.  Test infrastructure: plain NumPy float64,
independent of both the oracle's code and the HIP library.

Attention of query i over its visible keys j (all N keys, or j <= i under
the causal mask), O_i = sum_j P_ij V_j with P = softmax(scale q_i . k_j):

* Q = 0 makes every visible score 0, so P_ij = 1/n_i with n_i the number of
  visible keys (N, or i + 1 under the mask):
    O_i = mean of the visible V_j,        LSE_i = ln n_i.
  The gradients of L = sum(O * dO) at that point follow from the calculus
  of the definition (dV = P^T dO, dP = dO V^T, Delta_i = dO_i . O_i,
  dS = P * (dP - Delta), dQ = scale dS K, dK = scale dS^T Q):
    dV_j = sum over queries i that see j of dO_i / n_i,
    dK   = 0 (every term carries a factor Q_i = 0),
    dQ_i = scale / n_i * ( sum_{j visible} (dO_i . V_j) K_j
                           - (dO_i . O_i) sum_{j visible} K_j ).
* V = 1 (every element) gives O = 1 whatever the scores: the weights of a
  row sum to 1.
* Permuting keys and values by the same permutation leaves O and LSE
  unchanged without a mask: the softmax sum runs over the same pairs.

The method computes exactly this function ([csdn] adg.csdn.net/
6a311d0d10ee7a33f27dee1b.html, "在线Softmax：分块了还能算对吗？"; [guanweilu]
guanweilu.cn/article/445.html, table in "一张表看清：它比原生快在哪"), so the
fused kernels must reproduce these closed forms up to rounding.
"""
from __future__ import annotations

import numpy as np


def _visible_counts(N, causal):
    return np.arange(1, N + 1, dtype=np.float64) if causal else np.full(N, float(N))


def uniform_forward(v, causal):
    """O and LSE at Q = 0 for values v (B, H, N, D): the (prefix) mean of V
    and ln n_i.  Returns float64 arrays (B, H, N, D) and (B, H, N)."""
    v = np.asarray(v, dtype=np.float64)
    B, H, N, D = v.shape
    n = _visible_counts(N, causal)
    if causal:
        o = np.cumsum(v, axis=2) / n[:, None]
    else:
        o = np.broadcast_to(v.sum(axis=2, keepdims=True) / N, v.shape).copy()
    lse = np.broadcast_to(np.log(n), (B, H, N)).copy()
    return o, lse


def uniform_backward(k, v, do, scale, causal, block=256):
    """(dQ, dK, dV) of sum(O * dO) at Q = 0, float64, shaped like k.

    Under the mask the visible sums are prefix sums over keys; the term
    sum_{j <= i} (dO_i . V_j) K_j = dO_i C_i with C_i = sum_{j <= i} V_j K_j^T
    (a D x D prefix sum) is formed block by block: the prefix up to the
    block start plus a lower-triangular product inside the block."""
    k, v, do = (np.asarray(x, dtype=np.float64) for x in (k, v, do))
    B, H, N, D = k.shape
    n = _visible_counts(N, causal)
    o, _ = uniform_forward(v, causal)
    delta = np.einsum("bhnd,bhnd->bhn", do, o)
    w = do / n[:, None]  # dO_i / n_i
    if causal:
        # suffix sums: dV_j = sum_{i >= j} dO_i / n_i
        dv = np.flip(np.cumsum(np.flip(w, axis=2), axis=2), axis=2)
    else:
        dv = np.broadcast_to(w.sum(axis=2, keepdims=True), k.shape).copy()
    dk = np.zeros_like(k)
    dq = np.empty_like(k)
    if not causal:
        c = np.swapaxes(v, 2, 3) @ k                      # (B, H, D, D): sum_j V_j K_j^T
        ksum = k.sum(axis=2, keepdims=True)               # (B, H, 1, D)
        dq[:] = do @ c - delta[..., None] * ksum
    else:
        c = np.zeros((B, H, D, D))
        ksum = np.zeros((B, H, 1, D))
        tri = np.tril(np.ones((block, block)))
        for r0 in range(0, N, block):
            r1 = min(N, r0 + block)
            t = tri[: r1 - r0, : r1 - r0]
            g, vb, kb = do[:, :, r0:r1], v[:, :, r0:r1], k[:, :, r0:r1]
            inner = ((g @ np.swapaxes(vb, 2, 3)) * t) @ kb   # j in the block, j <= i
            kpre = ksum + np.cumsum(kb, axis=2)              # sum_{j <= i} K_j
            dq[:, :, r0:r1] = g @ c + inner - delta[:, :, r0:r1, None] * kpre
            c = c + np.swapaxes(vb, 2, 3) @ kb
            ksum = ksum + kb.sum(axis=2, keepdims=True)
    dq *= scale / n[:, None]
    return dq, dk, dv


def causal_uniform_forward_ranges(v, ranges):
    """Causal O at Q = 0 (prefix means of V) on row ranges [(r0, r1), ...] of
    one head v (N, D), without the whole prefix-sum array: each range starts
    from one sum of the rows before it.  Returns float64 (rows, D), the
    ranges' rows in order."""
    v = np.asarray(v)
    out = []
    for r0, r1 in ranges:
        start = np.add.reduce(v[:r0], axis=0, dtype=np.float64) if r0 else 0.0
        s = start + np.cumsum(v[r0:r1], axis=0, dtype=np.float64)
        out.append(s / np.arange(r0 + 1, r1 + 1, dtype=np.float64)[:, None])
    return np.concatenate(out)


def causal_uniform_dv_ranges(do, ranges):
    """Causal dV at Q = 0, dV_j = sum_{i >= j} dO_i / (i + 1), on row ranges
    of one head do (N, D) (float64 for the weighted sum of the rows after each
    range).  Returns float64 (rows, D)."""
    do = np.asarray(do)
    N = do.shape[0]
    out = []
    for r0, r1 in ranges:
        after = (1.0 / np.arange(r1 + 1, N + 1, dtype=np.float64)) @ do[r1:] if r1 < N else 0.0
        inner = do[r0:r1] / np.arange(r0 + 1, r1 + 1, dtype=np.float64)[:, None]
        out.append(after + np.cumsum(inner[::-1], axis=0)[::-1])
    return np.concatenate(out)


def within(got, ref, rel, slack):
    """Largest |got - ref| / (rel * |ref| + slack) over all elements: <= 1
    means every element lies within `rel` of its reference (relative) plus
    an absolute `slack`."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.shape != ref.shape:
        raise ValueError(f"shape {got.shape} != {ref.shape}")
    if got.size == 0:
        return 0.0
    bound = rel * np.abs(ref) + slack
    return float(np.max(np.abs(got - ref) / bound))


# One unit in the last place of bfloat16 relative to the value it rounds:
# round-to-nearest-even moves a value by at most half a spacing, and the
# spacing is at most 2^-7 of the value, so at most 2^-8 of it.
BF16_HALF_ULP_REL = 2.0 ** -8
