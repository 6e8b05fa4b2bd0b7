"""CPU float64 oracle for exact (softmax) attention, forward and backward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, header,
helper or constant with the HIP library and imports nothing from it.

Pages cited (by address and title):
  [csdn]      adg.csdn.net/6a311d0d10ee7a33f27dee1b.html
              "kk的大模型论文学习笔记 第8篇: FlashAttention"
  [guanweilu] guanweilu.cn/article/445.html
              "CUDA Kernel 级别的优化：Flash Attention 为什么比 PyTorch 原生实现快 5-10 倍"
  [ijyty]     ijyty.com/news/1153309
              "Flash Attention 技术原理让 Transformer 更快更高效"

What is computed.  The fused kernel the pages describe reaches exactly the
result of plain attention ([csdn] "在线Softmax：分块了还能算对吗？"; [guanweilu]
table in "一张表看清：它比原生快在哪", row on the mathematical result), so this
oracle is that plain definition written out, not the tiled algorithm:

  S = scale * Q K^T                      ([ijyty] "传统 Attention 的问题", the
                                          naive_attention snippet; [guanweilu]
                                          "三行 PyTorch，贵在搬数据")
  P = softmax(S) row-wise, stabilised by subtracting the row maximum
                                         ([ijyty] "数值稳定性", stable_softmax)
  O = P V
  LSE_i = m_i + ln(sum_j exp(S_ij - m_i))  (natural log of the row normaliser)

Readings where the pages are silent (each also listed with the design notes):
  * the causal mask keeps key j for query i iff j <= i (square N x N), so no
    row is ever fully masked;
  * LSE is the natural-log log-sum-exp of the scaled, masked scores;
  * the backward pass is ordinary calculus of the definition above (the pages
    only say that the fused backward recomputes S and P instead of storing
    them: [csdn] "重计算：扔掉比存着更快", [guanweilu] 第三招):
      dV = P^T dO,  dP = dO V^T,  Delta_i = sum_j P_ij dP_ij,
      dS = P * (dP - Delta),  dQ = scale dS K,  dK = scale dS^T Q.

Large N.  S is materialised one block of query rows at a time; each block
still sees every key of its rows, so this is the exact two-pass softmax per
row, not an online rescaling.

Partial attention and merging (the building block of sequence-parallel /
ring attention, not on the pages): a block of Nq queries at global positions
q_pos + i attends to a block of Nk keys at positions k_pos + j, the causal
mask keeping key j iff k_pos + j <= q_pos + i.  A row that sees no key has
O = 0 and LSE = -inf.  Two partial results of the same queries over disjoint
key sets combine exactly as the online softmax combines tiles ([guanweilu]
"FlashAttention 的三板斧", second technique, applied to whole blocks):
LSE = ln(e^LSE_a + e^LSE_b), O = e^(LSE_a - LSE) O_a + e^(LSE_b - LSE) O_b.

Parity pins (tests/test_oracle.py): closed forms (Q=0, one-hot keys, constant
V, N=1, scale=0, two-key log-sum-exp), invariants (joint key/value
permutation, query permutation, key shift), pure-Python brute force on tiny
inputs, central finite differences of the backward, and torch's CPU float64
scaled_dot_product_attention with autograd.  No function here is unpinned.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "attention_fwd",
    "attention_fwd_partial",
    "merge_partials",
    "attention_bwd",
    "attention_fwd_rows",
    "attention_bwd_query_rows",
    "attention_bwd_key_rows",
    "row_stats",
]

_DEFAULT_BLOCK = 512


def _as64(x):
    return np.asarray(x, dtype=np.float64)


def _check(q, k, v):
    if q.ndim != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("Q, K, V must share one (B, H, N, D) shape")


def _masked_scores(q2, k2, scale, causal, r0, r1):
    """Scores S[r0:r1, :] of one (batch, head), -inf where the causal mask
    hides a key ([ijyty] "传统 Attention 的问题": scores = Q K^T * scale)."""
    s = scale * (q2[r0:r1] @ k2.T)
    if causal:
        rows = np.arange(r0, r1)[:, None]
        cols = np.arange(k2.shape[0])[None, :]
        s = np.where(cols <= rows, s, -np.inf)
    return s


def _softmax_rows(s):
    """Stable softmax of each row plus its natural-log normaliser
    ([ijyty] "数值稳定性": subtract the row max, exponentiate, divide by the
    sum).  Returns (P, LSE)."""
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    l = e.sum(axis=1)
    return e / l[:, None], m + np.log(l)


def attention_fwd(q, k, v, scale, causal=False, block_rows=_DEFAULT_BLOCK):
    """O = softmax(scale Q K^T) V and LSE for every (b, h, i).

    q, k, v: (B, H, N, D) arrays (upcast to float64).  Returns O (B,H,N,D)
    and LSE (B,H,N), both float64.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    _check(q, k, v)
    B, H, N, D = q.shape
    o = np.empty_like(q)
    lse = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            for r0 in range(0, N, block_rows):
                r1 = min(N, r0 + block_rows)
                p, l = _softmax_rows(_masked_scores(q[b, h], k[b, h], scale, causal, r0, r1))
                o[b, h, r0:r1] = p @ v[b, h]
                lse[b, h, r0:r1] = l
    return o, lse


def attention_bwd(q, k, v, do, scale, causal=False, block_rows=_DEFAULT_BLOCK):
    """Gradients (dQ, dK, dV) of L = sum(O * dO), recomputing P from the
    definition.  All float64, shaped like q."""
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    _check(q, k, v)
    if do.shape != q.shape:
        raise ValueError("dO must have the shape of Q")
    B, H, N, D = q.shape
    dq = np.zeros_like(q)
    dk = np.zeros_like(q)
    dv = np.zeros_like(q)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, N, block_rows):
                r1 = min(N, r0 + block_rows)
                p, _ = _softmax_rows(_masked_scores(q[b, h], k[b, h], scale, causal, r0, r1))
                g = do[b, h, r0:r1]
                dv[b, h] += p.T @ g
                dp = g @ v[b, h].T
                delta = (p * dp).sum(axis=1)
                ds = p * (dp - delta[:, None])
                dq[b, h, r0:r1] = scale * (ds @ k[b, h])
                dk[b, h] += scale * (ds.T @ q[b, h, r0:r1])
    return dq, dk, dv


def _one_row(q, k, v, scale, causal, b, h, i):
    s = scale * (k[b, h] @ q[b, h, i])
    if causal:
        s = np.where(np.arange(k.shape[2]) <= i, s, -np.inf)
    m = s.max()
    e = np.exp(s - m)
    l = e.sum()
    return e / l, m + np.log(l)


def attention_fwd_rows(q, k, v, scale, causal, rows):
    """O and LSE for selected query rows only.

    rows: integer array (R, 3) of (b, h, i).  Returns O (R, D), LSE (R,).
    Each row is the same definition as attention_fwd, evaluated alone.
    """
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    out = np.empty((rows.shape[0], q.shape[3]))
    lse = np.empty(rows.shape[0])
    for n, (b, h, i) in enumerate(rows):
        p, l = _one_row(q, k, v, scale, causal, b, h, i)
        out[n] = p @ _as64(v[b, h])
        lse[n] = l
    return out, lse


def attention_bwd_query_rows(q, k, v, do, scale, causal, rows):
    """dQ for selected query rows (b, h, i): dQ_i = scale sum_j dS_ij K_j with
    dS_ij = P_ij (dP_ij - Delta_i).  Needs only row i.  Returns (R, D)."""
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    out = np.empty((rows.shape[0], q.shape[3]))
    for n, (b, h, i) in enumerate(rows):
        p, _ = _one_row(q, k, v, scale, causal, b, h, i)
        dp = _as64(v[b, h]) @ _as64(do[b, h, i])
        delta = p @ dp
        ds = p * (dp - delta)
        out[n] = scale * (ds @ _as64(k[b, h]))
    return out


def row_stats(q, k, v, do, scale, causal, b, h, block_rows=_DEFAULT_BLOCK):
    """(LSE, Delta) for every query row of one (b, h): LSE_i as in
    attention_fwd and Delta_i = sum_j P_ij dP_ij = dO_i . O_i."""
    q2, k2, v2, g2 = (_as64(x[b, h]) for x in (q, k, v, do))
    N = q2.shape[0]
    lse = np.empty(N)
    delta = np.empty(N)
    for r0 in range(0, N, block_rows):
        r1 = min(N, r0 + block_rows)
        p, l = _softmax_rows(_masked_scores(q2, k2, scale, causal, r0, r1))
        lse[r0:r1] = l
        delta[r0:r1] = ((p @ v2) * g2[r0:r1]).sum(axis=1)
    return lse, delta


def attention_bwd_key_rows(q, k, v, do, scale, causal, rows, block_rows=_DEFAULT_BLOCK,
                           stats=None):
    """dK and dV for selected key rows (b, h, j).

    Key row j collects a term from every query row i that sees it, so the
    row statistics (LSE_i, Delta_i) of the whole (b, h) are computed first
    (row_stats, cached per (b, h) in ``stats`` if a dict is given).  Then
      P_ij = exp(S_ij - LSE_i),  dV_j = sum_i P_ij dO_i,
      dS_ij = P_ij (dP_ij - Delta_i),  dK_j = scale sum_i dS_ij Q_i.
    Returns dK (R, D), dV (R, D).
    """
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    if stats is None:
        stats = {}
    dk = np.empty((rows.shape[0], q.shape[3]))
    dv = np.empty((rows.shape[0], q.shape[3]))
    for n, (b, h, j) in enumerate(rows):
        key = (int(b), int(h))
        if key not in stats:
            stats[key] = row_stats(q, k, v, do, scale, causal, b, h, block_rows)
        lse, delta = stats[key]
        q2 = _as64(q[b, h])
        g2 = _as64(do[b, h])
        s = scale * (q2 @ _as64(k[b, h, j]))
        if causal:
            s = np.where(np.arange(q2.shape[0]) >= j, s, -np.inf)
        p = np.exp(s - lse)
        dp = g2 @ _as64(v[b, h, j])
        ds = p * (dp - delta)
        dv[n] = p @ g2
        dk[n] = scale * (ds @ q2)
    return dk, dv


def attention_fwd_partial(q, k, v, scale, causal, q_pos=0, k_pos=0):
    """(O, LSE) of queries q (B, H, Nq, D) against keys/values k, v
    (B, H, Nk, D) whose rows sit at global positions q_pos + i and k_pos + j.
    Causal: key j is visible to query i iff k_pos + j <= q_pos + i.  Rows
    with no visible key get O = 0 and LSE = -inf."""
    q, k, v = _as64(q), _as64(k), _as64(v)
    if q.ndim != 4 or k.ndim != 4 or k.shape != v.shape or q.shape[:2] != k.shape[:2] \
            or q.shape[3] != k.shape[3]:
        raise ValueError("Q (B,H,Nq,D), K and V (B,H,Nk,D) expected")
    B, H, Nq, D = q.shape
    Nk = k.shape[2]
    o = np.zeros((B, H, Nq, D))
    lse = np.full((B, H, Nq), -np.inf)
    qpos = q_pos + np.arange(Nq)[:, None]
    kpos = k_pos + np.arange(Nk)[None, :]
    visible = (kpos <= qpos) if causal else np.ones((Nq, Nk), dtype=bool)
    rows = visible.any(axis=1)
    for b in range(B):
        for h in range(H):
            s = scale * (q[b, h] @ k[b, h].T)
            s = np.where(visible, s, -np.inf)[rows]
            if s.shape[0] == 0:
                continue
            p, l = _softmax_rows(s)
            o[b, h, rows] = p @ v[b, h]
            lse[b, h, rows] = l
    return o, lse


def merge_partials(o_a, lse_a, o_b, lse_b):
    """Combine two partial results of the same query rows over disjoint key
    sets: LSE = ln(e^LSE_a + e^LSE_b), O = e^(LSE_a-LSE) O_a + e^(LSE_b-LSE) O_b.
    Rows empty in both stay O = 0, LSE = -inf."""
    o_a, o_b = _as64(o_a), _as64(o_b)
    lse_a, lse_b = _as64(lse_a), _as64(lse_b)
    m = np.maximum(lse_a, lse_b)
    finite = np.isfinite(m)
    ms = np.where(finite, m, 0.0)
    wa = np.where(finite, np.exp(lse_a - ms), 0.0)
    wb = np.where(finite, np.exp(lse_b - ms), 0.0)
    tot = wa + wb
    lse = np.where(finite, ms + np.log(np.where(finite, tot, 1.0)), -np.inf)
    denom = np.where(finite, tot, 1.0)[..., None]
    o = (wa[..., None] * o_a + wb[..., None] * o_b) / denom
    return o, lse
