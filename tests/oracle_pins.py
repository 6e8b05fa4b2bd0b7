"""Pins for the attention oracle: facts fixed by the pages and by mathematics,
each written independently of the oracle's own code path.

Every pin takes the forward and backward callables to check,
  fwd(q, k, v, scale, causal) -> (O, LSE)
  bwd(q, k, v, dO, scale, causal) -> (dQ, dK, dV),
and raises AssertionError on a mismatch, so the same pins can be run against
deliberately broken copies of the oracle (tests/test_oracle_mutants.py).

The pages fix the definition O = softmax(scale Q K^T) V with a stable softmax
(ijyty.com/news/1153309 "Flash Attention 技术原理让 Transformer 更快更高效",
sections "传统 Attention 的问题" and "数值稳定性") and say the fused method's
result equals it exactly (guanweilu.cn/article/445.html, "一张表看清：它比原生
快在哪").  They print no worked numerical example, so the pins are closed
forms, invariants, brute force, finite differences and a library routine.
"""
from __future__ import annotations

import itertools
import math

import numpy as np

ATOL = 1e-12


def _close(a, b, atol=ATOL, rtol=1e-12, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    lim = atol + rtol * (np.max(np.abs(b)) if b.size else 0.0)
    assert err <= lim, f"{what}: max err {err:.3e} > {lim:.3e}"


def _rand(rng, shape):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------- closed forms

def pin_q_zero_uniform(fwd, bwd):
    """Q = 0 makes every visible score equal: O_i is the mean (causal: prefix
    mean) of V and LSE_i = ln(#visible keys)."""
    rng = np.random.default_rng(11)
    B, H, N, D = 2, 2, 7, 5
    k, v = _rand(rng, (B, H, N, D)), _rand(rng, (B, H, N, D))
    q = np.zeros((B, H, N, D))
    for causal in (False, True):
        o, lse = fwd(q, k, v, 0.7, causal)
        if causal:
            cnt = np.arange(1, N + 1, dtype=np.float64)
            exp_o = np.cumsum(v, axis=2) / cnt[:, None]
            exp_l = np.broadcast_to(np.log(cnt), (B, H, N))
        else:
            exp_o = np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape)
            exp_l = np.full((B, H, N), math.log(N))
        _close(o, exp_o, what=f"Q=0 O causal={causal}")
        _close(lse, exp_l, what=f"Q=0 LSE causal={causal}")


def pin_scale_zero_uniform(fwd, bwd):
    """scale = 0 ignores Q and K entirely: uniform weights over visible keys."""
    rng = np.random.default_rng(12)
    B, H, N, D = 1, 3, 6, 4
    q, k, v = (_rand(rng, (B, H, N, D)) for _ in range(3))
    for causal in (False, True):
        o, lse = fwd(q, k, v, 0.0, causal)
        if causal:
            cnt = np.arange(1, N + 1, dtype=np.float64)
            _close(o, np.cumsum(v, axis=2) / cnt[:, None], what="scale=0 causal")
            _close(lse, np.broadcast_to(np.log(cnt), (B, H, N)), what="scale=0 causal LSE")
        else:
            _close(o, np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape), what="scale=0")
            _close(lse, np.full((B, H, N), math.log(N)), what="scale=0 LSE")


def pin_one_hot_keys(fwd, bwd):
    """K_j = e_j (N <= D), Q_i = a e_s(i), scale 1: query i gives weight e^a to
    key s(i) and 1 to every other visible key, so
      O_i = (e^a V_s(i) + sum_{visible j != s(i)} V_j) / (e^a + n_i - 1),
      LSE_i = ln(e^a + n_i - 1),  n_i = number of visible keys.
    A transposed operand or a misplaced mask breaks this."""
    rng = np.random.default_rng(13)
    N, D = 6, 8
    k = np.zeros((1, 1, N, D))
    for j in range(N):
        k[0, 0, j, j] = 1.0
    v = _rand(rng, (1, 1, N, D))
    for causal in (False, True):
        for a in (3.0, 40.0):
            if causal:
                sel = np.array([rng.integers(0, i + 1) for i in range(N)])
            else:
                sel = rng.permutation(N)
            q = np.zeros((1, 1, N, D))
            for i in range(N):
                q[0, 0, i, sel[i]] = a
            o, lse = fwd(q, k, v, 1.0, causal)
            ea = math.exp(a)
            for i in range(N):
                vis = range(i + 1) if causal else range(N)
                n = len(vis)
                num = ea * v[0, 0, sel[i]] + sum(v[0, 0, j] for j in vis if j != sel[i])
                _close(o[0, 0, i], num / (ea + n - 1), what=f"one-hot O a={a} c={causal} i={i}")
                _close(lse[0, 0, i], math.log(ea + n - 1), what=f"one-hot LSE a={a} i={i}")


def pin_constant_values(fwd, bwd):
    """V = c everywhere gives O = c whatever the weights are."""
    rng = np.random.default_rng(14)
    B, H, N, D = 2, 2, 9, 3
    q, k = _rand(rng, (B, H, N, D)), _rand(rng, (B, H, N, D))
    v = np.full((B, H, N, D), -1.25)
    for causal in (False, True):
        o, _ = fwd(q, k, v, 0.9, causal)
        _close(o, v, what=f"constant V causal={causal}")


def pin_probability_rows(fwd, bwd):
    """With V = I (N = D) the output is P itself: rows are non-negative, sum
    to 1, vanish above the diagonal when causal, and P_ij = exp(S_ij - LSE_i)."""
    rng = np.random.default_rng(15)
    N = D = 7
    q, k = _rand(rng, (1, 1, N, D)), _rand(rng, (1, 1, N, D))
    v = np.eye(N)[None, None]
    for causal in (False, True):
        p, lse = fwd(q, k, v, 0.8, causal)
        p = p[0, 0]
        assert np.all(p >= 0.0), "negative probability"
        _close(p.sum(axis=1), np.ones(N), what=f"row sums causal={causal}")
        if causal:
            _close(np.triu(p, 1), np.zeros((N, N)), what="mass above the diagonal")
        for i in range(N):
            for j in range(N):
                if causal and j > i:
                    continue
                sij = 0.8 * float(np.dot(q[0, 0, i], k[0, 0, j]))
                _close(p[i, j], math.exp(sij - lse[0, 0, i]), what=f"P[{i},{j}] vs LSE")


def pin_single_token(fwd, bwd):
    """N = 1: O = V, LSE = scale q.k, dQ = dK = 0 and dV = dO."""
    rng = np.random.default_rng(16)
    q, k, v, g = (_rand(rng, (2, 3, 1, 5)) for _ in range(4))
    for causal in (False, True):
        o, lse = fwd(q, k, v, 0.6, causal)
        _close(o, v, what="N=1 O")
        _close(lse, 0.6 * np.sum(q * k, axis=-1), what="N=1 LSE")
        dq, dk, dv = bwd(q, k, v, g, 0.6, causal)
        _close(dq, np.zeros_like(q), what="N=1 dQ")
        _close(dk, np.zeros_like(k), what="N=1 dK")
        _close(dv, g, what="N=1 dV")


def pin_two_keys_extreme(fwd, bwd):
    """One visible pair of logits a, b: LSE = max + log1p(exp(-|a-b|)) and
    O = sigmoid(a-b) V_0 + sigmoid(b-a) V_1, also for logits near +-1000
    where an unstabilised exp overflows."""
    for a, b in ((1000.0, 0.0), (-1000.0, -999.0), (2.5, -1.0), (700.0, 710.0)):
        q = np.zeros((1, 1, 2, 2))
        k = np.zeros((1, 1, 2, 2))
        q[0, 0, :, 0] = 1.0
        k[0, 0, 0, 0], k[0, 0, 1, 0] = a, b
        v = np.array([[[[1.0, -2.0], [3.0, 0.5]]]])
        o, lse = fwd(q, k, v, 1.0, False)
        sig = 1.0 / (1.0 + math.exp(-(a - b))) if a - b > -700 else 0.0
        exp_o = sig * v[0, 0, 0] + (1.0 - sig) * v[0, 0, 1]
        exp_l = max(a, b) + math.log1p(math.exp(-abs(a - b)))
        for i in range(2):
            _close(o[0, 0, i], exp_o, atol=1e-12, what=f"two keys O a={a} b={b}")
            _close(lse[0, 0, i], exp_l, atol=1e-12, rtol=1e-15, what=f"two keys LSE a={a}")


def pin_q_zero_gradients(fwd, bwd):
    """Closed-form gradients at Q = 0 (weights 1/n_i over the n_i visible keys):
      dV_j = sum_{i sees j} dO_i / n_i,
      dQ_i = (scale / n_i) sum_{j visible} (dO_i . (V_j - Vbar_i)) K_j,
      dK = 0 (every dK term carries a factor Q)."""
    rng = np.random.default_rng(17)
    N, D, scale = 6, 3, 0.45
    k, v, g = (_rand(rng, (1, 1, N, D)) for _ in range(3))
    q = np.zeros((1, 1, N, D))
    for causal in (False, True):
        dq, dk, dv = bwd(q, k, v, g, scale, causal)
        edv = np.zeros((N, D))
        edq = np.zeros((N, D))
        for i in range(N):
            vis = list(range(i + 1)) if causal else list(range(N))
            n = len(vis)
            vbar = v[0, 0, vis].mean(axis=0)
            for j in vis:
                edv[j] += g[0, 0, i] / n
                edq[i] += (scale / n) * float(np.dot(g[0, 0, i], v[0, 0, j] - vbar)) * k[0, 0, j]
        _close(dv[0, 0], edv, what=f"Q=0 dV causal={causal}")
        _close(dq[0, 0], edq, what=f"Q=0 dQ causal={causal}")
        _close(dk, np.zeros_like(dk), what=f"Q=0 dK causal={causal}")


# ---------------------------------------------------------------- invariants

def pin_key_value_permutation(fwd, bwd):
    """Without a mask, attention is a set function of the (key, value) pairs."""
    rng = np.random.default_rng(21)
    B, H, N, D = 1, 2, 11, 4
    q, k, v = (_rand(rng, (B, H, N, D)) for _ in range(3))
    perm = rng.permutation(N)
    o1, l1 = fwd(q, k, v, 0.5, False)
    o2, l2 = fwd(q, k[:, :, perm], v[:, :, perm], 0.5, False)
    _close(o1, o2, atol=1e-13, what="key/value permutation O")
    _close(l1, l2, atol=1e-13, what="key/value permutation LSE")


def pin_query_permutation(fwd, bwd):
    """Without a mask, permuting queries permutes the output rows."""
    rng = np.random.default_rng(22)
    B, H, N, D = 1, 2, 9, 4
    q, k, v = (_rand(rng, (B, H, N, D)) for _ in range(3))
    perm = rng.permutation(N)
    o1, l1 = fwd(q, k, v, 0.5, False)
    o2, l2 = fwd(q[:, :, perm], k, v, 0.5, False)
    _close(o1[:, :, perm], o2, atol=1e-13, what="query permutation O")
    _close(l1[:, :, perm], l2, atol=1e-13, what="query permutation LSE")


def pin_key_shift(fwd, bwd):
    """Adding c to every key adds scale q_i.c to every score of row i: O is
    unchanged and LSE_i moves by exactly scale q_i.c (also when causal)."""
    rng = np.random.default_rng(23)
    B, H, N, D = 1, 1, 8, 4
    q, k, v = (_rand(rng, (B, H, N, D)) for _ in range(3))
    c = _rand(rng, (D,))
    for causal in (False, True):
        o1, l1 = fwd(q, k, v, 0.7, causal)
        o2, l2 = fwd(q, k + c, v, 0.7, causal)
        _close(o1, o2, atol=1e-12, what=f"key shift O causal={causal}")
        _close(l2 - l1, 0.7 * (q @ c), atol=1e-12, what=f"key shift LSE causal={causal}")


def pin_causal_first_row(fwd, bwd):
    """Under the causal mask query 0 sees only key 0: O_0 = V_0, LSE_0 = s_00;
    the last query sees every key, so its row equals the unmasked row."""
    rng = np.random.default_rng(24)
    B, H, N, D = 2, 2, 10, 4
    q, k, v = (_rand(rng, (B, H, N, D)) for _ in range(3))
    oc, lc = fwd(q, k, v, 0.3, True)
    on, ln = fwd(q, k, v, 0.3, False)
    _close(oc[:, :, 0], v[:, :, 0], what="causal row 0")
    _close(lc[:, :, 0], 0.3 * np.sum(q[:, :, 0] * k[:, :, 0], axis=-1), what="causal LSE 0")
    _close(oc[:, :, -1], on[:, :, -1], atol=1e-13, what="causal last row")
    _close(lc[:, :, -1], ln[:, :, -1], atol=1e-13, what="causal last LSE")


# ---------------------------------------------------------------- brute force

def _brute(q, k, v, scale, causal, q_pos=0, k_pos=0):
    """Pure-Python scalar attention: explicit loops, math.exp, no numpy.
    Query i sits at position q_pos + i, key j at k_pos + j; a row with no
    visible key gets O = 0, LSE = -inf."""
    B, H, N, D = q.shape
    Nk = k.shape[2]
    out = [[[[0.0] * D for _ in range(N)] for _ in range(H)] for _ in range(B)]
    lse = [[[0.0] * N for _ in range(H)] for _ in range(B)]
    for b, h, i in itertools.product(range(B), range(H), range(N)):
        keys = [j for j in range(Nk) if not causal or k_pos + j <= q_pos + i]
        if not keys:
            lse[b][h][i] = -math.inf
            continue
        s = {}
        for j in keys:
            acc = 0.0
            for d in range(D):
                acc += float(q[b, h, i, d]) * float(k[b, h, j, d])
            s[j] = scale * acc
        mx = max(s.values())
        w = {j: math.exp(x - mx) for j, x in s.items()}
        tot = sum(w.values())
        for d in range(D):
            out[b][h][i][d] = sum(w[j] * float(v[b, h, j, d]) for j in keys) / tot
        lse[b][h][i] = mx + math.log(tot)
    return np.array(out), np.array(lse)


def pin_brute_force(fwd, bwd):
    """Tiny random shapes against scalar loops, including a large scale."""
    rng = np.random.default_rng(31)
    for (B, H, N, D), scale in (((2, 2, 5, 3), 0.5), ((1, 3, 7, 2), 6.0), ((1, 1, 1, 4), 1.0)):
        q, k, v = (_rand(rng, (B, H, N, D)) for _ in range(3))
        for causal in (False, True):
            o, lse = fwd(q, k, v, scale, causal)
            bo, bl = _brute(q, k, v, scale, causal)
            _close(o, bo, atol=1e-12, what=f"brute O {B,H,N,D} c={causal}")
            _close(lse, bl, atol=1e-12, what=f"brute LSE {B,H,N,D} c={causal}")


# ---------------------------------------------------------------- backward

def pin_finite_differences(fwd, bwd):
    """Central differences of L = sum(O * dO) match dQ, dK, dV."""
    rng = np.random.default_rng(41)
    B, H, N, D = 1, 2, 5, 3
    scale, h = 0.8, 1e-6
    q, k, v, g = (_rand(rng, (B, H, N, D)) for _ in range(4))
    for causal in (False, True):
        grads = bwd(q, k, v, g, scale, causal)
        for which, x in enumerate((q, k, v)):
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p = [q, k, v]
                args_m = [q, k, v]
                args_p[which], args_m[which] = xp, xm
                lp = np.sum(fwd(*args_p, scale, causal)[0] * g)
                lm = np.sum(fwd(*args_m, scale, causal)[0] * g)
                num[idx] = (lp - lm) / (2 * h)
            _close(grads[which], num, atol=2e-8, rtol=1e-7,
                   what=f"finite differences d{'QKV'[which]} causal={causal}")


def pin_torch_sdpa(fwd, bwd):
    """torch's CPU float64 scaled_dot_product_attention (math backend) with
    autograd: an independent library routine for the same definition."""
    import torch

    rng = np.random.default_rng(51)
    B, H, N, D = 2, 3, 13, 8
    scale = 1.0 / math.sqrt(D)
    q, k, v, g = (_rand(rng, (B, H, N, D)) for _ in range(4))
    for causal in (False, True):
        tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
        to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal,
                                                              scale=scale)
        to.backward(torch.tensor(g))
        o, _ = fwd(q, k, v, scale, causal)
        _close(o, to.detach().numpy(), atol=1e-12, what=f"sdpa O causal={causal}")
        dq, dk, dv = bwd(q, k, v, g, scale, causal)
        _close(dq, tq.grad.numpy(), atol=1e-12, what=f"sdpa dQ causal={causal}")
        _close(dk, tk.grad.numpy(), atol=1e-12, what=f"sdpa dK causal={causal}")
        _close(dv, tv.grad.numpy(), atol=1e-12, what=f"sdpa dV causal={causal}")


FORWARD_PINS = [
    pin_q_zero_uniform,
    pin_scale_zero_uniform,
    pin_one_hot_keys,
    pin_constant_values,
    pin_probability_rows,
    pin_two_keys_extreme,
    pin_key_value_permutation,
    pin_query_permutation,
    pin_key_shift,
    pin_causal_first_row,
    pin_brute_force,
]
BACKWARD_PINS = [
    pin_single_token,
    pin_q_zero_gradients,
    pin_finite_differences,
    pin_torch_sdpa,
]
ALL_PINS = FORWARD_PINS + BACKWARD_PINS


# ---------------------------------------------------------------- partial + merge
# These take part(q, k, v, scale, causal, q_pos, k_pos) -> (O, LSE) and
# merge(o_a, lse_a, o_b, lse_b) -> (O, LSE).

def _close_lse(a, b, what):
    a, b = np.asarray(a), np.asarray(b)
    assert np.array_equal(np.isneginf(a), np.isneginf(b)), f"{what}: empty rows differ"
    fin = np.isfinite(b)
    _close(a[fin], b[fin], what=what)


def pin_partial_brute_force(part, merge):
    """Rectangular blocks at offset positions (including rows that see no key
    and blocks wholly visible) against scalar loops."""
    rng = np.random.default_rng(61)
    for Nq, Nk, q_pos, k_pos in ((5, 7, 10, 8), (4, 6, 0, 3), (6, 3, 0, 0), (3, 5, 20, 0),
                                 (4, 4, 0, 9)):
        q = rng.standard_normal((1, 2, Nq, 3))
        k, v = rng.standard_normal((1, 2, Nk, 3)), rng.standard_normal((1, 2, Nk, 3))
        for causal in (False, True):
            o, lse = part(q, k, v, 0.9, causal, q_pos, k_pos)
            bo, bl = _brute(q, k, v, 0.9, causal, q_pos, k_pos)
            _close(o, bo, what=f"partial O {Nq, Nk, q_pos, k_pos} c={causal}")
            _close_lse(lse, bl, what=f"partial LSE {Nq, Nk, q_pos, k_pos} c={causal}")


def pin_partial_empty_rows(part, merge):
    """Queries placed before every key see nothing under the causal mask."""
    rng = np.random.default_rng(62)
    q, k, v = (rng.standard_normal((1, 1, 4, 2)) for _ in range(3))
    o, lse = part(q, k, v, 1.0, True, 0, 100)
    _close(o, np.zeros_like(o), what="empty rows O")
    assert np.all(np.isneginf(lse)), "empty rows LSE"


def pin_merge_of_key_blocks_is_full_attention(part, merge):
    """Splitting the keys into blocks, attending to each block and merging the
    partial results gives plain attention over all keys (the online softmax
    applied to whole blocks)."""
    rng = np.random.default_rng(63)
    N, D = 11, 4
    q, k, v = (rng.standard_normal((2, 2, N, D)) for _ in range(3))
    for causal in (False, True):
        for cuts in ((5,), (3, 7), (1, 2, 10)):
            edges = [0, *cuts, N]
            o, lse = None, None
            for a, b in zip(edges[:-1], edges[1:]):
                po, pl = part(q, k[:, :, a:b], v[:, :, a:b], 0.7, causal, 0, a)
                o, lse = (po, pl) if o is None else merge(o, lse, po, pl)
            bo, bl = _brute(q, k, v, 0.7, causal)
            _close(o, bo, atol=1e-12, what=f"merged blocks O {cuts} c={causal}")
            _close(lse, bl, atol=1e-12, what=f"merged blocks LSE {cuts} c={causal}")


def pin_merge_identities(part, merge):
    """An empty partial is the identity; merging is symmetric; two single-key
    partials merge to the two-key softmax (sigmoid weights)."""
    rng = np.random.default_rng(64)
    o1, o2 = rng.standard_normal((1, 1, 3, 2)), rng.standard_normal((1, 1, 3, 2))
    l1, l2 = rng.standard_normal((1, 1, 3)), rng.standard_normal((1, 1, 3))
    empty_o, empty_l = np.zeros_like(o1), np.full_like(l1, -np.inf)
    mo, ml = merge(o1, l1, empty_o, empty_l)
    _close(mo, o1, what="merge with empty O")
    _close(ml, l1, what="merge with empty LSE")
    mo, ml = merge(empty_o, empty_l, empty_o, empty_l)
    _close(mo, empty_o, what="merge of empties O")
    assert np.all(np.isneginf(ml)), "merge of empties LSE"
    a_o, a_l = merge(o1, l1, o2, l2)
    b_o, b_l = merge(o2, l2, o1, l1)
    _close(a_o, b_o, what="merge symmetric O")
    _close(a_l, b_l, what="merge symmetric LSE")
    w = 1.0 / (1.0 + np.exp(l2 - l1))
    _close(a_o, w[..., None] * o1 + (1 - w)[..., None] * o2, what="merge sigmoid weights")
    _close(a_l, np.maximum(l1, l2) + np.log1p(np.exp(-np.abs(l1 - l2))), what="merge log-sum-exp")


PARTIAL_PINS = [
    pin_partial_brute_force,
    pin_partial_empty_rows,
    pin_merge_of_key_blocks_is_full_attention,
    pin_merge_identities,
]
