"""The pins are strong enough: each plausible mistake planted in the oracle
(on the CPU, in the oracle's own helpers or in a copy of its backward) makes
at least one pin fail."""
import numpy as np
import pytest

import oracle
import oracle.attention as oa
from tests import oracle_pins


def _fwd(q, k, v, scale, causal):
    return oa.attention_fwd(q, k, v, scale, causal)


def _bwd(q, k, v, g, scale, causal):
    return oa.attention_bwd(q, k, v, g, scale, causal)


def _some_pin_fails(fwd, bwd, pins):
    failed = []
    for pin in pins:
        try:
            with np.errstate(all="ignore"):
                pin(fwd, bwd)
        except (AssertionError, FloatingPointError, ValueError):
            failed.append(pin.__name__)
    return failed


# ------------------------------------------------------------ forward mutants

def _scores_strict_mask(q2, k2, scale, causal, r0, r1):
    s = scale * (q2[r0:r1] @ k2.T)
    if causal:
        rows = np.arange(r0, r1)[:, None]
        cols = np.arange(k2.shape[0])[None, :]
        s = np.where(cols < rows, s, -np.inf)          # planted: diagonal hidden
    return s


def _scores_reversed_mask(q2, k2, scale, causal, r0, r1):
    s = scale * (q2[r0:r1] @ k2.T)
    if causal:
        rows = np.arange(r0, r1)[:, None]
        cols = np.arange(k2.shape[0])[None, :]
        s = np.where(cols >= rows, s, -np.inf)         # planted: future keys kept
    return s


def _scores_swapped_qk(q2, k2, scale, causal, r0, r1):
    s = scale * (k2[r0:r1] @ q2.T)                     # planted: Q and K swapped
    if causal:
        rows = np.arange(r0, r1)[:, None]
        cols = np.arange(k2.shape[0])[None, :]
        s = np.where(cols <= rows, s, -np.inf)
    return s


def _scores_no_scale(q2, k2, scale, causal, r0, r1):
    s = q2[r0:r1] @ k2.T                               # planted: scale dropped
    if causal:
        rows = np.arange(r0, r1)[:, None]
        cols = np.arange(k2.shape[0])[None, :]
        s = np.where(cols <= rows, s, -np.inf)
    return s


def _softmax_unstable(s):
    e = np.exp(s)                                      # planted: no max subtraction
    l = e.sum(axis=1)
    return e / l[:, None], np.log(l)


def _softmax_log2(s):
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    l = e.sum(axis=1)
    return e / l[:, None], m + np.log2(l)              # planted: base-2 LSE


def _softmax_unnormalised(s):
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    l = e.sum(axis=1)
    return e, m + np.log(l)                            # planted: final divide dropped


FWD_MUTANTS = {
    "strict_mask": ("_masked_scores", _scores_strict_mask),
    "reversed_mask": ("_masked_scores", _scores_reversed_mask),
    "swapped_qk": ("_masked_scores", _scores_swapped_qk),
    "no_scale": ("_masked_scores", _scores_no_scale),
    "unstable_softmax": ("_softmax_rows", _softmax_unstable),
    "log2_lse": ("_softmax_rows", _softmax_log2),
    "unnormalised": ("_softmax_rows", _softmax_unnormalised),
}


@pytest.mark.parametrize("name", sorted(FWD_MUTANTS))
def test_forward_mutant_is_caught(name, monkeypatch):
    attr, fn = FWD_MUTANTS[name]
    monkeypatch.setattr(oa, attr, fn)
    failed = _some_pin_fails(_fwd, _bwd, oracle_pins.ALL_PINS)
    assert failed, f"mutant {name} passed every pin"


# ------------------------------------------------------------ backward mutants

def _bwd_copy(mutation):
    """A copy of the oracle's backward with one planted change."""
    def bwd(q, k, v, do, scale, causal):
        q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
        B, H, N, D = q.shape
        dq, dk, dv = np.zeros_like(q), np.zeros_like(q), np.zeros_like(q)
        for b in range(B):
            for h in range(H):
                p, _ = oa._softmax_rows(oa._masked_scores(q[b, h], k[b, h], scale, causal, 0, N))
                g = do[b, h]
                dv[b, h] = p.T @ g if mutation != "dv_untransposed" else p @ g
                dp = g @ v[b, h].T
                delta = (p * dp).sum(axis=1)
                if mutation == "no_delta":
                    ds = p * dp
                elif mutation == "delta_sign":
                    ds = p * (dp + delta[:, None])
                else:
                    ds = p * (dp - delta[:, None])
                dq[b, h] = scale * (ds @ k[b, h])
                if mutation == "dk_no_scale":
                    dk[b, h] = ds.T @ q[b, h]
                elif mutation == "dk_untransposed":
                    dk[b, h] = scale * (ds @ q[b, h])
                else:
                    dk[b, h] = scale * (ds.T @ q[b, h])
                if mutation == "dq_wrong_operand":
                    dq[b, h] = scale * (ds @ v[b, h])
        return dq, dk, dv
    return bwd


BWD_MUTANTS = ["dv_untransposed", "no_delta", "delta_sign", "dk_no_scale",
               "dk_untransposed", "dq_wrong_operand"]


def test_unmutated_backward_copy_passes():
    """The copy used for backward mutants is itself correct when unmutated."""
    failed = _some_pin_fails(_fwd, _bwd_copy(None), oracle_pins.BACKWARD_PINS)
    assert not failed, failed


@pytest.mark.parametrize("name", BWD_MUTANTS)
def test_backward_mutant_is_caught(name):
    failed = _some_pin_fails(_fwd, _bwd_copy(name), oracle_pins.BACKWARD_PINS)
    assert failed, f"mutant {name} passed every backward pin"


# ------------------------------------------------------------ partial / merge mutants

def _merge_swapped(o_a, lse_a, o_b, lse_b):
    o, l = oa.merge_partials(o_a, lse_a, o_b, lse_b)
    m = np.maximum(lse_a, lse_b)
    wa = np.exp(lse_b - m)                              # planted: weights swapped
    wb = np.exp(lse_a - m)
    return (wa[..., None] * o_a + wb[..., None] * o_b) / (wa + wb)[..., None], l


def _merge_max_only(o_a, lse_a, o_b, lse_b):
    o, _ = oa.merge_partials(o_a, lse_a, o_b, lse_b)
    return o, np.maximum(lse_a, lse_b)                  # planted: LSE not summed


def _partial_shifted(q, k, v, scale, causal, q_pos=0, k_pos=0):
    return oa.attention_fwd_partial(q, k, v, scale, causal, q_pos + 1, k_pos)  # off by one


@pytest.mark.parametrize("name,part,merge", [
    ("merge_swapped", oa.attention_fwd_partial, _merge_swapped),
    ("merge_max_only", oa.attention_fwd_partial, _merge_max_only),
    ("partial_shifted", _partial_shifted, oa.merge_partials),
])
def test_partial_mutant_is_caught(name, part, merge):
    failed = []
    for pin in oracle_pins.PARTIAL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(part, merge)
        except (AssertionError, FloatingPointError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every partial pin"
