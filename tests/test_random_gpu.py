"""Seeded random-shape parity of the HIP path (through the C ABI) with the
CPU float64 oracle.

The hand-picked cases elsewhere cover tile edges one at a time; here each
case draws batch, heads, sequence length, head dimension, mask, dtype and
score scale together from a fixed seed, so combinations nobody listed (a
ragged tail in a multi-head batch with a non-default scale, say) are run
too.  The same draws every time: a failure names its case and reproduces.
Every output element is compared, to the same tolerances as the other
parity tests.
"""
import numpy as np
import pytest

import oracle
from exact_io_aware_58_amd import inputs
from tests.gpu_util import TOL, max_abs, rel_to_max, say, to_device, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

from exact_io_aware_58_amd import fa  # noqa: E402  (fails loudly if libfa.so is missing)


def _case(i):
    r = np.random.default_rng([2024, i])
    B = int(r.integers(1, 4))
    H = int(r.integers(1, 6))
    N = int(r.integers(1, 700))
    D = int(r.choice([64, 128]))
    causal = bool(r.integers(0, 2))
    dtype = str(r.choice(["bf16", "f16"]))
    scale = float(r.uniform(0.5, 2.0) / np.sqrt(D))
    return B, H, N, D, causal, dtype, scale


def _draw(seed, shapes, dtype):
    vals, devs = {}, {}
    for name, shape in shapes.items():
        x, raw = inputs.draw(seed, name, shape, dtype)
        vals[name] = x.astype(np.float64)
        devs[name] = to_device(raw, dtype)
    return vals, devs


@pytest.mark.parametrize("i", range(16))
def test_random_forward_backward(i):
    B, H, N, D, causal, dtype, scale = _case(i)
    say(f"[random {i}] B={B} H={H} N={N} D={D} causal={causal} {dtype} scale={scale:.4f}")
    shape = (B, H, N, D)
    vals, devs = _draw(3000 + i, {n: shape for n in ("q", "k", "v", "do")}, dtype)
    o, lse = fa.forward(devs["q"], devs["k"], devs["v"], scale, causal)
    dq, dk, dv = fa.backward(devs["q"], devs["k"], devs["v"], o, devs["do"], lse, scale, causal)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_fwd(vals["q"], vals["k"], vals["v"], scale, causal)
    rq, rk, rv = oracle.attention_bwd(vals["q"], vals["k"], vals["v"], vals["do"], scale, causal)
    tol = TOL[dtype]
    eo, el = max_abs(to_f64(o), ro), max_abs(to_f64(lse), rl)
    eq, ek, ev = rel_to_max(to_f64(dq), rq), rel_to_max(to_f64(dk), rk), rel_to_max(to_f64(dv), rv)
    say(f"    O {eo:.2e} LSE {el:.2e} dQ/dK/dV rel {eq:.2e}/{ek:.2e}/{ev:.2e}")
    assert eo <= tol["o"] and el <= tol["lse"]
    assert max(eq, ek, ev) <= tol["grad_rel"]


def _wide_case(i):
    r = np.random.default_rng([2026, i])
    B = int(r.integers(1, 3))
    H = int(r.integers(260, 521)) // B
    N = int(r.integers(260, 641))
    D = int(r.choice([64, 128]))
    causal = bool(r.integers(0, 2))
    dtype = str(r.choice(["bf16", "f16"]))
    scale = float(r.uniform(0.5, 2.0) / np.sqrt(D))
    return B, H, N, D, causal, dtype, scale


@pytest.mark.parametrize("i", range(4))
def test_random_many_heads(i):
    """As test_random_forward_backward, on grids of 260-520 (batch, head)
    pairs: the forward takes the ping-pong kernel and the D = 64 backward
    the separate dK/dV and dQ kernels (the small random cases above take the
    4-wave forward and the combined backward launch)."""
    B, H, N, D, causal, dtype, scale = _wide_case(i)
    say(f"[random wide {i}] B={B} H={H} N={N} D={D} causal={causal} {dtype} scale={scale:.4f}")
    shape = (B, H, N, D)
    vals, devs = _draw(6000 + i, {n: shape for n in ("q", "k", "v", "do")}, dtype)
    o, lse = fa.forward(devs["q"], devs["k"], devs["v"], scale, causal)
    dq, dk, dv = fa.backward(devs["q"], devs["k"], devs["v"], o, devs["do"], lse, scale, causal)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_fwd(vals["q"], vals["k"], vals["v"], scale, causal)
    rq, rk, rv = oracle.attention_bwd(vals["q"], vals["k"], vals["v"], vals["do"], scale, causal)
    tol = TOL[dtype]
    eo, el = max_abs(to_f64(o), ro), max_abs(to_f64(lse), rl)
    eq, ek, ev = rel_to_max(to_f64(dq), rq), rel_to_max(to_f64(dk), rk), rel_to_max(to_f64(dv), rv)
    say(f"    O {eo:.2e} LSE {el:.2e} dQ/dK/dV rel {eq:.2e}/{ek:.2e}/{ev:.2e}")
    assert eo <= tol["o"] and el <= tol["lse"]
    assert max(eq, ek, ev) <= tol["grad_rel"]


@pytest.mark.parametrize("i", range(8))
def test_random_partial(i):
    """Partial attention of a query block over a key block at random
    position offsets (some rows may see no key: O = 0, LSE = -inf)."""
    r = np.random.default_rng([2025, i])
    B, H = int(r.integers(1, 3)), int(r.integers(1, 5))
    Nq, Nk = int(r.integers(1, 500)), int(r.integers(1, 500))
    D = int(r.choice([64, 128]))
    dtype = str(r.choice(["bf16", "f16", "f32"]))
    q_pos, k_pos = int(r.integers(0, 800)), int(r.integers(0, 800))
    causal = bool(r.integers(0, 2))
    scale = 1.0 / np.sqrt(D)
    say(f"[random partial {i}] B={B} H={H} Nq={Nq} Nk={Nk} D={D} {dtype} "
        f"q_pos={q_pos} k_pos={k_pos} causal={causal}")
    vals, devs = _draw(4000 + i, {"q": (B, H, Nq, D), "k": (B, H, Nk, D), "v": (B, H, Nk, D)},
                       dtype)
    o, lse = fa.forward_partial(devs["q"], devs["k"], devs["v"], scale, causal, q_pos, k_pos)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_fwd_partial(vals["q"], vals["k"], vals["v"], scale, causal,
                                          q_pos, k_pos)
    o, lse = to_f64(o), to_f64(lse)
    empty = np.isneginf(rl)
    assert np.array_equal(np.isneginf(lse), empty)
    assert np.all(o[empty] == 0.0)
    eo = max_abs(o, ro)
    el = max_abs(lse[~empty], rl[~empty])
    say(f"    O {eo:.2e} LSE {el:.2e} empty rows {int(empty.sum())}")
    assert eo <= TOL[dtype]["o"] and el <= TOL[dtype]["lse"]


@pytest.mark.parametrize("N", [1, 5, 33])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_tiny_sequences_on_large_grids(causal, D, N):
    """512 (batch, head) pairs of a handful of tokens: the forward takes the
    ping-pong kernel, whose 256-row workgroups then hold at most N valid rows
    (most waves have none), and the backward grids are as wide."""
    say(f"[tiny-N] B=4 H=128 N={N} D={D} causal={causal}")
    shape = (4, 128, N, D)
    vals, devs = _draw(5000 + N + D, {n: shape for n in ("q", "k", "v", "do")}, "bf16")
    scale = 1.0 / np.sqrt(D)
    o, lse = fa.forward(devs["q"], devs["k"], devs["v"], scale, causal)
    dq, dk, dv = fa.backward(devs["q"], devs["k"], devs["v"], o, devs["do"], lse, scale, causal)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_fwd(vals["q"], vals["k"], vals["v"], scale, causal)
    rq, rk, rv = oracle.attention_bwd(vals["q"], vals["k"], vals["v"], vals["do"], scale, causal)
    tol = TOL["bf16"]
    eo, el = max_abs(to_f64(o), ro), max_abs(to_f64(lse), rl)
    eq, ek, ev = rel_to_max(to_f64(dq), rq), rel_to_max(to_f64(dk), rk), rel_to_max(to_f64(dv), rv)
    say(f"    O {eo:.2e} LSE {el:.2e} dQ/dK/dV rel {eq:.2e}/{ek:.2e}/{ev:.2e}")
    assert eo <= tol["o"] and el <= tol["lse"]
    assert max(eq, ek, ev) <= tol["grad_rel"]
