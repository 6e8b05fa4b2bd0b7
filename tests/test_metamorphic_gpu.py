"""Full-size checks of every output row through closed forms.

At N = 16384 and 65536 the float64 oracle checks seeded row subsets only.
These tests cover every row of O (and, at the long causal shape, of dQ, dK
and dV) at those exact shapes and in the launch configuration the bench
times, using inputs whose attention has a closed form (tests/closed_forms.py):

  * V = 1: O = 1 up to one bf16 ulp below (see test_constant_values), and
    LSE does not depend on V at all, so it must equal the LSE of the
    ordinary run bit for bit.
  * Q = 0: uniform weights, O = (prefix) mean of V, LSE = ln n; at the causal
    shape also dK = 0 exactly, dV = suffix sums of dO_i / (i + 1) and dQ in
    closed form.
  * Permuting keys and values together (no mask) leaves O and LSE unchanged.

K, V and dO are the workloads' own seeded draws; only the structured tensor
is replaced.
"""
import numpy as np
import pytest

from exact_io_aware_58_amd import inputs
from tests.closed_forms import (BF16_HALF_ULP_REL, causal_uniform_dv_ranges,
                                causal_uniform_forward_ranges, uniform_backward,
                                uniform_forward, within)
import oracle
from tests.gpu_util import TOL, max_abs, rel_to_max, say, to_device, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

from exact_io_aware_58_amd import fa  # noqa: E402  (fails loudly if libfa.so is missing)

# O at Q = 0: round-to-nearest-even to bf16 (at most 2^-8 of the value) on
# top of an fp32 sum of up to 65536 unit-weight terms, divided by n (a few
# 1e-6 at most, bounded here by 5e-6).
O_SLACK = 5e-6
# LSE at Q = 0 is (0 + log2(n)) * ln 2 in fp32: a few ulps of ln 65536.
LSE_CLOSED_TOL = 1e-5


def _draw(w, name, mult=None):
    x, raw = inputs.draw(w.seed, name, w.shape, w.dtype,
                         w.input_mult if mult is None else mult)
    return x.astype(np.float64), to_device(raw, w.dtype)


def _zeros(w):
    return torch.zeros(w.shape, dtype=torch.bfloat16, device="cuda")


def _ones(w):
    return torch.ones(w.shape, dtype=torch.bfloat16, device="cuda")


@pytest.mark.parametrize("wname", ["c4", "c5"])
def test_constant_values(wname):
    """V = 1.  O_i = sum_j bf16(p_j) / sum_j p_j: the weights are rounded to
    bf16 for the PV product but summed in fp32, so the ratio is a weighted
    mean of (1 + d_j) with |d_j| <= 2^-8, and bf16 rounding of a value in
    [1 - 2^-8, 1 + 2^-8] gives 1 - 2^-8 or 1 (never 1 + 2^-7: the tie at
    1 + 2^-8 goes to the even 1.0).  Every element of O must be one of those
    two values; LSE does not depend on V and must equal the ordinary run's
    bit for bit."""
    w = inputs.WORKLOADS[wname]
    say(f"[V=1 {w.name}] all {w.B * w.H * w.N} rows")
    _, q = _draw(w, "q")
    _, k = _draw(w, "k")
    _, v = _draw(w, "v")
    _, lse_ref = fa.forward(q, k, v, w.scale, w.causal)
    o, lse = fa.forward(q, k, _ones(w), w.scale, w.causal)
    torch.cuda.synchronize()
    go = to_f64(o)
    worst = float(np.max(np.abs(go - 1.0)))
    below = int(np.count_nonzero(go != 1.0))
    same = torch.equal(lse, lse_ref)
    say(f"    max |O - 1| = {worst:.3e} ({below} elements at 1 - 2^-8); LSE equal: {same}")
    assert within(go, np.ones_like(go), 0.0, 2.0 ** -8) <= 1.0
    assert same


def test_zero_queries_long_forward():
    """Q = 0 at N = 16384, D = 128 (no mask): every row is the mean of V."""
    w = inputs.WORKLOADS["c4"]
    say(f"[Q=0 {w.name}] all rows")
    vv, v = _draw(w, "v")
    _, k = _draw(w, "k")
    o, lse = fa.forward(_zeros(w), k, v, w.scale, w.causal)
    torch.cuda.synchronize()
    ro, rl = uniform_forward(vv, w.causal)
    go, gl = to_f64(o), to_f64(lse)
    ratio = within(go, ro, BF16_HALF_ULP_REL, O_SLACK)
    el = max_abs(gl, rl)
    say(f"    O: worst |err| / (2^-8 |ref| + {O_SLACK}) = {ratio:.3f}; "
        f"rel-to-max {rel_to_max(go, ro):.2e}; LSE max abs {el:.2e}")
    assert ratio <= 1.0 and el <= LSE_CLOSED_TOL


def test_zero_queries_long_causal_training():
    """Q = 0 at N = 65536, D = 64, causal: forward and backward on every row
    of every head against the closed forms (prefix means, ln(i + 1), dK = 0,
    dV suffix sums, dQ)."""
    w = inputs.WORKLOADS["c5"]
    say(f"[Q=0 {w.name}] all rows, forward and backward")
    kk, k = _draw(w, "k")
    vv, v = _draw(w, "v")
    gg, do = _draw(w, "do", 1.0)
    q = _zeros(w)
    o, lse = fa.forward(q, k, v, w.scale, True)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, w.scale, True)
    torch.cuda.synchronize()
    ro, rl = uniform_forward(vv, True)
    go, gl = to_f64(o), to_f64(lse)
    ratio = within(go, ro, BF16_HALF_ULP_REL, O_SLACK)
    el = max_abs(gl, rl)
    say(f"    O: worst |err| / (2^-8 |ref| + {O_SLACK}) = {ratio:.3f}; LSE max abs {el:.2e}")
    assert ratio <= 1.0 and el <= LSE_CLOSED_TOL
    nz = int((dk != 0).sum())
    say(f"    dK nonzero at {nz} elements")
    assert nz == 0
    say("    closed-form gradients ...")
    rq, _, rv = uniform_backward(kk, vv, gg, w.scale, True)
    eq, ev = rel_to_max(to_f64(dq), rq), rel_to_max(to_f64(dv), rv)
    say(f"    rel-to-max dQ={eq:.2e} dV={ev:.2e}")
    assert eq <= 5e-2 and ev <= 5e-2


def test_joint_key_value_permutation_long_forward():
    """Unmasked N = 16384, D = 128: keys and values permuted by one seeded
    permutation give the same O and LSE on every row (up to the rounding of
    summing in another order)."""
    w = inputs.WORKLOADS["c4"]
    say(f"[permutation {w.name}] all rows")
    _, q = _draw(w, "q")
    _, k = _draw(w, "k")
    _, v = _draw(w, "v")
    o, lse = fa.forward(q, k, v, w.scale, False)
    perm = torch.from_numpy(np.random.default_rng(w.seed + 3000).permutation(w.N)).cuda()
    kp, vp = k[:, :, perm].contiguous(), v[:, :, perm].contiguous()
    o2, lse2 = fa.forward(q, kp, vp, w.scale, False)
    torch.cuda.synchronize()
    a, b = to_f64(o), to_f64(o2)
    eo, er = max_abs(a, b), rel_to_max(b, a)
    el = max_abs(to_f64(lse), to_f64(lse2))
    say(f"    O max abs {eo:.2e} (rel-to-max {er:.2e}); LSE max abs {el:.2e}")
    assert eo <= 2e-2 and er <= 2e-2 and el <= 1e-4


@pytest.mark.parametrize("wname", ["c4", "c5"])
def test_key_shift_long(wname):
    """Adding one vector c to every key changes every visible score of row i
    by the same scale * q_i . c: O is unchanged and LSE_i moves by exactly
    that amount.  P is then unchanged, so are dV = P^T dO and dS, and since
    every row of dS sums to zero (sum_j P_ij (dP_ij - Delta_i) = 0) dQ =
    scale dS (K + c) and dK = scale dS^T Q are unchanged too: at c5 the
    backward is checked as well.  Grid-valued Q, K, V, dO (inputs.draw_grid:
    multiples of 1/16) and c in {+1/4, -1/4}^D keep K + c exact in bf16, so
    the shifted run sees exactly the shifted inputs; every row is checked
    (c4 no mask, c5 causal)."""
    w = inputs.WORKLOADS[wname]
    say(f"[key shift {w.name}] all rows")
    qx, q = _grid(w, "q")
    _, k = _grid(w, "k")
    _, v = _grid(w, "v")
    sign = np.random.default_rng(w.seed + 4000).integers(0, 2, w.D) * 2 - 1
    cvec = 0.25 * sign.astype(np.float64)
    kc = (k.float() + torch.from_numpy(cvec).float().cuda()).to(torch.bfloat16)
    o, lse = fa.forward(q, k, v, w.scale, w.causal)
    o2, lse2 = fa.forward(q, kc, v, w.scale, w.causal)
    torch.cuda.synchronize()
    a, b = to_f64(o), to_f64(o2)
    eo, er = max_abs(a, b), rel_to_max(b, a)
    shift = w.scale * (qx.astype(np.float64) @ cvec)
    el = max_abs(to_f64(lse2) - to_f64(lse), shift)
    say(f"    O max abs {eo:.2e} (rel-to-max {er:.2e}); LSE shift max abs err {el:.2e}")
    assert eo <= 2e-2 and er <= 2e-2 and el <= 1e-3
    if w.backward:
        _, do = _grid(w, "do")
        g1 = fa.backward(q, k, v, o, do, lse, w.scale, w.causal)
        g2 = fa.backward(q, kc, v, o2, do, lse2, w.scale, w.causal)
        torch.cuda.synchronize()
        errs = [rel_to_max(to_f64(b2), to_f64(b1)) for b1, b2 in zip(g1, g2)]
        say("    rel-to-max dQ={:.2e} dK={:.2e} dV={:.2e}".format(*errs))
        assert max(errs) <= 5e-2


def test_query_permutation_long_forward():
    """Unmasked N = 16384, D = 128: permuting the queries permutes the rows
    of O and LSE (each row is computed from its own query alone)."""
    w = inputs.WORKLOADS["c4"]
    say(f"[query permutation {w.name}] all rows")
    _, q = _draw(w, "q")
    _, k = _draw(w, "k")
    _, v = _draw(w, "v")
    o, lse = fa.forward(q, k, v, w.scale, False)
    perm = torch.from_numpy(np.random.default_rng(w.seed + 5000).permutation(w.N)).cuda()
    o2, lse2 = fa.forward(q[:, :, perm].contiguous(), k, v, w.scale, False)
    torch.cuda.synchronize()
    a, b = to_f64(o[:, :, perm]), to_f64(o2)
    eo, er = max_abs(a, b), rel_to_max(b, a)
    el = max_abs(to_f64(lse[:, :, perm]), to_f64(lse2))
    say(f"    O max abs {eo:.2e} (rel-to-max {er:.2e}); LSE max abs {el:.2e}")
    assert eo <= 2e-2 and er <= 2e-2 and el <= 1e-4


def test_zero_queries_d128_training():
    """Q = 0 at the D = 128 training shape (B=1, H=16, N=16384, no mask):
    every row of O is the mean of V, dK = 0 exactly, and dQ, dV match their
    closed forms on every row."""
    w = inputs.WORKLOADS["train_d128"]
    say(f"[Q=0 {w.name}] all rows, forward and backward")
    kk, k = _draw(w, "k")
    vv, v = _draw(w, "v")
    gg, do = _draw(w, "do", 1.0)
    q = _zeros(w)
    o, lse = fa.forward(q, k, v, w.scale, False)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, w.scale, False)
    torch.cuda.synchronize()
    ro, rl = uniform_forward(vv, False)
    go, gl = to_f64(o), to_f64(lse)
    ratio = within(go, ro, BF16_HALF_ULP_REL, O_SLACK)
    el = max_abs(gl, rl)
    say(f"    O: worst |err| / (2^-8 |ref| + {O_SLACK}) = {ratio:.3f}; LSE max abs {el:.2e}")
    assert ratio <= 1.0 and el <= LSE_CLOSED_TOL
    nz = int((dk != 0).sum())
    say(f"    dK nonzero at {nz} elements")
    assert nz == 0
    rq, _, rv = uniform_backward(kk, vv, gg, w.scale, False)
    eq, ev = rel_to_max(to_f64(dq), rq), rel_to_max(to_f64(dv), rv)
    say(f"    rel-to-max dQ={eq:.2e} dV={ev:.2e}")
    assert eq <= 5e-2 and ev <= 5e-2




# The longest head the library accepts: N = 2^23 at D = 128, 2 GiB per
# tensor, so the kernels' 32-bit byte offsets inside a head come within one
# row of 2^31.  Grid-valued inputs (inputs.draw_grid) keep drawing them to a
# few seconds and make every prefix sum of V exact.  Closed forms are checked
# on the first 2^16 and the last 2^18 rows (the largest offsets), the oracle
# on single rows near the end.  Progress lines bypass pytest's capture: each
# pass runs for tens of seconds.
LONG_N, LONG_D = 1 << 23, 128
LONG_RANGES = [(0, 1 << 16), (LONG_N - (1 << 18), LONG_N)]
LONG_PICKS = [LONG_N // 2 + 3, LONG_N - 2, LONG_N - 1]


def _long(seed):
    return inputs.Workload(f"longest_head_b1h1n{LONG_N}d{LONG_D}", seed, 1, 1, LONG_N, LONG_D,
                           "bf16", True, True)


def _grid(w, name):
    x, raw = inputs.draw_grid(w.seed, name, w.shape, w.dtype)
    return x, to_device(raw, w.dtype)


def _range_rows(t):
    """Rows LONG_RANGES of head (0, 0) of a device tensor, as float64."""
    return np.concatenate([to_f64(t[0, 0, r0:r1]) for r0, r1 in LONG_RANGES])


def _row_rel(got, ref):
    """Largest per-row max|err| / max|ref| over the rows of (R, D) arrays."""
    den = np.maximum(np.max(np.abs(ref), axis=1), 1e-30)
    return float(np.max(np.max(np.abs(got - ref), axis=1) / den))


def _note(capsys, msg):
    with capsys.disabled():
        print(msg, flush=True)


@pytest.mark.timeout(600)
def test_longest_head_forward(capsys):
    """Causal forward at N = 2^23, D = 128.  Q = 0: O on the checked ranges
    (prefix means of V, exact sums, so only the bf16 rounding of O remains)
    and LSE = ln(i + 1) on every row.  Grid-valued Q: O and LSE of three rows
    near the end against the oracle."""
    w = _long(11)
    N = w.N
    _note(capsys, f"\n[{w.name}] forward: drawing K, V, Q")
    kx, k = _grid(w, "k")
    vx, v = _grid(w, "v")
    qx, q = _grid(w, "q")
    _note(capsys, "    Q = 0 ...")
    o, lse = fa.forward(_zeros(w), k, v, w.scale, True)
    torch.cuda.synchronize()
    go, gl = _range_rows(o), to_f64(lse)[0, 0]
    ro = causal_uniform_forward_ranges(vx[0, 0], LONG_RANGES)
    ratio = within(go, ro, BF16_HALF_ULP_REL, O_SLACK)
    el = max_abs(gl, np.log(np.arange(1, N + 1, dtype=np.float64)))
    _note(capsys, f"    O on {len(go)} rows: worst |err| / (2^-8 |ref| + {O_SLACK}) = {ratio:.3f}; "
                  f"LSE on every row: max abs {el:.2e}")
    assert ratio <= 1.0 and el <= LSE_CLOSED_TOL
    del o, lse, go, gl, ro
    _note(capsys, "    grid-valued Q ...")
    o, lse = fa.forward(q, k, v, w.scale, True)
    torch.cuda.synchronize()
    rows = np.array([(0, 0, i) for i in LONG_PICKS], dtype=np.int64)
    go = to_f64(o[0, 0, LONG_PICKS])
    gl = to_f64(lse[0, 0, LONG_PICKS])
    del o, lse, q, k, v
    qq, kk, vv = (x.astype(np.float64) for x in (qx, kx, vx))
    ro, rl = oracle.attention_fwd_rows(qq, kk, vv, w.scale, True, rows)
    eo, el = _row_rel(go, ro), max_abs(gl, rl)
    _note(capsys, f"    rows {LONG_PICKS}: O worst per-row rel-to-max {eo:.2e}; LSE max abs {el:.2e}")
    assert eo <= TOL["bf16"]["o_rel"] and el <= TOL["bf16"]["lse"]


@pytest.mark.timeout(600)
def test_longest_head_backward(capsys):
    """Causal forward and backward at N = 2^23, D = 128 with Q = 0: dK = 0 on
    every row, dV (suffix sums of dO_i / (i + 1)) on the checked ranges, dQ
    of three rows near the end against the oracle (which takes the zero
    queries like any other input)."""
    w = _long(12)
    _note(capsys, f"\n[{w.name}] backward: drawing K, V, dO")
    kx, k = _grid(w, "k")
    vx, v = _grid(w, "v")
    gx, do = _grid(w, "do")
    q = _zeros(w)
    _note(capsys, "    Q = 0: forward and backward ...")
    o, lse = fa.forward(q, k, v, w.scale, True)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, w.scale, True)
    torch.cuda.synchronize()
    nz = int(torch.count_nonzero(dk))
    gq = to_f64(dq[0, 0, LONG_PICKS])
    gv = _range_rows(dv)
    del o, lse, dq, dk, dv, q, k, v, do
    gg = gx.astype(np.float64)
    rv = causal_uniform_dv_ranges(gg[0, 0], LONG_RANGES)
    ev = _row_rel(gv, rv)
    _note(capsys, f"    dK nonzero at {nz} elements; dV on {len(gv)} rows: "
                  f"worst per-row rel-to-max {ev:.2e}")
    assert nz == 0 and ev <= TOL["bf16"]["grad_rel"]
    rows = np.array([(0, 0, i) for i in LONG_PICKS], dtype=np.int64)
    kk, vv = kx.astype(np.float64), vx.astype(np.float64)
    q0 = np.zeros(w.shape)  # pages never touched except the picked rows
    rq = oracle.attention_bwd_query_rows(q0, kk, vv, gg, w.scale, True, rows)
    eq = _row_rel(gq, rq)
    _note(capsys, f"    dQ rows {LONG_PICKS}: worst per-row rel-to-max {eq:.2e}")
    assert eq <= TOL["bf16"]["grad_rel"]
