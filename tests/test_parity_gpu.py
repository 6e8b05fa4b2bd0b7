"""Parity of the HIP path (through the C ABI) with the CPU float64 oracle.

Small shapes are compared element by element over every output; they span
several tiles and ragged tails (N not a multiple of any tile size), both
masks, both head dims and every dtype.  The five workloads run at full size
in the same launch configuration the bench times; where the oracle cannot
cover every row (N = 16384 and 65536) it checks seeded row subsets that
always include tile edges and the causal diagonal.
"""
import numpy as np
import pytest

import oracle
from exact_io_aware_58_amd import inputs
from tests.gpu_util import TOL, draw_case, max_abs, o_ok, rel_to_max, say, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

from exact_io_aware_58_amd import fa  # noqa: E402  (fails loudly if libfa.so is missing)

SHAPES_N = [1, 17, 63, 64, 65, 127, 128, 129, 255, 1000]


def _fwd(devs, scale, causal):
    o, lse = fa.forward(devs["q"], devs["k"], devs["v"], scale, causal)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", SHAPES_N)
def test_forward_small(N, causal, D, dtype):
    say(f"[fwd] N={N} D={D} causal={causal} dtype={dtype}")
    shape = (1, 2, N, D)
    vals, devs = draw_case(100 + N, shape, dtype)
    scale = 1.0 / np.sqrt(D)
    o, lse = _fwd(devs, scale, causal)
    ro, rl = oracle.attention_fwd(vals["q"], vals["k"], vals["v"], scale, causal)
    tol = TOL[dtype]
    assert max_abs(to_f64(o), ro) <= tol["o"]
    assert max_abs(to_f64(lse), rl) <= tol["lse"]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [257, 600])
def test_forward_many_heads(N, causal, D, dtype):
    """Grids with at least two 256-row workgroups per CU take the ping-pong
    forward kernel (8 waves, 256 rows); ragged N covers its tail handling."""
    say(f"[fwd-many-heads] N={N} D={D} causal={causal} dtype={dtype}")
    shape = (2, 256, N, D)
    vals, devs = draw_case(300 + N, shape, dtype)
    scale = 1.0 / np.sqrt(D)
    o, lse = _fwd(devs, scale, causal)
    ro, rl = oracle.attention_fwd(vals["q"], vals["k"], vals["v"], scale, causal)
    tol = TOL[dtype]
    eo, el = max_abs(to_f64(o), ro), max_abs(to_f64(lse), rl)
    say(f"    max abs O={eo:.2e} LSE={el:.2e}")
    assert eo <= tol["o"] and el <= tol["lse"]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_one_round_of_pingpong(causal, D):
    """A grid of exactly one 256-row workgroup per CU (128 heads x 2 query
    blocks) also takes the ping-pong kernel; N = 300 leaves a ragged tail."""
    say(f"[fwd-one-round] D={D} causal={causal}")
    shape = (1, 128, 300, D)
    vals, devs = draw_case(500 + D, shape, "bf16")
    scale = 1.0 / np.sqrt(D)
    o, lse = _fwd(devs, scale, causal)
    ro, rl = oracle.attention_fwd(vals["q"], vals["k"], vals["v"], scale, causal)
    eo, el = max_abs(to_f64(o), ro), max_abs(to_f64(lse), rl)
    say(f"    max abs O={eo:.2e} LSE={el:.2e}")
    assert eo <= TOL["bf16"]["o"] and el <= TOL["bf16"]["lse"]


@pytest.mark.parametrize("heads", [1, 512], ids=["4wave", "pingpong"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fp16_weight_near_the_rescale_bound(causal, D, heads):
    """The forward keeps a row's reference maximum until some lane's tile
    sum passes a bound, so one weight can come close to that bound before a
    rescale.  Built case: every query is a*e0, keys 0..127 are zero (the
    reference settles at score 0 on the first tile), key 128 is b*e0 with
    a*b = 16 - 2^-14 and scale = ln 2, i.e. its weight against that
    reference is 2^15.99994 = 65533; every later key scores -30.  That
    weight does not fit fp16 (largest finite 65504); packed as the PV
    operand it would become +inf.  O must stay finite and match the oracle."""
    say(f"[fwd-f16-bound] D={D} causal={causal} heads={heads}")
    N = 300
    a, b = 1.0 + 2.0 / 1024, 16.0 - 2.0 / 64  # both exact in fp16; a*b exact in fp32
    q = np.zeros((1, heads, N, D), np.float16)
    k = np.zeros((1, heads, N, D), np.float16)
    q[..., 0] = a
    k[:, :, 128, 0] = b
    k[:, :, 129:, 0] = -30.0
    rng = np.random.default_rng(7)
    v = rng.standard_normal((1, heads, N, D)).astype(np.float16)
    devs = {n: torch.from_numpy(x).cuda() for n, x in (("q", q), ("k", k), ("v", v))}
    scale = float(np.log(2.0))
    o, lse = _fwd(devs, scale, causal)
    got_o, got_l = to_f64(o), to_f64(lse)
    assert np.isfinite(got_o).all() and np.isfinite(got_l).all()
    h = [0, heads - 1]  # identical heads: check the first and the last
    ro, rl = oracle.attention_fwd(q[:, h].astype(np.float64), k[:, h].astype(np.float64),
                                  v[:, h].astype(np.float64), scale, causal)
    eo, el = max_abs(got_o[:, h], ro), max_abs(got_l[:, h], rl)
    say(f"    max abs O={eo:.2e} LSE={el:.2e}")
    assert eo <= TOL["f16"]["o"] and el <= TOL["f16"]["lse"]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("mult", [None, 2.0 ** -10, 8.0, 64.0],
                         ids=["scale2^-32", "scale2^-10", "scale8", "scale64"])
def test_extreme_scales(mult, causal, D, dtype):
    """scale = mult/sqrt(D), from the smallest scale the ABI accepts (2^-32:
    every weight is 1 to fp32 precision, so O is the mean of the visible
    values) to 64/sqrt(D) (scores spread over hundreds of log units: nearly
    one-hot rows, and the lazily kept reference maximum moves often);
    forward and, for 16-bit types, backward against the oracle.

    Two tolerances follow the arithmetic rather than the defaults.  fp32:
    a score's rounding error grows with its terms, up to D * 2^-24 *
    scale * sum_d |q_d k_d| (recursive summation over d), which at scale
    64/sqrt(D) is far above 1e-5; LSE may move by that much and O by twice
    that times max|V|.  fp16 gradients: dQ and dK are scale times O(1), below
    fp16's smallest subnormal at scale 2^-32, so the reference is the
    oracle's value rounded to fp16 (zero there): the best the output can
    hold."""
    scale = 2.0 ** -32 if mult is None else mult / np.sqrt(D)
    say(f"[extreme scale] scale={scale:g} D={D} causal={causal} dtype={dtype}")
    shape = (1, 2, 300, D)
    grad = dtype != "f32"
    vals, devs = draw_case(900 + D + causal, shape, dtype, grad=grad)
    o, lse = _fwd(devs, scale, causal)
    ro, rl = oracle.attention_fwd(vals["q"], vals["k"], vals["v"], scale, causal)
    tol = TOL[dtype]
    tol_o, tol_l = tol["o"], tol["lse"]
    if dtype == "f32":
        terms = np.einsum("bhid,bhjd->bhij", np.abs(vals["q"]), np.abs(vals["k"]))
        bound = D * 2.0 ** -24 * scale * float(terms.max())
        tol_o += 2 * bound * float(np.abs(vals["v"]).max())
        tol_l += bound
    eo, el = max_abs(to_f64(o), ro), max_abs(to_f64(lse), rl)
    say(f"    O {eo:.2e} LSE {el:.2e} (tolerances {tol_o:.2e}, {tol_l:.2e})")
    assert eo <= tol_o and el <= tol_l
    if not grad:
        return
    dq, dk, dv = fa.backward(devs["q"], devs["k"], devs["v"], o, devs["do"], lse, scale, causal)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_bwd(vals["q"], vals["k"], vals["v"], vals["do"], scale, causal)
    if dtype == "f16":
        rq, rk, rv = (r.astype(np.float16).astype(np.float64) for r in (rq, rk, rv))
    eq, ek, ev = rel_to_max(to_f64(dq), rq), rel_to_max(to_f64(dk), rk), rel_to_max(to_f64(dv), rv)
    say(f"    rel-to-max dQ={eq:.2e} dK={ek:.2e} dV={ev:.2e}")
    assert max(eq, ek, ev) <= tol["grad_rel"]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", SHAPES_N)
def test_backward_small(N, causal, D, dtype):
    say(f"[bwd] N={N} D={D} causal={causal} dtype={dtype}")
    shape = (1, 2, N, D)
    vals, devs = draw_case(200 + N, shape, dtype, grad=True)
    scale = 1.0 / np.sqrt(D)
    o, lse = _fwd(devs, scale, causal)
    dq, dk, dv = fa.backward(devs["q"], devs["k"], devs["v"], o, devs["do"], lse, scale, causal)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_bwd(vals["q"], vals["k"], vals["v"], vals["do"], scale, causal)
    tol = TOL[dtype]["grad_rel"]
    eq, ek, ev = rel_to_max(to_f64(dq), rq), rel_to_max(to_f64(dk), rk), rel_to_max(to_f64(dv), rv)
    say(f"    rel-to-max dQ={eq:.2e} dK={ek:.2e} dV={ev:.2e}")
    assert eq <= tol and ek <= tol and ev <= tol


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 128, 300, 64), (2, 256, 257, 64)],
                         ids=["128heads", "512heads"])
def test_backward_many_heads(shape, causal, dtype):
    """Grids of hundreds of heads (one or more full rounds of workgroups on
    every CU) with ragged N: the last query block and key tile are partial in
    every head; every element of dQ, dK, dV."""
    say(f"[bwd-many-heads] shape={shape} causal={causal} dtype={dtype}")
    vals, devs = draw_case(700 + shape[2], shape, dtype, grad=True)
    scale = 1.0 / np.sqrt(shape[3])
    o, lse = _fwd(devs, scale, causal)
    dq, dk, dv = fa.backward(devs["q"], devs["k"], devs["v"], o, devs["do"], lse, scale, causal)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_bwd(vals["q"], vals["k"], vals["v"], vals["do"], scale, causal)
    tol = TOL[dtype]["grad_rel"]
    eq, ek, ev = rel_to_max(to_f64(dq), rq), rel_to_max(to_f64(dk), rk), rel_to_max(to_f64(dv), rv)
    say(f"    rel-to-max dQ={eq:.2e} dK={ek:.2e} dV={ev:.2e}")
    assert eq <= tol and ek <= tol and ev <= tol


@pytest.mark.parametrize("D", [64, 128])
def test_timing_hooks_count_and_bound_the_launches(D):
    """The per-kernel timing the bench reports: with timing on, every launch
    is counted under its kernel, each duration is positive, and the summed
    kernel times fit inside the wall time of the same launches (events on
    the same stream around all of them).  At D = 64 this grid takes the
    combined dK/dV + dQ launch, at D = 128 the two separate kernels."""
    say(f"[timing] B=1 H=16 N=2048 D={D} causal, 3 fwd+bwd")
    shape = (1, 16, 2048, D)
    vals, devs = draw_case(41, shape, "bf16", grad=True)
    scale = 1.0 / np.sqrt(D)
    o, lse = _fwd(devs, scale, True)
    dq, dk, dv = fa.backward(devs["q"], devs["k"], devs["v"], o, devs["do"], lse, scale, True)
    torch.cuda.synchronize()
    assert fa.fa_timing_enable(True) == fa.FA_OK
    try:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(3):
            fa.forward(devs["q"], devs["k"], devs["v"], scale, True, out=o, lse=lse)
            fa.backward(devs["q"], devs["k"], devs["v"], o, devs["do"], lse, scale, True,
                        dq=dq, dk=dk, dv=dv)
        e1.record()
        torch.cuda.synchronize()
        wall = e0.elapsed_time(e1)
        used = [fa.FA_KERNEL_FWD, fa.FA_KERNEL_BWD_DELTA]
        used += [fa.FA_KERNEL_BWD_DKDV_DQ] if D == 64 else [fa.FA_KERNEL_BWD_DKDV,
                                                            fa.FA_KERNEL_BWD_DQ]
        total = 0.0
        for kid in range(fa.FA_KERNEL_COUNT):
            n, ms, dropped = fa.fa_timing_read(kid)
            say(f"    {fa.fa_kernel_name(kid)}: {n} launches, {ms:.4f} ms")
            if kid in used:
                assert n == 3 and dropped == 0 and ms > 0.0
                total += ms
            else:
                assert n == 0 and ms == 0.0
        say(f"    kernels {total:.4f} ms within {wall:.4f} ms of wall time")
        assert total <= wall * 1.02
    finally:
        fa.fa_timing_enable(False)


def test_output_rounding_is_nearest_even():
    """N = 2 with identical keys gives weights of exactly 1/2, so O is the
    exact fp32 mean of two bf16 values; pick means that sit exactly halfway
    between two bf16 numbers (ties go to the even one) and just above a
    halfway point (must round up, where truncation would round down)."""
    D = 64
    q = np.zeros((1, 1, 2, D), np.float32)
    k = np.zeros((1, 1, 2, D), np.float32)
    v = np.zeros((1, 1, 2, D), np.float32)
    u = 2.0 ** -7
    pairs = [(1.0, 1.0 + 2 * u), (1.0 + u, 1.0 + 2 * u), (1.0 + u, 1.0 + 4 * u),
             (-1.0 - u, -1.0 - 2 * u), (2.0, 2.0 + 4 * u)]
    exp_bits = []
    for d in range(D):
        a, b = pairs[d % len(pairs)]
        v[0, 0, 0, d], v[0, 0, 1, d] = a, b
    from exact_io_aware_58_amd.inputs import round_bf16_bits
    mean = ((v[0, 0, 0].astype(np.float64) + v[0, 0, 1]) / 2).astype(np.float32)
    exp_bits = round_bf16_bits(mean)
    devs = {n: torch.from_numpy(x).cuda().to(torch.bfloat16) for n, x in (("q", q), ("k", k), ("v", v))}
    o, _ = _fwd(devs, 0.125, False)
    got = o.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got[0, 0, 0], exp_bits)
    assert np.array_equal(got[0, 0, 1], exp_bits)


def test_forward_and_backward_are_repeatable():
    """No atomics anywhere: two runs give identical bits."""
    w = inputs.WORKLOADS["c3"]
    vals, devs = draw_case(w.seed, (2, 4, 700, 64), "bf16", grad=True)
    outs = []
    for _ in range(2):
        o, lse = _fwd(devs, 0.125, True)
        g = fa.backward(devs["q"], devs["k"], devs["v"], o, devs["do"], lse, 0.125, True)
        torch.cuda.synchronize()
        outs.append([t.clone() for t in (o, lse, *g)])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_side_stream_gives_the_same_bits():
    """The stream argument: forward, backward and partial attention enqueued
    on a non-default stream (the binding passes torch's current stream)
    produce the bits of the default-stream run, with the inputs written on
    the default stream first and an event ordering the two."""
    vals, devs = draw_case(4321, (2, 3, 500, 128), "bf16", grad=True)

    def run():
        o, lse = fa.forward(devs["q"], devs["k"], devs["v"], 0.09, True)
        g = fa.backward(devs["q"], devs["k"], devs["v"], o, devs["do"], lse, 0.09, True)
        op, lp = fa.forward_partial(devs["q"], devs["k"], devs["v"], 0.09, True, 100, 0)
        return [o, lse, *g, op, lp]

    ref = [t.clone() for t in run()]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        got = run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)


@pytest.mark.parametrize("D", [64, 128])
def test_graph_capture_replays_match_eager(D):
    """A training step's forward and backward captured into a HIP graph
    (torch.cuda.CUDAGraph; the library only launches kernels, no memset or
    allocation) and replayed three times, new input values written eagerly
    between replays: every replay equals the eager run on the same values,
    bit for bit."""
    B, H, N, scale = 1, 4, 700, D ** -0.5
    draws = [draw_case(7000 + 10 * r + D, (B, H, N, D), "bf16", grad=True)[1] for r in range(4)]
    q, k, v, do = (draws[0][n].clone() for n in ("q", "k", "v", "do"))
    o, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    ws = torch.empty(max(fa.workspace_bytes(q, True), 16), dtype=torch.uint8, device=q.device)

    def step():
        fa.forward(q, k, v, scale, True, out=o, lse=lse)
        fa.backward(q, k, v, o, do, lse, scale, True, dq=dq, dk=dk, dv=dv, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the capture
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for r in range(1, 4):
        for name, t in (("q", q), ("k", k), ("v", v), ("do", do)):
            t.copy_(draws[r][name])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (o, lse, dq, dk, dv)]
        eo, el = fa.forward(draws[r]["q"], draws[r]["k"], draws[r]["v"], scale, True)
        eg = fa.backward(draws[r]["q"], draws[r]["k"], draws[r]["v"], eo, draws[r]["do"], el,
                         scale, True)
        torch.cuda.synchronize()
        for a, b in zip(got, [eo, el, *eg]):
            assert torch.equal(a, b)


# ------------------------------------------------------------ five workloads

def _workload_devs(w):
    return draw_case(w.seed, w.shape, w.dtype, w.input_mult, grad=w.backward)


def test_workload_c1_fp32_forward():
    w = inputs.WORKLOADS["c1"]
    say(f"[{w.name}]")
    vals, devs = _workload_devs(w)
    o, lse = _fwd(devs, w.scale, w.causal)
    ro, rl = oracle.attention_fwd(vals["q"], vals["k"], vals["v"], w.scale, w.causal)
    eo, el = max_abs(to_f64(o), ro), max_abs(to_f64(lse), rl)
    say(f"    max abs O={eo:.2e} LSE={el:.2e}")
    assert eo <= 1e-5 and el <= 1e-5


def test_workload_c2_bf16_forward():
    w = inputs.WORKLOADS["c2"]
    say(f"[{w.name}]")
    vals, devs = _workload_devs(w)
    o, lse = _fwd(devs, w.scale, w.causal)
    ro, rl = oracle.attention_fwd(vals["q"], vals["k"], vals["v"], w.scale, w.causal)
    eo, er, ok = o_ok(to_f64(o), ro, "bf16")
    el = max_abs(to_f64(lse), rl)
    say(f"    max abs O={eo:.2e} (rel-to-max {er:.2e}) LSE={el:.2e}")
    assert ok and el <= 1e-3


def test_workload_c3_causal_training_step():
    w = inputs.WORKLOADS["c3"]
    say(f"[{w.name}]")
    vals, devs = _workload_devs(w)
    o, lse = _fwd(devs, w.scale, True)
    dq, dk, dv = fa.backward(devs["q"], devs["k"], devs["v"], o, devs["do"], lse, w.scale, True)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_fwd(vals["q"], vals["k"], vals["v"], w.scale, True)
    rq, rk, rv = oracle.attention_bwd(vals["q"], vals["k"], vals["v"], vals["do"], w.scale, True)
    eo, er, ok = o_ok(to_f64(o), ro, "bf16")
    el = max_abs(to_f64(lse), rl)
    eq, ek, ev = rel_to_max(to_f64(dq), rq), rel_to_max(to_f64(dk), rk), rel_to_max(to_f64(dv), rv)
    say(f"    O={eo:.2e} (rel-to-max {er:.2e}) LSE={el:.2e} dQ={eq:.2e} dK={ek:.2e} dV={ev:.2e}")
    assert ok and el <= 1e-3
    assert eq <= 5e-2 and ek <= 5e-2 and ev <= 5e-2


def _sampled(t, rows):
    idx = torch.from_numpy(rows).to(t.device)
    return to_f64(t[idx[:, 0], idx[:, 1], idx[:, 2]])


def test_workload_c4_long_forward_subset():
    w = inputs.WORKLOADS["c4"]
    say(f"[{w.name}]")
    vals, devs = _workload_devs(w)
    before = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    o, lse = _fwd(devs, w.scale, w.causal)
    peak_extra = torch.cuda.max_memory_allocated() - before
    # O(N) device memory: the outputs (O and LSE) and nothing of size N x N
    assert peak_extra <= o.numel() * 2 + lse.numel() * 4 + (1 << 21)
    rows = inputs.check_row_subset(w)
    ro, rl = oracle.attention_fwd_rows(vals["q"], vals["k"], vals["v"], w.scale, w.causal, rows)
    eo, er, ok = o_ok(_sampled(o, rows), ro, "bf16")
    el = max_abs(to_f64(lse)[tuple(rows.T)], rl)
    say(f"    {len(rows)} rows: max abs O={eo:.2e} (rel-to-max {er:.2e}, max |O_ref| "
        f"{np.max(np.abs(ro)):.3e}) LSE={el:.2e}")
    assert ok and el <= 1e-3


def _key_rows_two_heads(w, count=128):
    """Key rows for dK/dV at N = 65536: the tile-edge rows of the first and
    last head plus seeded rows of those two heads (each checked key row needs
    a full pass over its head's queries in the oracle)."""
    fixed = inputs.check_row_subset(w, count=16)[:16]
    rng = np.random.default_rng(w.seed + 2000)
    rows = [tuple(r) for r in fixed]
    seen = set(rows)
    while len(rows) < count:
        h = (0, w.H - 1)[int(rng.integers(2))]
        r = (0, h, int(rng.integers(w.N)))
        if r not in seen:
            seen.add(r)
            rows.append(r)
    return np.array(rows, dtype=np.int64)


def test_workload_c5_long_causal_training_subset():
    w = inputs.WORKLOADS["c5"]
    say(f"[{w.name}]")
    vals, devs = _workload_devs(w)
    o, lse = _fwd(devs, w.scale, True)
    dq, dk, dv = fa.backward(devs["q"], devs["k"], devs["v"], o, devs["do"], lse, w.scale, True)
    torch.cuda.synchronize()
    qrows = inputs.check_row_subset(w)
    ro, rl = oracle.attention_fwd_rows(vals["q"], vals["k"], vals["v"], w.scale, True, qrows)
    rq = oracle.attention_bwd_query_rows(vals["q"], vals["k"], vals["v"], vals["do"], w.scale,
                                         True, qrows)
    eo, er, ok = o_ok(_sampled(o, qrows), ro, "bf16")
    el = max_abs(to_f64(lse)[tuple(qrows.T)], rl)
    eq = rel_to_max(_sampled(dq, qrows), rq)
    say(f"    {len(qrows)} query rows: O={eo:.2e} (rel-to-max {er:.2e}) LSE={el:.2e} dQ={eq:.2e}")
    krows = _key_rows_two_heads(w)
    stats = {}
    for h in sorted({int(r[1]) for r in krows}):
        say(f"    oracle row statistics of head {h} ...")
        stats[(0, h)] = oracle.row_stats(vals["q"], vals["k"], vals["v"], vals["do"], w.scale,
                                         True, 0, h, block_rows=1024)
    rk, rv = oracle.attention_bwd_key_rows(vals["q"], vals["k"], vals["v"], vals["do"], w.scale,
                                           True, krows, stats=stats)
    ek, ev = rel_to_max(_sampled(dk, krows), rk), rel_to_max(_sampled(dv, krows), rv)
    say(f"    {len(krows)} key rows: dK={ek:.2e} dV={ev:.2e}")
    assert ok and el <= 1e-3 and eq <= 5e-2
    assert ek <= 5e-2 and ev <= 5e-2


def test_workload_n128k_causal_training_subset():
    """A 131072-token causal forward + backward on one GPU (device memory
    stays linear in N: the library allocates nothing), checked on seeded
    query rows (O, LSE, dQ) and key rows of head 0 (dK, dV)."""
    w = inputs.WORKLOADS["n128k"]
    say(f"[{w.name}]")
    vals, devs = _workload_devs(w)
    before = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    o, lse = _fwd(devs, w.scale, True)
    dq, dk, dv = fa.backward(devs["q"], devs["k"], devs["v"], o, devs["do"], lse, w.scale, True)
    torch.cuda.synchronize()
    peak_extra = torch.cuda.max_memory_allocated() - before
    # outputs (O, dQ, dK, dV, LSE) and the workspace (two float32 row
    # statistics per query row, -Delta and -LSE/scale); nothing N x N
    ws = fa.workspace_bytes(devs["q"], True)
    assert ws <= 2 * lse.numel() * 4 + 512
    assert peak_extra <= 4 * o.numel() * 2 + lse.numel() * 4 + ws + (1 << 22)
    qrows = inputs.check_row_subset(w)
    ro, rl = oracle.attention_fwd_rows(vals["q"], vals["k"], vals["v"], w.scale, True, qrows)
    rq = oracle.attention_bwd_query_rows(vals["q"], vals["k"], vals["v"], vals["do"], w.scale,
                                         True, qrows)
    eo, er, ok = o_ok(_sampled(o, qrows), ro, "bf16")
    el = max_abs(to_f64(lse)[tuple(qrows.T)], rl)
    eq = rel_to_max(_sampled(dq, qrows), rq)
    say(f"    {len(qrows)} query rows: O={eo:.2e} (rel-to-max {er:.2e}) LSE={el:.2e} dQ={eq:.2e}")
    krows = np.array([r for r in _key_rows_two_heads(w, count=48) if r[1] == 0][:32], dtype=np.int64)
    say("    oracle row statistics of head 0 ...")
    stats = {(0, 0): oracle.row_stats(vals["q"], vals["k"], vals["v"], vals["do"], w.scale, True,
                                      0, 0, block_rows=1024)}
    rk, rv = oracle.attention_bwd_key_rows(vals["q"], vals["k"], vals["v"], vals["do"], w.scale,
                                           True, krows, stats=stats)
    ek, ev = rel_to_max(_sampled(dk, krows), rk), rel_to_max(_sampled(dv, krows), rv)
    say(f"    {len(krows)} key rows: dK={ek:.2e} dV={ev:.2e}")
    assert ok and el <= 1e-3 and eq <= 5e-2
    assert ek <= 5e-2 and ev <= 5e-2


def test_workload_d128_training_subset():
    """The D = 128 training step (B=1, H=16, N=16384, no mask; the unmasked
    D = 128 dK/dV kernel has its own build unit): seeded query rows (O, LSE,
    dQ) and key rows of the first and last head (dK, dV) against the
    oracle."""
    w = inputs.WORKLOADS["train_d128"]
    say(f"[{w.name}]")
    vals, devs = _workload_devs(w)
    o, lse = _fwd(devs, w.scale, w.causal)
    dq, dk, dv = fa.backward(devs["q"], devs["k"], devs["v"], o, devs["do"], lse, w.scale,
                             w.causal)
    torch.cuda.synchronize()
    qrows = inputs.check_row_subset(w)
    ro, rl = oracle.attention_fwd_rows(vals["q"], vals["k"], vals["v"], w.scale, w.causal, qrows)
    rq = oracle.attention_bwd_query_rows(vals["q"], vals["k"], vals["v"], vals["do"], w.scale,
                                         w.causal, qrows)
    eo, er, ok = o_ok(_sampled(o, qrows), ro, "bf16")
    el = max_abs(to_f64(lse)[tuple(qrows.T)], rl)
    eq = rel_to_max(_sampled(dq, qrows), rq)
    say(f"    {len(qrows)} query rows: O={eo:.2e} (rel-to-max {er:.2e}) LSE={el:.2e} dQ={eq:.2e}")
    krows = _key_rows_two_heads(w, count=64)
    stats = {}
    for h in sorted({int(r[1]) for r in krows}):
        say(f"    oracle row statistics of head {h} ...")
        stats[(0, h)] = oracle.row_stats(vals["q"], vals["k"], vals["v"], vals["do"], w.scale,
                                         w.causal, 0, h, block_rows=1024)
    rk, rv = oracle.attention_bwd_key_rows(vals["q"], vals["k"], vals["v"], vals["do"], w.scale,
                                           w.causal, krows, stats=stats)
    ek, ev = rel_to_max(_sampled(dk, krows), rk), rel_to_max(_sampled(dv, krows), rv)
    say(f"    {len(krows)} key rows: dK={ek:.2e} dV={ev:.2e}")
    assert ok and el <= 1e-3 and eq <= 5e-2
    assert ek <= 5e-2 and ev <= 5e-2
