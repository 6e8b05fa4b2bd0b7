"""Parity of fa_fwd_partial and fa_merge (through the C ABI) with the CPU
float64 oracle.

fa_fwd_partial: rectangular query/key blocks at position offsets, element by
element over every output, for every offset regime of the causal rule (rows
that see part of the block, none of it, all of it), both head dims, every
dtype, and a grid large enough for the 8-wave kernel.  fa_merge: on its own,
over synthetic partial results that include rows empty on one or both sides,
and composed with fa_fwd_partial: splitting the keys of a sequence into
blocks and merging the blocks' results reproduces attention over the whole
sequence (the single-GPU building block of key/value passing across
devices).  At full size (a 65536-token causal sequence split four ways) the
composition is checked on seeded rows.
"""
import numpy as np
import pytest

import oracle
from exact_io_aware_58_amd import inputs
from tests.gpu_util import TOL, max_abs, o_ok, say, to_device, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

from exact_io_aware_58_amd import fa  # noqa: E402  (fails loudly if libfa.so is missing)


def _draw_blocks(seed, B, H, Nq, Nk, D, dtype, mult=1.0):
    vals, devs = {}, {}
    for name, n in (("q", Nq), ("k", Nk), ("v", Nk)):
        x, raw = inputs.draw(seed, name, (B, H, n, D), dtype, mult)
        vals[name] = x.astype(np.float64)
        devs[name] = to_device(raw, dtype)
    return vals, devs


def _check(o, lse, ro, rl, dtype, what):
    o, lse = to_f64(o), to_f64(lse)
    empty = np.isneginf(rl)
    assert np.array_equal(np.isneginf(lse), empty), f"{what}: empty rows differ"
    assert np.all(o[empty] == 0.0), f"{what}: O of empty rows is not zero"
    eo = max_abs(o, ro)
    el = max_abs(lse[~empty], rl[~empty])
    say(f"    {what}: max abs O={eo:.2e} LSE={el:.2e} empty rows={int(empty.sum())}")
    assert eo <= TOL[dtype]["o"] and el <= TOL[dtype]["lse"], what


# (Nq, Nk, q_pos, k_pos, causal)
PARTIAL_CASES = [
    (300, 457, 1000, 900, True),   # keys up to i + 100: partly visible, ragged tiles
    (300, 457, 0, 200, True),      # first 200 rows see nothing
    (129, 65, 70, 0, True),        # every key visible to every row
    (64, 1000, 500, 0, True),      # few queries, long key block
    (200, 100, 0, 500, True),      # no row sees anything
    (17, 300, 0, 0, True),         # Nq < Nk, aligned starts
    (257, 129, 0, 0, False),       # rectangular, unmasked
    (1, 1, 5, 5, True),
]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("case", PARTIAL_CASES, ids=lambda c: "nq{}-nk{}-qp{}-kp{}-c{}".format(*c))
def test_partial_small(case, D, dtype):
    Nq, Nk, qp, kp, causal = case
    say(f"[partial] Nq={Nq} Nk={Nk} q_pos={qp} k_pos={kp} causal={causal} D={D} {dtype}")
    vals, devs = _draw_blocks(500 + Nq + Nk, 1, 2, Nq, Nk, D, dtype)
    scale = 1.0 / np.sqrt(D)
    o, lse = fa.forward_partial(devs["q"], devs["k"], devs["v"], scale, causal, qp, kp)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_fwd_partial(vals["q"], vals["k"], vals["v"], scale, causal, qp, kp)
    _check(o, lse, ro, rl, dtype, "partial")


@pytest.mark.parametrize("causal", [False, True])
def test_partial_at_equal_positions_is_fa_fwd(causal):
    """Nq = Nk and q_pos = k_pos run the same kernel with the same arguments
    as fa_fwd: identical bits."""
    vals, devs = _draw_blocks(77, 2, 4, 700, 700, 64, "bf16")
    o1, l1 = fa.forward(devs["q"], devs["k"], devs["v"], 0.125, causal)
    o2, l2 = fa.forward_partial(devs["q"], devs["k"], devs["v"], 0.125, causal, 12345, 12345)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("qp,kp", [(400, 0), (0, 300)])
def test_partial_many_heads(qp, kp, D):
    """Enough 256-row workgroups for the ping-pong kernel, with rows that see
    part of the block (q_pos 400) or, for the first 300 rows, nothing."""
    B, H, Nq, Nk = 1, 192, 600, 900
    say(f"[partial-many-heads] H={H} Nq={Nq} Nk={Nk} q_pos={qp} k_pos={kp} D={D}")
    vals, devs = _draw_blocks(900 + D + qp, B, H, Nq, Nk, D, "bf16")
    scale = 1.0 / np.sqrt(D)
    o, lse = fa.forward_partial(devs["q"], devs["k"], devs["v"], scale, True, qp, kp)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_fwd_partial(vals["q"], vals["k"], vals["v"], scale, True, qp, kp)
    _check(o, lse, ro, rl, "bf16", "partial pp")


# ------------------------------------------------------------------ merge

def _merge_inputs(seed, shape, dtype):
    B, H, N, D = shape
    oa, oa_raw = inputs.draw(seed, "oa", shape, dtype)
    ob, ob_raw = inputs.draw(seed, "ob", shape, dtype)
    la, _ = inputs.draw(seed, "la", (B, H, N), "f32", 3.0)
    lb, _ = inputs.draw(seed, "lb", (B, H, N), "f32", 3.0)
    i = np.arange(N)
    la[..., i % 7 == 0] = -np.inf    # rows empty in partial a
    lb[..., i % 11 == 0] = -np.inf   # rows empty in partial b (both at i % 77 == 0)
    oa[..., i % 7 == 0, :] = 0.0     # an empty partial has O = 0
    ob[..., i % 11 == 0, :] = 0.0
    oa_raw = inputs.round_to_dtype(oa.astype(np.float32), dtype)[1]
    ob_raw = inputs.round_to_dtype(ob.astype(np.float32), dtype)[1]
    return (oa.astype(np.float64), la.astype(np.float64), ob.astype(np.float64),
            lb.astype(np.float64), to_device(oa_raw, dtype),
            torch.from_numpy(np.ascontiguousarray(la)).cuda(), to_device(ob_raw, dtype),
            torch.from_numpy(np.ascontiguousarray(lb)).cuda())


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("N", [1, 77, 1000])
def test_merge_kernel(N, D, dtype):
    say(f"[merge] N={N} D={D} {dtype}")
    oa, la, ob, lb, d_oa, d_la, d_ob, d_lb = _merge_inputs(40 + N, (2, 3, N, D), dtype)
    fa.merge(d_oa, d_la, d_ob, d_lb)
    torch.cuda.synchronize()
    ro, rl = oracle.merge_partials(oa, la, ob, lb)
    o, lse = to_f64(d_oa), to_f64(d_la)
    empty = np.isneginf(rl)
    assert np.array_equal(np.isneginf(lse), empty)
    assert np.all(o[empty] == 0.0)
    eo, el = max_abs(o, ro), max_abs(lse[~empty], rl[~empty])
    say(f"    max abs O={eo:.2e} LSE={el:.2e}")
    assert eo <= TOL[dtype]["o"] and el <= 1e-5


def test_merge_with_itself():
    """Merging a result with itself keeps O (weights 1/2 each, exact) and
    adds ln 2 to the LSE; O_part may alias O."""
    oa, la, _, _, d_oa, d_la, _, _ = _merge_inputs(3, (1, 2, 300, 64), "bf16")
    before = d_oa.clone()
    fa.merge(d_oa, d_la, d_oa, d_la)
    torch.cuda.synchronize()
    assert torch.equal(d_oa, before)
    fin = np.isfinite(la)
    got = to_f64(d_la)
    assert np.all(np.isneginf(got[~fin]))
    assert max_abs(got[fin], la[fin] + np.log(2.0)) <= 1e-5


# ------------------------------------------------- split keys, merge blocks

def _split_attention(devs, scale, causal, q_cuts, k_cuts):
    """Attention over the whole sequence assembled from blocks: every query
    block attends to every key block it can see through fa_fwd_partial and
    the results are combined with fa_merge."""
    q, k, v = devs["q"], devs["k"], devs["v"]
    outs, lses = [], []
    for qa, qb in zip(q_cuts[:-1], q_cuts[1:]):
        qs = q[:, :, qa:qb].contiguous()
        acc = None
        for ka, kb in zip(k_cuts[:-1], k_cuts[1:]):
            if causal and ka > qb - 1:
                continue  # a block wholly in the future contributes nothing
            o, l = fa.forward_partial(qs, k[:, :, ka:kb].contiguous(), v[:, :, ka:kb].contiguous(),
                                      scale, causal, qa, ka)
            acc = (o, l) if acc is None else fa.merge(acc[0], acc[1], o, l)
        outs.append(acc[0])
        lses.append(acc[1])
    torch.cuda.synchronize()
    return torch.cat(outs, dim=2), torch.cat(lses, dim=2)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("cuts", [(0, 1024, 2048, 3072, 4096), (0, 1000, 2500, 4096)],
                         ids=["even4", "uneven3"])
def test_key_blocks_merge_to_full_attention(cuts, causal, D):
    say(f"[split-merge] cuts={cuts} causal={causal} D={D}")
    N = cuts[-1]
    vals, devs = _draw_blocks(4000 + D, 1, 4, N, N, D, "bf16")
    scale = 1.0 / np.sqrt(D)
    o, lse = _split_attention(devs, scale, causal, cuts, cuts)
    ro, rl = oracle.attention_fwd(vals["q"], vals["k"], vals["v"], scale, causal)
    eo, el = max_abs(to_f64(o), ro), max_abs(to_f64(lse), rl)
    say(f"    max abs O={eo:.2e} LSE={el:.2e}")
    assert eo <= TOL["bf16"]["o"] and el <= TOL["bf16"]["lse"]


def test_long_sequence_split_four_ways_subset():
    """The 65536-token causal workload (16 heads, D = 64) with its keys and
    queries split into four 16384-row blocks, as four devices would hold
    them; the assembled result is checked on seeded rows of every block."""
    w = inputs.WORKLOADS["c5"]
    say(f"[split-merge {w.name}]")
    vals, devs = _draw_blocks(w.seed, w.B, w.H, w.N, w.N, w.D, w.dtype, w.input_mult)
    cuts = tuple(range(0, w.N + 1, w.N // 4))
    o, lse = _split_attention(devs, w.scale, True, cuts, cuts)
    rows = inputs.check_row_subset(w)
    ro, rl = oracle.attention_fwd_rows(vals["q"], vals["k"], vals["v"], w.scale, True, rows)
    idx = torch.from_numpy(rows).to(o.device)
    got_o = to_f64(o[idx[:, 0], idx[:, 1], idx[:, 2]])
    eo, er, ok = o_ok(got_o, ro, "bf16")
    el = max_abs(to_f64(lse)[tuple(rows.T)], rl)
    say(f"    {len(rows)} rows: max abs O={eo:.2e} (rel-to-max {er:.2e}) LSE={el:.2e}")
    assert ok and el <= TOL["bf16"]["lse"]
