"""The oracle against its pins (CPU only)."""
import numpy as np
import pytest

import oracle
from tests import oracle_pins
from exact_io_aware_58_amd import inputs


def _fwd(q, k, v, scale, causal):
    return oracle.attention_fwd(q, k, v, scale, causal)


def _bwd(q, k, v, g, scale, causal):
    return oracle.attention_bwd(q, k, v, g, scale, causal)


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(_fwd, _bwd)


@pytest.mark.parametrize("pin", oracle_pins.PARTIAL_PINS, ids=lambda p: p.__name__)
def test_partial_pin(pin):
    pin(oracle.attention_fwd_partial, oracle.merge_partials)


def test_partial_at_equal_positions_is_plain_attention():
    rng = np.random.default_rng(7)
    q, k, v = (rng.standard_normal((1, 2, 9, 4)) for _ in range(3))
    for causal in (False, True):
        o, l = oracle.attention_fwd_partial(q, k, v, 0.5, causal, 3, 3)
        ro, rl = oracle.attention_fwd(q, k, v, 0.5, causal)
        np.testing.assert_allclose(o, ro, atol=1e-13, rtol=0)
        np.testing.assert_allclose(l, rl, atol=1e-13, rtol=0)


def test_pins_hold_with_small_row_blocks():
    """Row blocking is a memory device only: every pin holds when S is built
    two rows at a time."""
    f = lambda q, k, v, s, c: oracle.attention_fwd(q, k, v, s, c, block_rows=2)
    b = lambda q, k, v, g, s, c: oracle.attention_bwd(q, k, v, g, s, c, block_rows=2)
    for pin in oracle_pins.ALL_PINS:
        pin(f, b)


@pytest.mark.parametrize("causal", [False, True])
def test_row_subsets_match_full(causal):
    """The per-row entry points used at full size give the full-tensor values."""
    rng = np.random.default_rng(5)
    B, H, N, D = 2, 3, 37, 6
    q, k, v, g = (rng.standard_normal((B, H, N, D)) for _ in range(4))
    o, lse = oracle.attention_fwd(q, k, v, 0.4, causal, block_rows=8)
    dq, dk, dv = oracle.attention_bwd(q, k, v, g, 0.4, causal, block_rows=8)
    rows = np.array([(b, h, i) for b in range(B) for h in range(H) for i in (0, 1, 17, N - 1)])
    ro, rl = oracle.attention_fwd_rows(q, k, v, 0.4, causal, rows)
    rdq = oracle.attention_bwd_query_rows(q, k, v, g, 0.4, causal, rows)
    rdk, rdv = oracle.attention_bwd_key_rows(q, k, v, g, 0.4, causal, rows, block_rows=5)
    sel = tuple(rows.T)
    np.testing.assert_allclose(ro, o[sel], atol=1e-13, rtol=0)
    np.testing.assert_allclose(rl, lse[sel], atol=1e-13, rtol=0)
    np.testing.assert_allclose(rdq, dq[sel], atol=1e-13, rtol=0)
    np.testing.assert_allclose(rdk, dk[sel], atol=1e-13, rtol=0)
    np.testing.assert_allclose(rdv, dv[sel], atol=1e-13, rtol=0)


def test_row_stats_delta_is_rowsum_do_o():
    """Delta_i computed from the row statistics equals dO_i . O_i."""
    rng = np.random.default_rng(6)
    q, k, v, g = (rng.standard_normal((1, 2, 20, 4)) for _ in range(4))
    for causal in (False, True):
        o, lse = oracle.attention_fwd(q, k, v, 0.9, causal)
        l2, d2 = oracle.row_stats(q, k, v, g, 0.9, causal, 0, 1, block_rows=7)
        np.testing.assert_allclose(l2, lse[0, 1], atol=1e-13, rtol=0)
        np.testing.assert_allclose(d2, np.sum(o[0, 1] * g[0, 1], axis=-1), atol=1e-13, rtol=0)


def test_inputs_are_seeded_and_rounded():
    """The shared generator is deterministic and its bf16 values are exactly
    representable (round trip through the raw bits is the identity)."""
    a, abits = inputs.draw(3, "q", (4, 8), "bf16")
    b, bbits = inputs.draw(3, "q", (4, 8), "bf16")
    assert np.array_equal(abits, bbits)
    assert np.array_equal(inputs.bf16_bits_to_f32(inputs.round_bf16_bits(a)), a)
    # round-to-nearest-even on hand-picked bit patterns
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20], dtype=np.float32)
    got = inputs.bf16_bits_to_f32(inputs.round_bf16_bits(x))
    np.testing.assert_array_equal(got, np.array([1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7], np.float32))
    h, hraw = inputs.draw(3, "k", (4, 8), "f16")
    assert hraw.dtype == np.float16 and np.array_equal(hraw.astype(np.float32), h)


def test_check_rows_cover_tile_edges():
    for key in ("c4", "c5"):
        w = inputs.WORKLOADS[key]
        rows = inputs.check_row_subset(w)
        assert len(rows) == w.check_rows
        assert len({tuple(r) for r in rows}) == len(rows)
        for h in (0, w.H - 1):
            for i in (0, 63, 64, 127, 128, w.N - 1):
                assert any((r == (0, h, i)).all() for r in rows)
