"""fa_bwd_noalloc through the C ABI: the backward with its row statistics in
the library's fixed per-GPU scratch instead of a caller workspace must give
exactly what fa_bwd gives (same kernels), on two calls in a row, the second
on a smaller problem (the scratch keeps the first call's contents)."""
import numpy as np
import pytest

from tests.gpu_util import draw_case, rel_to_max, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

from exact_io_aware_58_amd import fa  # noqa: E402

import oracle  # noqa: E402


def _run_both(shape, causal, seed):
    B, H, N, D = shape
    vals, devs = draw_case(seed, shape, "bf16", grad=True)
    q, k, v, do = devs["q"], devs["k"], devs["v"], devs["do"]
    scale = 1.0 / np.sqrt(D)
    o, lse = fa.forward(q, k, v, scale, causal)
    ref = fa.backward(q, k, v, o, do, lse, scale, causal)
    got = [torch.full_like(q, float("nan")) for _ in range(3)]
    sh = torch.cuda.current_stream().cuda_stream
    rc = fa.fa_bwd_noalloc(fa.FA_BF16, B, H, N, D, scale, causal, q.data_ptr(), k.data_ptr(),
                           v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                           got[0].data_ptr(), got[1].data_ptr(), got[2].data_ptr(), sh)
    assert rc == fa.FA_OK, fa.fa_status_string(rc)
    torch.cuda.synchronize()
    return vals, ref, got, scale


def test_noalloc_backward_matches_fa_bwd_twice():
    cases = [((2, 8, 1000, 64), True, 901), ((1, 4, 300, 128), False, 902)]
    for shape, causal, seed in cases:  # the second call is the smaller problem
        say(f"[noalloc] shape={shape} causal={causal}")
        vals, ref, got, scale = _run_both(shape, causal, seed)
        for name, r, g in zip(("dQ", "dK", "dV"), ref, got):
            assert torch.equal(r, g), f"{name} differs from fa_bwd"
        rq, rk, rv = oracle.attention_bwd(vals["q"], vals["k"], vals["v"], vals["do"], scale,
                                          causal)
        errs = [rel_to_max(g.float().cpu().numpy().astype(np.float64), r)
                for g, r in zip(got, (rq, rk, rv))]
        say(f"    bit-identical to fa_bwd; rel-to-max vs oracle {errs}")
        assert max(errs) <= 5e-2


def test_noalloc_rejects_problems_beyond_its_scratch():
    cap = fa.fa_bwd_noalloc_max_bytes()
    # 2^22 rows fill the scratch exactly; one more row of heads does not fit
    B, H, N, D = 1, 65, 65536, 64
    assert fa.fa_bwd_workspace_bytes(fa.FA_BF16, B, H, N, D, 1) > cap
    t = torch.empty(16, dtype=torch.uint8, device="cuda")
    p = t.data_ptr()
    rc = fa.fa_bwd_noalloc(fa.FA_BF16, B, H, N, D, 0.125, 1, p, p, p, p, p, p, p, p, p,
                           torch.cuda.current_stream().cuda_stream)
    assert rc == fa.FA_ERR_WORKSPACE
