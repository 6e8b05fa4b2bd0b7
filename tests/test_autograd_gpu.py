"""fa.attention: the autograd wrapper over fa_fwd / fa_bwd.  Its output and
gradients are the C ABI's own (bit for bit: the wrapper only marshals), and
it takes part in an ordinary torch graph (a loss built on its output)."""
import pytest

from tests.gpu_util import draw_case, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
def test_autograd_matches_the_c_abi(causal, D):
    from exact_io_aware_58_amd import fa
    say(f"[autograd] D={D} causal={causal}")
    shape = (2, 3, 333, D)
    vals, devs = draw_case(700 + D + causal, shape, "bf16", grad=True)
    q, k, v, do = devs["q"], devs["k"], devs["v"], devs["do"]
    scale = D ** -0.5
    o_ref, lse = fa.forward(q, k, v, scale, causal)
    dq_ref, dk_ref, dv_ref = fa.backward(q, k, v, o_ref, do, lse, scale, causal)

    qg, kg, vg = (t.detach().clone().requires_grad_(True) for t in (q, k, v))
    o = fa.attention(qg, kg, vg, causal=causal)  # default scale 1/sqrt(D)
    # the same dO through an ordinary loss: d(sum(O * dO))/dO = dO
    (o.float() * do.float()).sum().backward()
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o_ref)
    assert torch.equal(qg.grad, dq_ref)
    assert torch.equal(kg.grad, dk_ref)
    assert torch.equal(vg.grad, dv_ref)
