"""The C-ABI library without a GPU: it loads, exports every symbol the header
declares, and rejects bad arguments before making any HIP call."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")
LIB = os.path.join(ROOT, "exact_io_aware_58_amd", "libfa.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libfa.so not built")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_api():
    assert {"fa_fwd", "fa_bwd", "fa_bwd_workspace_bytes", "fa_status_string", "fa_fwd_partial",
            "fa_merge"} <= set(_declared())


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    missing = [s for s in _declared() if s not in exported]
    assert not missing, missing


def test_binding_names_match_header():
    from exact_io_aware_58_amd import fa
    assert sorted(fa.SIGNATURES) == _declared()
    for name in _declared():
        assert callable(getattr(fa, name))


@pytest.fixture(scope="module")
def fa():
    from exact_io_aware_58_amd import fa as mod
    return mod


A = 0x10000  # aligned fake device addresses: validation rejects before any use
P = [A + 0x1000 * i for i in range(12)]


def test_version_and_status_strings(fa):
    assert fa.fa_version() >= 4
    for code in (0, -1, -2, -3, -4):
        assert fa.fa_status_string(code) != "unknown status"
    assert fa.fa_status_string(99) == "unknown status"


@pytest.mark.parametrize("args,status", [
    (dict(dtype=7), -2),
    (dict(D=96), -2),
    (dict(D=32), -2),
    (dict(B=0), -1),
    (dict(H=-1), -1),
    (dict(N=0), -1),
    (dict(N=1 << 25), -1),
    (dict(B=1 << 10, H=1 << 10, N=1 << 11), -1),  # B*H*N > 2^30
    (dict(B=1, H=1 << 23, N=1), -1),   # B*H*ceil(N/64) = 2^23: a grid of 2^32 work-items
    (dict(B=1 << 12, H=1 << 11, N=64), -1),
    (dict(B=1 << 10, H=1 << 10, N=520), -1),  # 2^20 heads x 9 padded 64-row blocks
    (dict(scale=0.0), -1),
    (dict(scale=-0.125), -1),
    (dict(scale=float("inf")), -1),
    (dict(scale=float("nan")), -1),
    (dict(scale=2.0 ** -33), -1),  # scale * log2(e) must stay a normal fp32
    (dict(scale=2.0 ** 33), -1),
    (dict(scale=1e-45), -1),       # fp32 denormal
])
def test_fwd_rejects_bad_problem(fa, args, status):
    kw = dict(dtype=fa.FA_BF16, B=1, H=2, N=128, D=64, scale=0.125)
    kw.update(args)
    rc = fa.fa_fwd(kw["dtype"], kw["B"], kw["H"], kw["N"], kw["D"], kw["scale"], 0,
                   P[0], P[1], P[2], P[3], P[4], None)
    assert rc == status


@pytest.mark.parametrize("which", range(5))
@pytest.mark.parametrize("bad", [0, A + 8])
def test_fwd_rejects_null_or_misaligned(fa, which, bad):
    ptrs = P[:5]
    ptrs[which] = bad
    assert fa.fa_fwd(fa.FA_BF16, 1, 2, 128, 64, 0.125, 0, *ptrs, None) == fa.FA_ERR_INVALID_ARG


def test_workspace_bytes(fa):
    assert fa.fa_bwd_workspace_bytes(fa.FA_BF16, 8, 12, 1024, 64, 1) == 2 * 8 * 12 * 1024 * 4
    assert fa.fa_bwd_workspace_bytes(fa.FA_BF16, 1, 1, 3, 64, 0) == 2 * 256  # padded
    assert fa.fa_bwd_workspace_bytes(fa.FA_BF16, 1, 1, 3, 96, 0) == 0
    assert fa.fa_bwd_workspace_bytes(fa.FA_F32, 1, 1, 128, 64, 0) == 0


def _bwd(fa, dtype=None, ws_bytes=None, ws=P[10], ptr_over=None, D=64, N=128, scale=0.125):
    dtype = fa.FA_BF16 if dtype is None else dtype
    ptrs = P[:9]
    if ptr_over:
        ptrs[ptr_over[0]] = ptr_over[1]
    if ws_bytes is None:
        ws_bytes = fa.fa_bwd_workspace_bytes(fa.FA_BF16, 1, 2, N, 64, 0)
    return fa.fa_bwd(dtype, 1, 2, N, D, scale, 0, *ptrs, ws, ws_bytes, None)


def test_bwd_validation(fa):
    assert _bwd(fa, ws_bytes=16) == fa.FA_ERR_WORKSPACE
    assert _bwd(fa, ws=0) == fa.FA_ERR_WORKSPACE
    assert _bwd(fa, ws=A + 4) == fa.FA_ERR_INVALID_ARG
    assert _bwd(fa, dtype=fa.FA_F32) == fa.FA_ERR_UNSUPPORTED
    assert _bwd(fa, D=80) == fa.FA_ERR_UNSUPPORTED
    for bad in (0.0, 2.0 ** -33, 2.0 ** 33, float("nan")):
        assert _bwd(fa, scale=bad) == fa.FA_ERR_INVALID_ARG
    for i in range(9):
        assert _bwd(fa, ptr_over=(i, 0)) == fa.FA_ERR_INVALID_ARG
        assert _bwd(fa, ptr_over=(i, A + 2)) == fa.FA_ERR_INVALID_ARG


def test_timing_read_bounds(fa):
    with pytest.raises(fa.FAError):
        fa.fa_timing_read(fa.FA_KERNEL_COUNT)
    n, ms, dropped = fa.fa_timing_read(fa.FA_KERNEL_FWD)
    assert n == 0 and ms == 0.0 and dropped == 0
    assert [fa.fa_kernel_name(i) for i in range(fa.FA_KERNEL_COUNT)] == [
        "fwd", "bwd_delta", "bwd_dkdv", "bwd_dq", "merge", "bwd_dkdv_dq"]
    assert fa.fa_kernel_name(fa.FA_KERNEL_COUNT) == "unknown"


@pytest.mark.parametrize("args,status", [
    (dict(dtype=7), -2),
    (dict(D=96), -2),
    (dict(Nq=0), -1),
    (dict(Nk=0), -1),
    (dict(Nk=1 << 24), -1),
    (dict(Nq=1 << 24), -1),
    (dict(q_pos=-1), -1),
    (dict(k_pos=-5), -1),
    (dict(k_pos=(1 << 62) + 1), -1),
    (dict(scale=0.0), -1),
    (dict(scale=float("nan")), -1),
    (dict(scale=2.0 ** -40), -1),
])
def test_fwd_partial_rejects_bad_problem(fa, args, status):
    kw = dict(dtype=fa.FA_BF16, Nq=100, Nk=300, D=64, scale=0.125, q_pos=0, k_pos=0)
    kw.update(args)
    rc = fa.fa_fwd_partial(kw["dtype"], 1, 2, kw["Nq"], kw["Nk"], kw["D"], kw["scale"], 1,
                           kw["q_pos"], kw["k_pos"], P[0], P[1], P[2], P[3], P[4], None)
    assert rc == status


@pytest.mark.parametrize("which", range(5))
def test_fwd_partial_rejects_null_or_misaligned(fa, which):
    for bad in (0, A + 8):
        ptrs = P[:5]
        ptrs[which] = bad
        assert fa.fa_fwd_partial(fa.FA_BF16, 1, 2, 100, 300, 64, 0.125, 1, 0, 0, *ptrs,
                                 None) == fa.FA_ERR_INVALID_ARG


def test_merge_validation(fa):
    ok = (P[0], P[1], P[2], P[3])
    assert fa.fa_merge(7, 1, 2, 100, 64, *ok, None) == fa.FA_ERR_UNSUPPORTED
    assert fa.fa_merge(fa.FA_BF16, 1, 2, 100, 80, *ok, None) == fa.FA_ERR_UNSUPPORTED
    assert fa.fa_merge(fa.FA_BF16, 1, 0, 100, 64, *ok, None) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_merge(fa.FA_BF16, 1, 2, 0, 64, *ok, None) == fa.FA_ERR_INVALID_ARG
    for which in range(4):
        for bad in (0, A + 4):
            ptrs = list(ok)
            ptrs[which] = bad
            assert fa.fa_merge(fa.FA_F16, 1, 2, 100, 64, *ptrs, None) == fa.FA_ERR_INVALID_ARG


class _FakeTensor:
    """Stands in for a device tensor in the binding's argument checks (no
    GPU here): only the attributes the checks read."""

    def __init__(self, shape, dtype, cuda=True, contiguous=True, device="cuda:0"):
        self.shape, self.dtype, self.is_cuda, self.device = tuple(shape), dtype, cuda, device
        self._contiguous = contiguous

    def is_contiguous(self):
        return self._contiguous


def test_binding_rejects_bad_caller_outputs(fa):
    torch = pytest.importorskip("torch")
    q = _FakeTensor((1, 2, 64, 64), torch.bfloat16)
    fa._check_out(_FakeTensor(q.shape, q.dtype), q, "out")
    for bad in (_FakeTensor((1, 2, 32, 64), q.dtype), _FakeTensor(q.shape, torch.float16),
                _FakeTensor(q.shape, q.dtype, contiguous=False),
                _FakeTensor(q.shape, q.dtype, cuda=False, device="cpu"),
                _FakeTensor(q.shape, q.dtype, device="cuda:1")):
        with pytest.raises(ValueError):
            fa._check_out(bad, q, "out")
    fa._check_lse(_FakeTensor((1, 2, 64), torch.float32), 1, 2, 64, q)
    for bad in (_FakeTensor((1, 2, 64), torch.bfloat16), _FakeTensor((1, 2, 63), torch.float32),
                _FakeTensor((1, 2, 64), torch.float32, contiguous=False),
                _FakeTensor((1, 2, 64), torch.float32, device="cuda:1")):
        with pytest.raises(ValueError):
            fa._check_lse(bad, 1, 2, 64, q)


def test_noalloc_backward_validation(fa):
    """Argument checks of fa_bwd_noalloc happen before any HIP call."""
    cap = fa.fa_bwd_noalloc_max_bytes()
    assert cap == 32 << 20
    # the scratch holds the workspace of 2^22 rows and no more
    assert fa.fa_bwd_workspace_bytes(fa.FA_BF16, 1, 64, 65536, 64, 1) == cap
    assert fa.fa_bwd_workspace_bytes(fa.FA_BF16, 1, 65, 65536, 64, 1) > cap

    def call(dtype=fa.FA_BF16, H=2, N=128, D=64, scale=0.125, ptr_over=None):
        ptrs = P[:9]
        if ptr_over:
            ptrs[ptr_over[0]] = ptr_over[1]
        return fa.fa_bwd_noalloc(dtype, 1, H, N, D, scale, 0, *ptrs, None)

    assert call(H=65, N=65536) == fa.FA_ERR_WORKSPACE
    assert call(dtype=fa.FA_F32) == fa.FA_ERR_UNSUPPORTED
    assert call(D=80) == fa.FA_ERR_UNSUPPORTED
    assert call(scale=0.0) == fa.FA_ERR_INVALID_ARG
    for i in range(9):
        assert call(ptr_over=(i, 0)) == fa.FA_ERR_INVALID_ARG
        assert call(ptr_over=(i, A + 2)) == fa.FA_ERR_INVALID_ARG
