"""ctypes binding of libfa.so (C ABI in include/fa.h).

Argument marshalling only: every step of attention runs in the library's HIP
kernels.  The raw entry points keep the C names and take integers (device
addresses, stream handles); ``forward``/``backward`` are conveniences that
allocate outputs with torch (device memory and streams are the only things
torch is used for) and pass ``tensor.data_ptr()`` and the current stream.

Loading fails loudly if the library has not been built: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_F32, FA_BF16, FA_F16 = 0, 1, 2
FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE, FA_ERR_HIP = 0, -1, -2, -3, -4
FA_KERNEL_FWD, FA_KERNEL_BWD_DELTA, FA_KERNEL_BWD_DKDV, FA_KERNEL_BWD_DQ = 0, 1, 2, 3
FA_KERNEL_MERGE = 4
FA_KERNEL_BWD_DKDV_DQ = 5
FA_KERNEL_COUNT = 6

# Every symbol include/fa.h declares, with (restype, argtypes).
_c_int, _c_size, _vp, _f = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
_ll = ctypes.c_longlong
SIGNATURES = {
    "fa_fwd": (_c_int, [_c_int] * 5 + [_f, _c_int] + [_vp] * 6),
    "fa_fwd_partial": (_c_int, [_c_int] * 6 + [_f, _c_int, _ll, _ll] + [_vp] * 6),
    "fa_merge": (_c_int, [_c_int] * 5 + [_vp] * 5),
    "fa_bwd_workspace_bytes": (_c_size, [_c_int] * 6),
    "fa_bwd": (_c_int, [_c_int] * 5 + [_f, _c_int] + [_vp] * 10 + [_c_size, _vp]),
    "fa_bwd_noalloc": (_c_int, [_c_int] * 5 + [_f, _c_int] + [_vp] * 10),
    "fa_bwd_noalloc_max_bytes": (_c_size, []),
    "fa_status_string": (ctypes.c_char_p, [_c_int]),
    "fa_version": (_c_int, []),
    "fa_timing_enable": (_c_int, [_c_int]),
    "fa_timing_read": (_c_int, [_c_int, ctypes.POINTER(ctypes.c_longlong),
                                ctypes.POINTER(ctypes.c_double),
                                ctypes.POINTER(ctypes.c_longlong)]),
    "fa_kernel_name": (ctypes.c_char_p, [_c_int]),
}


class FAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {fa_status_string(status)} ({status})")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                          "(the HIP library is the only compute path)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


# ---------------------------------------------------------------- raw C ABI

def fa_fwd(dtype, B, H, N, D, scale, causal, Q, K, V, O, LSE, stream) -> int:
    return _lib.fa_fwd(dtype, B, H, N, D, scale, int(causal), Q, K, V, O, LSE, stream)


def fa_fwd_partial(dtype, B, H, Nq, Nk, D, scale, causal, q_pos, k_pos, Q, K, V, O, LSE,
                   stream) -> int:
    return _lib.fa_fwd_partial(dtype, B, H, Nq, Nk, D, scale, int(causal), q_pos, k_pos,
                               Q, K, V, O, LSE, stream)


def fa_merge(dtype, B, H, N, D, O, LSE, O_part, LSE_part, stream) -> int:
    return _lib.fa_merge(dtype, B, H, N, D, O, LSE, O_part, LSE_part, stream)


def fa_bwd_workspace_bytes(dtype, B, H, N, D, causal) -> int:
    return _lib.fa_bwd_workspace_bytes(dtype, B, H, N, D, int(causal))


def fa_bwd(dtype, B, H, N, D, scale, causal, Q, K, V, O, dO, LSE, dQ, dK, dV,
           workspace, workspace_bytes, stream) -> int:
    return _lib.fa_bwd(dtype, B, H, N, D, scale, int(causal), Q, K, V, O, dO, LSE,
                       dQ, dK, dV, workspace, workspace_bytes, stream)


def fa_bwd_noalloc(dtype, B, H, N, D, scale, causal, Q, K, V, O, dO, LSE, dQ, dK, dV,
                   stream) -> int:
    return _lib.fa_bwd_noalloc(dtype, B, H, N, D, scale, int(causal), Q, K, V, O, dO, LSE,
                               dQ, dK, dV, stream)


def fa_bwd_noalloc_max_bytes() -> int:
    return _lib.fa_bwd_noalloc_max_bytes()


def fa_status_string(status: int) -> str:
    return _lib.fa_status_string(status).decode()


def fa_version() -> int:
    return _lib.fa_version()


def fa_timing_enable(on: bool) -> int:
    return _lib.fa_timing_enable(1 if on else 0)


def fa_timing_read(kernel_id: int):
    """(launches, total_ms, dropped) for one kernel id."""
    n, ms, dr = ctypes.c_longlong(), ctypes.c_double(), ctypes.c_longlong()
    rc = _lib.fa_timing_read(kernel_id, ctypes.byref(n), ctypes.byref(ms), ctypes.byref(dr))
    if rc != FA_OK:
        raise FAError(rc, "fa_timing_read")
    return n.value, ms.value, dr.value


def fa_kernel_name(kernel_id: int) -> str:
    return _lib.fa_kernel_name(kernel_id).decode()


# ---------------------------------------------------------------- torch helpers

def _dtype_code(t):
    import torch
    codes = {torch.float32: FA_F32, torch.bfloat16: FA_BF16, torch.float16: FA_F16}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return codes[t.dtype]


def _check_qkv(*ts):
    shape, dtype, dev = ts[0].shape, ts[0].dtype, ts[0].device
    for t in ts:
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("tensors must be contiguous device tensors")
        if t.shape != shape or t.dtype != dtype or t.device != dev:
            raise ValueError("tensors must share one (B, H, N, D) shape, dtype and device")
    if len(shape) != 4:
        raise ValueError("expected (B, H, N, D) tensors")
    return shape


def _check_out(t, like, name):
    """A caller-supplied output must be a contiguous device tensor of the
    input's shape and dtype on the same device (the kernels write every
    element of it)."""
    if (not t.is_cuda or not t.is_contiguous() or t.shape != like.shape
            or t.dtype != like.dtype or t.device != like.device):
        raise ValueError(f"{name} must be a contiguous {tuple(like.shape)} {like.dtype} tensor "
                         f"on {like.device}")


def _check_lse(t, B, H, N, like, name="lse"):
    import torch
    if (not t.is_cuda or not t.is_contiguous() or tuple(t.shape) != (B, H, N)
            or t.dtype != torch.float32 or t.device != like.device):
        raise ValueError(f"{name} must be a contiguous float32 ({B}, {H}, {N}) tensor on "
                         f"{like.device}")


def _stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


def forward(q, k, v, scale, causal=False, out=None, lse=None):
    """(O, LSE) for (B, H, N, D) tensors; LSE is float32 (B, H, N)."""
    import torch
    B, H, N, D = _check_qkv(q, k, v)
    if out is None:
        out = torch.empty_like(q)
    _check_out(out, q, "out")
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check_lse(lse, B, H, N, q)
    rc = fa_fwd(_dtype_code(q), B, H, N, D, float(scale), causal, q.data_ptr(), k.data_ptr(),
                v.data_ptr(), out.data_ptr(), lse.data_ptr(), _stream())
    if rc != FA_OK:
        raise FAError(rc, "fa_fwd")
    return out, lse


def forward_partial(q, k, v, scale, causal=False, q_pos=0, k_pos=0, out=None, lse=None):
    """(O, LSE) of (B, H, Nq, D) queries at positions q_pos.. over (B, H, Nk, D)
    keys/values at positions k_pos..; rows that see no key get O = 0, LSE = -inf."""
    import torch
    _check_qkv(k, v)
    if q.dim() != 4:
        raise ValueError("expected (B, H, Nq, D) queries")
    B, H, Nq, D = q.shape
    Nk = k.shape[2]
    if (not q.is_cuda or not q.is_contiguous() or q.dtype != k.dtype
            or tuple(k.shape) != (B, H, Nk, D)):
        raise ValueError("q must be a contiguous (B, H, Nq, D) device tensor matching k, v")
    if k.device != q.device:
        raise ValueError("q, k, v must be on one device")
    if out is None:
        out = torch.empty_like(q)
    _check_out(out, q, "out")
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    _check_lse(lse, B, H, Nq, q)
    rc = fa_fwd_partial(_dtype_code(q), B, H, Nq, Nk, D, float(scale), causal, int(q_pos),
                        int(k_pos), q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                        lse.data_ptr(), _stream())
    if rc != FA_OK:
        raise FAError(rc, "fa_fwd_partial")
    return out, lse


def merge(o, lse, o_part, lse_part):
    """Merges (o_part, lse_part) into (o, lse) in place and returns them."""
    _check_qkv(o, o_part)
    B, H, N, D = o.shape
    _check_lse(lse, B, H, N, o)
    _check_lse(lse_part, B, H, N, o, "lse_part")
    rc = fa_merge(_dtype_code(o), B, H, N, D, o.data_ptr(), lse.data_ptr(), o_part.data_ptr(),
                  lse_part.data_ptr(), _stream())
    if rc != FA_OK:
        raise FAError(rc, "fa_merge")
    return o, lse


def workspace_bytes(q, causal=False):
    B, H, N, D = q.shape
    return fa_bwd_workspace_bytes(_dtype_code(q), B, H, N, D, causal)


def backward(q, k, v, o, do, lse, scale, causal=False, dq=None, dk=None, dv=None,
             workspace=None):
    """(dQ, dK, dV) of sum(O * dO), recomputing P from LSE."""
    import torch
    B, H, N, D = _check_qkv(q, k, v, o, do)
    _check_lse(lse, B, H, N, q)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for t, name in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _check_out(t, q, name)
    need = workspace_bytes(q, causal)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if (not workspace.is_cuda or not workspace.is_contiguous()
            or workspace.device != q.device):
        raise ValueError("workspace must be a contiguous tensor on the inputs' device")
    rc = fa_bwd(_dtype_code(q), B, H, N, D, float(scale), causal, q.data_ptr(), k.data_ptr(),
                v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(), dq.data_ptr(),
                dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(),
                workspace.numel() * workspace.element_size(), _stream())
    if rc != FA_OK:
        raise FAError(rc, "fa_bwd")
    return dq, dk, dv


_attention_fn = None


def _attention_function():
    """The torch.autograd.Function behind attention(), built on first use
    (torch is imported lazily, like everywhere in this module)."""
    global _attention_fn
    if _attention_fn is None:
        import torch

        class _Attention(torch.autograd.Function):
            @staticmethod
            def forward(ctx, q, k, v, scale, causal):
                o, lse = forward(q, k, v, scale, causal)
                ctx.save_for_backward(q, k, v, o, lse)
                ctx.scale, ctx.causal = scale, causal
                return o

            @staticmethod
            def backward(ctx, do):
                q, k, v, o, lse = ctx.saved_tensors
                dq, dk, dv = backward(q, k, v, o, do.contiguous(), lse, ctx.scale, ctx.causal)
                return dq, dk, dv, None, None

        _attention_fn = _Attention
    return _attention_fn


def attention(q, k, v, scale=None, causal=False):
    """O = softmax(scale Q K^T) V for (B, H, N, D) contiguous device tensors,
    differentiable through torch autograd: the forward runs fa_fwd and keeps
    Q, K, V, O and LSE; the backward runs fa_bwd on the incoming dO (16-bit
    dtypes; the fp32 path is forward only).  scale defaults to 1/sqrt(D)."""
    if scale is None:
        scale = q.shape[-1] ** -0.5
    return _attention_function().apply(q, k, v, float(scale), bool(causal))

