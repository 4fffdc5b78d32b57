"""Python binding of libvdn_hybrid_attn.so, the gfx950 Video DeltaNet hybrid
video-to-video attention layer (see include/vdn_hybrid_attn.h for the ABI).

The binding only marshals arguments: it checks devices, dtypes, shapes and
contiguity, allocates outputs and the workspace with torch, and passes raw device
pointers and torch's current HIP stream to the C entry points.  Every step of the
computation runs in the library's HIP kernels; if the library is not built the
calls raise instead of computing anything another way.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libvdn_hybrid_attn.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP, ERR_TOO_LARGE = 0, -1, -2, -3, -4, -5
NOALLOC_SCRATCH_BYTES = 64 << 20          # VDN_NOALLOC_SCRATCH_BYTES
PREC_FP32, PREC_BF16, PREC_BF16_FP8QK, PREC_FP8 = 0, 1, 2, 3
PRECISIONS = {"fp32": PREC_FP32, "bf16": PREC_BF16, "bf16_fp8qk": PREC_BF16_FP8QK, "fp8": PREC_FP8}
SCHED_COLS = 13
STAGES = ("prep", "factor", "scan", "wprep", "attn", "combine", "readout", "quant", "proj")

# C signatures: (name, restype, argtypes)
_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t
_SIGS = {
    "vdn_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I]),
    "vdn_hybrid_attn": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _SZ, _P]),
    "vdn_workspace_bytes_mixed": (_SZ, [_I, _I, _I, _I, _I, _I]),
    "vdn_workspace_bytes_proj": (_SZ, [_I, _I, _I, _I, _I, _I]),
    "vdn_hybrid_attn_proj": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _SZ, _P]),
    "vdn_out_proj": (_I, [_P, _P, _I, _I, _I, _P, _P]),
    "vdn_hybrid_attn_noalloc": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P]),
    "vdn_hybrid_attn_mixed": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _SZ, _P]),
    "vdn_softmax_branch": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _SZ, _P]),
    "vdn_vda_states": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _SZ, _P]),
    "vdn_vda_linear": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _SZ, _P]),
    "vdn_fp8_quantize": (_I, [_P, _I, _I, _I, _I, ctypes.c_float, _P, _P, _P]),
    "vdn_schedule": (_I, [_I, ctypes.POINTER(ctypes.c_int), _I]),
    "vdn_set_stage_events": (_I, [_I, _P, _P]),
    "vdn_status_string": (ctypes.c_char_p, [_I]),
    "vdn_last_hip_error": (_I, []),
}
EXPORTS = tuple(_SIGS)

_lib = None


class VdnError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = load()
        msg = lib.vdn_status_string(status).decode()
        if status == ERR_HIP:
            msg += f" (hipError_t {lib.vdn_last_hip_error()})"
        super().__init__(f"{where}: {msg} [{status}]")
        self.status = status


def load(path: str | None = None):
    """Load the shared library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m hybrid_sparse_linear_chunked_amd.build`")
    lib = ctypes.CDLL(p)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def _check(status: int, where: str):
    if status != OK:
        raise VdnError(status, where)


def schedule(F: int) -> np.ndarray:
    """Frame partition table of the layer (host only): int32 [rows, 13]."""
    lib = load()
    n = lib.vdn_schedule(F, None, 0)
    if n < 0:
        raise VdnError(n, "vdn_schedule")
    buf = (ctypes.c_int * (n * SCHED_COLS))()
    lib.vdn_schedule(F, buf, n)
    return np.frombuffer(buf, dtype=np.int32).reshape(n, SCHED_COLS).copy()


def workspace_bytes(F: int, N: int, H: int, d: int, precision: int) -> int:
    return int(load().vdn_workspace_bytes(F, N, H, d, precision))


def workspace_bytes_mixed(F: int, N: int, T: int, H: int, d: int, precision: int) -> int:
    return int(load().vdn_workspace_bytes_mixed(F, N, T, H, d, precision))


# ------------------------------------------------------------------ torch side
def _torch():
    import torch
    return torch


def _precision_of(x, precision):
    torch = _torch()
    if precision is None:
        return PREC_FP32 if x.dtype == torch.float32 else PREC_BF16
    return PRECISIONS[precision] if isinstance(precision, str) else int(precision)


def _check_io(name, x, dtype, shape=None):
    torch = _torch()
    if not isinstance(x, torch.Tensor) or not x.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if x.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {x.dtype}")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(x.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(x.shape)}")


def _span(x):
    p = x.data_ptr()
    return p, p + x.numel() * x.element_size()


def _check_no_alias(what, x, **others):
    """Raise if tensor `x` shares memory with any of `others` (outputs must not
    alias inputs, and the workspace must alias neither)."""
    a0, a1 = _span(x)
    for name, y in others.items():
        if y is None:
            continue
        b0, b1 = _span(y)
        if a0 < b1 and b0 < a1:
            raise ValueError(f"{what} overlaps {name}: outputs and workspace must not alias inputs")


def _io_dtype(prec):
    torch = _torch()
    return torch.float32 if prec == PREC_FP32 else torch.bfloat16


def _stream():
    return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)


def _workspace(F, N, H, d, prec, device, workspace=None):
    torch = _torch()
    need = workspace_bytes(F, N, H, d, prec)
    if need == 0:
        raise VdnError(ERR_UNSUPPORTED, "vdn_workspace_bytes")
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < need:
            raise VdnError(ERR_WORKSPACE, "workspace")
        return workspace
    return torch.empty(need, dtype=torch.uint8, device=device)


def new_workspace(F, N, H, d, precision, device="cuda"):
    """A workspace tensor for repeated calls with this shape."""
    return _workspace(F, N, H, d, precision if isinstance(precision, int) else PRECISIONS[precision], device)


def hybrid_attn(q, k, v, beta, gate, precision=None, out=None, workspace=None):
    """O = O_soft + g (.) O_lin for q, k, v [F, N, H, d]; beta fp32 [F, H]; gate fp32 [H, d]."""
    torch = _torch()
    prec = _precision_of(q, precision)
    F, N, H, d = q.shape
    dt = _io_dtype(prec)
    for name, x in (("q", q), ("k", k), ("v", v)):
        _check_io(name, x, dt, (F, N, H, d))
    _check_io("beta", beta, torch.float32, (F, H))
    _check_io("gate", gate, torch.float32, (H, d))
    O = torch.empty_like(q) if out is None else out
    _check_io("out", O, dt, (F, N, H, d))
    ws = _workspace(F, N, H, d, prec, q.device, workspace)
    _check_no_alias("out", O, q=q, k=k, v=v, beta=beta, gate=gate, workspace=ws)
    _check_no_alias("workspace", ws, q=q, k=k, v=v, beta=beta, gate=gate)
    st = load().vdn_hybrid_attn(q.data_ptr(), k.data_ptr(), v.data_ptr(), beta.data_ptr(),
                                gate.data_ptr(), F, N, H, d, prec, O.data_ptr(), ws.data_ptr(),
                                ws.numel() * ws.element_size(), _stream())
    _check(st, "vdn_hybrid_attn")
    return O


def hybrid_attn_noalloc(q, k, v, beta, gate, precision=None, out=None):
    """hybrid_attn with the library's built-in scratch instead of a workspace: the
    call allocates nothing on the device beyond `out` (pass it to allocate
    nothing at all).  Shapes needing more than NOALLOC_SCRATCH_BYTES of workspace
    raise; concurrent calls on one GPU race (they share its scratch)."""
    torch = _torch()
    prec = _precision_of(q, precision)
    F, N, H, d = q.shape
    dt = _io_dtype(prec)
    for name, x in (("q", q), ("k", k), ("v", v)):
        _check_io(name, x, dt, (F, N, H, d))
    _check_io("beta", beta, torch.float32, (F, H))
    _check_io("gate", gate, torch.float32, (H, d))
    O = torch.empty_like(q) if out is None else out
    _check_io("out", O, dt, (F, N, H, d))
    _check_no_alias("out", O, q=q, k=k, v=v, beta=beta, gate=gate)
    st = load().vdn_hybrid_attn_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), beta.data_ptr(),
                                        gate.data_ptr(), F, N, H, d, prec, O.data_ptr(), _stream())
    _check(st, "vdn_hybrid_attn_noalloc")
    return O


def new_workspace_mixed(F, N, T, H, d, precision, device="cuda"):
    """A workspace tensor for repeated hybrid_attn_mixed calls with this shape."""
    prec = precision if isinstance(precision, int) else PRECISIONS[precision]
    need = workspace_bytes_mixed(F, N, T, H, d, prec)
    if need == 0:
        raise VdnError(ERR_UNSUPPORTED, "vdn_workspace_bytes_mixed")
    return _torch().empty(need, dtype=_torch().uint8, device=device)


def hybrid_attn_mixed(q, k, v, beta, gate, F, N, precision=None, out=None, workspace=None):
    """The layer with extra (text / audio) tokens: q, k, v [F*N + T, H, d], the
    F*N video tokens (frame-major) then T extra tokens; beta fp32 [F, H]; gate fp32
    [H, d].  Returns O of q's shape."""
    torch = _torch()
    prec = _precision_of(q, precision)
    L, H, d = q.shape
    T = L - F * N
    if T < 0:
        raise ValueError(f"q has {L} tokens, fewer than F*N = {F * N}")
    dt = _io_dtype(prec)
    for name, x in (("q", q), ("k", k), ("v", v)):
        _check_io(name, x, dt, (L, H, d))
    _check_io("beta", beta, torch.float32, (F, H))
    _check_io("gate", gate, torch.float32, (H, d))
    O = torch.empty_like(q) if out is None else out
    _check_io("out", O, dt, (L, H, d))
    need = workspace_bytes_mixed(F, N, T, H, d, prec)
    if need == 0:
        raise VdnError(ERR_UNSUPPORTED, "vdn_workspace_bytes_mixed")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    elif workspace.numel() * workspace.element_size() < need:
        raise VdnError(ERR_WORKSPACE, "workspace")
    _check_no_alias("out", O, q=q, k=k, v=v, beta=beta, gate=gate, workspace=workspace)
    _check_no_alias("workspace", workspace, q=q, k=k, v=v, beta=beta, gate=gate)
    st = load().vdn_hybrid_attn_mixed(q.data_ptr(), k.data_ptr(), v.data_ptr(), beta.data_ptr(),
                                      gate.data_ptr(), F, N, T, H, d, prec, O.data_ptr(),
                                      workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream())
    _check(st, "vdn_hybrid_attn_mixed")
    return O


def new_workspace_proj(F, N, H, d, D, precision, device="cuda"):
    """A workspace tensor for repeated hybrid_attn_proj calls with this shape."""
    prec = precision if isinstance(precision, int) else PRECISIONS[precision]
    need = int(load().vdn_workspace_bytes_proj(F, N, H, d, D, prec))
    if need == 0:
        raise VdnError(ERR_UNSUPPORTED, "vdn_workspace_bytes_proj")
    return _torch().empty(need, dtype=_torch().uint8, device=device)


def hybrid_attn_proj(q, k, v, beta, gate, Wp, precision=None, out=None, workspace=None):
    """Y = O_soft W_s^T + (g (.) O_lin) W_l^T: q, k, v bf16 [F, N, H, d]; Wp bf16
    [D, 2*H*d] = [W_s | W_l].  Returns Y bf16 [F*N, D]."""
    torch = _torch()
    prec = _precision_of(q, precision)
    F, N, H, d = q.shape
    D = Wp.shape[0]
    for name, x in (("q", q), ("k", k), ("v", v)):
        _check_io(name, x, torch.bfloat16, (F, N, H, d))
    _check_io("beta", beta, torch.float32, (F, H))
    _check_io("gate", gate, torch.float32, (H, d))
    _check_io("Wp", Wp, torch.bfloat16, (D, 2 * H * d))
    Y = torch.empty((F * N, D), dtype=torch.bfloat16, device=q.device) if out is None else out
    _check_io("out", Y, torch.bfloat16, (F * N, D))
    if workspace is None:
        workspace = new_workspace_proj(F, N, H, d, D, prec, device=q.device)
    wbytes = workspace.numel() * workspace.element_size()
    if wbytes < int(load().vdn_workspace_bytes_proj(F, N, H, d, D, prec)):
        raise VdnError(ERR_WORKSPACE, "workspace")
    _check_no_alias("out", Y, q=q, k=k, v=v, beta=beta, gate=gate, Wp=Wp, workspace=workspace)
    _check_no_alias("workspace", workspace, q=q, k=k, v=v, beta=beta, gate=gate, Wp=Wp)
    st = load().vdn_hybrid_attn_proj(q.data_ptr(), k.data_ptr(), v.data_ptr(), beta.data_ptr(), gate.data_ptr(),
                                     Wp.data_ptr(), F, N, H, d, D, prec, Y.data_ptr(), workspace.data_ptr(),
                                     wbytes, _stream())
    _check(st, "vdn_hybrid_attn_proj")
    return Y


def out_proj(A, B, out=None):
    """Y[M, N] = A[M, K] B[N, K]^T in bf16 (fp32 accumulation)."""
    torch = _torch()
    M, K = A.shape
    N = B.shape[0]
    _check_io("A", A, torch.bfloat16, (M, K))
    _check_io("B", B, torch.bfloat16, (N, K))
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=A.device) if out is None else out
    _check_io("out", Y, torch.bfloat16, (M, N))
    _check_no_alias("out", Y, A=A, B=B)
    _check(load().vdn_out_proj(A.data_ptr(), B.data_ptr(), M, K, N, Y.data_ptr(), _stream()), "vdn_out_proj")
    return Y


def softmax_branch(q, k, v, precision=None, out=None, workspace=None):
    prec = _precision_of(q, precision)
    F, N, H, d = q.shape
    dt = _io_dtype(prec)
    for name, x in (("q", q), ("k", k), ("v", v)):
        _check_io(name, x, dt, (F, N, H, d))
    O = _torch().empty_like(q) if out is None else out
    _check_io("out", O, dt, (F, N, H, d))
    ws = _workspace(F, N, H, d, prec, q.device, workspace)
    _check_no_alias("out", O, q=q, k=k, v=v, workspace=ws)
    _check_no_alias("workspace", ws, q=q, k=k, v=v)
    st = load().vdn_softmax_branch(q.data_ptr(), k.data_ptr(), v.data_ptr(), F, N, H, d, prec,
                                   O.data_ptr(), ws.data_ptr(), ws.numel() * ws.element_size(), _stream())
    _check(st, "vdn_softmax_branch")
    return O


def vda_states(k, v, beta, precision=None, workspace=None):
    """(S_fwd, S_bwd), each fp32 [C, H, d, d]."""
    torch = _torch()
    prec = _precision_of(k, precision)
    F, N, H, d = k.shape
    dt = _io_dtype(prec)
    _check_io("k", k, dt, (F, N, H, d))
    _check_io("v", v, dt, (F, N, H, d))
    _check_io("beta", beta, torch.float32, (F, H))
    C = (F + 4) // 5
    Sf = torch.empty((C, H, d, d), dtype=torch.float32, device=k.device)
    Sb = torch.empty_like(Sf)
    ws = _workspace(F, N, H, d, prec, k.device, workspace)
    _check_no_alias("workspace", ws, k=k, v=v, beta=beta)
    st = load().vdn_vda_states(k.data_ptr(), v.data_ptr(), beta.data_ptr(), F, N, H, d, prec,
                               Sf.data_ptr(), Sb.data_ptr(), ws.data_ptr(), ws.numel() * ws.element_size(), _stream())
    _check(st, "vdn_vda_states")
    return Sf, Sb


def vda_linear(q, S_fwd, S_bwd, precision=None, workspace=None):
    """Ungated O_lin [F, N, H, d]."""
    torch = _torch()
    prec = _precision_of(q, precision)
    F, N, H, d = q.shape
    C = (F + 4) // 5
    _check_io("q", q, _io_dtype(prec), (F, N, H, d))
    _check_io("S_fwd", S_fwd, torch.float32, (C, H, d, d))
    _check_io("S_bwd", S_bwd, torch.float32, (C, H, d, d))
    O = torch.empty_like(q)
    ws = _workspace(F, N, H, d, prec, q.device, workspace)
    _check_no_alias("workspace", ws, q=q, S_fwd=S_fwd, S_bwd=S_bwd)
    st = load().vdn_vda_linear(q.data_ptr(), S_fwd.data_ptr(), S_bwd.data_ptr(), F, N, H, d, prec,
                               O.data_ptr(), ws.data_ptr(), ws.numel() * ws.element_size(), _stream())
    _check(st, "vdn_vda_linear")
    return O


def fp8_quantize(x, prescale=1.0):
    """(codes uint8 [F, N, H, d], scale_exp int32 [H]) of a bf16 tensor: E4M3 codes
    of fp32(x * prescale) with per-head power-of-two scales 2^scale_exp."""
    torch = _torch()
    F, N, H, d = x.shape
    _check_io("x", x, torch.bfloat16)
    codes = torch.empty((F, N, H, d), dtype=torch.uint8, device=x.device)
    sexp = torch.empty((H,), dtype=torch.int32, device=x.device)
    st = load().vdn_fp8_quantize(x.data_ptr(), F, N, H, d, float(prescale), codes.data_ptr(), sexp.data_ptr(),
                                 _stream())
    _check(st, "vdn_fp8_quantize")
    return codes, sexp


def set_stage_events(stage: int, before=None, after=None):
    """Record torch.cuda.Event pairs around a stage's kernels (None, None stops)."""
    b = None if before is None else ctypes.c_void_p(before.cuda_event)
    a = None if after is None else ctypes.c_void_p(after.cuda_event)
    _check(load().vdn_set_stage_events(stage, b, a), "vdn_set_stage_events")
