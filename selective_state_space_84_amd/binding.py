"""ctypes binding of the gfx950 selective-scan library (libssm_scan.so).

Argument marshalling only: the functions here check tensor placement,
allocate outputs or workspace when the caller passes none, and hand raw device
pointers and the current HIP stream to the C ABI declared in
``include/ssm_scan.h``.  Every step of the computation runs in the library's
kernels.  There is no fallback: if the library is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libssm_scan.so")

SSM_DTYPE_F32 = 0
SSM_DTYPE_BF16 = 1
SSM_FLAG_DELTA_SOFTPLUS = 0x1
SSM_FLAG_EXACT_ZOH = 0x2
SSM_FLAG_A_LINEAR_N = 0x4

SSM_OK = 0
SSM_ERR_NULL_ARG = -1
SSM_ERR_BAD_DIM = -2
SSM_ERR_UNSUPPORTED = -3
SSM_ERR_MISALIGNED = -4
SSM_ERR_WORKSPACE = -5
SSM_ERR_HIP = -6
SSM_ERR_ALIAS = -7

# Every symbol the header declares, with its ctypes signature.
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_U32 = ctypes.c_uint32
_SZ = ctypes.c_size_t


class ScanOpts(ctypes.Structure):
    """Mirror of ssm_scan_opts_t."""
    _fields_ = [("n_split", ctypes.c_int32), ("reserved0", ctypes.c_int32), ("chunk_len", ctypes.c_int64),
                ("flags", ctypes.c_uint32), ("reserved1", ctypes.c_uint32), ("dt_bias", ctypes.c_void_p),
                ("ckpt_out", ctypes.c_void_p)]


SIGNATURES = {
    "ssm_abi_version": ([], ctypes.c_int),
    "ssm_strerror": ([ctypes.c_int], ctypes.c_char_p),
    "ssm_scan_fwd_workspace_size": ([_I64, _I64, _I64, _I64], _SZ),
    "ssm_scan_fwd_ex_workspace_size": ([_I64, _I64, _I64, _I64, ctypes.POINTER(ScanOpts)], _SZ),
    "ssm_scan_fwd_plan": ([_I64, _I64, _I64, _I64, ctypes.POINTER(ScanOpts), ctypes.POINTER(_I32),
                           ctypes.POINTER(_I64), ctypes.POINTER(_I64)], ctypes.c_int),
    "ssm_scan_fwd": ([_P] * 10 + [_I64] * 4 + [_I32, _P, _SZ, _P], ctypes.c_int),
    "ssm_scan_fwd_ex": ([_P] * 10 + [_I64] * 4 + [_I32, ctypes.POINTER(ScanOpts), _P, _SZ, _P], ctypes.c_int),
    "ssm_scan_fwd_noalloc": ([_P] * 10 + [_I64] * 4 + [_I32, ctypes.POINTER(ScanOpts), _P], ctypes.c_int),
    "ssm_scan_fwd_noalloc_max_bytes": ([], _SZ),
    "ssm_state_update": ([_P] * 9 + [_I64] * 3 + [_I32, _P], ctypes.c_int),
    "ssm_state_update_ex": ([_P] * 9 + [_I64] * 3 + [_I32, _U32, _P, _P], ctypes.c_int),
    "ssm_scan_bwd_workspace_size": ([_I64, _I64, _I64, _I64], _SZ),
    "ssm_scan_bwd_workspace_size_ex": ([_I64, _I64, _I64, _I64, _I32], _SZ),
    "ssm_scan_ckpt_bytes": ([_I64, _I64, _I64, _I64], _SZ),
    "ssm_scan_bwd": ([_P] * 21 + [_I64] * 4 + [_I32, _U32, _P, _SZ, _P], ctypes.c_int),
    "ssm_ssd_fwd": ([_P] * 10 + [_I64] * 6 + [_I32, _U32, _P, _P], ctypes.c_int),
    "ssm_conv1d_fwd": ([_P] * 6 + [_I64] * 4 + [_I32, _I32, _P], ctypes.c_int),
    "ssm_conv1d_update": ([_P] * 5 + [_I64] * 3 + [_I32, _I32, _P], ctypes.c_int),
}

_lib = None


class SsmError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s failed: %s (%d)" % (what, strerror(status), status))


def load_library(path: Optional[str] = None):
    """Load libssm_scan.so (built in-tree by build_lib.build()); raises if absent."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError("libssm_scan.so is not built (%s); run python -m selective_state_space_84_amd.build_lib" % p)
    lib = ctypes.CDLL(p)
    for name, (args, res) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    if path is None:
        _lib = lib
    return lib


def abi_version() -> int:
    return load_library().ssm_abi_version()


def strerror(status: int) -> str:
    return load_library().ssm_strerror(status).decode()


def _opts(n_split=0, chunk_len=0, flags=0, dt_bias=None, ckpt_out=None) -> ScanOpts:
    return ScanOpts(n_split, 0, chunk_len, flags, 0, _ptr(dt_bias), _ptr(ckpt_out))


def scan_ckpt_bytes(batch, seqlen, d_inner, d_state) -> int:
    """Bytes of the block-start state checkpoints a forward call can save."""
    n = load_library().ssm_scan_ckpt_bytes(batch, seqlen, d_inner, d_state)
    if n == ctypes.c_size_t(-1).value:
        raise SsmError(SSM_ERR_BAD_DIM, "ssm_scan_ckpt_bytes")
    return n


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr() or None


def _io_dtype(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return SSM_DTYPE_BF16
    if t.dtype == torch.float32:
        return SSM_DTYPE_F32
    raise ValueError("io tensors must be bfloat16 or float32, got %s" % t.dtype)


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream or None
    if isinstance(stream, int):
        return stream or None
    return stream.cuda_stream or None


def scan_plan(batch, seqlen, d_inner, d_state, n_split=0, chunk_len=0, flags=0) -> Tuple[int, int, int]:
    """(n_split, chunk_len, n_chunks) the library launches for these sizes."""
    g = _I32()
    cl = _I64()
    nc = _I64()
    o = _opts(n_split, chunk_len, flags)
    rc = load_library().ssm_scan_fwd_plan(batch, seqlen, d_inner, d_state, ctypes.byref(o), ctypes.byref(g),
                                          ctypes.byref(cl), ctypes.byref(nc))
    if rc != SSM_OK:
        raise SsmError(rc, "ssm_scan_fwd_plan")
    return g.value, cl.value, nc.value


def scan_workspace_size(batch, seqlen, d_inner, d_state, n_split=0, chunk_len=0, flags=0) -> int:
    o = _opts(n_split, chunk_len, flags)
    n = load_library().ssm_scan_fwd_ex_workspace_size(batch, seqlen, d_inner, d_state, ctypes.byref(o))
    if n == ctypes.c_size_t(-1).value:
        raise SsmError(SSM_ERR_BAD_DIM, "ssm_scan_fwd_ex_workspace_size")
    return n


def ssm_scan_fwd(x, delta, A, B, C, D=None, z=None, h0=None, *, y=None, h_last=None, want_h_last=True,
                 workspace=None, n_split=0, chunk_len=0, flags=0, dt_bias=None, ckpt_out=None, stream=None):
    """Selective scan over the sequence; returns (y, h_last).

    x, delta, z: (batch, seqlen, d_inner); A: (d_inner, d_state) fp32;
    B, C: (batch, seqlen, d_state); D: (d_inner,) fp32; h0: (batch, d_inner, d_state) fp32.
    io tensors are all bfloat16 or all float32.  Outputs are allocated when not given.
    ckpt_out: optional fp32 buffer of scan_ckpt_bytes() bytes that receives the
    state before every 8-step block (for ssm_scan_bwd(ckpt=...)).
    """
    import torch
    batch, seqlen, d_inner = x.shape
    d_state = A.shape[1]
    dt = _io_dtype(x)
    if y is None:
        y = torch.empty_like(x)
    if h_last is None and want_h_last:
        h_last = torch.empty((batch, d_inner, d_state), dtype=torch.float32, device=x.device)
    ws_bytes = scan_workspace_size(batch, seqlen, d_inner, d_state, n_split, chunk_len, flags)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device)
    ws_have = 0 if workspace is None else workspace.numel() * workspace.element_size()
    o = _opts(n_split, chunk_len, flags, dt_bias, ckpt_out)
    rc = load_library().ssm_scan_fwd_ex(
        _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0), _ptr(y), _ptr(h_last),
        batch, seqlen, d_inner, d_state, dt, ctypes.byref(o), _ptr(workspace), ws_have, _stream(stream))
    if rc != SSM_OK:
        raise SsmError(rc, "ssm_scan_fwd")
    return y, h_last


def ssm_scan_fwd_noalloc(x, delta, A, B, C, D=None, z=None, h0=None, *, y, h_last=None, n_split=0, chunk_len=0,
                         flags=0, dt_bias=None, stream=None):
    """ssm_scan_fwd without a workspace: the library's per-device scratch holds
    the chunk carries and nothing is allocated (y and h_last must be given)."""
    batch, seqlen, d_inner = x.shape
    d_state = A.shape[1]
    o = _opts(n_split, chunk_len, flags, dt_bias, None)
    rc = load_library().ssm_scan_fwd_noalloc(
        _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0), _ptr(y), _ptr(h_last),
        batch, seqlen, d_inner, d_state, _io_dtype(x), ctypes.byref(o), _stream(stream))
    if rc != SSM_OK:
        raise SsmError(rc, "ssm_scan_fwd_noalloc")
    return y, h_last


def ssm_state_update(h, x_t, delta_t, A, B_t, C_t, D=None, z_t=None, *, y_t=None, flags=0, dt_bias=None,
                     stream=None):
    """One decode step, in place on h (batch, d_inner, d_state) fp32; returns y_t."""
    import torch
    batch, d_inner, d_state = h.shape
    dt = _io_dtype(x_t)
    if y_t is None:
        y_t = torch.empty_like(x_t)
    rc = load_library().ssm_state_update_ex(
        _ptr(h), _ptr(x_t), _ptr(delta_t), _ptr(A), _ptr(B_t), _ptr(C_t), _ptr(D), _ptr(z_t), _ptr(y_t),
        batch, d_inner, d_state, dt, flags, _ptr(dt_bias), _stream(stream))
    if rc != SSM_OK:
        raise SsmError(rc, "ssm_state_update")
    return y_t


def scan_bwd_workspace_size(batch, seqlen, d_inner, d_state, ckpt_given=False) -> int:
    """Backward workspace bytes; smaller when the forward call's checkpoints are passed."""
    n = load_library().ssm_scan_bwd_workspace_size_ex(batch, seqlen, d_inner, d_state, 1 if ckpt_given else 0)
    if n == ctypes.c_size_t(-1).value:
        raise SsmError(SSM_ERR_BAD_DIM, "ssm_scan_bwd_workspace_size_ex")
    return n


def ssm_scan_bwd(x, delta, A, B, C, D=None, z=None, h0=None, *, dy, dh_last=None, flags=0, dt_bias=None,
                 ckpt=None, want_dh0=True, grads=None, workspace=None, stream=None):
    """Gradient of ssm_scan_fwd for L = sum(dy * y) + sum(dh_last * h_last).

    ckpt: optional checkpoints saved by the forward call (ssm_scan_fwd(ckpt_out=...)).

    Returns a dict with dx, ddelta (w.r.t. the delta argument as passed), dA,
    dB, dC (fp32), and dD, dz, dh0, d_dt_bias when D, z, want_dh0, the softplus
    flag are used.  Outputs are allocated unless given in ``grads``.
    """
    import torch
    batch, seqlen, d_inner = x.shape
    d_state = A.shape[1]
    dt = _io_dtype(x)
    dev = x.device
    g = dict(grads or {})
    f32 = dict(dtype=torch.float32, device=dev)
    if "dx" not in g:
        g["dx"] = torch.empty_like(x)
    if "ddelta" not in g:
        g["ddelta"] = torch.empty_like(x)
    if "dA" not in g:
        g["dA"] = torch.empty((d_inner, d_state), **f32)
    if "dB" not in g:
        g["dB"] = torch.empty((batch, seqlen, d_state), **f32)
    if "dC" not in g:
        g["dC"] = torch.empty((batch, seqlen, d_state), **f32)
    if D is not None and "dD" not in g:
        g["dD"] = torch.empty((d_inner,), **f32)
    if z is not None and "dz" not in g:
        g["dz"] = torch.empty_like(x)
    if want_dh0 and "dh0" not in g:
        g["dh0"] = torch.empty((batch, d_inner, d_state), **f32)
    if (flags & SSM_FLAG_DELTA_SOFTPLUS) and "d_dt_bias" not in g:
        g["d_dt_bias"] = torch.empty((d_inner,), **f32)
    ws_bytes = scan_bwd_workspace_size(batch, seqlen, d_inner, d_state, ckpt_given=ckpt is not None)
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ws_have = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = load_library().ssm_scan_bwd(
        _ptr(x), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0), _ptr(dt_bias), _ptr(dy),
        _ptr(dh_last), _ptr(ckpt), _ptr(g["dx"]), _ptr(g["ddelta"]), _ptr(g["dA"]), _ptr(g["dB"]), _ptr(g["dC"]),
        _ptr(g.get("dD")), _ptr(g.get("dz")), _ptr(g.get("dh0")), _ptr(g.get("d_dt_bias")), batch, seqlen, d_inner,
        d_state, dt, flags, _ptr(workspace), ws_have, _stream(stream))
    if rc != SSM_OK:
        raise SsmError(rc, "ssm_scan_bwd")
    return g


def ssm_ssd_fwd(x, dt, A, B, C, D=None, z=None, h0=None, *, y=None, h_last=None, want_h_last=True, flags=0,
                dt_bias=None, stream=None):
    """Scan with a scalar decay per head (Mamba-2 / SSD form); returns (y, h_last).

    x, z: (batch, seqlen, nheads, 64) bf16; dt: (batch, seqlen, nheads) bf16;
    A, D, dt_bias: (nheads,) fp32; B, C: (batch, seqlen, ngroups, d_state) bf16;
    h0: (batch, nheads, 64, d_state) fp32.
    """
    import torch
    batch, seqlen, nheads, headdim = x.shape
    ngroups, d_state = B.shape[2], B.shape[3]
    if y is None:
        y = torch.empty_like(x)
    if h_last is None and want_h_last:
        h_last = torch.empty((batch, nheads, headdim, d_state), dtype=torch.float32, device=x.device)
    rc = load_library().ssm_ssd_fwd(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(h0),
                                    _ptr(y), _ptr(h_last), batch, seqlen, nheads, headdim, ngroups, d_state,
                                    _io_dtype(x), flags, _ptr(dt_bias), _stream(stream))
    if rc != SSM_OK:
        raise SsmError(rc, "ssm_ssd_fwd")
    return y, h_last


def ssm_conv1d_fwd(x, w, bias=None, state_in=None, *, y=None, state_out=None, want_state=True, silu=True,
                   stream=None):
    """Causal depthwise conv1d (+ SiLU); returns (y, state_out).

    x: (batch, seqlen, d_inner) bf16/fp32; w: (d_inner, d_conv) fp32;
    bias: (d_inner,) fp32; state_in / state_out: (batch, d_inner, d_conv-1) fp32.
    """
    import torch
    batch, seqlen, d_inner = x.shape
    d_conv = w.shape[1]
    if y is None:
        y = torch.empty_like(x)
    if state_out is None and want_state:
        state_out = torch.empty((batch, d_inner, d_conv - 1), dtype=torch.float32, device=x.device)
    rc = load_library().ssm_conv1d_fwd(_ptr(x), _ptr(w), _ptr(bias), _ptr(state_in), _ptr(y), _ptr(state_out),
                                       batch, seqlen, d_inner, d_conv, _io_dtype(x), 1 if silu else 0,
                                       _stream(stream))
    if rc != SSM_OK:
        raise SsmError(rc, "ssm_conv1d_fwd")
    return y, state_out


def ssm_conv1d_update(state, x_t, w, bias=None, *, y_t=None, silu=True, stream=None):
    """One decode step of the conv, in place on state (batch, d_inner, d_conv-1); returns y_t."""
    import torch
    batch, d_inner = x_t.shape
    d_conv = w.shape[1]
    if y_t is None:
        y_t = torch.empty_like(x_t)
    rc = load_library().ssm_conv1d_update(_ptr(state), _ptr(x_t), _ptr(w), _ptr(bias), _ptr(y_t), batch, d_inner,
                                          d_conv, _io_dtype(x_t), 1 if silu else 0, _stream(stream))
    if rc != SSM_OK:
        raise SsmError(rc, "ssm_conv1d_update")
    return y_t
