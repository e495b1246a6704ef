"""ctypes binding of libm3.so (include/m3.h).  Argument marshalling only.

Every call passes raw device pointers and the current HIP stream of the tensors'
device; all arithmetic runs in the library's HIP kernels.  There is no fallback:
if the library is missing or the tensors are not on a GPU the call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libm3.so")

M3_FP32, M3_BF16 = 0, 1
STATUS = {0: "M3_OK", 1: "M3_ERR_NULL", 2: "M3_ERR_SHAPE", 3: "M3_ERR_DTYPE",
          4: "M3_ERR_WORKSPACE", 5: "M3_ERR_DEVICE", 6: "M3_ERR_ALIAS", 7: "M3_ERR_TIMEOUT"}
EXPORTS = ("m3_prefill_workspace_bytes", "m3_prefill_chunk_used", "m3_prefill_max_chunk",
           "m3_prefill_gated_chunk_used", "m3_prefill_prologue_chunk_used", "m3_prefill_status",
           "m3_debug_set_spin_limit", "m3_scan_prefill", "m3_scan_prefill_noalloc",
           "m3_scan_backward", "m3_scan_backward_workspace_bytes",
           "m3_scan_prefill_gated", "m3_decode_step", "m3_decode_step_bf16_state",
           "m3_decode_step_gated", "m3_decode_step_prologue", "m3_scan_prefill_prologue",
           "m3_prefill_kernel_used", "m3_debug_set_prefill_kernel",
           "m3_prefill_prologue_mode", "m3_prefill_prologue_workspace_bytes", "m3_prefill_prologue_kernel_used",
           "m3_prefill_gated_kernel_used",
           "m3_status_str", "m3_version")
M3_KERNEL_PER_CHUNK, M3_KERNEL_STREAM = 1, 2
M3_PROLOGUE_FUSED, M3_PROLOGUE_STAGED = 1, 2


class M3Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seqlen", ctypes.c_int32),
                ("nheads", ctypes.c_int32), ("headdim", ctypes.c_int32),
                ("dstate", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class M3Prologue(ctypes.Structure):
    _fields_ = [("eps", ctypes.c_float), ("bias_B", ctypes.c_void_p), ("bias_C", ctypes.c_void_p)]


class M3Error(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


_lib = None


def load_library(path: str = LIB_PATH):
    """Loads libm3.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m state_space_sequence_02_amd.build`")
    lib = ctypes.CDLL(path)
    vp, fp, sz = ctypes.c_void_p, ctypes.POINTER(ctypes.c_float), ctypes.c_size_t
    sp = ctypes.POINTER(M3Shape)
    lib.m3_prefill_workspace_bytes.restype = sz
    lib.m3_prefill_workspace_bytes.argtypes = [sp]
    for fn in ("m3_prefill_chunk_used", "m3_prefill_max_chunk", "m3_prefill_gated_chunk_used",
               "m3_prefill_prologue_chunk_used"):
        getattr(lib, fn).restype = ctypes.c_int32
        getattr(lib, fn).argtypes = [sp]
    lib.m3_prefill_status.restype = ctypes.c_int
    lib.m3_prefill_status.argtypes = [vp, sz, vp]
    lib.m3_debug_set_spin_limit.restype = None
    lib.m3_debug_set_spin_limit.argtypes = [ctypes.c_uint32]
    lib.m3_prefill_kernel_used.restype = ctypes.c_int32
    lib.m3_prefill_kernel_used.argtypes = [sp]
    lib.m3_debug_set_prefill_kernel.restype = ctypes.c_int
    lib.m3_debug_set_prefill_kernel.argtypes = [ctypes.c_int32]
    lib.m3_scan_prefill.restype = ctypes.c_int
    lib.m3_scan_prefill.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.m3_scan_backward_workspace_bytes.restype = sz
    lib.m3_scan_backward_workspace_bytes.argtypes = [sp]
    lib.m3_scan_backward.restype = ctypes.c_int
    lib.m3_scan_backward.argtypes = [sp] + [vp] * 23 + [sz, vp]
    lib.m3_scan_prefill_noalloc.restype = ctypes.c_int
    lib.m3_scan_prefill_noalloc.argtypes = [sp] + [vp] * 13
    lib.m3_decode_step.restype = ctypes.c_int
    lib.m3_decode_step.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.m3_decode_step_bf16_state.restype = ctypes.c_int
    lib.m3_decode_step_bf16_state.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.m3_scan_prefill_gated.restype = ctypes.c_int
    lib.m3_scan_prefill_gated.argtypes = [sp] + [vp] * 16 + [sz, vp]
    lib.m3_decode_step_gated.restype = ctypes.c_int
    lib.m3_decode_step_gated.argtypes = [sp] + [vp] * 15
    lib.m3_prefill_prologue_mode.restype = ctypes.c_int32
    lib.m3_prefill_prologue_mode.argtypes = [sp]
    lib.m3_prefill_prologue_kernel_used.restype = ctypes.c_int32
    lib.m3_prefill_prologue_kernel_used.argtypes = [sp]
    lib.m3_prefill_gated_kernel_used.restype = ctypes.c_int32
    lib.m3_prefill_gated_kernel_used.argtypes = [sp]
    lib.m3_prefill_prologue_workspace_bytes.restype = sz
    lib.m3_prefill_prologue_workspace_bytes.argtypes = [sp]
    lib.m3_scan_prefill_prologue.restype = ctypes.c_int
    lib.m3_scan_prefill_prologue.argtypes = [sp, ctypes.POINTER(M3Prologue)] + [vp] * 13 + [sz, vp]
    lib.m3_decode_step_prologue.restype = ctypes.c_int
    lib.m3_decode_step_prologue.argtypes = [sp, ctypes.POINTER(M3Prologue)] + [vp] * 12
    lib.m3_status_str.restype = ctypes.c_char_p
    lib.m3_status_str.argtypes = [ctypes.c_int]
    lib.m3_version.restype = ctypes.c_int32
    lib.m3_version.argtypes = []
    _lib = lib
    return lib


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return M3_BF16
    if t.dtype == torch.float32:
        return M3_FP32
    raise TypeError(f"x/B/C must be float32 or bfloat16, got {t.dtype}")


def _ptr(t: Optional[torch.Tensor], dtype=None, device=None) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("all tensors must be on the GPU")
    if device is not None and t.device != device:
        raise ValueError(f"tensor on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _check(code: int):
    if code != 0:
        raise M3Error(code, load_library().m3_status_str(code).decode())


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def make_shape(batch, seqlen, nheads, headdim, dstate, rank, chunk=0, dtype=M3_BF16) -> M3Shape:
    return M3Shape(int(batch), int(seqlen), int(nheads), int(headdim), int(dstate), int(rank),
                   int(chunk), int(dtype))


def prefill_workspace_bytes(shape: M3Shape) -> int:
    return int(load_library().m3_prefill_workspace_bytes(ctypes.byref(shape)))


def prefill_chunk_used(shape: M3Shape, variant: str = "plain") -> int:
    """Chunk (tokens) the prefill entry point `variant` ("plain", "gated" or
    "prologue") uses for this shape; 0 when it refuses the shape."""
    fn = {"plain": "m3_prefill_chunk_used", "gated": "m3_prefill_gated_chunk_used",
          "prologue": "m3_prefill_prologue_chunk_used"}[variant]
    return int(getattr(load_library(), fn)(ctypes.byref(shape)))


def prefill_prologue_mode(shape: M3Shape) -> int:
    """m3_prefill_prologue_mode: M3_PROLOGUE_FUSED (1), M3_PROLOGUE_STAGED (2),
    or 0 when m3_scan_prefill_prologue refuses the shape."""
    return int(load_library().m3_prefill_prologue_mode(ctypes.byref(shape)))


def prefill_prologue_kernel_used(shape: M3Shape) -> int:
    """m3_prefill_prologue_kernel_used: the prefill kernel a prologue call runs."""
    return int(load_library().m3_prefill_prologue_kernel_used(ctypes.byref(shape)))


def prefill_gated_kernel_used(shape: M3Shape) -> int:
    """m3_prefill_gated_kernel_used: the prefill kernel a gated call runs."""
    return int(load_library().m3_prefill_gated_kernel_used(ctypes.byref(shape)))


def prefill_prologue_workspace_bytes(shape: M3Shape) -> int:
    return int(load_library().m3_prefill_prologue_workspace_bytes(ctypes.byref(shape)))


def prefill_max_chunk(shape: M3Shape) -> int:
    return int(load_library().m3_prefill_max_chunk(ctypes.byref(shape)))


def prefill_status(workspace: torch.Tensor) -> int:
    """m3_prefill_status: waits for the workspace's stream, returns (and clears)
    the status its error word records (0 = M3_OK)."""
    return int(load_library().m3_prefill_status(
        _ptr(workspace, None, workspace.device), workspace.numel() * workspace.element_size(),
        _stream(workspace.device)))


def debug_set_spin_limit(polls: int) -> None:
    load_library().m3_debug_set_spin_limit(int(polls))


def prefill_kernel_used(shape: M3Shape) -> int:
    """m3_prefill_kernel_used: M3_KERNEL_STREAM (2), M3_KERNEL_PER_CHUNK (1) or
    0 when m3_scan_prefill refuses the shape."""
    return int(load_library().m3_prefill_kernel_used(ctypes.byref(shape)))


def debug_set_prefill_kernel(which: int) -> None:
    """m3_debug_set_prefill_kernel: 0 the library's choice, 1 the per-chunk
    kernel only, 2 the streaming kernel wherever it takes the shape."""
    _check(load_library().m3_debug_set_prefill_kernel(int(which)))


def scan_prefill(x, B, C, dt, A, lam, theta=None, h0=None, B_prev=None, x_prev=None,
                 y=None, h_out=None, chunk: int = 0, workspace=None,
                 want_state: bool = True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunked prefill (m3_scan_prefill).

    x [b,L,H,R,P], B/C [b,L,H,R,N] (fp32 or bf16, same dtype); dt/lam [b,L,H],
    A [H], theta [b,L,H,N/2] fp32 or None; h0 [b,H,N,P] fp32 or None; B_prev
    [b,H,R,N] / x_prev [b,H,R,P] or None.  Returns (y, h_out).  Output and
    workspace tensors are allocated with torch when not given (the workspace
    zero-filled); a workspace passed in must have been zero-filled before its
    first use and may then be passed to every later call on the same stream.
    """
    lib = load_library()
    b, L, H, R, P = x.shape
    N = B.shape[-1]
    dev = x.device
    dcode = _dtype_code(x)
    shape = make_shape(b, L, H, P, N, R, chunk, dcode)
    if y is None:
        y = torch.empty_like(x)
    if h_out is None and want_state:
        h_out = torch.empty((b, H, N, P), dtype=torch.float32, device=dev)
    need = int(lib.m3_prefill_workspace_bytes(ctypes.byref(shape)))
    if workspace is None:
        workspace = torch.zeros(max(need, 1), dtype=torch.uint8, device=dev)
    f32 = torch.float32
    code = lib.m3_scan_prefill(
        ctypes.byref(shape), _ptr(x, x.dtype, dev), _ptr(B, x.dtype, dev), _ptr(C, x.dtype, dev),
        _ptr(dt, f32, dev), _ptr(A, f32, dev), _ptr(lam, f32, dev), _ptr(theta, f32, dev),
        _ptr(h0, f32, dev), _ptr(B_prev, x.dtype, dev), _ptr(x_prev, x.dtype, dev),
        _ptr(y, x.dtype, dev), _ptr(h_out, f32, dev),
        _ptr(workspace, None, dev), workspace.numel() * workspace.element_size(), _stream(dev))
    _check(code)
    return y, h_out


def scan_prefill_gated(x, B, C, dt, A, lam, theta=None, h0=None, B_prev=None, x_prev=None,
                       z=None, w_y=None, w_z=None, out=None, h_out=None, chunk: int = 0,
                       workspace=None, want_state: bool = True):
    """Chunked prefill with the gated readout fused (m3_scan_prefill_gated):
    out[b,t,h,p] = sum_r w_y[h,r,p] y[b,t,h,r,p] silu(w_z[h,r,p] z[b,t,h,p]).
    z [b,L,H,P] (x's dtype) or None; w_y, w_z [H,R,P] fp32 or None.  Other
    arguments as scan_prefill.  Returns (out, h_out)."""
    lib = load_library()
    b, L, H, R, P = x.shape
    N = B.shape[-1]
    dev = x.device
    dcode = _dtype_code(x)
    shape = make_shape(b, L, H, P, N, R, chunk, dcode)
    if out is None:
        out = torch.empty((b, L, H, P), dtype=x.dtype, device=dev)
    if h_out is None and want_state:
        h_out = torch.empty((b, H, N, P), dtype=torch.float32, device=dev)
    need = int(lib.m3_prefill_workspace_bytes(ctypes.byref(shape)))
    if workspace is None:
        workspace = torch.zeros(max(need, 1), dtype=torch.uint8, device=dev)
    f32 = torch.float32
    code = lib.m3_scan_prefill_gated(
        ctypes.byref(shape), _ptr(x, x.dtype, dev), _ptr(B, x.dtype, dev), _ptr(C, x.dtype, dev),
        _ptr(dt, f32, dev), _ptr(A, f32, dev), _ptr(lam, f32, dev), _ptr(theta, f32, dev),
        _ptr(h0, f32, dev), _ptr(B_prev, x.dtype, dev), _ptr(x_prev, x.dtype, dev),
        _ptr(z, x.dtype, dev), _ptr(w_y, f32, dev), _ptr(w_z, f32, dev),
        _ptr(out, x.dtype, dev), _ptr(h_out, f32, dev),
        _ptr(workspace, None, dev), workspace.numel() * workspace.element_size(), _stream(dev))
    _check(code)
    return out, h_out


def decode_step_gated(h, x, B, C, dt, A, lam, theta=None, B_prev=None, x_prev=None,
                      z=None, w_y=None, w_z=None, out=None):
    """One decode step (fp32 state h, updated in place) with the gated readout
    fused (m3_decode_step_gated); z [b,H,P] or None, w_y/w_z [H,R,P] or None.
    Returns out [b,H,P]."""
    lib = load_library()
    b, H, R, P = x.shape
    N = B.shape[-1]
    dev = x.device
    shape = make_shape(b, 1, H, P, N, R, 0, _dtype_code(x))
    if out is None:
        out = torch.empty((b, H, P), dtype=x.dtype, device=dev)
    f32 = torch.float32
    code = lib.m3_decode_step_gated(
        ctypes.byref(shape), _ptr(h, f32, dev),
        _ptr(B_prev, x.dtype, dev), _ptr(x_prev, x.dtype, dev),
        _ptr(x, x.dtype, dev), _ptr(B, x.dtype, dev), _ptr(C, x.dtype, dev),
        _ptr(dt, f32, dev), _ptr(A, f32, dev), _ptr(lam, f32, dev), _ptr(theta, f32, dev),
        _ptr(z, x.dtype, dev), _ptr(w_y, f32, dev), _ptr(w_z, f32, dev),
        _ptr(out, x.dtype, dev), _stream(dev))
    _check(code)
    return out


def _prologue(eps, bias_B, bias_C, dev):
    return M3Prologue(float(eps), _ptr(bias_B, torch.float32, dev), _ptr(bias_C, torch.float32, dev))


def scan_prefill_prologue(x, B, C, dt, A, lam, theta=None, h0=None, B_prev=None, x_prev=None,
                          y=None, h_out=None, chunk: int = 0, workspace=None, want_state: bool = True,
                          eps: float = 1e-6, bias_B=None, bias_C=None):
    """Chunked prefill with the prologue (m3_scan_prefill_prologue; fused into
    the prefill kernel or staged before it, see prefill_prologue_mode): B, C
    and B_prev RMS-normalised per column over N (+ eps) plus bias_B / bias_C
    [H,R,N] fp32 (or None); theta holds raw angles, the step angle being
    dt * theta.  Other arguments as scan_prefill; a workspace passed in must
    hold prefill_prologue_workspace_bytes.  Returns (y, h_out)."""
    lib = load_library()
    b, L, H, R, P = x.shape
    N = B.shape[-1]
    dev = x.device
    shape = make_shape(b, L, H, P, N, R, chunk, _dtype_code(x))
    if y is None:
        y = torch.empty_like(x)
    if h_out is None and want_state:
        h_out = torch.empty((b, H, N, P), dtype=torch.float32, device=dev)
    need = int(lib.m3_prefill_prologue_workspace_bytes(ctypes.byref(shape)))
    if workspace is None:
        workspace = torch.zeros(max(need, 1), dtype=torch.uint8, device=dev)
    f32 = torch.float32
    pro = _prologue(eps, bias_B, bias_C, dev)
    code = lib.m3_scan_prefill_prologue(
        ctypes.byref(shape), ctypes.byref(pro), _ptr(x, x.dtype, dev), _ptr(B, x.dtype, dev),
        _ptr(C, x.dtype, dev), _ptr(dt, f32, dev), _ptr(A, f32, dev), _ptr(lam, f32, dev), _ptr(theta, f32, dev),
        _ptr(h0, f32, dev), _ptr(B_prev, x.dtype, dev), _ptr(x_prev, x.dtype, dev),
        _ptr(y, x.dtype, dev), _ptr(h_out, f32, dev),
        _ptr(workspace, None, dev), workspace.numel() * workspace.element_size(), _stream(dev))
    _check(code)
    return y, h_out


def decode_step_prologue(h, x, B, C, dt, A, lam, theta=None, B_prev=None, x_prev=None, y=None,
                         eps: float = 1e-6, bias_B=None, bias_C=None):
    """One decode step (fp32 state h, in place) with the fused prologue
    (m3_decode_step_prologue): B, C, B_prev RMS-normalised per column over N
    (+ eps) plus bias_B / bias_C [H,R,N] fp32 (or None); theta holds raw angles,
    the step angle being dt * theta.  Returns y."""
    lib = load_library()
    b, H, R, P = x.shape
    N = B.shape[-1]
    dev = x.device
    shape = make_shape(b, 1, H, P, N, R, 0, _dtype_code(x))
    if y is None:
        y = torch.empty_like(x)
    f32 = torch.float32
    pro = _prologue(eps, bias_B, bias_C, dev)
    code = lib.m3_decode_step_prologue(
        ctypes.byref(shape), ctypes.byref(pro), _ptr(h, f32, dev),
        _ptr(B_prev, x.dtype, dev), _ptr(x_prev, x.dtype, dev),
        _ptr(x, x.dtype, dev), _ptr(B, x.dtype, dev), _ptr(C, x.dtype, dev),
        _ptr(dt, f32, dev), _ptr(A, f32, dev), _ptr(lam, f32, dev), _ptr(theta, f32, dev),
        _ptr(y, x.dtype, dev), _stream(dev))
    _check(code)
    return y


def decode_step(h, x, B, C, dt, A, lam, theta=None, B_prev=None, x_prev=None, y=None):
    """One decode step; updates h [b,H,N,P] in place, returns y.  An fp32 h calls
    m3_decode_step, a bf16 h m3_decode_step_bf16_state."""
    lib = load_library()
    b, H, R, P = x.shape
    N = B.shape[-1]
    dev = x.device
    dcode = _dtype_code(x)
    shape = make_shape(b, 1, H, P, N, R, 0, dcode)
    if y is None:
        y = torch.empty_like(x)
    f32 = torch.float32
    fn = lib.m3_decode_step_bf16_state if h.dtype == torch.bfloat16 else lib.m3_decode_step
    code = fn(
        ctypes.byref(shape), _ptr(h, h.dtype if h.dtype == torch.bfloat16 else f32, dev),
        _ptr(B_prev, x.dtype, dev), _ptr(x_prev, x.dtype, dev),
        _ptr(x, x.dtype, dev), _ptr(B, x.dtype, dev), _ptr(C, x.dtype, dev),
        _ptr(dt, f32, dev), _ptr(A, f32, dev), _ptr(lam, f32, dev), _ptr(theta, f32, dev),
        _ptr(y, x.dtype, dev), _stream(dev))
    _check(code)
    return y


def backward_workspace_bytes(shape: M3Shape) -> int:
    return int(load_library().m3_scan_backward_workspace_bytes(ctypes.byref(shape)))


def scan_backward(x, B, C, dt, A, lam, theta=None, h0=None, B_prev=None, x_prev=None,
                  dy=None, dh_out=None, workspace=None, want=("h0", "B_prev", "x_prev")) -> dict:
    """Gradients of <dy, y> + <dh_out, h_out> for the prefill (m3_scan_backward).

    Inputs as scan_prefill; dy [b,L,H,R,P] in x's dtype; dh_out [b,H,N,P] fp32
    or None.  Returns a dict of fp32 gradients: x, B, C, dt, A, lam, theta (None
    without theta), h0, B_prev, x_prev (computed when named in `want` and, for
    the previous write, given).  The workspace (every forward state) is
    allocated with torch when not given."""
    lib = load_library()
    b, L, H, R, P = x.shape
    N = B.shape[-1]
    dev = x.device
    shape = make_shape(b, L, H, P, N, R, 0, _dtype_code(x))
    need = int(lib.m3_scan_backward_workspace_bytes(ctypes.byref(shape)))
    if need == 0:
        raise M3Error(2, "the backward does not take this shape")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    g = dict(x=torch.empty((b, L, H, R, P), **f32), B=torch.empty((b, L, H, R, N), **f32),
             C=torch.empty((b, L, H, R, N), **f32), dt=torch.empty((b, L, H), **f32),
             A=torch.empty((H,), **f32), lam=torch.empty((b, L, H), **f32),
             theta=None if theta is None else torch.empty((b, L, H, N // 2), **f32),
             h0=torch.empty((b, H, N, P), **f32) if "h0" in want else None,
             B_prev=torch.empty((b, H, R, N), **f32) if ("B_prev" in want and B_prev is not None) else None,
             x_prev=torch.empty((b, H, R, P), **f32) if ("x_prev" in want and B_prev is not None) else None)
    f = torch.float32
    code = lib.m3_scan_backward(
        ctypes.byref(shape), _ptr(x, x.dtype, dev), _ptr(B, x.dtype, dev), _ptr(C, x.dtype, dev),
        _ptr(dt, f, dev), _ptr(A, f, dev), _ptr(lam, f, dev), _ptr(theta, f, dev),
        _ptr(h0, f, dev), _ptr(B_prev, x.dtype, dev), _ptr(x_prev, x.dtype, dev),
        _ptr(dy, x.dtype, dev), _ptr(dh_out, f, dev),
        _ptr(g["x"], f, dev), _ptr(g["B"], f, dev), _ptr(g["C"], f, dev), _ptr(g["dt"], f, dev),
        _ptr(g["A"], f, dev), _ptr(g["lam"], f, dev), _ptr(g["theta"], f, dev), _ptr(g["h0"], f, dev),
        _ptr(g["B_prev"], f, dev), _ptr(g["x_prev"], f, dev),
        _ptr(workspace, None, dev), workspace.numel() * workspace.element_size(), _stream(dev))
    _check(code)
    return g
