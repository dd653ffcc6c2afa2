"""Thin Python binding of libw2a8.so (the MI355X W2A8 linear layer).

Every function marshals arguments (dtype, shape, device, contiguity checks;
pointers and the current HIP stream) and calls the C ABI of the same name in
``include/w2a8.h``; all computation happens in the library.  PyTorch supplies
device memory and streams only.  If the library has not been built, importing
the binding's functions raises; there is no fallback path.

Host functions take/return CPU tensors; device functions take CUDA (HIP)
tensors on the current device and enqueue work on the current stream (or on
``stream=`` if given).
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

__all__ = [
    "W2A8Error", "lib", "packed_bytes", "workspace_bytes", "layout_version",
    "ternarize_absmean", "pack_ternary", "unpack_ternary", "quant_act_int8",
    "w2a8_gemv", "w2a8_gemv_noalloc", "w2a8_gemm", "gemv", "gemm", "linear", "Workspace",
    "w2a8_linear_gemv", "tune_gemv", "tune_gemv_force", "gemv_plan", "linear_plan", "DEFAULT_GEMV_POLICY",
    "tune_gemm", "tune_gemm_ring", "tune_gemm_pipe",
    "act4_bytes", "pack_act_int4", "quant_act_int4", "w2a4_gemv", "w2a4_linear_gemv",
    "linear_a4", "w2a8_gemv_grouped", "w2a8_linear_gemv_grouped", "linear_grouped",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libw2a8.so")
LAYOUT_VERSION = 1

_lib = None
_lib_lock = threading.Lock()


class W2A8Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {lib().w2a8_status_str(status).decode()} (status {status})")


def lib():
    """The loaded library (built in-tree); raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    with _lib_lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
                "or `python w2a8_gemv_amd/build.py`")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I32, F32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
        L.w2a8_status_str.argtypes = [I32]
        L.w2a8_status_str.restype = ctypes.c_char_p
        L.w2a8_layout_version.argtypes = []
        L.w2a8_layout_version.restype = I32
        L.w2a8_packed_bytes.argtypes = [I64, I64]
        L.w2a8_packed_bytes.restype = I64
        L.w2a8_workspace_bytes.argtypes = [I64, I64, I64]
        L.w2a8_workspace_bytes.restype = I64
        L.w2a8_ternarize_absmean.argtypes = [P, I64, I64, P, P]
        L.w2a8_ternarize_absmean.restype = I32
        L.pack_ternary.argtypes = [P, I64, I64, P, I64]
        L.pack_ternary.restype = I32
        L.unpack_ternary.argtypes = [P, I64, I64, I64, P]
        L.unpack_ternary.restype = I32
        L.quant_act_int8.argtypes = [P, I64, I64, P, P, P]
        L.quant_act_int8.restype = I32
        L.w2a8_gemv.argtypes = [P, P, I64, I64, P, P, F32, P, P, I64, P]
        L.w2a8_gemv.restype = I32
        L.w2a8_gemv_noalloc.argtypes = [P, P, I64, I64, P, P, F32, P, P]
        L.w2a8_gemv_noalloc.restype = I32
        L.w2a8_gemm.argtypes = [P, P, I64, I64, I64, P, P, F32, P, P, I64, P]
        L.w2a8_gemm.restype = I32
        L.w2a8_linear_gemv.argtypes = [P, P, I64, I64, F32, P, P, P, I64, P]
        L.w2a8_linear_gemv.restype = I32
        L.w2a4_act_bytes.argtypes = [I64, I64]
        L.w2a4_act_bytes.restype = I64
        L.pack_act_int4.argtypes = [P, I64, I64, P, I64]
        L.pack_act_int4.restype = I32
        L.quant_act_int4.argtypes = [P, I64, I64, P, P, P]
        L.quant_act_int4.restype = I32
        L.w2a4_gemv.argtypes = [P, P, I64, I64, P, P, F32, P, P, I64, P]
        L.w2a4_gemv.restype = I32
        L.w2a4_linear_gemv.argtypes = [P, P, I64, I64, F32, P, P, P, I64, P]
        L.w2a4_linear_gemv.restype = I32
        L.w2a8_gemv_grouped.argtypes = [I32, P, P, I64, P, P, P, P, P, P, I64, P]
        L.w2a8_gemv_grouped.restype = I32
        L.w2a8_linear_gemv_grouped.argtypes = [I32, P, P, I64, P, P, P, P, P, I64, P]
        L.w2a8_linear_gemv_grouped.restype = I32
        L.w2a8_tune_gemv.argtypes = [I32, I32, I32, I32, I32]
        L.w2a8_tune_gemv.restype = I32
        L.w2a8_gemv_plan.argtypes = [I64, I64, I32, P, P, P, P]
        L.w2a8_linear_plan.argtypes = [I64, I64, I32, I32, P, P, P, P, P]
        L.w2a8_linear_plan.restype = I32
        L.w2a8_tune_gemv_force.argtypes = [I32, I32, I32, I32, I32]
        L.w2a8_tune_gemv_force.restype = I32
        L.w2a8_tune_gemm.argtypes = [I32]
        L.w2a8_tune_gemm.restype = I32
        L.w2a8_tune_gemm_pipe.argtypes = [I32]
        L.w2a8_tune_gemm_pipe.restype = I32
        L.w2a8_tune_gemm_ring.argtypes = [I32, I32, I32]
        L.w2a8_tune_gemm_ring.restype = I32
        L.w2a8_gemv_plan.restype = I32
        if L.w2a8_layout_version() != LAYOUT_VERSION:
            raise RuntimeError("libw2a8.so layout version does not match the binding")
        _lib = L
        return L


def _check(status: int, where: str):
    if status != 0:
        raise W2A8Error(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, name, dtype, device=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device == "cuda" and not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device == "cpu" and t.is_cuda:
        raise ValueError(f"{name} must be a host tensor")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


# ---------------------------------------------------------------------------
# sizes
# ---------------------------------------------------------------------------
def layout_version() -> int:
    return int(lib().w2a8_layout_version())


def packed_bytes(N: int, K: int) -> int:
    n = int(lib().w2a8_packed_bytes(N, K))
    if n < 0:
        raise W2A8Error(2, "w2a8_packed_bytes")
    return n


def workspace_bytes(M: int, N: int, K: int) -> int:
    n = int(lib().w2a8_workspace_bytes(M, N, K))
    if n < 0:
        raise W2A8Error(2, "w2a8_workspace_bytes")
    return n


# ---------------------------------------------------------------------------
# offline host steps
# ---------------------------------------------------------------------------
def ternarize_absmean(W: torch.Tensor):
    """W fp32 [N, K] (CPU) -> (wq int8 [N, K] CPU, sw float)."""
    _need(W, "W", torch.float32, "cpu")
    N, K = W.shape
    wq = torch.empty((N, K), dtype=torch.int8)
    sw = torch.zeros(1, dtype=torch.float32)
    _check(lib().w2a8_ternarize_absmean(_ptr(W), N, K, _ptr(wq), _ptr(sw)),
           "w2a8_ternarize_absmean")
    return wq, float(sw[0])


def pack_ternary(w: torch.Tensor) -> torch.Tensor:
    """w int8 [N, K] in {-1,0,1} (CPU) -> packed uint8 [packed_bytes(N, K)] (CPU)."""
    _need(w, "w", torch.int8, "cpu")
    N, K = w.shape
    nb = packed_bytes(N, K)
    out = torch.empty(nb, dtype=torch.uint8)
    _check(lib().pack_ternary(_ptr(w), N, K, _ptr(out), nb), "pack_ternary")
    return out


def unpack_ternary(p: torch.Tensor, N: int, K: int) -> torch.Tensor:
    _need(p, "packed", torch.uint8, "cpu")
    w = torch.empty((N, K), dtype=torch.int8)
    _check(lib().unpack_ternary(_ptr(p), p.numel(), N, K, _ptr(w)), "unpack_ternary")
    return w


# ---------------------------------------------------------------------------
# workspace cache (one zeroed buffer per device and stream)
# ---------------------------------------------------------------------------
class Workspace:
    """Zero-initialised device workspace; each library call leaves it zeroed."""

    _cache = {}
    _lock = threading.Lock()

    @classmethod
    def get(cls, nbytes: int, device: torch.device, stream) -> torch.Tensor | None:
        if nbytes <= 0:
            return None
        key = (device.index, stream.cuda_stream)
        with cls._lock:
            buf = cls._cache.get(key)
            if buf is None or buf.numel() < nbytes:
                with torch.cuda.stream(stream):
                    buf = torch.zeros(max(nbytes, 4096), dtype=torch.uint8, device=device)
                cls._cache[key] = buf
            return buf


def _ws(nbytes, device, stream, workspace):
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, "cuda")
        return workspace
    s = torch.cuda.current_stream(device) if stream is None else stream
    return Workspace.get(nbytes, device, s)


# ---------------------------------------------------------------------------
# device steps
# ---------------------------------------------------------------------------
def quant_act_int8(x_bf16: torch.Tensor, x_q=None, s_a=None, stream=None):
    """x bf16 [M, K] (device) -> (x_q int8 [M, K], s_a fp32 [M])."""
    _need(x_bf16, "x_bf16", torch.bfloat16, "cuda")
    if x_bf16.dim() == 1:
        x_bf16 = x_bf16.view(1, -1)
    M, K = x_bf16.shape
    if x_q is None:
        x_q = torch.empty((M, K), dtype=torch.int8, device=x_bf16.device)
    if s_a is None:
        s_a = torch.empty(M, dtype=torch.float32, device=x_bf16.device)
    _need(x_q, "x_q", torch.int8, "cuda")
    _need(s_a, "s_a", torch.float32, "cuda")
    if x_q.numel() != M * K or s_a.numel() != M:
        raise ValueError("x_q / s_a have the wrong size")
    _check(lib().quant_act_int8(_ptr(x_bf16), M, K, _ptr(x_q), _ptr(s_a), _stream_handle(stream)),
           "quant_act_int8")
    return x_q, s_a


def w2a8_gemv(w_packed, x, N, K, y_i32=None, s_a=None, s_w=1.0, y_f32=None,
              workspace=None, stream=None):
    """Raw C-ABI call (outputs must be given); returns nothing."""
    _need(w_packed, "w_packed", torch.uint8, "cuda")
    _need(x, "x", torch.int8, "cuda")
    if x.numel() != K:
        raise ValueError("x must have K elements")
    if w_packed.numel() < packed_bytes(N, K):
        raise ValueError("w_packed is smaller than packed_bytes(N, K)")
    for t, nm, dt in ((y_i32, "y_i32", torch.int32), (y_f32, "y_f32", torch.float32)):
        if t is not None:
            _need(t, nm, dt, "cuda")
            if t.numel() != N:
                raise ValueError(f"{nm} must have N elements")
    if s_a is not None:
        _need(s_a, "s_a", torch.float32, "cuda")
    need = workspace_bytes(1, N, K)
    ws = _ws(need, x.device, stream, workspace)
    _check(lib().w2a8_gemv(_ptr(w_packed), _ptr(x), N, K, _ptr(y_i32), _ptr(s_a),
                           ctypes.c_float(s_w), _ptr(y_f32), _ptr(ws),
                           0 if ws is None else ws.numel(), _stream_handle(stream)),
           "w2a8_gemv")


def w2a8_gemv_noalloc(w_packed, x, N, K, y_i32=None, s_a=None, s_w=1.0, y_f32=None,
                      stream=None):
    """Raw C-ABI call: the GEMV with the library's static scratch instead of a
    workspace (allocates nothing); returns nothing."""
    _need(w_packed, "w_packed", torch.uint8, "cuda")
    _need(x, "x", torch.int8, "cuda")
    if x.numel() != K:
        raise ValueError("x must have K elements")
    if w_packed.numel() < packed_bytes(N, K):
        raise ValueError("w_packed is smaller than packed_bytes(N, K)")
    for t, nm, dt in ((y_i32, "y_i32", torch.int32), (y_f32, "y_f32", torch.float32)):
        if t is not None:
            _need(t, nm, dt, "cuda")
            if t.numel() != N:
                raise ValueError(f"{nm} must have N elements")
    if s_a is not None:
        _need(s_a, "s_a", torch.float32, "cuda")
    _check(lib().w2a8_gemv_noalloc(_ptr(w_packed), _ptr(x), N, K, _ptr(y_i32), _ptr(s_a),
                                   ctypes.c_float(s_w), _ptr(y_f32), _stream_handle(stream)),
           "w2a8_gemv_noalloc")


def w2a8_gemm(w_packed, x, M, N, K, y_i32=None, s_a=None, s_w=1.0, y_f32=None,
              workspace=None, stream=None):
    """Raw C-ABI call (outputs must be given); returns nothing."""
    _need(w_packed, "w_packed", torch.uint8, "cuda")
    _need(x, "x", torch.int8, "cuda")
    if x.numel() != M * K:
        raise ValueError("x must have M*K elements")
    if w_packed.numel() < packed_bytes(N, K):
        raise ValueError("w_packed is smaller than packed_bytes(N, K)")
    for t, nm, dt in ((y_i32, "y_i32", torch.int32), (y_f32, "y_f32", torch.float32)):
        if t is not None:
            _need(t, nm, dt, "cuda")
            if t.numel() != M * N:
                raise ValueError(f"{nm} must have M*N elements")
    if s_a is not None:
        _need(s_a, "s_a", torch.float32, "cuda")
        if s_a.numel() != M:
            raise ValueError("s_a must have M elements")
    need = workspace_bytes(M, N, K)
    ws = _ws(need, x.device, stream, workspace)
    _check(lib().w2a8_gemm(_ptr(w_packed), _ptr(x), M, N, K, _ptr(y_i32), _ptr(s_a),
                           ctypes.c_float(s_w), _ptr(y_f32), _ptr(ws),
                           0 if ws is None else ws.numel(), _stream_handle(stream)),
           "w2a8_gemm")


def w2a8_linear_gemv(w_packed, x_bf16, N, K, s_w, y_f32, y_i32=None, workspace=None,
                     stream=None):
    """Raw C-ABI call: fused quantize + GEMV + fp32 epilogue for one token."""
    _need(w_packed, "w_packed", torch.uint8, "cuda")
    if x_bf16.dtype not in (torch.bfloat16, torch.int16, torch.uint16) or not x_bf16.is_cuda:
        raise TypeError("x_bf16 must be a bfloat16 (or 16-bit bit pattern) CUDA tensor")
    if not x_bf16.is_contiguous() or x_bf16.numel() != K:
        raise ValueError("x_bf16 must be contiguous with K elements")
    if w_packed.numel() < packed_bytes(N, K):
        raise ValueError("w_packed is smaller than packed_bytes(N, K)")
    _need(y_f32, "y_f32", torch.float32, "cuda")
    if y_f32.numel() != N:
        raise ValueError("y_f32 must have N elements")
    if y_i32 is not None:
        _need(y_i32, "y_i32", torch.int32, "cuda")
        if y_i32.numel() != N:
            raise ValueError("y_i32 must have N elements")
    ws = _ws(workspace_bytes(1, N, K), x_bf16.device, stream, workspace)
    _check(lib().w2a8_linear_gemv(_ptr(w_packed), _ptr(x_bf16), N, K, ctypes.c_float(s_w),
                                  _ptr(y_f32), _ptr(y_i32), _ptr(ws),
                                  0 if ws is None else ws.numel(), _stream_handle(stream)),
           "w2a8_linear_gemv")


# ---------------------------------------------------------------------------
# W2A4 variant: int4 activations in the A4I layout (see include/w2a8.h)
# ---------------------------------------------------------------------------
def act4_bytes(M: int, K: int) -> int:
    v = int(lib().w2a4_act_bytes(M, K))
    if v < 0:
        raise ValueError("M or K out of range")
    return v


def pack_act_int4(q: torch.Tensor) -> torch.Tensor:
    """Host int8 [M, K] (values -8..7) -> host uint8 [act4_bytes(M, K)] (A4I layout)."""
    q2 = q.view(1, -1) if q.dim() == 1 else q
    _need(q2, "q", torch.int8, "cpu")
    M, K = q2.shape
    out = torch.empty(act4_bytes(M, K), dtype=torch.uint8)
    _check(lib().pack_act_int4(_ptr(q2), M, K, _ptr(out), out.numel()), "pack_act_int4")
    return out


def quant_act_int4(x_bf16: torch.Tensor, x_q4=None, s_a=None, stream=None):
    """x bf16 [M, K] (device) -> (A4I bytes uint8 [act4_bytes(M, K)], s_a fp32 [M])."""
    _need(x_bf16, "x_bf16", torch.bfloat16, "cuda")
    x2 = x_bf16.view(1, -1) if x_bf16.dim() == 1 else x_bf16
    M, K = x2.shape
    if x_q4 is None:
        x_q4 = torch.empty(act4_bytes(M, K), dtype=torch.uint8, device=x2.device)
    if s_a is None:
        s_a = torch.empty(M, dtype=torch.float32, device=x2.device)
    _need(x_q4, "x_q4", torch.uint8, "cuda")
    _need(s_a, "s_a", torch.float32, "cuda")
    if x_q4.numel() < act4_bytes(M, K) or s_a.numel() != M:
        raise ValueError("x_q4 / s_a have the wrong size")
    _check(lib().quant_act_int4(_ptr(x2), M, K, _ptr(x_q4), _ptr(s_a), _stream_handle(stream)),
           "quant_act_int4")
    return x_q4, s_a


def w2a4_gemv(w_packed, x_q4, N, K, y_i32=None, s_a=None, s_w=1.0, y_f32=None,
              workspace=None, stream=None):
    """Raw C-ABI call: W2A4 GEMV over one A4I activation row; returns nothing."""
    _need(w_packed, "w_packed", torch.uint8, "cuda")
    _need(x_q4, "x_q4", torch.uint8, "cuda")
    if x_q4.numel() < act4_bytes(1, K):
        raise ValueError("x_q4 must hold act4_bytes(1, K) bytes")
    if w_packed.numel() < packed_bytes(N, K):
        raise ValueError("w_packed is smaller than packed_bytes(N, K)")
    for t, nm, dt in ((y_i32, "y_i32", torch.int32), (y_f32, "y_f32", torch.float32)):
        if t is not None:
            _need(t, nm, dt, "cuda")
            if t.numel() != N:
                raise ValueError(f"{nm} must have N elements")
    if s_a is not None:
        _need(s_a, "s_a", torch.float32, "cuda")
    ws = _ws(workspace_bytes(1, N, K), x_q4.device, stream, workspace)
    _check(lib().w2a4_gemv(_ptr(w_packed), _ptr(x_q4), N, K, _ptr(y_i32), _ptr(s_a),
                           ctypes.c_float(s_w), _ptr(y_f32), _ptr(ws),
                           0 if ws is None else ws.numel(), _stream_handle(stream)),
           "w2a4_gemv")


def w2a4_linear_gemv(w_packed, x_bf16, N, K, s_w, y_f32, y_i32=None, workspace=None,
                     stream=None):
    """Raw C-ABI call: fused int4 quantize + W2A4 GEMV + fp32 epilogue for one token."""
    _need(w_packed, "w_packed", torch.uint8, "cuda")
    if x_bf16.dtype not in (torch.bfloat16, torch.int16, torch.uint16) or not x_bf16.is_cuda:
        raise TypeError("x_bf16 must be a bfloat16 (or 16-bit bit pattern) CUDA tensor")
    if not x_bf16.is_contiguous() or x_bf16.numel() != K:
        raise ValueError("x_bf16 must be contiguous with K elements")
    if w_packed.numel() < packed_bytes(N, K):
        raise ValueError("w_packed is smaller than packed_bytes(N, K)")
    _need(y_f32, "y_f32", torch.float32, "cuda")
    if y_f32.numel() != N:
        raise ValueError("y_f32 must have N elements")
    if y_i32 is not None:
        _need(y_i32, "y_i32", torch.int32, "cuda")
        if y_i32.numel() != N:
            raise ValueError("y_i32 must have N elements")
    ws = _ws(workspace_bytes(1, N, K), x_bf16.device, stream, workspace)
    _check(lib().w2a4_linear_gemv(_ptr(w_packed), _ptr(x_bf16), N, K, ctypes.c_float(s_w),
                                  _ptr(y_f32), _ptr(y_i32), _ptr(ws),
                                  0 if ws is None else ws.numel(), _stream_handle(stream)),
           "w2a4_linear_gemv")


def linear_a4(x_bf16, w_packed, s_w, N, K, stream=None, fused=True):
    """W2A4 linear layer for one token -> fp32 [1, N].  fused=True:
    w2a4_linear_gemv (one launch); otherwise quant_act_int4, then w2a4_gemv
    with the fp32 epilogue (two launches, no host synchronisation).  Both
    routes give bit-identical results."""
    if fused:
        y = torch.empty((1, N), dtype=torch.float32, device=x_bf16.device)
        w2a4_linear_gemv(w_packed, x_bf16.reshape(-1), N, K, s_w, y.view(-1), stream=stream)
        return y
    xq4, sa = quant_act_int4(x_bf16.reshape(1, -1), stream=stream)
    y = torch.empty((1, N), dtype=torch.float32, device=x_bf16.device)
    w2a4_gemv(w_packed, xq4, N, K, s_a=sa, s_w=s_w, y_f32=y.view(-1), stream=stream)
    return y


MAX_GROUPS = 8


def _host_array(ctype, values):
    return (ctype * len(values))(*values)


def _grouped_args(w_packed, Ns, K, s_w, y_i32, y_f32):
    G = len(w_packed)
    if not (1 <= G <= MAX_GROUPS) or len(Ns) != G or len(s_w) != G:
        raise ValueError(f"need 1..{MAX_GROUPS} projections with one N and one s_w each")
    for g, (w, n) in enumerate(zip(w_packed, Ns)):
        _need(w, f"w_packed[{g}]", torch.uint8, "cuda")
        if w.numel() < packed_bytes(n, K):
            raise ValueError(f"w_packed[{g}] is smaller than packed_bytes(N[{g}], K)")
    arrays = []
    for ys, nm, dt in ((y_i32, "y_i32", torch.int32), (y_f32, "y_f32", torch.float32)):
        if ys is None:
            arrays.append(None)
            continue
        if len(ys) != G:
            raise ValueError(f"{nm} must have one entry per projection")
        for g, (y, n) in enumerate(zip(ys, Ns)):
            if y is not None:
                _need(y, f"{nm}[{g}]", dt, "cuda")
                if y.numel() != n:
                    raise ValueError(f"{nm}[{g}] must have N[{g}] elements")
        arrays.append(_host_array(ctypes.c_void_p, [None if y is None else y.data_ptr() for y in ys]))
    need = sum(workspace_bytes(1, n, K) for n in Ns)
    return (G, _host_array(ctypes.c_void_p, [w.data_ptr() for w in w_packed]),
            _host_array(ctypes.c_int64, list(Ns)), _host_array(ctypes.c_float, list(s_w)),
            arrays[0], arrays[1], need)


def w2a8_gemv_grouped(w_packed, x, Ns, K, s_w, y_i32=None, y_f32=None, s_a=None,
                      workspace=None, stream=None):
    """Raw C-ABI call: several projections (lists of equal length) sharing one
    int8 activation row x [K], in one launch; returns nothing."""
    _need(x, "x", torch.int8, "cuda")
    if x.numel() != K:
        raise ValueError("x must have K elements")
    if s_a is not None:
        _need(s_a, "s_a", torch.float32, "cuda")
    G, wp, n_arr, sw_arr, yi_arr, yf_arr, need = _grouped_args(w_packed, Ns, K, s_w, y_i32, y_f32)
    ws = _ws(need, x.device, stream, workspace)
    _check(lib().w2a8_gemv_grouped(G, wp, n_arr, K, _ptr(x), _ptr(s_a), sw_arr, yi_arr, yf_arr,
                                   _ptr(ws), 0 if ws is None else ws.numel(),
                                   _stream_handle(stream)),
           "w2a8_gemv_grouped")


def w2a8_linear_gemv_grouped(w_packed, x_bf16, Ns, K, s_w, y_f32, y_i32=None, workspace=None,
                             stream=None):
    """Raw C-ABI call: quantize one bf16 token and apply several projections
    to it, in one launch; returns nothing."""
    if x_bf16.dtype not in (torch.bfloat16, torch.int16, torch.uint16) or not x_bf16.is_cuda:
        raise TypeError("x_bf16 must be a bfloat16 (or 16-bit bit pattern) CUDA tensor")
    if not x_bf16.is_contiguous() or x_bf16.numel() != K:
        raise ValueError("x_bf16 must be contiguous with K elements")
    G, wp, n_arr, sw_arr, yi_arr, yf_arr, need = _grouped_args(w_packed, Ns, K, s_w, y_i32, y_f32)
    ws = _ws(need, x_bf16.device, stream, workspace)
    _check(lib().w2a8_linear_gemv_grouped(G, wp, n_arr, K, _ptr(x_bf16), sw_arr, yf_arr, yi_arr,
                                          _ptr(ws), 0 if ws is None else ws.numel(),
                                          _stream_handle(stream)),
           "w2a8_linear_gemv_grouped")


def linear_grouped(x_bf16, w_packed, s_w, Ns, K, stream=None):
    """Several W2A8 linear layers applied to one bf16 token (one launch):
    returns a list of fp32 [1, N_g] outputs."""
    ys = [torch.empty((1, n), dtype=torch.float32, device=x_bf16.device) for n in Ns]
    w2a8_linear_gemv_grouped(w_packed, x_bf16.reshape(-1), Ns, K, s_w, [y.view(-1) for y in ys],
                             stream=stream)
    return ys


def gemv(w_packed, x, N, K, *, out_i32=True, s_a=None, s_w=1.0, stream=None):
    """y_i32 [N] (and y_f32 [N] when s_a is given) for one int8 activation row."""
    y_i32 = torch.empty(N, dtype=torch.int32, device=x.device) if out_i32 else None
    y_f32 = torch.empty(N, dtype=torch.float32, device=x.device) if s_a is not None else None
    w2a8_gemv(w_packed, x, N, K, y_i32=y_i32, s_a=s_a, s_w=s_w, y_f32=y_f32, stream=stream)
    return y_i32 if y_f32 is None else (y_i32, y_f32)


def gemm(w_packed, x, N, K, *, out_i32=True, s_a=None, s_w=1.0, stream=None):
    """Y_i32 [M, N] (and Y_f32 when s_a is given) for int8 activations [M, K]."""
    M = x.shape[0]
    y_i32 = torch.empty((M, N), dtype=torch.int32, device=x.device) if out_i32 else None
    y_f32 = torch.empty((M, N), dtype=torch.float32, device=x.device) if s_a is not None else None
    w2a8_gemm(w_packed, x, M, N, K, y_i32=y_i32, s_a=s_a, s_w=s_w, y_f32=y_f32, stream=stream)
    return y_i32 if y_f32 is None else (y_i32, y_f32)


def linear(x_bf16, w_packed, s_w, N, K, stream=None, fused=True):
    """Full W2A8 linear layer: bf16 activations [M, K] -> fp32 [M, N].

    M == 1 with fused=True: w2a8_linear_gemv (one launch).  Otherwise
    quant_act_int8, then w2a8_gemv (M == 1) or w2a8_gemm (M > 1) with the
    fp32 epilogue, all enqueued on one stream with no host synchronisation.
    Both routes give bit-identical results.
    """
    x2 = x_bf16.view(1, -1) if x_bf16.dim() == 1 else x_bf16
    M = x2.shape[0]
    if M == 1 and fused:
        y = torch.empty((1, N), dtype=torch.float32, device=x2.device)
        w2a8_linear_gemv(w_packed, x2.reshape(-1), N, K, s_w, y.view(-1), stream=stream)
        return y
    xq, sa = quant_act_int8(x2, stream=stream)
    y = torch.empty((M, N), dtype=torch.float32, device=x2.device)
    if M == 1:
        w2a8_gemv(w_packed, xq.view(-1), N, K, s_a=sa, s_w=s_w, y_f32=y.view(-1), stream=stream)
    else:
        w2a8_gemm(w_packed, xq, M, N, K, s_a=sa, s_w=s_w, y_f32=y, stream=stream)
    return y


# ---------------------------------------------------------------------------
# tuning knobs (w2a8_tuning.h)
# ---------------------------------------------------------------------------
DEFAULT_GEMV_POLICY = (4, 6, 8, 256, 48)


def tune_gemv(wg_per_cu: int, tiles_per_wave: int, unroll: int, krange_tiles: int = 256,
              split_min_tiles: int = 48):
    _check(lib().w2a8_tune_gemv(wg_per_cu, tiles_per_wave, unroll, krange_tiles,
                                split_min_tiles), "w2a8_tune_gemv")


def tune_gemv_force(kernel: int, waves_per_wg: int = 1, wgs_per_strip: int = 1, depth: int = 2,
                    direct_x: int = 0):
    """Force a GEMV plan (kernel 1: batch kernel, 2: ring kernel, 3: row-slice
    kernel with waves_per_wg 1 and wgs_per_strip 8; 0: automatic)."""
    _check(lib().w2a8_tune_gemv_force(kernel, waves_per_wg, wgs_per_strip, depth, direct_x),
           "w2a8_tune_gemv_force")


def tune_gemm(kernel: int):
    """Batched-product kernel: 0 automatic, 1 pipelined whenever K allows, 2 general,
    3 few-row whenever M <= 8, 4 short-batch MFMA ring whenever M <= 32 and K allows."""
    _check(lib().w2a8_tune_gemm(kernel), "w2a8_tune_gemm")


def tune_gemm_pipe(config: int = -1):
    """Forced configuration (0..9) of the pipelined MFMA GEMM (-1: automatic)."""
    _check(lib().w2a8_tune_gemm_pipe(config), "w2a8_tune_gemm_pipe")


def tune_gemm_ring(waves_per_wg: int = 0, wgs_per_strip: int = 0, depth: int = 0):
    """Forced plan of the short-batch MFMA ring kernel (all 0: automatic)."""
    _check(lib().w2a8_tune_gemm_ring(waves_per_wg, wgs_per_strip, depth), "w2a8_tune_gemm_ring")


def linear_plan(N: int, K: int, cus: int, int4: bool = False):
    """Automatic launch plan of the fused linear layer (w2a8_linear_gemv, or
    w2a4_linear_gemv with int4=True): (kernel, waves per workgroup,
    workgroups per strip, run, depth); kernel 1 is the workgroup kernel's
    fused variant, 3 the ring kernel over shared k-ranges, 4 the ring kernel
    with per-wave runs."""
    v = [ctypes.c_int(0) for _ in range(5)]
    _check(lib().w2a8_linear_plan(N, K, cus, int(bool(int4)), *[ctypes.byref(x) for x in v]),
           "w2a8_linear_plan")
    return tuple(x.value for x in v)


def gemv_plan(N: int, K: int, cus: int):
    """Automatic launch plan of w2a8_gemv: (kernel, waves per workgroup,
    workgroups per strip, depth); kernel 2 is the ring kernel (K a multiple
    of 16), 1 the batch kernel."""
    kern, wk, sg, d = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int(0)
    _check(lib().w2a8_gemv_plan(N, K, cus, ctypes.byref(kern), ctypes.byref(wk), ctypes.byref(sg),
                                ctypes.byref(d)), "w2a8_gemv_plan")
    return kern.value, wk.value, sg.value, d.value
