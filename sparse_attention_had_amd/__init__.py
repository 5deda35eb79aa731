"""HAD (Hamming Attention Distillation) inference attention for AMD MI355X.

Thin ctypes binding of libhad.so.  Every step of the path runs in the HIP
kernels of that library; this module only checks tensor metadata, passes
device pointers and the current HIP stream, and turns status codes into
exceptions.  PyTorch provides device memory and streams.

    bits, sigma = pack(x)                       # sign bits + sigma of x
    out = attention(qbits, kbits, v, topn, scale, causal)
    s   = logits(qbits, kbits, dim, ...)        # inspection export
    idx = select(qbits, kbits, dim, topn, ...)  # inspection export

There is no CPU fallback: if the library is missing, every call raises.
"""

from __future__ import annotations

import ctypes
import os
import threading

import torch

__all__ = [
    "HadError",
    "library_path",
    "load_library",
    "words_per_row",
    "pack_workspace_bytes",
    "pack",
    "attention",
    "logits",
    "select",
    "DEV_NAN_INPUT",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
DEV_NAN_INPUT = 1

HAD_F32 = 0
HAD_BF16 = 1


class HadError(RuntimeError):
    """A libhad call returned a non-zero status."""

    def __init__(self, fn: str, status: int, name: str, detail: str):
        super().__init__(f"{fn} failed with {name} ({status}): {detail}")
        self.status = status
        self.status_name = name


class Shape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64),
        ("heads", ctypes.c_int64),
        ("seq", ctypes.c_int64),
        ("dim", ctypes.c_int64),
    ]


class DecodeShape(ctypes.Structure):
    """had_decode_shape: B, H, new query rows, valid cache rows, cache rows, d."""

    _fields_ = [("batch", ctypes.c_int64), ("heads", ctypes.c_int64), ("n_q", ctypes.c_int64),
                ("n_k", ctypes.c_int64), ("k_stride", ctypes.c_int64), ("dim", ctypes.c_int64)]


_lib = None
_lib_lock = threading.Lock()


def library_path() -> str:
    return os.environ.get("HAD_LIBRARY", os.path.join(_PKG, "libhad.so"))


def load_library():
    """Load libhad.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    with _lib_lock:
        if _lib is not None:
            return _lib
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(
                f"libhad.so not found at {path}; build it first "
                "(python -m sparse_attention_had_amd.build)")
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I = ctypes.c_int
        lib.had_words_per_row.argtypes = [I64]
        lib.had_words_per_row.restype = I64
        lib.had_pack_workspace_bytes.argtypes = [Shape]
        lib.had_pack_workspace_bytes.restype = ctypes.c_size_t
        lib.had_pack.argtypes = [P, Shape, P, P, P, ctypes.c_size_t, P, P]
        lib.had_pack.restype = I
        lib.had_attention.argtypes = [P, P, P, I, Shape, I64, ctypes.c_float, I, P, P]
        lib.had_attention.restype = I
        lib.had_logits.argtypes = [P, P, Shape, I64, I64, I64, I64, P, P]
        lib.had_logits.restype = I
        lib.had_select.argtypes = [P, P, Shape, I64, I, I64, I64, P, P]
        lib.had_select.restype = I
        lib.had_forward_workspace_bytes.argtypes = [Shape]
        lib.had_forward_workspace_bytes.restype = ctypes.c_size_t
        lib.had_forward.argtypes = [P, P, P, I, Shape, I64, ctypes.c_float, I, P, P, P, P, P, P,
                                    ctypes.c_size_t, P, P]
        lib.had_forward.restype = I
        lib.had_forward_noalloc.argtypes = [P, P, P, I, Shape, I64, ctypes.c_float, I, P, P, P, P, P,
                                            P, P]
        lib.had_forward_noalloc.restype = I
        lib.had_backward_workspace_bytes.argtypes = [Shape]
        lib.had_backward_workspace_bytes.restype = ctypes.c_size_t
        lib.had_backward.argtypes = [P, P, P, I, Shape, I64, ctypes.c_float, I, P, P, P, P, P, P, P, P,
                                     ctypes.c_size_t, P]
        lib.had_backward.restype = I
        lib.had_soft_workspace_bytes.argtypes = [Shape]
        lib.had_soft_workspace_bytes.restype = ctypes.c_size_t
        lib.had_soft_forward.argtypes = [P, P, P, I, Shape, I64, ctypes.c_float, ctypes.c_float, I, P, P,
                                         P, P, ctypes.c_size_t, P]
        lib.had_soft_forward.restype = I
        lib.had_soft_select.argtypes = [P, P, Shape, I64, ctypes.c_float, I, P, P, I64, I64, P, P,
                                        ctypes.c_size_t, P]
        lib.had_soft_select.restype = I
        lib.had_pack_calibrate.argtypes = [P, Shape, P, P, P, ctypes.c_size_t, P, P]
        lib.had_pack_calibrate.restype = I
        lib.had_sigma_from_state.argtypes = [P, P, P]
        lib.had_sigma_from_state.restype = I
        lib.had_topn_mass.argtypes = [P, P, Shape, ctypes.c_float, I, ctypes.c_double, I64, I64, P, P]
        lib.had_topn_mass.restype = I
        lib.had_decode_workspace_bytes.argtypes = [DecodeShape]
        lib.had_decode_workspace_bytes.restype = ctypes.c_size_t
        lib.had_decode.argtypes = [P, P, P, I, DecodeShape, I64, I64, ctypes.c_float, I, P, P,
                                   ctypes.c_size_t, P]
        lib.had_decode.restype = I
        lib.had_decode_forward.argtypes = [P, P, P, I, DecodeShape, I64, I64, ctypes.c_float, I, P, P,
                                   ctypes.c_size_t, P]
        lib.had_decode_forward.restype = I
        lib.had_status_string.argtypes = [I]
        lib.had_status_string.restype = ctypes.c_char_p
        lib.had_last_error.argtypes = []
        lib.had_last_error.restype = ctypes.c_char_p
        _lib = lib
        return lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        lib = load_library()
        name = lib.had_status_string(status).decode()
        detail = lib.had_last_error().decode()
        raise HadError(fn, status, name, detail)


def _stream_of(device: torch.device, stream):
    return torch.cuda.current_stream(device) if stream is None else stream


def _stream_handle(device: torch.device, stream) -> int:
    return int(_stream_of(device, stream).cuda_stream)


def _need_cuda(t: torch.Tensor, name: str, dtype=None):
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must have dtype {dtype}, got {t.dtype}")


def _shape4(t: torch.Tensor, name: str):
    if t.dim() != 4:
        raise ValueError(f"{name} must have shape [B, H, n, d]")
    return t.shape


def words_per_row(dim: int) -> int:
    return int(load_library().had_words_per_row(int(dim)))


def pack_workspace_bytes(shape) -> int:
    return int(load_library().had_pack_workspace_bytes(Shape(*[int(x) for x in shape])))


_ws_cache = {}


def _workspace(device: torch.device, stream, nbytes: int) -> torch.Tensor:
    """A cached workspace of at least nbytes for calls on `stream` (None: the
    current stream).  It is allocated while that stream is current, so the
    caching allocator orders its reuse after the stream's work; no initial
    contents are needed by any call."""
    s = _stream_of(device, stream)
    key = (device.index, int(s.cuda_stream))
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < nbytes:
        with torch.cuda.stream(s):
            ws = torch.empty(max(nbytes, 4096), dtype=torch.uint8, device=device)
        _ws_cache[key] = ws
    return ws


def pack(x: torch.Tensor, *, with_sigma: bool = True, out: torch.Tensor | None = None,
         sigma: torch.Tensor | None = None, dev_status: torch.Tensor | None = None,
         workspace: torch.Tensor | None = None, stream=None):
    """Sign bits ([B,H,n,W] int32 view of uint32 words) and sigma of x.

    Returns (bits, sigma) where sigma is a 1-element float32 device tensor,
    or None when with_sigma is False.
    """
    lib = load_library()
    _need_cuda(x, "x", torch.float32)
    B, H, n, d = _shape4(x, "x")
    W = words_per_row(d)
    if out is None:
        out = torch.empty((B, H, n, W), dtype=torch.int32, device=x.device)
    _need_cuda(out, "out", torch.int32)
    if tuple(out.shape) != (B, H, n, W):
        raise ValueError("out must have shape [B, H, n, W]")
    shape = Shape(B, H, n, d)
    sh = _stream_handle(x.device, stream)
    sig_ptr = None
    ws_ptr = None
    ws_bytes = 0
    if with_sigma:
        if sigma is None:
            sigma = torch.empty(1, dtype=torch.float32, device=x.device)
        _need_cuda(sigma, "sigma", torch.float32)
        need = int(lib.had_pack_workspace_bytes(shape))
        if workspace is None:
            workspace = _workspace(x.device, stream, need)
        _need_cuda(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
        sig_ptr = sigma.data_ptr()
        ws_ptr = workspace.data_ptr()
    st_ptr = None
    if dev_status is not None:
        _need_cuda(dev_status, "dev_status", torch.int32)
        st_ptr = dev_status.data_ptr()
    _check("had_pack", lib.had_pack(x.data_ptr(), shape, out.data_ptr(), sig_ptr, ws_ptr,
                                    ws_bytes, st_ptr, sh))
    return out, (sigma if with_sigma else None)


def attention(qbits: torch.Tensor, kbits: torch.Tensor, v: torch.Tensor, topn: int,
              scale: float, causal: bool = False, *, out: torch.Tensor | None = None,
              stream=None) -> torch.Tensor:
    """Fused HAD attention; returns out [B,H,n,d] float32."""
    lib = load_library()
    _need_cuda(qbits, "qbits", torch.int32)
    _need_cuda(kbits, "kbits", torch.int32)
    _need_cuda(v, "v")
    B, H, n, d = _shape4(v, "v")
    W = words_per_row(d)
    if tuple(qbits.shape) != (B, H, n, W) or tuple(kbits.shape) != (B, H, n, W):
        raise ValueError("qbits/kbits must have shape [B, H, n, ceil(d/32)]")
    if v.dtype == torch.float32:
        vdt = HAD_F32
    elif v.dtype == torch.bfloat16:
        vdt = HAD_BF16
    else:
        raise ValueError("v must be float32 or bfloat16")
    if out is None:
        out = torch.empty((B, H, n, d), dtype=torch.float32, device=v.device)
    _need_cuda(out, "out", torch.float32)
    if tuple(out.shape) != (B, H, n, d):
        raise ValueError("out must have the shape of v")
    _check("had_attention", lib.had_attention(
        qbits.data_ptr(), kbits.data_ptr(), v.data_ptr(), vdt, Shape(B, H, n, d), int(topn),
        float(scale), int(bool(causal)), out.data_ptr(), _stream_handle(v.device, stream)))
    return out


def _v_dtype(v: torch.Tensor) -> int:
    if v.dtype == torch.float32:
        return HAD_F32
    if v.dtype == torch.bfloat16:
        return HAD_BF16
    raise ValueError("v must be float32 or bfloat16")


def forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, topn: int, scale: float,
            causal: bool = False, *, with_sigma: bool = True, out: torch.Tensor | None = None,
            qbits: torch.Tensor | None = None, kbits: torch.Tensor | None = None,
            sigma_q: torch.Tensor | None = None, sigma_k: torch.Tensor | None = None,
            dev_status: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
            stream=None):
    """Pack Q and K and run the attention in two launches (had_forward).

    Returns (out, qbits, kbits, sigma_q, sigma_k); the sigmas are None when
    with_sigma is False.
    """
    lib = load_library()
    _need_cuda(q, "q", torch.float32)
    _need_cuda(k, "k", torch.float32)
    _need_cuda(v, "v")
    B, H, n, d = _shape4(q, "q")
    if tuple(k.shape) != (B, H, n, d) or tuple(v.shape) != (B, H, n, d):
        raise ValueError("q, k and v must have the same shape [B, H, n, d]")
    W = words_per_row(d)
    dev = q.device
    if qbits is None:
        qbits = torch.empty((B, H, n, W), dtype=torch.int32, device=dev)
    if kbits is None:
        kbits = torch.empty((B, H, n, W), dtype=torch.int32, device=dev)
    for t, name in ((qbits, "qbits"), (kbits, "kbits")):
        _need_cuda(t, name, torch.int32)
        if tuple(t.shape) != (B, H, n, W):
            raise ValueError(f"{name} must have shape [B, H, n, ceil(d/32)]")
    if out is None:
        out = torch.empty((B, H, n, d), dtype=torch.float32, device=dev)
    _need_cuda(out, "out", torch.float32)
    if tuple(out.shape) != (B, H, n, d):
        raise ValueError("out must have the shape of v")
    shape = Shape(B, H, n, d)
    sh = _stream_handle(dev, stream)
    sq_ptr = sk_ptr = ws_ptr = None
    ws_bytes = 0
    if with_sigma:
        if sigma_q is None:
            sigma_q = torch.empty(1, dtype=torch.float32, device=dev)
        if sigma_k is None:
            sigma_k = torch.empty(1, dtype=torch.float32, device=dev)
        _need_cuda(sigma_q, "sigma_q", torch.float32)
        _need_cuda(sigma_k, "sigma_k", torch.float32)
        need = int(lib.had_forward_workspace_bytes(shape))
        if workspace is None:
            workspace = _workspace(dev, stream, need)
        _need_cuda(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
        sq_ptr, sk_ptr, ws_ptr = sigma_q.data_ptr(), sigma_k.data_ptr(), workspace.data_ptr()
    st_ptr = None
    if dev_status is not None:
        _need_cuda(dev_status, "dev_status", torch.int32)
        st_ptr = dev_status.data_ptr()
    _check("had_forward", lib.had_forward(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), _v_dtype(v), shape, int(topn), float(scale),
        int(bool(causal)), qbits.data_ptr(), kbits.data_ptr(), out.data_ptr(), sq_ptr, sk_ptr,
        ws_ptr, ws_bytes, st_ptr, sh))
    if not with_sigma:
        return out, qbits, kbits, None, None
    return out, qbits, kbits, sigma_q, sigma_k


def forward_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, topn: int, scale: float,
                    causal: bool = False, *, with_sigma: bool = True, out: torch.Tensor | None = None,
                    qbits: torch.Tensor | None = None, kbits: torch.Tensor | None = None,
                    sigma_q: torch.Tensor | None = None, sigma_k: torch.Tensor | None = None,
                    dev_status: torch.Tensor | None = None, stream=None):
    """had_forward_noalloc: forward() without a workspace (the sigma partials
    live in the library's own device array; calls that overlap on one GPU
    race).  The library allocates nothing; tensors not passed in are
    allocated here by torch.  Returns (out, qbits, kbits, sigma_q, sigma_k)."""
    lib = load_library()
    _need_cuda(q, "q", torch.float32)
    _need_cuda(k, "k", torch.float32)
    _need_cuda(v, "v")
    B, H, n, d = _shape4(q, "q")
    if tuple(k.shape) != (B, H, n, d) or tuple(v.shape) != (B, H, n, d):
        raise ValueError("q, k and v must have the same shape [B, H, n, d]")
    W = words_per_row(d)
    dev = q.device
    qbits = torch.empty((B, H, n, W), dtype=torch.int32, device=dev) if qbits is None else qbits
    kbits = torch.empty((B, H, n, W), dtype=torch.int32, device=dev) if kbits is None else kbits
    for t, name in ((qbits, "qbits"), (kbits, "kbits")):
        _need_cuda(t, name, torch.int32)
        if tuple(t.shape) != (B, H, n, W):
            raise ValueError(f"{name} must have shape [B, H, n, ceil(d/32)]")
    out = torch.empty((B, H, n, d), dtype=torch.float32, device=dev) if out is None else out
    _need_cuda(out, "out", torch.float32)
    if tuple(out.shape) != (B, H, n, d):
        raise ValueError("out must have the shape of v")
    sq_ptr = sk_ptr = None
    if with_sigma:
        sigma_q = torch.empty(1, dtype=torch.float32, device=dev) if sigma_q is None else sigma_q
        sigma_k = torch.empty(1, dtype=torch.float32, device=dev) if sigma_k is None else sigma_k
        _need_cuda(sigma_q, "sigma_q", torch.float32)
        _need_cuda(sigma_k, "sigma_k", torch.float32)
        sq_ptr, sk_ptr = sigma_q.data_ptr(), sigma_k.data_ptr()
    st_ptr = None
    if dev_status is not None:
        _need_cuda(dev_status, "dev_status", torch.int32)
        st_ptr = dev_status.data_ptr()
    _check("had_forward_noalloc", lib.had_forward_noalloc(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), _v_dtype(v), Shape(B, H, n, d), int(topn),
        float(scale), int(bool(causal)), qbits.data_ptr(), kbits.data_ptr(), out.data_ptr(),
        sq_ptr, sk_ptr, st_ptr, _stream_handle(dev, stream)))
    if not with_sigma:
        return out, qbits, kbits, None, None
    return out, qbits, kbits, sigma_q, sigma_k


def backward(qbits: torch.Tensor, kbits: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
             dout: torch.Tensor, topn: int, scale: float, causal: bool = False, *,
             sigma_q: torch.Tensor | None = None, sigma_k: torch.Tensor | None = None,
             dq: torch.Tensor | None = None, dk: torch.Tensor | None = None,
             dv: torch.Tensor | None = None, workspace: torch.Tensor | None = None, stream=None):
    """Straight-through backward of attention() (had_backward): returns (dq, dk, dv)
    float32 [B,H,n,d].  out is attention()'s output for the same inputs, dout
    the gradient at out; sigma_q / sigma_k (1-element device tensors, e.g. from
    pack()) divide dq / dk, None meaning 1."""
    lib = load_library()
    _need_cuda(qbits, "qbits", torch.int32)
    _need_cuda(kbits, "kbits", torch.int32)
    _need_cuda(v, "v")
    _need_cuda(out, "out", torch.float32)
    _need_cuda(dout, "dout", torch.float32)
    B, H, n, d = _shape4(v, "v")
    W = words_per_row(d)
    if tuple(qbits.shape) != (B, H, n, W) or tuple(kbits.shape) != (B, H, n, W):
        raise ValueError("qbits/kbits must have shape [B, H, n, ceil(d/32)]")
    if tuple(out.shape) != (B, H, n, d) or tuple(dout.shape) != (B, H, n, d):
        raise ValueError("out and dout must have the shape of v")
    dev = v.device
    grads = []
    for t, name in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        t = torch.empty((B, H, n, d), dtype=torch.float32, device=dev) if t is None else t
        _need_cuda(t, name, torch.float32)
        if tuple(t.shape) != (B, H, n, d):
            raise ValueError(f"{name} must have the shape of v")
        grads.append(t)
    ptrs = []
    for t, name in ((sigma_q, "sigma_q"), (sigma_k, "sigma_k")):
        if t is not None:
            _need_cuda(t, name, torch.float32)
        ptrs.append(None if t is None else t.data_ptr())
    shape = Shape(B, H, n, d)
    need = int(lib.had_backward_workspace_bytes(shape))
    if workspace is None:
        workspace = _workspace(dev, stream, need)
    _need_cuda(workspace, "workspace")
    _check("had_backward", lib.had_backward(
        qbits.data_ptr(), kbits.data_ptr(), v.data_ptr(), _v_dtype(v), shape, int(topn),
        float(scale), int(bool(causal)), out.data_ptr(), dout.data_ptr(), ptrs[0], ptrs[1],
        grads[0].data_ptr(), grads[1].data_ptr(), grads[2].data_ptr(), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream_handle(dev, stream)))
    return tuple(grads)


def _soft_common(q, k, sigma_q, sigma_k):
    _need_cuda(q, "q", torch.float32)
    _need_cuda(k, "k", torch.float32)
    B, H, n, d = _shape4(q, "q")
    if tuple(k.shape) != (B, H, n, d):
        raise ValueError("k must have the shape of q")
    ptrs = []
    for t, name in ((sigma_q, "sigma_q"), (sigma_k, "sigma_k")):
        if t is not None:
            _need_cuda(t, name, torch.float32)
        ptrs.append(None if t is None else t.data_ptr())
    return Shape(B, H, n, d), ptrs


def soft_forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, topn: int, scale: float, c: float,
                 causal: bool = False, *, sigma_q: torch.Tensor | None = None,
                 sigma_k: torch.Tensor | None = None, out: torch.Tensor | None = None,
                 workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """had_soft_forward: the path with tanh(x / (sigma c)) in place of sign;
    returns out float32 [B,H,n,d].  sigma_q / sigma_k are 1-element device
    tensors (e.g. from pack()), None meaning 1."""
    lib = load_library()
    shape, ptrs = _soft_common(q, k, sigma_q, sigma_k)
    _need_cuda(v, "v")
    if tuple(v.shape) != tuple(q.shape):
        raise ValueError("v must have the shape of q")
    dev = q.device
    if out is None:
        out = torch.empty(tuple(q.shape), dtype=torch.float32, device=dev)
    _need_cuda(out, "out", torch.float32)
    need = int(lib.had_soft_workspace_bytes(shape))
    if workspace is None:
        workspace = _workspace(dev, stream, max(need, 256))
    _need_cuda(workspace, "workspace")
    _check("had_soft_forward", lib.had_soft_forward(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), _v_dtype(v), shape, int(topn), float(scale), float(c),
        int(bool(causal)), ptrs[0], ptrs[1], out.data_ptr(), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream_handle(dev, stream)))
    return out


def soft_select(q: torch.Tensor, k: torch.Tensor, topn: int, c: float, causal: bool = False, *,
                sigma_q: torch.Tensor | None = None, sigma_k: torch.Tensor | None = None,
                bh_begin: int = 0, bh_count: int | None = None, workspace: torch.Tensor | None = None,
                stream=None) -> torch.Tensor:
    """had_soft_select: keep mask [bh_count, n, n] uint8 of soft_forward()'s kept sets."""
    lib = load_library()
    shape, ptrs = _soft_common(q, k, sigma_q, sigma_k)
    dev = q.device
    n = shape.seq
    bh_count = shape.batch * shape.heads - bh_begin if bh_count is None else bh_count
    keep = torch.empty((bh_count, n, n), dtype=torch.uint8, device=dev)
    need = int(lib.had_soft_workspace_bytes(shape))
    if workspace is None:
        workspace = _workspace(dev, stream, max(need, 256))
    _need_cuda(workspace, "workspace")
    _check("had_soft_select", lib.had_soft_select(
        q.data_ptr(), k.data_ptr(), shape, int(topn), float(c), int(bool(causal)), ptrs[0], ptrs[1],
        int(bh_begin), int(bh_count), keep.data_ptr(), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), _stream_handle(dev, stream)))
    return keep


def decode_workspace_bytes(batch: int, heads: int, n_q: int, n_k: int, k_stride: int,
                           dim: int) -> int:
    return int(load_library().had_decode_workspace_bytes(
        DecodeShape(batch, heads, n_q, n_k, k_stride, dim)))


def decode(qbits: torch.Tensor, kbits: torch.Tensor, v: torch.Tensor, topn: int, scale: float,
           q_pos0: int = 0, causal: bool = True, *, n_k: int | None = None,
           out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
           stream=None) -> torch.Tensor:
    """New query rows against a key/value cache (had_decode).

    qbits [B,H,n_q,W] int32 (had_pack of the new rows), kbits [B,H,k_stride,W]
    int32, v [B,H,k_stride,d] float32 or bfloat16; the first n_k cache rows are
    valid (default: all).  Returns out [B,H,n_q,d] float32.
    """
    return _decode_call("had_decode", qbits, kbits, v, topn, scale, q_pos0, causal, n_k, out,
                        workspace, stream)


def decode_forward(q: torch.Tensor, kbits: torch.Tensor, v: torch.Tensor, topn: int, scale: float,
                   q_pos0: int = 0, causal: bool = True, *, n_k: int | None = None,
                   out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                   stream=None) -> torch.Tensor:
    """had_decode_forward: as decode(), with the new rows q [B,H,n_q,d] float32
    (their sign words are built inside the first launch; equal to pack + decode)."""
    return _decode_call("had_decode_forward", q, kbits, v, topn, scale, q_pos0, causal, n_k, out,
                        workspace, stream)


def _decode_call(name, qarg, kbits, v, topn, scale, q_pos0, causal, n_k, out, workspace, stream):
    lib = load_library()
    _need_cuda(kbits, "kbits", torch.int32)
    _need_cuda(v, "v")
    B, H, ks, d = _shape4(v, "v")
    W = words_per_row(d)
    if name == "had_decode":
        _need_cuda(qarg, "qbits", torch.int32)
        nq = qarg.shape[2]
        if qarg.dim() != 4 or tuple(qarg.shape) != (B, H, nq, W):
            raise ValueError("qbits must have shape [B, H, n_q, ceil(d/32)]")
    else:
        _need_cuda(qarg, "q", torch.float32)
        nq = qarg.shape[2]
        if qarg.dim() != 4 or tuple(qarg.shape) != (B, H, nq, d):
            raise ValueError("q must have shape [B, H, n_q, d]")
    if tuple(kbits.shape) != (B, H, ks, W):
        raise ValueError("kbits must have shape [B, H, k_stride, ceil(d/32)]")
    nk = ks if n_k is None else int(n_k)
    shape = DecodeShape(B, H, nq, nk, ks, d)
    if out is None:
        out = torch.empty((B, H, nq, d), dtype=torch.float32, device=v.device)
    _need_cuda(out, "out", torch.float32)
    if tuple(out.shape) != (B, H, nq, d):
        raise ValueError("out must have shape [B, H, n_q, d]")
    sh = _stream_handle(v.device, stream)
    need = int(lib.had_decode_workspace_bytes(shape))
    if workspace is None:
        workspace = _workspace(v.device, stream, need)
    _need_cuda(workspace, "workspace")
    _check(name, getattr(lib, name)(
        qarg.data_ptr(), kbits.data_ptr(), v.data_ptr(), _v_dtype(v), shape, int(q_pos0),
        int(topn), float(scale), int(bool(causal)), out.data_ptr(), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), sh))
    return out


def topn_mass(qbits: torch.Tensor, kbits: torch.Tensor, dim: int, scale: float, mass: float,
              causal: bool = False, *, bh_begin: int = 0, bh_count: int | None = None,
              stream=None) -> torch.Tensor:
    """Smallest N per row whose top-N softmax weights reach mass: [bh_count, n] int32."""
    lib = load_library()
    _need_cuda(qbits, "qbits", torch.int32)
    _need_cuda(kbits, "kbits", torch.int32)
    B, H, n, W = _shape4(qbits, "qbits")
    if W != words_per_row(dim) or tuple(kbits.shape) != (B, H, n, W):
        raise ValueError("qbits/kbits must have shape [B, H, n, ceil(dim/32)]")
    if bh_count is None:
        bh_count = B * H - bh_begin
    nout = torch.empty((bh_count, n), dtype=torch.int32, device=qbits.device)
    _check("had_topn_mass", lib.had_topn_mass(
        qbits.data_ptr(), kbits.data_ptr(), Shape(B, H, n, dim), float(scale), int(bool(causal)),
        float(mass), int(bh_begin), int(bh_count), nout.data_ptr(),
        _stream_handle(qbits.device, stream)))
    return nout


def sigma_state(device="cuda") -> torch.Tensor:
    """A zeroed had_sigma_state (4 float64 on the device) for pack_calibrate."""
    return torch.zeros(4, dtype=torch.float64, device=device)


def pack_calibrate(x: torch.Tensor, state: torch.Tensor, *, out: torch.Tensor | None = None,
                   dev_status: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                   stream=None) -> torch.Tensor:
    """Sign bits of x (as pack) and x's count / sum / sum of squares added to state."""
    lib = load_library()
    _need_cuda(x, "x", torch.float32)
    _need_cuda(state, "state", torch.float64)
    if state.numel() != 4:
        raise ValueError("state must hold 4 float64 (had_sigma_state)")
    B, H, n, d = _shape4(x, "x")
    W = words_per_row(d)
    if out is None:
        out = torch.empty((B, H, n, W), dtype=torch.int32, device=x.device)
    _need_cuda(out, "out", torch.int32)
    shape = Shape(B, H, n, d)
    sh = _stream_handle(x.device, stream)
    need = int(lib.had_pack_workspace_bytes(shape))
    if workspace is None:
        workspace = _workspace(x.device, stream, need)
    st_ptr = None
    if dev_status is not None:
        _need_cuda(dev_status, "dev_status", torch.int32)
        st_ptr = dev_status.data_ptr()
    _check("had_pack_calibrate", lib.had_pack_calibrate(
        x.data_ptr(), shape, out.data_ptr(), state.data_ptr(), workspace.data_ptr(),
        workspace.numel() * workspace.element_size(), st_ptr, sh))
    return out


def sigma_from_state(state: torch.Tensor, stream=None) -> torch.Tensor:
    """Population standard deviation of everything added to state (1-element float32)."""
    lib = load_library()
    _need_cuda(state, "state", torch.float64)
    sigma = torch.empty(1, dtype=torch.float32, device=state.device)
    _check("had_sigma_from_state", lib.had_sigma_from_state(
        state.data_ptr(), sigma.data_ptr(), _stream_handle(state.device, stream)))
    return sigma


def logits(qbits: torch.Tensor, kbits: torch.Tensor, dim: int, *, bh_begin: int = 0,
           bh_count: int | None = None, row_begin: int = 0, row_count: int | None = None,
           stream=None) -> torch.Tensor:
    """Integer logits [bh_count, row_count, n] int16 from the kernel's logit stage."""
    lib = load_library()
    _need_cuda(qbits, "qbits", torch.int32)
    _need_cuda(kbits, "kbits", torch.int32)
    B, H, n, W = _shape4(qbits, "qbits")
    if tuple(kbits.shape) != tuple(qbits.shape):
        raise ValueError("kbits must have the shape of qbits")
    bh_count = B * H - bh_begin if bh_count is None else bh_count
    row_count = n - row_begin if row_count is None else row_count
    out = torch.empty((bh_count, row_count, n), dtype=torch.int16, device=qbits.device)
    _check("had_logits", lib.had_logits(
        qbits.data_ptr(), kbits.data_ptr(), Shape(B, H, n, int(dim)), int(bh_begin), int(bh_count),
        int(row_begin), int(row_count), out.data_ptr(), _stream_handle(qbits.device, stream)))
    return out


def select(qbits: torch.Tensor, kbits: torch.Tensor, dim: int, topn: int, causal: bool = False,
           *, bh_begin: int = 0, bh_count: int | None = None, stream=None) -> torch.Tensor:
    """Kept key indices [bh_count, n, topn] int32 (ascending, -1 padded)."""
    lib = load_library()
    _need_cuda(qbits, "qbits", torch.int32)
    _need_cuda(kbits, "kbits", torch.int32)
    B, H, n, W = _shape4(qbits, "qbits")
    if tuple(kbits.shape) != tuple(qbits.shape):
        raise ValueError("kbits must have the shape of qbits")
    bh_count = B * H - bh_begin if bh_count is None else bh_count
    out = torch.empty((bh_count, n, int(topn)), dtype=torch.int32, device=qbits.device)
    _check("had_select", lib.had_select(
        qbits.data_ptr(), kbits.data_ptr(), Shape(B, H, n, int(dim)), int(topn),
        int(bool(causal)), int(bh_begin), int(bh_count), out.data_ptr(),
        _stream_handle(qbits.device, stream)))
    return out
