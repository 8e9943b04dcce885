"""Thin ctypes binding of libqlora_nf4.so.

Argument marshalling only: every step of quantisation, dequantisation and the
linear layer runs in the library's HIP kernels.  PyTorch provides device
memory (tensors) and the current HIP stream.  Functions carry the names of
the C entry points (include/qlora_nf4.h) they call.

The library is loaded on first use from this package directory; if it is
missing or cannot be loaded, every call raises QLoraLibraryError (there is no
fallback).
"""

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqlora_nf4.so")

QLORA_OK = 0
QLORA_ERR_INVALID_ARG = -1
QLORA_ERR_UNSUPPORTED_DTYPE = -2
QLORA_ERR_WORKSPACE_TOO_SMALL = -3
QLORA_ERR_MISALIGNED = -4
QLORA_ERR_HIP = -5
QLORA_ERR_INTERNAL = -6
QLORA_DTYPE_F32 = 0
QLORA_DTYPE_BF16 = 1

# qlora_code_type: the codebook of a quantised weight.  CODE_TYPES are the
# 4-bit types; INT8 (one byte per weight) is QLORA_CODE_INT8.  Every entry
# point takes every type; the linear layer runs Int8 weights on its 256 x 256
# GEMM kernel at every token count (the weight-streaming kernel for few
# tokens takes 4-bit codes only).
QLORA_CODE_NF4 = 0
QLORA_CODE_FP4_E2M1 = 1
QLORA_CODE_FP4_E3M0 = 2
QLORA_CODE_INT4 = 3
QLORA_CODE_INT8 = 4
CODE_TYPES = {"nf4": QLORA_CODE_NF4, "fp4_e2m1": QLORA_CODE_FP4_E2M1, "fp4_e3m0": QLORA_CODE_FP4_E3M0,
              "int4": QLORA_CODE_INT4}
BLOCKSIZE = 64
BLOCKSIZE2 = 256
MAX_RANK = 256

# Every function declared in include/qlora_nf4.h.
EXPORTED = (
    "qlora_nf4_storage_bytes", "qlora_storage_bytes", "qlora_nf4_quantize_workspace", "qlora_linear_workspace",
    "qlora_nf4_codebook", "qlora_codebook", "qlora_status_string", "qlora_last_error",
    "qlora_nf4_quantize", "qlora_nf4_dequantize", "qlora_linear_fwd", "qlora_linear_bwd",
    "qlora_linear_fwd_dropout", "qlora_linear_bwd_dropout",
    "qlora_clip_scale_workspace", "qlora_clip_scale", "qlora_adamw_step",
    "qlora_profile_events", "qlora_linear_fwd_noalloc", "qlora_dropout_mask",
    "qlora_nf4_quantize_batched_workspace", "qlora_nf4_quantize_batched", "qlora_adamw_step_paged",
    "qlora_probe_read",
)
QLORA_KERNEL = {"quantize": 0, "dequantize": 1, "fwd_main": 2, "bwd_dx": 3}


class QLoraLibraryError(RuntimeError):
    pass


class QLoraError(RuntimeError):
    def __init__(self, status, fn, message):
        self.status = status
        super().__init__(f"{fn} failed ({status}: {_status_text(status)}): {message}")


class qlora_nf4_t(ctypes.Structure):
    _fields_ = [
        ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
        ("blocksize", ctypes.c_int32), ("blocksize2", ctypes.c_int32),
        ("double_quant", ctypes.c_int32), ("code_type", ctypes.c_int32),
        ("codes", ctypes.c_void_p), ("absmax_q", ctypes.c_void_p), ("absmax", ctypes.c_void_p),
        ("scale2", ctypes.c_void_p), ("offset", ctypes.c_void_p),
    ]


_lib = None
_vp, _i64, _i32, _f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
_pdesc = ctypes.POINTER(qlora_nf4_t)


def lib():
    """The loaded library (raises QLoraLibraryError if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise QLoraLibraryError(f"{LIB_PATH} not found: build it with "
                                "`python -m bit_nf4_quantized_quantize_amd.build`")
    try:
        L = ctypes.CDLL(LIB_PATH)
    except OSError as e:
        raise QLoraLibraryError(f"cannot load {LIB_PATH}: {e}") from e
    sig = {
        "qlora_nf4_storage_bytes": (_i32, [_i64, _i32, ctypes.POINTER(_i64)]),
        "qlora_storage_bytes": (_i32, [_i64, _i32, _i32, ctypes.POINTER(_i64)]),
        "qlora_nf4_quantize_workspace": (_i32, [_i64, _i32, ctypes.POINTER(_i64)]),
        "qlora_linear_workspace": (_i32, [_i64, _i64, _i64, _i32, ctypes.POINTER(_i64), ctypes.POINTER(_i64)]),
        "qlora_nf4_codebook": (_i32, [ctypes.POINTER(_f32)]),
        "qlora_codebook": (_i32, [_i32, ctypes.POINTER(_f32)]),
        "qlora_status_string": (ctypes.c_char_p, [_i32]),
        "qlora_last_error": (ctypes.c_char_p, []),
        "qlora_nf4_quantize": (_i32, [_vp, _i32, _pdesc, _vp, _i64, _vp]),
        "qlora_nf4_dequantize": (_i32, [_pdesc, _vp, _i32, _vp]),
        "qlora_linear_fwd": (_i32, [_vp, _i64, _pdesc, _vp, _vp, _i32, _f32, _vp, _vp, _vp, _i64, _vp]),
        "qlora_linear_bwd": (_i32, [_vp, _vp, _vp, _i64, _pdesc, _vp, _vp, _i32, _f32, _vp, _vp, _vp, _i32, _vp, _i64,
                                    _vp]),
        "qlora_linear_fwd_dropout": (_i32, [_vp, _i64, _pdesc, _vp, _vp, _i32, _f32, _vp, _f32, _vp, _vp, _vp, _i64,
                                            _vp]),
        "qlora_clip_scale_workspace": (_i32, [_i64, ctypes.POINTER(_i64)]),
        "qlora_clip_scale": (_i32, [_vp, _i64, _f32, _vp, _vp, _i64, _vp]),
        "qlora_adamw_step": (_i32, [_vp, _vp, _vp, _vp, _vp, _i64, _vp, _f32, _f32, _f32, _f32, _f32, _i32, _vp]),
        "qlora_linear_bwd_dropout": (_i32, [_vp, _vp, _vp, _i64, _pdesc, _vp, _vp, _i32, _f32, _vp, _f32, _vp, _vp,
                                            _vp, _i32, _vp, _i64, _vp]),
        "qlora_profile_events": (_i32, [_i32, _vp, _vp]),
        "qlora_linear_fwd_noalloc": (_i32, [_vp, _i64, _pdesc, _vp, _vp, _i32, _f32, _vp, _vp, _vp]),
        "qlora_dropout_mask": (_i32, [ctypes.c_uint64, ctypes.c_uint64, _i64, _i64, _f32, _vp, _vp]),
        "qlora_nf4_quantize_batched_workspace": (_i32, [_pdesc, _i32, ctypes.POINTER(_i64)]),
        "qlora_nf4_quantize_batched": (_i32, [ctypes.POINTER(_vp), _i32, _pdesc, _i32, _vp, _i64, _vp]),
        "qlora_adamw_step_paged": (_i32, [_vp, _vp, _vp, _vp, _vp, _i64, _vp, _f32, _f32, _f32, _f32, _f32, _i32,
                                          _vp, _i64, _vp, _vp]),
        "qlora_probe_read": (_i32, [_vp, _i64, _vp, _vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype, f.argtypes = res, args
    _lib = L
    return L


def _status_text(status):
    try:
        return lib().qlora_status_string(status).decode()
    except QLoraLibraryError:
        return "?"


def _check(status, fn):
    if status != QLORA_OK:
        raise QLoraError(status, fn, lib().qlora_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("qlora_nf4 tensors must live on a HIP device")


# ------------------------------------------------------------ host queries

def qlora_nf4_storage_bytes(numel, double_quant=True):
    out = (_i64 * 5)()
    _check(lib().qlora_nf4_storage_bytes(numel, int(double_quant), out), "qlora_nf4_storage_bytes")
    return dict(zip(("codes", "absmax_q", "absmax", "scale2", "offset"), list(out)))


def qlora_storage_bytes(numel, double_quant=True, code_type=QLORA_CODE_NF4):
    out = (_i64 * 5)()
    _check(lib().qlora_storage_bytes(numel, int(double_quant), int(code_type), out), "qlora_storage_bytes")
    return dict(zip(("codes", "absmax_q", "absmax", "scale2", "offset"), list(out)))


def qlora_nf4_quantize_workspace(numel, double_quant=True):
    ws = _i64(0)
    _check(lib().qlora_nf4_quantize_workspace(numel, int(double_quant), ctypes.byref(ws)),
           "qlora_nf4_quantize_workspace")
    return ws.value


def qlora_linear_workspace(M, N, K, r):
    f, b = _i64(0), _i64(0)
    _check(lib().qlora_linear_workspace(M, N, K, r, ctypes.byref(f), ctypes.byref(b)), "qlora_linear_workspace")
    return f.value, b.value


def qlora_codebook(code_type):
    out = (_f32 * (256 if int(code_type) == QLORA_CODE_INT8 else 16))()
    _check(lib().qlora_codebook(int(code_type), out), "qlora_codebook")
    return list(out)


def qlora_nf4_codebook():
    out = (_f32 * 16)()
    _check(lib().qlora_nf4_codebook(out), "qlora_nf4_codebook")
    return list(out)


def qlora_profile_events(kernel, start=None, stop=None):
    """Attach (or detach, with None) a pair of hipEvent_t handles (ints or
    ctypes.c_void_p, created with hipEventCreate) to a kernel of the library
    for the calling thread."""
    kid = QLORA_KERNEL[kernel]
    _check(lib().qlora_profile_events(kid, start, stop), "qlora_profile_events")


def qlora_probe_read(buf, out, stream=None):
    """Measurement probe: one streaming read of the device tensor `buf`
    (contiguous, 16-byte aligned, a multiple of 16 bytes); `out` is a device
    tensor of at least 4 bytes the kernel may write."""
    _need_cuda(buf, out)
    _check(lib().qlora_probe_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(out), _stream(stream)),
           "qlora_probe_read")


# ----------------------------------------------------------- quantised weight

class NF4Weight:
    """Device buffers of one NF4-quantised weight [rows, cols] (or one of
    another storage type, `code_type`) plus the C descriptor that points at
    them."""

    def __init__(self, rows, cols, double_quant=True, device=None, code_type=QLORA_CODE_NF4):
        self.rows, self.cols, self.double_quant = int(rows), int(cols), bool(double_quant)
        self.code_type = int(code_type)
        sizes = qlora_storage_bytes(self.rows * self.cols, self.double_quant, self.code_type)
        dev = device if device is not None else torch.device("cuda", torch.cuda.current_device())
        u8 = torch.uint8
        # Pad every buffer to a 16-byte multiple so vector accesses never leave it.
        pad = lambda n: max(16, (n + 15) // 16 * 16)  # noqa: E731
        self.codes = torch.empty(pad(sizes["codes"]), dtype=u8, device=dev)
        self.absmax_q = torch.empty(pad(sizes["absmax_q"]), dtype=u8, device=dev) if double_quant else None
        self.absmax = torch.empty(pad(sizes["absmax"]) // 4, dtype=torch.float32, device=dev) if not double_quant else None
        self.scale2 = torch.empty(pad(sizes["scale2"]) // 4, dtype=torch.float32, device=dev) if double_quant else None
        self.offset = torch.empty(4, dtype=torch.float32, device=dev) if double_quant else None
        self.sizes = sizes

    @property
    def numel(self):
        return self.rows * self.cols

    def desc(self):
        d = qlora_nf4_t()
        d.rows, d.cols = self.rows, self.cols
        d.blocksize, d.blocksize2 = BLOCKSIZE, BLOCKSIZE2
        d.double_quant = int(self.double_quant)
        d.code_type = self.code_type
        d.codes = self.codes.data_ptr()
        d.absmax_q = self.absmax_q.data_ptr() if self.absmax_q is not None else None
        d.absmax = self.absmax.data_ptr() if self.absmax is not None else None
        d.scale2 = self.scale2.data_ptr() if self.scale2 is not None else None
        d.offset = self.offset.data_ptr() if self.offset is not None else None
        return d

    # host copies of the stored buffers, trimmed to their true sizes
    def host(self):
        s = self.sizes
        out = {"codes": self.codes[:s["codes"]].cpu().numpy()}
        if self.double_quant:
            out["absmax_q"] = self.absmax_q[:s["absmax_q"]].cpu().numpy()
            out["scale2"] = self.scale2[:s["scale2"] // 4].cpu().numpy()
            out["offset"] = self.offset[:1].cpu().numpy()
        else:
            out["absmax"] = self.absmax[:s["absmax"] // 4].cpu().numpy()
        return out


# ---------------------------------------------------------- device entry points

def qlora_nf4_quantize(w, double_quant=True, out=None, workspace=None, stream=None, code_type=QLORA_CODE_NF4):
    """Quantise fp32 or bf16 tensor `w` ([rows, cols] or 1-D) into an
    NF4Weight (new or `out`; `out` keeps its own code_type).  `code_type`
    (a QLORA_CODE_* value) picks the codebook of a new weight.
    `workspace`: optional uint8 device tensor of at least
    qlora_nf4_quantize_workspace bytes."""
    _need_cuda(w)
    if not w.is_contiguous():
        raise ValueError("w must be contiguous")
    dtype = {torch.float32: QLORA_DTYPE_F32, torch.bfloat16: QLORA_DTYPE_BF16}.get(w.dtype)
    if dtype is None:
        raise ValueError("w must be float32 or bfloat16")
    rows, cols = (w.shape[0], w.shape[1]) if w.dim() == 2 else (1, w.numel())
    q = out if out is not None else NF4Weight(rows, cols, double_quant, w.device, code_type)
    nws = qlora_nf4_quantize_workspace(q.numel, q.double_quant)
    ws = workspace if workspace is not None else torch.empty(max(nws, 16), dtype=torch.uint8, device=w.device)
    if ws.numel() < nws:
        raise ValueError(f"quantize workspace needs {nws} bytes")
    nws = ws.numel()
    d = q.desc()
    _check(lib().qlora_nf4_quantize(_ptr(w), dtype, ctypes.byref(d), _ptr(ws), nws, _stream(stream)),
           "qlora_nf4_quantize")
    q._ws = ws  # keep the workspace alive until the stream has used it
    return q


def qlora_nf4_quantize_batched(ws_list, outs, workspace=None, stream=None):
    """Quantise the tensors in ws_list (all float32 or all bfloat16) into the
    NF4Weight objects in outs (sharing code_type and double_quant) with one
    batched call; returns outs."""
    n = len(ws_list)
    if n != len(outs):
        raise ValueError("one output weight per input tensor")
    if n == 0:
        return outs
    _need_cuda(*ws_list)
    dtype = {torch.float32: QLORA_DTYPE_F32, torch.bfloat16: QLORA_DTYPE_BF16}.get(ws_list[0].dtype)
    if dtype is None or any(w.dtype != ws_list[0].dtype or not w.is_contiguous() for w in ws_list):
        raise ValueError("inputs must be contiguous and all float32 or all bfloat16")
    for w, q in zip(ws_list, outs):
        if w.numel() != q.numel:
            raise ValueError("each input must have its weight's number of elements")
    descs = (qlora_nf4_t * n)(*[q.desc() for q in outs])
    ptrs = (_vp * n)(*[w.data_ptr() for w in ws_list])
    nws = _i64(0)
    _check(lib().qlora_nf4_quantize_batched_workspace(descs, n, ctypes.byref(nws)), "qlora_nf4_quantize_batched_workspace")
    ws = workspace if workspace is not None else torch.empty(max(nws.value, 16), dtype=torch.uint8,
                                                             device=ws_list[0].device)
    if ws.numel() < nws.value:
        raise ValueError(f"batched quantize workspace needs {nws.value} bytes")
    _check(lib().qlora_nf4_quantize_batched(ptrs, dtype, descs, n, _ptr(ws), ws.numel(), _stream(stream)),
           "qlora_nf4_quantize_batched")
    for q in outs:
        q._ws = ws
    return outs


def qlora_nf4_dequantize(q, dtype=torch.bfloat16, out=None, stream=None):
    code = {torch.float32: QLORA_DTYPE_F32, torch.bfloat16: QLORA_DTYPE_BF16}.get(dtype)
    if code is None:
        raise ValueError("dtype must be float32 or bfloat16")
    if out is None:
        out = torch.empty((q.rows, q.cols), dtype=dtype, device=q.codes.device)
    _need_cuda(out)
    d = q.desc()
    _check(lib().qlora_nf4_dequantize(ctypes.byref(d), _ptr(out), code, _stream(stream)), "qlora_nf4_dequantize")
    return out


def _bf16_2d(t, name, shape):
    if t.dtype != torch.bfloat16 or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be a contiguous bfloat16 tensor of shape {tuple(shape)}")


class Workspace:
    """Grow-only device scratch for the linear entry points."""

    def __init__(self):
        self.buf = None

    def get(self, nbytes, device):
        if self.buf is None or self.buf.numel() < nbytes or self.buf.device != device:
            self.buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        return self.buf


_default_ws = {}


def _ws(nbytes, device, ws):
    if ws is None:
        ws = _default_ws.setdefault((device.type, device.index), Workspace())
    return ws.get(nbytes, device)


def pack_keep_mask(keep):
    """Bit-pack a boolean keep mask [M, K] (K % 8 == 0) into the uint8 [M, K/8]
    layout the dropout entry points take: bit j of byte (m, c) is keep[m, 8c + j]."""
    if keep.dtype != torch.bool or keep.dim() != 2 or keep.shape[1] % 8:
        raise ValueError("keep must be a bool [M, K] tensor with K % 8 == 0")
    w = (1 << torch.arange(8, device=keep.device, dtype=torch.int32))
    return (keep.view(keep.shape[0], -1, 8).to(torch.int32) * w).sum(-1).to(torch.uint8).contiguous()


def qlora_dropout_mask(seed, offset, M, K, p, out=None, device=None, stream=None):
    """The packed keep mask u8 [M, K/8] of LoRA dropout with drop probability
    p, drawn on the device from Philox4x64-10 keyed by (seed, offset)."""
    if out is None:
        dev = device if device is not None else torch.device("cuda", torch.cuda.current_device())
        out = torch.empty((M, K // 8), dtype=torch.uint8, device=dev)
    _need_cuda(out)
    if out.dtype != torch.uint8 or tuple(out.shape) != (M, K // 8) or not out.is_contiguous():
        raise ValueError("out must be a contiguous uint8 [M, K/8] tensor")
    _check(lib().qlora_dropout_mask(int(seed) & (2 ** 64 - 1), int(offset) & (2 ** 64 - 1), M, K, float(p),
                                    _ptr(out), _stream(stream)), "qlora_dropout_mask")
    return out


def _keep_arg(keep, X, p):
    if keep is None:
        return None
    _need_cuda(keep)
    if keep.dtype != torch.uint8 or tuple(keep.shape) != (X.shape[0], X.shape[1] // 8) or not keep.is_contiguous():
        raise ValueError("keep must be a contiguous uint8 [M, K/8] bit mask (see pack_keep_mask)")
    if not 0.0 <= float(p) < 1.0:
        raise ValueError("dropout p must be in [0, 1)")
    return keep


def qlora_linear_fwd(X, q, A, B, s, save_xa=True, Y=None, XA=None, workspace=None, stream=None, keep=None, p=0.0):
    """Y = X W_bf16^T + s (X A) B.  Returns (Y, XA or None).  With `keep`
    (a pack_keep_mask bit mask of X) and drop probability p the adapter sees
    X * keep / (1 - p) (LoRA dropout)."""
    _need_cuda(X, A, B)
    M, K = X.shape
    N, r = q.rows, A.shape[1]
    _bf16_2d(X, "X", (M, q.cols))
    _bf16_2d(A, "A", (K, r))
    _bf16_2d(B, "B", (r, N))
    keep = _keep_arg(keep, X, p)
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=X.device)
    if save_xa and XA is None:
        XA = torch.empty((M, r), dtype=torch.bfloat16, device=X.device)
    nws, _ = qlora_linear_workspace(M, N, K, r)
    ws = _ws(nws, X.device, workspace)
    d = q.desc()
    if keep is None:
        _check(lib().qlora_linear_fwd(_ptr(X), M, ctypes.byref(d), _ptr(A), _ptr(B), r, float(s), _ptr(Y),
                                      _ptr(XA) if save_xa else None, _ptr(ws), ws.numel(), _stream(stream)),
               "qlora_linear_fwd")
    else:
        _check(lib().qlora_linear_fwd_dropout(_ptr(X), M, ctypes.byref(d), _ptr(A), _ptr(B), r, float(s),
                                              _ptr(keep), float(p), _ptr(Y), _ptr(XA) if save_xa else None,
                                              _ptr(ws), ws.numel(), _stream(stream)),
               "qlora_linear_fwd_dropout")
    return Y, (XA if save_xa else None)


def qlora_linear_bwd(dY, X, XA, q, A, B, s, need_dx=True, dX=None, dA=None, dB=None, workspace=None, stream=None,
                     keep=None, p=0.0, accumulate=False):
    """Returns (dX or None, dA, dB) for Y = X W_bf16^T + s (X A) B; with
    `keep` and p, the gradients of the dropout forward (same mask).  XA may
    be None: the library then recomputes it (bit-identical to the forward's).
    With `accumulate` the gradients are added to the given dA and dB."""
    _need_cuda(dY, X, XA, A, B)
    M, K = X.shape
    N, r = q.rows, A.shape[1]
    keep = _keep_arg(keep, X, p)
    _bf16_2d(dY, "dY", (M, N))
    _bf16_2d(X, "X", (M, q.cols))
    if XA is not None:
        _bf16_2d(XA, "XA", (M, r))
    _bf16_2d(A, "A", (K, r))
    _bf16_2d(B, "B", (r, N))
    dev = X.device
    if accumulate and (dA is None or dB is None):
        raise ValueError("accumulate needs the dA and dB to add to")
    if need_dx and dX is None:
        dX = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    if dA is None:
        dA = torch.empty((K, r), dtype=torch.bfloat16, device=dev)
    if dB is None:
        dB = torch.empty((r, N), dtype=torch.bfloat16, device=dev)
    _bf16_2d(dA, "dA", (K, r))
    _bf16_2d(dB, "dB", (r, N))
    _need_cuda(dA, dB)
    _, nws = qlora_linear_workspace(M, N, K, r)
    ws = _ws(nws, dev, workspace)
    d = q.desc()
    acc = 1 if accumulate else 0
    if keep is None:
        _check(lib().qlora_linear_bwd(_ptr(dY), _ptr(X), _ptr(XA), M, ctypes.byref(d), _ptr(A), _ptr(B), r, float(s),
                                      _ptr(dX) if need_dx else None, _ptr(dA), _ptr(dB), acc, _ptr(ws), ws.numel(),
                                      _stream(stream)),
               "qlora_linear_bwd")
    else:
        _check(lib().qlora_linear_bwd_dropout(_ptr(dY), _ptr(X), _ptr(XA), M, ctypes.byref(d), _ptr(A), _ptr(B), r,
                                              float(s), _ptr(keep), float(p), _ptr(dX) if need_dx else None,
                                              _ptr(dA), _ptr(dB), acc, _ptr(ws), ws.numel(), _stream(stream)),
               "qlora_linear_bwd_dropout")
    return (dX if need_dx else None), dA, dB


# ------------------------------------------------------ LoRA optimizer step

def qlora_clip_scale(grad, max_norm=0.3, scale=None, workspace=None, stream=None):
    """Device fp32 scalar min(1, max_norm / (||grad|| + 1e-6)) for a flat bf16
    gradient tensor (all LoRA gradients)."""
    _need_cuda(grad)
    if grad.dtype != torch.bfloat16 or not grad.is_contiguous():
        raise ValueError("grad must be a contiguous bf16 tensor")
    n = grad.numel()
    if scale is None:
        scale = torch.empty(4, dtype=torch.float32, device=grad.device)
    nws = _i64(0)
    _check(lib().qlora_clip_scale_workspace(n, ctypes.byref(nws)), "qlora_clip_scale_workspace")
    ws = _ws(nws.value, grad.device, workspace)
    _check(lib().qlora_clip_scale(_ptr(grad), n, float(max_norm), _ptr(scale), _ptr(ws), ws.numel(), _stream(stream)),
           "qlora_clip_scale")
    return scale


def qlora_adamw_step(param, grad, exp_avg, exp_avg_sq, step, lr, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.0,
                     grad_scale=None, param_bf16=None, stream=None):
    """One AdamW step in place on flat fp32 `param`, `exp_avg`, `exp_avg_sq`
    (device or pinned host tensors for the states) with flat bf16 `grad`;
    `grad_scale` a device fp32 scalar (qlora_clip_scale) or None; writes the
    bf16 copy of the updated parameters into `param_bf16` when given."""
    _need_cuda(param, grad)
    n = param.numel()
    for t, name, dt in ((param, "param", torch.float32), (grad, "grad", torch.bfloat16),
                        (exp_avg, "exp_avg", torch.float32), (exp_avg_sq, "exp_avg_sq", torch.float32)):
        if t.dtype != dt or t.numel() != n or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dt} tensor of {n} elements")
    for t, name in ((exp_avg, "exp_avg"), (exp_avg_sq, "exp_avg_sq")):
        if not (t.is_cuda or t.is_pinned()):
            raise ValueError(f"{name} must be on the GPU or in pinned host memory")
    if param_bf16 is not None and (param_bf16.dtype != torch.bfloat16 or param_bf16.numel() != n):
        raise ValueError("param_bf16 must be a bf16 tensor of the parameters' size")
    _check(lib().qlora_adamw_step(_ptr(param), _ptr(param_bf16) if param_bf16 is not None else None, _ptr(grad),
                                  _ptr(exp_avg), _ptr(exp_avg_sq), n,
                                  _ptr(grad_scale) if grad_scale is not None else None, float(lr), float(betas[0]),
                                  float(betas[1]), float(eps), float(weight_decay), int(step), _stream(stream)),
           "qlora_adamw_step")
    return param


def qlora_adamw_step_paged(param, grad, exp_avg, exp_avg_sq, step, lr, staging, betas=(0.9, 0.999), eps=1e-8,
                           weight_decay=0.0, grad_scale=None, param_bf16=None, stream=None, copy_stream=None):
    """qlora_adamw_step with exp_avg and exp_avg_sq in pinned host memory,
    paged through the uint8 device tensor `staging` chunk by chunk; copies
    run on `copy_stream` (a torch.cuda.Stream) when given, overlapping the
    updates."""
    _need_cuda(param, grad, staging)
    n = param.numel()
    for t, name, dt in ((param, "param", torch.float32), (grad, "grad", torch.bfloat16),
                        (exp_avg, "exp_avg", torch.float32), (exp_avg_sq, "exp_avg_sq", torch.float32)):
        if t.dtype != dt or t.numel() != n or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dt} tensor of {n} elements")
    for t, name in ((exp_avg, "exp_avg"), (exp_avg_sq, "exp_avg_sq")):
        if t.is_cuda or not t.is_pinned():
            raise ValueError(f"{name} must be in pinned host memory")
    if param_bf16 is not None and (param_bf16.dtype != torch.bfloat16 or param_bf16.numel() != n):
        raise ValueError("param_bf16 must be a bf16 tensor of the parameters' size")
    cs = ctypes.c_void_p(copy_stream.cuda_stream) if copy_stream is not None else None
    _check(lib().qlora_adamw_step_paged(_ptr(param), _ptr(param_bf16) if param_bf16 is not None else None, _ptr(grad),
                                        _ptr(exp_avg), _ptr(exp_avg_sq), n,
                                        _ptr(grad_scale) if grad_scale is not None else None, float(lr),
                                        float(betas[0]), float(betas[1]), float(eps), float(weight_decay), int(step),
                                        _ptr(staging), staging.numel(), _stream(stream), cs),
           "qlora_adamw_step_paged")
    return param
