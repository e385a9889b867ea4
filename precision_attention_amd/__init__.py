"""FP4 attention with Direct-P for MI355X (gfx950): Python binding of ``libfp4attn.so``.

Argument marshalling only: every step of the computation runs in the HIP kernels behind the
C ABI in ``include/fp4attn.h``. PyTorch supplies device memory and the current stream. The
library must be built (``__graft_entry__.build()`` or ``python -m precision_attention_amd.build``);
there is no fallback of any kind when it is missing.

Method: "Hardware-Aware FP4 FlashAttention-4" (arXiv:2609.04105), gist.science technical
summary (Methodology 1 "Direct-P for Forward Inference", Methodology 2 "Quantized Causal
Backward") and the arXiv abstract.
"""
from __future__ import annotations

import ctypes
import functools
import os
from dataclasses import dataclass

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_lib", "libfp4attn.so")

MXFP4 = 1
MXFP8 = 2
ALONG_D = 0
ALONG_SEQ = 1

STATUS = {0: "OK", 1: "ERR_NULL", 2: "ERR_SHAPE", 3: "ERR_UNSUPPORTED", 4: "ERR_ALIGN", 5: "ERR_FORMAT",
          6: "ERR_LAUNCH", 7: "ERR_SCRATCH"}
NOALLOC_SCRATCH_BYTES = 72 << 20  # FP4ATTN_NOALLOC_SCRATCH_BYTES

EXPORTED = [
    "fp4attn_mx_codes_bytes", "fp4attn_mx_scales_bytes", "fp4attn_quantize_mx", "fp4attn_quantize_mx_batch",
    "fp4attn_project_qkv", "fp4attn_project_qkv_ex", "fp4attn_quantize_nvfp4", "fp4attn_fwd_nvfp4", "fp4attn_fwd", "fp4attn_fwd_ex",
    "fp4attn_fwd_bf16",
    "fp4attn_bwd_workspace_bytes", "fp4attn_bwd", "fp4attn_bwd_noalloc", "fp4attn_key_block", "fp4attn_status_str",
    "fp4attn_clock_probe",
]


class Fp4AttnError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__("%s failed: %s (%s)" % (what, STATUS.get(status, status), _status_str(status)))
        self.status = status


class _MX(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("axis", ctypes.c_int32), ("codes", ctypes.c_void_p),
                ("scales", ctypes.c_void_p)]


class _QuantJob(ctypes.Structure):
    _fields_ = [("x_bf16", ctypes.c_void_p), ("heads", ctypes.c_int64), ("out", _MX)]


MAX_QUANT_JOBS = 4

_lib = None


def library_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """Load libfp4attn.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError("libfp4attn.so is not built (%s); run __graft_entry__.build()" % _LIB_PATH)
        L = ctypes.CDLL(_LIB_PATH)
        i64, i32, vp, sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
        mxp = ctypes.POINTER(_MX)
        L.fp4attn_mx_codes_bytes.argtypes = [i32, i64, i64, i64, i64]
        L.fp4attn_mx_codes_bytes.restype = sz
        L.fp4attn_mx_scales_bytes.argtypes = [i64, i64, i64, i64]
        L.fp4attn_mx_scales_bytes.restype = sz
        L.fp4attn_quantize_mx.argtypes = [vp, mxp, i64, i64, i64, i64, vp]
        L.fp4attn_quantize_mx.restype = i32
        L.fp4attn_quantize_mx_batch.argtypes = [ctypes.POINTER(_QuantJob), i32, i64, i64, i64, vp]
        L.fp4attn_quantize_mx_batch.restype = i32
        L.fp4attn_project_qkv.argtypes = [vp, vp, mxp, mxp, mxp, mxp, mxp, mxp, i64, i64, i64, i64, i64, i64, vp]
        L.fp4attn_project_qkv.restype = i32
        L.fp4attn_project_qkv_ex.argtypes = [vp, vp, mxp, mxp, mxp, mxp, mxp, mxp, i64, i64, i64, i64, i64, i64, i32, vp]
        L.fp4attn_project_qkv_ex.restype = i32
        L.fp4attn_quantize_nvfp4.argtypes = [vp, vp, vp, vp, i32, i64, i64, i64, i64, vp]
        L.fp4attn_quantize_nvfp4.restype = i32
        L.fp4attn_fwd_nvfp4.argtypes = [vp, vp, mxp, vp, vp, i64, i64, i64, i64, i64, vp, vp, vp]
        L.fp4attn_fwd_nvfp4.restype = i32
        L.fp4attn_fwd.argtypes = [mxp, mxp, mxp, vp, vp, i64, i64, i64, i64, i64, i32, vp]
        L.fp4attn_fwd.restype = i32
        L.fp4attn_fwd_ex.argtypes = [mxp, mxp, mxp, vp, vp, i64, i64, i64, i64, i64, i32, ctypes.c_uint, vp, vp, vp]
        L.fp4attn_fwd_ex.restype = i32
        L.fp4attn_fwd_bf16.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, vp]
        L.fp4attn_fwd_bf16.restype = i32
        L.fp4attn_bwd_workspace_bytes.argtypes = [i64, i64, i64, i64, i64]
        L.fp4attn_bwd_workspace_bytes.restype = sz
        L.fp4attn_bwd.argtypes = [mxp, mxp, mxp, mxp, mxp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i32,
                                  vp]
        L.fp4attn_bwd.restype = i32
        L.fp4attn_bwd_noalloc.argtypes = [mxp, mxp, mxp, mxp, mxp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                          i32, vp]
        L.fp4attn_bwd_noalloc.restype = i32
        L.fp4attn_key_block.argtypes = [i64, i32]
        L.fp4attn_key_block.restype = i32
        L.fp4attn_status_str.argtypes = [i32]
        L.fp4attn_status_str.restype = ctypes.c_char_p
        L.fp4attn_clock_probe.argtypes = [vp, i32, i32, ctypes.POINTER(i32), vp]
        L.fp4attn_clock_probe.restype = i32
        _lib = L
    return _lib


def _status_str(status: int) -> str:
    try:
        return lib().fp4attn_status_str(status).decode()
    except Exception:  # noqa: BLE001 - only used to decorate an error message
        return "?"


def _check(status: int, what: str):
    if status != 0:
        raise Fp4AttnError(status, what)


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


# ---- host-side checks: the C ABI receives raw pointers and cannot check buffer sizes, so every
# tensor is checked here (shape, dtype, contiguity, device) before any call; a mismatch raises
# ValueError and nothing is enqueued.

def _check_tensor(t, name: str, dtype, shape, device):
    if not isinstance(t, torch.Tensor):
        raise ValueError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))


def _check_mx(m, name: str, fmt: int | None, axis: int | None, shape, device):
    """An MXTensor of logical shape `shape` whose code and scale buffers hold at least the bytes
    the library reads and writes for it."""
    if not isinstance(m, MXTensor):
        raise ValueError("%s must be an MXTensor" % name)
    if fmt is not None and m.fmt != fmt:
        raise ValueError("%s must have format %d, got %d" % (name, fmt, m.fmt))
    if axis is not None and m.axis != axis:
        raise ValueError("%s must be blocked along axis %d, got %d" % (name, axis, m.axis))
    if tuple(m.shape) != tuple(shape):
        raise ValueError("%s must have logical shape %s, got %s" % (name, tuple(shape), tuple(m.shape)))
    need_c, need_s = _mx_bytes(m.fmt, *shape)
    for buf, need, what in ((m.codes, need_c, "codes"), (m.scales, need_s, "scales")):
        if not isinstance(buf, torch.Tensor) or buf.dtype != torch.uint8 or not buf.is_contiguous():
            raise ValueError("%s.%s must be a contiguous uint8 tensor" % (name, what))
        if buf.numel() < need:
            raise ValueError("%s.%s holds %d bytes, %d needed" % (name, what, buf.numel(), need))
        if device is not None and buf.device != device:
            raise ValueError("%s.%s is on %s, expected %s" % (name, what, buf.device, device))


@functools.lru_cache(maxsize=256)
def _mx_bytes(fmt: int, B: int, heads: int, N: int, D: int):
    """(codes bytes, scales bytes) of an MX tensor, as the library computes them."""
    return (int(lib().fp4attn_mx_codes_bytes(fmt, B, heads, N, D)), int(lib().fp4attn_mx_scales_bytes(B, heads, N, D)))


def _check_heads(H: int, Hkv: int):
    if Hkv < 1 or H % Hkv != 0:
        raise ValueError("the query heads (%d) must be a multiple of the key/value heads (%d)" % (H, Hkv))


def _require_gpu_device(device):
    if device.type != "cuda":
        raise ValueError("the tensors must be on a GPU device, got %s" % device)


@dataclass
class MXTensor:
    """One MX-quantized [B, heads, N, D] tensor on the device (layout: include/fp4attn.h)."""
    codes: torch.Tensor  # uint8
    scales: torch.Tensor  # uint8
    fmt: int
    axis: int
    shape: tuple

    def c_struct(self) -> _MX:
        return _MX(self.fmt, self.axis, self.codes.data_ptr(), self.scales.data_ptr())


def mx_empty(B, heads, N, D, fmt, axis, device) -> MXTensor:
    L = lib()
    nc = L.fp4attn_mx_codes_bytes(fmt, B, heads, N, D)
    ns = L.fp4attn_mx_scales_bytes(B, heads, N, D)
    codes = torch.empty(max(nc, 16), dtype=torch.uint8, device=device)[:nc]
    scales = torch.empty(max(ns, 16), dtype=torch.uint8, device=device)[:ns]
    return MXTensor(codes, scales, fmt, axis, (B, heads, N, D))


def quantize_mx(x: torch.Tensor, fmt: int, axis: int, out: MXTensor | None = None) -> MXTensor:
    """MX-quantize a bf16 [B, heads, N, D] device tensor (fp4attn_quantize_mx)."""
    if x.dtype != torch.bfloat16 or not x.is_contiguous() or x.dim() != 4:
        raise ValueError("x must be a contiguous 4-D bfloat16 tensor")
    B, heads, N, D = x.shape
    if out is None:
        out = mx_empty(B, heads, N, D, fmt, axis, x.device)
    _check_mx(out, "out", fmt, axis, (B, heads, N, D), x.device)
    _require_gpu_device(x.device)
    s = out.c_struct()
    _check(lib().fp4attn_quantize_mx(x.data_ptr(), ctypes.byref(s), B, heads, N, D, _stream(x.device)),
           "fp4attn_quantize_mx")
    return out


class QuantizeBatchCall:
    """A validated fp4attn_quantize_mx_batch call over fixed buffers: the checks run once, here;
    each call then passes the stored arguments and the stream (default: the current stream of the
    tensors' device). The tensors must stay alive and keep their shapes while the object is used."""

    def __init__(self, xs, fmts, axes, outs=None):
        xs = list(xs)
        if not 1 <= len(xs) <= MAX_QUANT_JOBS or len(fmts) != len(xs) or len(axes) != len(xs):
            raise ValueError("one to %d tensors, each with a format and an axis" % MAX_QUANT_JOBS)
        B, _, N, D = xs[0].shape
        for x in xs:
            if x.dtype != torch.bfloat16 or not x.is_contiguous() or x.dim() != 4:
                raise ValueError("every x must be a contiguous 4-D bfloat16 tensor")
            if x.shape[0] != B or x.shape[2] != N or x.shape[3] != D:
                raise ValueError("the tensors must share B, N and D")
        if outs is None:
            outs = [mx_empty(B, x.shape[1], N, D, f, a, x.device) for x, f, a in zip(xs, fmts, axes)]
        if len(outs) != len(xs):
            raise ValueError("one output per input tensor")
        for i, (x, o, f, a) in enumerate(zip(xs, outs, fmts, axes)):
            if x.device != xs[0].device:
                raise ValueError("the tensors must share one device")
            _check_mx(o, "outs[%d]" % i, f, a, tuple(x.shape), x.device)
        _require_gpu_device(xs[0].device)
        self.jobs = (_QuantJob * len(xs))()
        for i, (x, o) in enumerate(zip(xs, outs)):
            self.jobs[i].x_bf16 = x.data_ptr()
            self.jobs[i].heads = x.shape[1]
            self.jobs[i].out = o.c_struct()
        self.args = (self.jobs, len(xs), B, N, D)
        self.device = xs[0].device
        self.outs, self._keep = outs, xs
        self._fn = lib().fp4attn_quantize_mx_batch

    def __call__(self, stream=None):
        _check(self._fn(*self.args, _stream(self.device) if stream is None else stream), "fp4attn_quantize_mx_batch")
        return self.outs


def quantize_mx_batch(xs, fmts, axes, outs=None) -> list:
    """MX-quantize up to four bf16 [B, heads_i, N, D] device tensors sharing B, N and D in one launch
    (fp4attn_quantize_mx_batch); job i uses fmts[i] and axes[i]."""
    return QuantizeBatchCall(xs, fmts, axes, outs)()


class ProjectCall:
    """A validated fp4attn_project_qkv call over fixed buffers (see QuantizeBatchCall): the QKV
    projection X [B, N, Dm] times the weight W [(H + 2 Hkv) D, Dm] (rows of Wq, then Wk, then Wv)
    with the MX quantization in its epilogue. ``outs`` holds the MXTensors q, k (MXFP4 along D), v
    (along the sequence, ``v_fmt``) and, with ``fp8_views``, q8, k8 (MXFP8 along the sequence) and
    v8 (MXFP8 along D); missing ones are allocated. ``tile``: 0 lets the library choose, 128 or 256
    fixes the workgroup tile at 256 tokens by that many features (fp4attn_project_qkv_ex; every
    tile gives the same bytes)."""

    def __init__(self, x: torch.Tensor, w: torch.Tensor, H: int, Hkv: int, D: int, v_fmt: int = MXFP4,
                 fp8_views: bool = False, outs: dict | None = None, tile: int = 0):
        if x.dim() != 3 or w.dim() != 2:
            raise ValueError("x must be [B, N, Dm] and w [(H + 2 Hkv) D, Dm]")
        if tile not in (0, 128, 256):
            raise ValueError("tile must be 0, 128 or 256")
        B, N, Dm = x.shape
        dev = x.device
        _check_heads(H, Hkv)
        if v_fmt not in (MXFP4, MXFP8):
            raise ValueError("v_fmt must be MXFP4 or MXFP8")
        _check_tensor(x, "x", torch.bfloat16, (B, N, Dm), dev)
        _check_tensor(w, "w", torch.bfloat16, ((H + 2 * Hkv) * D, Dm), dev)
        spec = {"q": (H, MXFP4, ALONG_D), "k": (Hkv, MXFP4, ALONG_D), "v": (Hkv, v_fmt, ALONG_SEQ)}
        if fp8_views:
            spec.update({"q8": (H, MXFP8, ALONG_SEQ), "k8": (Hkv, MXFP8, ALONG_SEQ), "v8": (Hkv, MXFP8, ALONG_D)})
        outs = dict(outs or {})
        if set(outs) - set(spec):
            raise ValueError("unexpected outputs %s" % sorted(set(outs) - set(spec)))
        for name, (heads, fmt, axis) in spec.items():
            if name not in outs:
                outs[name] = mx_empty(B, heads, N, D, fmt, axis, dev)
            _check_mx(outs[name], name, fmt, axis, (B, heads, N, D), dev)
        _require_gpu_device(dev)
        names = ("q", "k", "v", "q8", "k8", "v8")
        self.structs = tuple(outs[n].c_struct() if n in outs else None for n in names)
        self.args = (x.data_ptr(), w.data_ptr()) + tuple(
            ctypes.byref(t) if t is not None else None for t in self.structs) + (B, N, Dm, H, Hkv, D, int(tile))
        self.device, self.outs, self._keep = dev, outs, (x, w)
        self._fn = lib().fp4attn_project_qkv_ex

    def __call__(self, stream=None):
        _check(self._fn(*self.args, _stream(self.device) if stream is None else stream), "fp4attn_project_qkv_ex")
        return self.outs


def project_qkv(x: torch.Tensor, w: torch.Tensor, H: int, Hkv: int, D: int, v_fmt: int = MXFP4,
                fp8_views: bool = False, outs: dict | None = None, tile: int = 0) -> dict:
    """QKV projection with the MX quantization in its epilogue (fp4attn_project_qkv_ex); returns the
    dict of MXTensors described at ProjectCall."""
    return ProjectCall(x, w, H, Hkv, D, v_fmt, fp8_views, outs, tile)()


@dataclass
class NVFP4Tensor:
    """One NVFP4-style [B, heads, N, D] tensor on the device (fp4attn_quantize_nvfp4): E2M1 codes
    [B, heads, N, D/2], E4M3 block scales [B, heads, N, D/16], the per-tensor exponent, and the
    represented values as bf16 [B, heads, N, D] (the operand of fwd_nvfp4)."""
    codes: torch.Tensor
    scales: torch.Tensor
    xhat: torch.Tensor
    tensor_exp: int
    shape: tuple


def quantize_nvfp4(x: torch.Tensor, tensor_exp: int = 0, out: NVFP4Tensor | None = None) -> NVFP4Tensor:
    """NVFP4-style quantization of a bf16 [B, heads, N, D] device tensor along D
    (fp4attn_quantize_nvfp4): blocks of 16, E4M3 scales, the per-tensor scale 2^tensor_exp."""
    if x.dim() != 4:
        raise ValueError("x must be a 4-D bfloat16 tensor [B, heads, N, D]")
    B, heads, N, D = x.shape
    dev = x.device
    _check_tensor(x, "x", torch.bfloat16, (B, heads, N, D), dev)
    if out is None:
        out = NVFP4Tensor(torch.empty((B, heads, N, D // 2), dtype=torch.uint8, device=dev),
                          torch.empty((B, heads, N, D // 16), dtype=torch.uint8, device=dev),
                          torch.empty((B, heads, N, D), dtype=torch.bfloat16, device=dev), int(tensor_exp),
                          (B, heads, N, D))
    _check_tensor(out.codes, "out.codes", torch.uint8, (B, heads, N, D // 2), dev)
    _check_tensor(out.scales, "out.scales", torch.uint8, (B, heads, N, D // 16), dev)
    _check_tensor(out.xhat, "out.xhat", torch.bfloat16, (B, heads, N, D), dev)
    _require_gpu_device(dev)
    out.tensor_exp = int(tensor_exp)
    _check(lib().fp4attn_quantize_nvfp4(x.data_ptr(), out.codes.data_ptr(), out.scales.data_ptr(), out.xhat.data_ptr(),
                                        int(tensor_exp), B, heads, N, D, _stream(dev)), "fp4attn_quantize_nvfp4")
    return out


class FwdNvCall:
    """A validated fp4attn_fwd_nvfp4 call over fixed buffers (see FwdCall): Direct-P on the
    integer-log2 anchor with S from the bf16 expansions of NVFP4-style Q and K and MXFP4 V."""

    def __init__(self, q: NVFP4Tensor, k: NVFP4Tensor, v: MXTensor, out: torch.Tensor | None = None,
                 lse: torch.Tensor | None = None):
        B, H, N, D = q.shape
        Hkv = k.shape[1]
        dev = q.xhat.device
        _check_heads(H, Hkv)
        _check_tensor(q.xhat, "q.xhat", torch.bfloat16, (B, H, N, D), dev)
        _check_tensor(k.xhat, "k.xhat", torch.bfloat16, (B, Hkv, N, D), dev)
        _check_mx(v, "v", MXFP4, ALONG_SEQ, (B, Hkv, N, D), dev)
        if out is None:
            out = torch.empty((B, H, N, D), dtype=torch.bfloat16, device=dev)
        if lse is None:
            lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        _check_tensor(out, "out", torch.bfloat16, (B, H, N, D), dev)
        _check_tensor(lse, "lse", torch.float32, (B, H, N), dev)
        _require_gpu_device(dev)
        self.vs = v.c_struct()
        self.args = (q.xhat.data_ptr(), k.xhat.data_ptr(), ctypes.byref(self.vs), out.data_ptr(), lse.data_ptr(), B, H,
                     Hkv, N, D)
        self.device, self.out, self.lse = dev, out, lse
        self._keep = (q, k, v)
        self._fn = lib().fp4attn_fwd_nvfp4

    def __call__(self, stream=None, events=None):
        st = _stream(self.device) if stream is None else stream
        ev = (None, None) if events is None else (events[0].cuda_event, events[1].cuda_event)
        _check(self._fn(*self.args, st, *ev), "fp4attn_fwd_nvfp4")
        return self.out, self.lse


def fwd_nvfp4(q: NVFP4Tensor, k: NVFP4Tensor, v: MXTensor, out: torch.Tensor | None = None,
              lse: torch.Tensor | None = None, events=None):
    """Direct-P forward with NVFP4-style Q and K (fp4attn_fwd_nvfp4). Returns (O, LSE)."""
    return FwdNvCall(q, k, v, out, lse)(events=events)


FWD_ANCHORED = 1  # FP4ATTN_FWD_ANCHORED


class FwdCall:
    """A validated fp4attn_fwd_ex call over fixed buffers (see QuantizeBatchCall). anchored=True
    selects Direct-P on the integer-log2 anchor with the range guard (noncausal, MXFP4 V). Calling
    it with events=(start, stop), a pair of timing-enabled torch.cuda.Event objects, binds them to
    the attention kernel's own dispatch, so start.elapsed_time(stop) is the kernel's duration."""

    def __init__(self, q: MXTensor, k: MXTensor, v: MXTensor, causal: bool = False, out: torch.Tensor | None = None,
                 lse: torch.Tensor | None = None, anchored: bool = False):
        B, H, N, D = q.shape
        Hkv = k.shape[1]
        dev = q.codes.device
        _check_heads(H, Hkv)
        _check_mx(q, "q", MXFP4, ALONG_D, (B, H, N, D), dev)
        _check_mx(k, "k", MXFP4, ALONG_D, (B, Hkv, N, D), dev)
        _check_mx(v, "v", None, ALONG_SEQ, (B, Hkv, N, D), dev)
        if out is None:
            out = torch.empty((B, H, N, D), dtype=torch.bfloat16, device=dev)
        if lse is None:
            lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        _check_tensor(out, "out", torch.bfloat16, (B, H, N, D), dev)
        _check_tensor(lse, "lse", torch.float32, (B, H, N), dev)
        _require_gpu_device(dev)
        self.structs = (q.c_struct(), k.c_struct(), v.c_struct())
        self.args = tuple(ctypes.byref(t) for t in self.structs) + (out.data_ptr(), lse.data_ptr(), B, H, Hkv, N, D,
                                                                     int(bool(causal)),
                                                                     FWD_ANCHORED if anchored else 0)
        self.device, self.out, self.lse = dev, out, lse
        self._keep = (q, k, v)
        self._fn = lib().fp4attn_fwd_ex

    def __call__(self, stream=None, events=None):
        st = _stream(self.device) if stream is None else stream
        ev = (None, None) if events is None else (events[0].cuda_event, events[1].cuda_event)
        _check(self._fn(*self.args, st, *ev), "fp4attn_fwd_ex")
        return self.out, self.lse


def fwd(q: MXTensor, k: MXTensor, v: MXTensor, causal: bool = False, out: torch.Tensor | None = None,
        lse: torch.Tensor | None = None, events=None, anchored: bool = False):
    """FP4 attention forward (fp4attn_fwd_ex). Returns (O bf16 [B,H,N,D], LSE fp32 [B,H,N]).

    anchored: Direct-P on the integer-log2 anchor (noncausal, MXFP4 V). events: optional (start,
    stop) pair of timing-enabled torch.cuda.Event objects bound to the attention kernel's own
    dispatch."""
    return FwdCall(q, k, v, causal, out, lse, anchored)(events=events)


def fwd_bf16(q: torch.Tensor, k: torch.Tensor, vt: torch.Tensor, causal: bool = False,
             out: torch.Tensor | None = None, lse: torch.Tensor | None = None):
    """BF16-MFMA forward of the same loop (fp4attn_fwd_bf16). q [B, H, N, D], k [B, Hkv, N, D] and
    V transposed, vt [B, Hkv, D, N] (e.g. v.transpose(-1, -2).contiguous()), all bf16."""
    if q.dim() != 4 or k.dim() != 4 or vt.dim() != 4:
        raise ValueError("q, k must be 4-D [B, heads, N, D] and vt 4-D [B, heads, D, N]")
    B, H, N, D = q.shape
    Hkv = k.shape[1]
    dev = q.device
    _check_heads(H, Hkv)
    _check_tensor(q, "q", torch.bfloat16, (B, H, N, D), dev)
    _check_tensor(k, "k", torch.bfloat16, (B, Hkv, N, D), dev)
    _check_tensor(vt, "vt", torch.bfloat16, (B, Hkv, D, N), dev)
    if out is None:
        out = torch.empty((B, H, N, D), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check_tensor(out, "out", torch.bfloat16, (B, H, N, D), dev)
    _check_tensor(lse, "lse", torch.float32, (B, H, N), dev)
    _require_gpu_device(dev)
    _check(lib().fp4attn_fwd_bf16(q.data_ptr(), k.data_ptr(), vt.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, Hkv,
                                  N, D, int(bool(causal)), _stream(q.device)), "fp4attn_fwd_bf16")
    return out, lse


def bwd_workspace_bytes(B, H, Hkv, N, D) -> int:
    return int(lib().fp4attn_bwd_workspace_bytes(B, H, Hkv, N, D))


def _bwd_checked(q, k, q8, k8, v8, o, do, lse):
    B, H, N, D = q.shape
    Hkv = k.shape[1]
    dev = o.device
    _check_heads(H, Hkv)
    _check_mx(q, "q", MXFP4, ALONG_D, (B, H, N, D), dev)
    _check_mx(k, "k", MXFP4, ALONG_D, (B, Hkv, N, D), dev)
    _check_mx(q8, "q8", MXFP8, ALONG_SEQ, (B, H, N, D), dev)
    _check_mx(k8, "k8", MXFP8, ALONG_SEQ, (B, Hkv, N, D), dev)
    _check_mx(v8, "v8", MXFP8, ALONG_D, (B, Hkv, N, D), dev)
    _check_tensor(o, "o", torch.bfloat16, (B, H, N, D), dev)
    _check_tensor(do, "do", torch.bfloat16, (B, H, N, D), dev)
    _check_tensor(lse, "lse", torch.float32, (B, H, N), dev)
    return B, H, Hkv, N, D, dev


def bwd(q: MXTensor, k: MXTensor, q8: MXTensor, k8: MXTensor, v8: MXTensor, o: torch.Tensor, do: torch.Tensor,
        lse: torch.Tensor, causal: bool = True, workspace: torch.Tensor | None = None):
    """Causal FP8 backward (fp4attn_bwd). Returns (dQ, dK, dV) bf16."""
    B, H, Hkv, N, D, dev = _bwd_checked(q, k, q8, k8, v8, o, do, lse)
    nbytes = bwd_workspace_bytes(B, H, Hkv, N, D)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    if workspace.dtype != torch.uint8 or not workspace.is_contiguous() or workspace.device != dev:
        raise ValueError("workspace must be a contiguous uint8 tensor on %s" % dev)
    if workspace.numel() < nbytes:
        raise ValueError("workspace holds %d bytes, %d needed" % (workspace.numel(), nbytes))
    _require_gpu_device(dev)
    dq = torch.empty((B, H, N, D), dtype=torch.bfloat16, device=dev)
    dk = torch.empty((B, Hkv, N, D), dtype=torch.bfloat16, device=dev)
    dv = torch.empty((B, Hkv, N, D), dtype=torch.bfloat16, device=dev)
    structs = [t.c_struct() for t in (q, k, q8, k8, v8)]
    _check(lib().fp4attn_bwd(*[ctypes.byref(s) for s in structs], o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                             dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(), B, H, Hkv, N, D,
                             int(bool(causal)), _stream(dev)), "fp4attn_bwd")
    return dq, dk, dv


def bwd_noalloc(q: MXTensor, k: MXTensor, q8: MXTensor, k8: MXTensor, v8: MXTensor, o: torch.Tensor,
                do: torch.Tensor, lse: torch.Tensor, dq: torch.Tensor, dk: torch.Tensor, dv: torch.Tensor,
                causal: bool = True):
    """The causal FP8 backward without any device allocation (fp4attn_bwd_noalloc): the library's
    static scratch array replaces the workspace, and the caller passes the outputs dq [B,H,N,D],
    dk, dv [B,Hkv,N,D] (bf16). Calls that overlap on one device race on that array."""
    B, H, Hkv, N, D, dev = _bwd_checked(q, k, q8, k8, v8, o, do, lse)
    _check_tensor(dq, "dq", torch.bfloat16, (B, H, N, D), dev)
    _check_tensor(dk, "dk", torch.bfloat16, (B, Hkv, N, D), dev)
    _check_tensor(dv, "dv", torch.bfloat16, (B, Hkv, N, D), dev)
    _require_gpu_device(dev)
    structs = [t.c_struct() for t in (q, k, q8, k8, v8)]
    _check(lib().fp4attn_bwd_noalloc(*[ctypes.byref(s) for s in structs], o.data_ptr(), do.data_ptr(),
                                     lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Hkv, N, D,
                                     int(bool(causal)), _stream(dev)), "fp4attn_bwd_noalloc")
    return dq, dk, dv


def key_block(D: int, causal: bool) -> int:
    return int(lib().fp4attn_key_block(D, int(bool(causal))))


def directp_forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor):
    """Quantize bf16 Q/K (along D) and V (along the sequence) to MXFP4 and run Direct-P."""
    qm, km, vm = quantize_mx_batch((q, k, v), (MXFP4, MXFP4, MXFP4), (ALONG_D, ALONG_D, ALONG_SEQ))
    return fwd(qm, km, vm, causal=False)


def clock_probe(iters: int = 24000, nblocks: int = 512, device=None) -> dict:
    """The shader clock under an MFMA + VALU load on every CU (fp4attn_clock_probe): GHz from each
    workgroup's shader-cycle and real-time counters over its loop (median, min, max over the
    workgroups) and the loop's wall time in ms (the median workgroup's ticks)."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else device
    counts = torch.empty(2 * nblocks, dtype=torch.int64, device=dev)
    khz = ctypes.c_int32(0)
    st = lib().fp4attn_clock_probe(ctypes.c_void_p(counts.data_ptr()), int(nblocks), int(iters), ctypes.byref(khz),
                                   ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
    _check(st, "fp4attn_clock_probe")
    c = counts.view(nblocks, 2).cpu().double()
    ghz = (c[:, 0] / c[:, 1] * khz.value / 1e6).sort().values
    return {"ghz_median": float(ghz[nblocks // 2]), "ghz_min": float(ghz[0]), "ghz_max": float(ghz[-1]),
            "loop_ms": float(c[:, 1].median()) / khz.value, "realtime_khz": khz.value}
