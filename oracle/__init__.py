"""CPU oracle for FP4 attention with Direct-P -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package. It shares no code with the GPU library (``precision_attention_amd``)
and never imports it; the GPU path never imports this package.

The arithmetic lives in ``fp4attn_oracle.c`` (plain C, built with gcc -O2
-ffp-contract=off -fopenmp). This module only compiles it, marshals NumPy arrays and
reshapes tensors for the two quantization axes. ``textbook.py`` holds the fp64 textbook
softmax attention used to pin the C code.

Method: "Hardware-Aware FP4 FlashAttention-4" (arXiv:2609.04105), gist.science technical
summary (Methodology 1 "Direct-P for Forward Inference", Methodology 2 "Quantized Causal
Backward") and the arXiv abstract.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_DIR = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_DIR, "fp4attn_oracle.c")
_BUILD = os.path.join(_DIR, "_build")
_SO = os.path.join(_BUILD, "libfp4attn_oracle.so")

FMT_E2M1 = 1
FMT_E4M3 = 2
P_DIRECT = 0
P_E4M3 = 1
P_EXACT = 2
P_DIRECT_ANCHOR = 3

OK = 0
ERR_ARG = 1
ERR_INEXACT = 2
ERR_NOMEM = 3


class OracleError(RuntimeError):
    pass


def build(force: bool = True) -> str:
    """Compile the C oracle into ``oracle/_build``. Returns the shared-library path."""
    os.makedirs(_BUILD, exist_ok=True)
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
               "-Wall", "-Wextra", "-Wno-unused-parameter", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _SO)
    return _SO


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_SO)
        P = ctypes.POINTER
        dp, u8p, u16p, i64p, fp = P(ctypes.c_double), P(ctypes.c_uint8), P(ctypes.c_uint16), P(ctypes.c_int64), P(ctypes.c_float)
        i64, i32 = ctypes.c_int64, ctypes.c_int
        L.orc_e2m1_decode.argtypes = [i32]; L.orc_e2m1_decode.restype = ctypes.c_double
        L.orc_e4m3_decode.argtypes = [i32]; L.orc_e4m3_decode.restype = ctypes.c_double
        L.orc_e8m0_decode.argtypes = [i32]; L.orc_e8m0_decode.restype = ctypes.c_double
        L.orc_e2m1_encode.argtypes = [ctypes.c_double]; L.orc_e2m1_encode.restype = i32
        L.orc_e4m3_encode.argtypes = [ctypes.c_double]; L.orc_e4m3_encode.restype = i32
        L.orc_mx_block_exponent.argtypes = [ctypes.c_double, i32]; L.orc_mx_block_exponent.restype = i32
        L.orc_mx_quantize_f64.argtypes = [dp, i64, i64, i32, u8p, u8p]; L.orc_mx_quantize_f64.restype = i32
        L.orc_mx_quantize_bf16.argtypes = [u16p, i64, i64, i32, u8p, u8p]; L.orc_mx_quantize_bf16.restype = i32
        L.orc_mx_dequantize.argtypes = [u8p, u8p, i64, i64, i32, dp]; L.orc_mx_dequantize.restype = i32
        L.orc_nvfp4_quantize.argtypes = [dp, i64, i64, i32, u8p, u8p, dp]; L.orc_nvfp4_quantize.restype = i32
        L.orc_bf16_to_f64.argtypes = [u16p, i64, dp]; L.orc_bf16_to_f64.restype = i32
        L.orc_f64_to_bf16.argtypes = [dp, i64, u16p]; L.orc_f64_to_bf16.restype = i32
        L.orc_directp_code.argtypes = [ctypes.c_float]; L.orc_directp_code.restype = i32
        L.orc_directp_thresholds.argtypes = [fp]; L.orc_directp_thresholds.restype = None
        L.orc_e4m3_code_of_exp2.argtypes = [ctypes.c_float]; L.orc_e4m3_code_of_exp2.restype = i32
        L.orc_log2e_scale.argtypes = [i64]; L.orc_log2e_scale.restype = ctypes.c_float
        L.orc_block_probs.argtypes = [fp, i32, ctypes.c_float, ctypes.c_float, i32, dp]; L.orc_block_probs.restype = i32
        L.orc_attn_fwd.argtypes = [dp, dp, dp, i64, i64, i64, i64, i64, i64, i32, i32, i32, i64p, i64, dp, dp, dp, dp]
        L.orc_attn_fwd.restype = i32
        L.orc_attn_bwd.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, i64, i64, i64, i64, i64, i32, i32,
                                   i64p, i64, dp, i64p, i64, dp, dp]
        L.orc_attn_bwd.restype = i32
        L.orc_num_threads.argtypes = []; L.orc_num_threads.restype = i32
        L.orc_block_probs_anchored.argtypes = [fp, i32, ctypes.c_float, dp]
        L.orc_block_probs_anchored.restype = i32
        L.orc_bwd_prob.argtypes = [ctypes.c_float, ctypes.c_float, i64]; L.orc_bwd_prob.restype = ctypes.c_double
        _lib = L
    return _lib


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _check(rc, what):
    if rc != OK:
        raise OracleError("%s failed with oracle status %d" % (what, rc))


def num_threads() -> int:
    return int(lib().orc_num_threads())


# ------------------------------------------------------------------ formats

def e2m1_decode(code: int) -> float:
    return lib().orc_e2m1_decode(int(code))


def e4m3_decode(code: int) -> float:
    return lib().orc_e4m3_decode(int(code))


def e8m0_decode(code: int) -> float:
    return lib().orc_e8m0_decode(int(code))


def e2m1_encode(x: float) -> int:
    return lib().orc_e2m1_encode(float(x))


def e4m3_encode(x: float) -> int:
    return lib().orc_e4m3_encode(float(x))


def mx_block_exponent(amax: float, fmt: int) -> int:
    return lib().orc_mx_block_exponent(float(amax), int(fmt))


def directp_code(u) -> int:
    return lib().orc_directp_code(ctypes.c_float(float(np.float32(u))))


def directp_thresholds() -> np.ndarray:
    out = np.zeros(7, np.float32)
    lib().orc_directp_thresholds(_ptr(out, ctypes.c_float))
    return out


def e4m3_code_of_exp2(u) -> int:
    return lib().orc_e4m3_code_of_exp2(ctypes.c_float(float(np.float32(u))))


def log2e_scale(D: int) -> np.float32:
    return np.float32(lib().orc_log2e_scale(int(D)))


def block_probs(s, m, D: int, pmode: int):
    """Probabilities of one (<= 32)-key block relative to running max m. Returns (e_b, P)."""
    s = np.ascontiguousarray(s, np.float32)
    if s.size > 32:
        raise ValueError("a probability block holds at most 32 keys")
    p = np.zeros(s.size, np.float64)
    eb = lib().orc_block_probs(_ptr(s, ctypes.c_float), s.size, ctypes.c_float(float(np.float32(m))),
                               ctypes.c_float(float(log2e_scale(D))), pmode, _ptr(p, ctypes.c_double))
    return int(eb), p


def block_probs_anchored(s, D: int):
    """Direct-P probabilities of one (<= 32)-key block on the integer-log2 anchor. Returns
    (t_b - 2, P) with P absolute (P approximates 2^(S c))."""
    s = np.ascontiguousarray(s, np.float32)
    if s.size > 32:
        raise ValueError("a probability block holds at most 32 keys")
    p = np.zeros(s.size, np.float64)
    e = lib().orc_block_probs_anchored(_ptr(s, ctypes.c_float), s.size, ctypes.c_float(float(log2e_scale(D))),
                                       _ptr(p, ctypes.c_double))
    return int(e), p


def bwd_prob(s, lse, D: int) -> float:
    """The quantized backward's rebuilt probability of one score s (binary32) for a row with
    log-sum-exp lse (binary32): fp32(2^(fmaf(s, c, -fp32(lse * log2 e))))."""
    return float(lib().orc_bwd_prob(ctypes.c_float(float(np.float32(s))), ctypes.c_float(float(np.float32(lse))),
                                     int(D)))


def bf16_to_f64(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.uint16)
    out = np.empty(x.shape, np.float64)
    _check(lib().orc_bf16_to_f64(_ptr(x, ctypes.c_uint16), x.size, _ptr(out, ctypes.c_double)), "bf16_to_f64")
    return out


def f64_to_bf16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, np.uint16)
    _check(lib().orc_f64_to_bf16(_ptr(x, ctypes.c_double), x.size, _ptr(out, ctypes.c_uint16)), "f64_to_bf16")
    return out


# ------------------------------------------------------------------ MX quantization

def mx_quantize(x: np.ndarray, fmt: int, axis: str = "d"):
    """MX-quantize a [..., N, D] tensor in blocks of 32 along ``axis``.

    axis "d": blocks along the last dim; codes [..., N, D], scales [..., N, D/32].
    axis "seq": blocks along N; codes [..., N, D], scales [..., N/32, D].
    ``x`` is either uint16 (bfloat16 bits) or float64. Codes are logical, one per element.
    """
    if axis not in ("d", "seq"):
        raise ValueError(axis)
    work = x if axis == "d" else np.swapaxes(x, -1, -2)
    work = np.ascontiguousarray(work)
    length = work.shape[-1]
    nvec = work.size // length
    codes = np.empty(work.shape, np.uint8)
    scales = np.empty(work.shape[:-1] + (length // 32,), np.uint8)
    L = lib()
    if work.dtype == np.uint16:
        rc = L.orc_mx_quantize_bf16(_ptr(work, ctypes.c_uint16), nvec, length, fmt, _ptr(codes, ctypes.c_uint8),
                                    _ptr(scales, ctypes.c_uint8))
    else:
        work = np.ascontiguousarray(work, dtype=np.float64)
        rc = L.orc_mx_quantize_f64(_ptr(work, ctypes.c_double), nvec, length, fmt, _ptr(codes, ctypes.c_uint8),
                                   _ptr(scales, ctypes.c_uint8))
    _check(rc, "mx_quantize")
    if axis == "seq":
        codes = np.ascontiguousarray(np.swapaxes(codes, -1, -2))
        scales = np.ascontiguousarray(np.swapaxes(scales, -1, -2))
    return codes, scales


def nvfp4_quantize(x: np.ndarray, g: int = 0):
    """NVFP4-style quantization of a [..., D] tensor along its last axis (see orc_nvfp4_quantize):
    blocks of 16, E2M1 codes, one E4M3 scale per block, the per-tensor scale 2^g.

    ``x`` is uint16 (bfloat16 bits) or float64. Returns (codes [..., D], scale codes [..., D/16],
    x_hat [..., D] float64, the represented values)."""
    x = np.asarray(x)
    xd = bf16_to_f64(x) if x.dtype == np.uint16 else np.ascontiguousarray(x, dtype=np.float64)
    length = xd.shape[-1]
    nvec = xd.size // length
    codes = np.empty(xd.shape, np.uint8)
    scales = np.empty(xd.shape[:-1] + (length // 16,), np.uint8)
    xhat = np.empty(xd.shape, np.float64)
    _check(lib().orc_nvfp4_quantize(_ptr(xd, ctypes.c_double), nvec, length, int(g), _ptr(codes, ctypes.c_uint8),
                                    _ptr(scales, ctypes.c_uint8), _ptr(xhat, ctypes.c_double)), "nvfp4_quantize")
    return codes, scales, xhat


def mx_dequantize(codes: np.ndarray, scales: np.ndarray, fmt: int, axis: str = "d") -> np.ndarray:
    if axis == "seq":
        codes = np.swapaxes(codes, -1, -2)
        scales = np.swapaxes(scales, -1, -2)
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    length = codes.shape[-1]
    out = np.empty(codes.shape, np.float64)
    _check(lib().orc_mx_dequantize(_ptr(codes, ctypes.c_uint8), _ptr(scales, ctypes.c_uint8), codes.size // length,
                                   length, fmt, _ptr(out, ctypes.c_double)), "mx_dequantize")
    if axis == "seq":
        out = np.ascontiguousarray(np.swapaxes(out, -1, -2))
    return out


# ------------------------------------------------------------------ attention

def attn_fwd(Q, K, V, KB: int, causal: bool, pmode: int, rows=None, check_exact: bool = True):
    """Online-softmax forward on dequantized operands (see orc_attn_fwd).

    Q [B,H,N,D], K/V [B,Hkv,N,D] float64. rows: optional flattened [B,H,N] indices.
    Returns dict(O [nrows,D] or [B,H,N,D], lse, l, m).
    """
    Q = np.ascontiguousarray(Q, np.float64)
    K = np.ascontiguousarray(K, np.float64)
    V = np.ascontiguousarray(V, np.float64)
    B, H, N, D = Q.shape
    Hkv = K.shape[1]
    if rows is None:
        nrows = B * H * N
        rows_p = None
    else:
        rows = np.ascontiguousarray(rows, np.int64)
        nrows = rows.size
        rows_p = _ptr(rows, ctypes.c_int64)
    O = np.empty((nrows, D), np.float64)
    lse = np.empty(nrows, np.float64)
    lsum = np.empty(nrows, np.float64)
    m = np.empty(nrows, np.float64)
    rc = lib().orc_attn_fwd(_ptr(Q, ctypes.c_double), _ptr(K, ctypes.c_double), _ptr(V, ctypes.c_double), B, H, Hkv,
                            N, D, KB, int(bool(causal)), pmode, int(bool(check_exact)), rows_p, nrows,
                            _ptr(O, ctypes.c_double), _ptr(lse, ctypes.c_double), _ptr(lsum, ctypes.c_double),
                            _ptr(m, ctypes.c_double))
    _check(rc, "attn_fwd")
    if rows is None:
        O = O.reshape(B, H, N, D)
        lse = lse.reshape(B, H, N)
        lsum = lsum.reshape(B, H, N)
        m = m.reshape(B, H, N)
    return {"O": O, "lse": lse, "l": lsum, "m": m}


def attn_bwd(Qs, Ks, dOd, Vd, dOq, Kk, Qq, O, dO, lse, causal: bool, quant: bool, qrows=None, kcols=None,
             want_dq: bool = True, want_dkv: bool = True):
    """Backward on dequantized operand views (see orc_attn_bwd). Returns dict(dQ, dK, dV)."""
    arrs = [np.ascontiguousarray(a, np.float64) for a in (Qs, Ks, dOd, Vd, dOq, Kk, Qq, O, dO, lse)]
    Qs, Ks, dOd, Vd, dOq, Kk, Qq, O, dO, lse = arrs
    B, H, N, D = Qs.shape
    Hkv = Ks.shape[1]
    if not want_dq:
        nq, qp = 0, None
    elif qrows is None:
        nq, qp = B * H * N, None
    else:
        qrows = np.ascontiguousarray(qrows, np.int64)
        nq, qp = qrows.size, _ptr(qrows, ctypes.c_int64)
    if not want_dkv:
        nk, kp = 0, None
    elif kcols is None:
        nk, kp = B * Hkv * N, None
    else:
        kcols = np.ascontiguousarray(kcols, np.int64)
        nk, kp = kcols.size, _ptr(kcols, ctypes.c_int64)
    dQ = np.zeros((max(nq, 1), D), np.float64)
    dK = np.zeros((max(nk, 1), D), np.float64)
    dV = np.zeros((max(nk, 1), D), np.float64)
    P = ctypes.c_double
    rc = lib().orc_attn_bwd(*[_ptr(a, P) for a in arrs], B, H, Hkv, N, D, int(bool(causal)), int(bool(quant)), qp, nq,
                            _ptr(dQ, P), kp, nk, _ptr(dK, P), _ptr(dV, P))
    _check(rc, "attn_bwd")
    out = {}
    if want_dq:
        out["dQ"] = dQ[:nq].reshape(B, H, N, D) if qrows is None else dQ[:nq]
    if want_dkv:
        out["dK"] = dK[:nk].reshape(B, Hkv, N, D) if kcols is None else dK[:nk]
        out["dV"] = dV[:nk].reshape(B, Hkv, N, D) if kcols is None else dV[:nk]
    return out


# ------------------------------------------------------------------ end-to-end paths from bf16 inputs

def quantize_directp_operands(q16, k16, v16):
    """MXFP4 Q/K along D and MXFP4 V along the sequence (noncausal Direct-P route)."""
    qc, qs = mx_quantize(q16, FMT_E2M1, "d")
    kc, ks = mx_quantize(k16, FMT_E2M1, "d")
    vc, vs = mx_quantize(v16, FMT_E2M1, "seq")
    return {"q": (qc, qs), "k": (kc, ks), "v": (vc, vs)}


def directp_forward(q16, k16, v16, KB: int, rows=None):
    """Noncausal Direct-P forward from bf16 inputs: returns O (fp64 and bf16 bits), LSE and codes."""
    ops = quantize_directp_operands(q16, k16, v16)
    Qd = mx_dequantize(*ops["q"], FMT_E2M1, "d")
    Kd = mx_dequantize(*ops["k"], FMT_E2M1, "d")
    Vd = mx_dequantize(*ops["v"], FMT_E2M1, "seq")
    res = attn_fwd(Qd, Kd, Vd, KB, False, P_DIRECT, rows=rows)
    res["O_bf16"] = f64_to_bf16(res["O"])
    res["ops"] = ops
    return res


def directp_anchored_forward(q16, k16, v16, rows=None):
    """Noncausal Direct-P on the integer-log2 anchor from bf16 inputs (MXFP4 Q/K/V as for
    directp_forward): returns O (fp64 and bf16 bits), LSE and the operands."""
    ops = quantize_directp_operands(q16, k16, v16)
    Qd = mx_dequantize(*ops["q"], FMT_E2M1, "d")
    Kd = mx_dequantize(*ops["k"], FMT_E2M1, "d")
    Vd = mx_dequantize(*ops["v"], FMT_E2M1, "seq")
    res = attn_fwd(Qd, Kd, Vd, 32, False, P_DIRECT_ANCHOR, rows=rows)
    res["O_bf16"] = f64_to_bf16(res["O"])
    res["ops"] = ops
    return res


def nvfp4_anchored_forward(q16, k16, v16, gq: int = 0, gk: int = 0, rows=None):
    """Direct-P on the integer-log2 anchor with NVFP4-style Q and K (summary, Methodology 1
    "Format Selection"): Q and K quantized by ``nvfp4_quantize`` (per-tensor scales 2^gq, 2^gk),
    V MXFP4 along the sequence; S is the binary32 rounding of the exact dot product of the
    represented values (exact in binary64: every product has at most 12 significant bits)."""
    qc, qs, Qd = nvfp4_quantize(q16, gq)
    kc, ks, Kd = nvfp4_quantize(k16, gk)
    vc, vs = mx_quantize(v16, FMT_E2M1, "seq")
    Vd = mx_dequantize(vc, vs, FMT_E2M1, "seq")
    res = attn_fwd(Qd, Kd, Vd, 32, False, P_DIRECT_ANCHOR, rows=rows, check_exact=False)
    res["O_bf16"] = f64_to_bf16(res["O"])
    res["q_hat"], res["k_hat"] = Qd, Kd
    res["ops"] = {"q": (qc, qs), "k": (kc, ks), "v": (vc, vs)}
    return res


def quantize_causal_operands(q16, k16, v16):
    """Causal training route: MXFP4 Q/K along D (the saved state), MXFP8 V along the sequence."""
    qc, qs = mx_quantize(q16, FMT_E2M1, "d")
    kc, ks = mx_quantize(k16, FMT_E2M1, "d")
    vc, vs = mx_quantize(v16, FMT_E4M3, "seq")
    return {"q": (qc, qs), "k": (kc, ks), "v8": (vc, vs)}


def fp8_forward(q16, k16, v16, KB: int, causal: bool, rows=None):
    """FP8 P/V forward (MXFP4 Q/K, E4M3 P, MXFP8 V) from bf16 inputs; causal=True is the training
    route, causal=False the noncausal FP8 route the pages compare Direct-P with."""
    ops = quantize_causal_operands(q16, k16, v16)
    Qd = mx_dequantize(*ops["q"], FMT_E2M1, "d")
    Kd = mx_dequantize(*ops["k"], FMT_E2M1, "d")
    Vd = mx_dequantize(*ops["v8"], FMT_E4M3, "seq")
    res = attn_fwd(Qd, Kd, Vd, KB, causal, P_E4M3, rows=rows)
    res["O_bf16"] = f64_to_bf16(res["O"])
    res["ops"] = ops
    return res


def causal_forward(q16, k16, v16, KB: int, rows=None):
    return fp8_forward(q16, k16, v16, KB, True, rows=rows)


def backward_views(q16, k16, v16, do16):
    """MXFP8 operand views of the backward's gradient products, dequantized."""
    return {
        "dOd": mx_dequantize(*mx_quantize(do16, FMT_E4M3, "d"), FMT_E4M3, "d"),
        "Vd": mx_dequantize(*mx_quantize(v16, FMT_E4M3, "d"), FMT_E4M3, "d"),
        "dOq": mx_dequantize(*mx_quantize(do16, FMT_E4M3, "seq"), FMT_E4M3, "seq"),
        "Kk": mx_dequantize(*mx_quantize(k16, FMT_E4M3, "seq"), FMT_E4M3, "seq"),
        "Qq": mx_dequantize(*mx_quantize(q16, FMT_E4M3, "seq"), FMT_E4M3, "seq"),
    }


def causal_backward(q16, k16, v16, do16, o16, lse32, qrows=None, kcols=None, want_dq=True, want_dkv=True,
                    causal=True):
    """FP8 backward of the causal route from bf16 inputs, the forward's bf16 O and fp32 LSE.
    causal=False drops the mask (the same gradient formats over all keys)."""
    Qs = mx_dequantize(*mx_quantize(q16, FMT_E2M1, "d"), FMT_E2M1, "d")
    Ks = mx_dequantize(*mx_quantize(k16, FMT_E2M1, "d"), FMT_E2M1, "d")
    v = backward_views(q16, k16, v16, do16)
    O = bf16_to_f64(o16)
    dO = bf16_to_f64(do16)
    lse = np.asarray(lse32, np.float32).astype(np.float64)
    return attn_bwd(Qs, Ks, v["dOd"], v["Vd"], v["dOq"], v["Kk"], v["Qq"], O, dO, lse, causal=causal, quant=True,
                    qrows=qrows, kcols=kcols, want_dq=want_dq, want_dkv=want_dkv)


# ------------------------------------------------------------------ QKV projection

def project_qkv(x16, w16, H: int, Hkv: int, D: int):
    """Q, K, V = X Wq^T, X Wk^T, X Wv^T in binary64, each as [B, heads, N, D].

    Reading (gist.science summary, Methodology 2 "Quantized Causal Backward", *Gradient Formats*,
    and Results, *Training Performance*: the projection epilogues publish the quantized Q, K, V and
    their FP8 views): x16 holds bf16 bits [B, N, Dm]; w16 holds bf16 bits [(H + 2 Hkv) D, Dm], the
    weight of one linear layer (output features by input features) whose rows are Wq (H heads of
    D rows each), then Wk (Hkv heads), then Wv (Hkv heads). Every bf16 x bf16 product is exact in
    binary64; the sums over Dm are the library's binary64 matrix product.
    """
    X = bf16_to_f64(np.asarray(x16))
    W = bf16_to_f64(np.asarray(w16))
    if X.ndim != 3 or W.ndim != 2 or W.shape != ((H + 2 * Hkv) * D, X.shape[2]):
        raise ValueError("x must be [B, N, Dm] and w [(H + 2 Hkv) D, Dm]")
    B, N, _ = X.shape
    Y = np.matmul(X, W.T)  # [B, N, F]
    Y = np.ascontiguousarray(Y.reshape(B, N, H + 2 * Hkv, D).transpose(0, 2, 1, 3))
    return Y[:, :H], Y[:, H:H + Hkv], Y[:, H + Hkv:]


def project_qkv_views(x16, w16, H: int, Hkv: int, D: int, v_fmt: int = FMT_E2M1, fp8_views: bool = False):
    """The MX tensors a fused projection epilogue writes, quantized from the binary64 products.

    Reading: the epilogue quantizes the accumulated product itself; no bf16 copy of Q, K or V is
    formed, so there is no intermediate rounding. Returns (views, (q, k, v)) with views holding
    (codes, scales) per name, in the logical layout of ``mx_quantize``:
    q, k MXFP4 (E2M1) along D; v along the sequence in ``v_fmt`` (E2M1 for Direct-P, E4M3 for the
    causal route); with ``fp8_views`` also the backward's q8, k8 (E4M3 along the sequence) and v8
    (E4M3 along D).
    """
    q, k, v = project_qkv(x16, w16, H, Hkv, D)
    views = {"q": mx_quantize(q, FMT_E2M1, "d"), "k": mx_quantize(k, FMT_E2M1, "d"),
             "v": mx_quantize(v, v_fmt, "seq")}
    if fp8_views:
        views["q8"] = mx_quantize(q, FMT_E4M3, "seq")
        views["k8"] = mx_quantize(k, FMT_E4M3, "seq")
        views["v8"] = mx_quantize(v, FMT_E4M3, "d")
    return views, (q, k, v)
