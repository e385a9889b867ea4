"""GPU backward (fp4attn_bwd) versus the oracle's FP8 backward.

Both sides get the same O and LSE: the oracle's forward of the same inputs (never the GPU's).
Tolerance: cosine similarity >= 0.999 for each of dQ, dK, dV and each head of them; besides,
the relative RMS error must stay <= 5e-3 (the two sides differ only in accumulation order,
fp32 versus binary64 for Delta and the score products, and the occasional E4M3 rounding of a
P or dS element that lies within an fp32 ulp of a rounding midpoint).

Small shapes compare every element and span several key tiles, several query blocks, ragged
tails (N % 128 != 0 and N % 64 != 0) and grouped-query heads. The full-size training shape
(B=1, H=32, Hkv=8, N=8192, D=128) is compared in tests/test_gpu_fullsize.py.
"""
import numpy as np
import pytest

from precision_attention_amd.inputs import attention_inputs
from tests.gpuhelpers import bf16_to_np, require_gpu, to_dev
from tests.mxlayout import unpack_codes, unpack_scales

pytestmark = pytest.mark.gpu

COS_MIN = 0.999
REL_RMS_MAX = 5e-3


def gpu_backward(x, o16, lse32, causal, dev):
    import precision_attention_amd as pa
    import torch

    q, k, v, do = (to_dev(x[n], dev) for n in ("q", "k", "v", "do"))
    o = to_dev(o16, dev)
    lse = torch.from_numpy(np.ascontiguousarray(lse32, np.float32)).to(dev)
    qm = pa.quantize_mx(q, pa.MXFP4, pa.ALONG_D)
    km = pa.quantize_mx(k, pa.MXFP4, pa.ALONG_D)
    q8 = pa.quantize_mx(q, pa.MXFP8, pa.ALONG_SEQ)
    k8 = pa.quantize_mx(k, pa.MXFP8, pa.ALONG_SEQ)
    v8 = pa.quantize_mx(v, pa.MXFP8, pa.ALONG_D)
    dq, dk, dv = pa.bwd(qm, km, q8, k8, v8, o, do, lse, causal=causal)
    torch.cuda.synchronize()
    return bf16_to_np(dq), bf16_to_np(dk), bf16_to_np(dv)


def metrics(g, r):
    g = np.asarray(g, np.float64).ravel()
    r = np.asarray(r, np.float64).ravel()
    cos = float(g @ r / max(np.sqrt((g @ g) * (r @ r)), 1e-300))
    rel = float(np.sqrt(np.sum((g - r) ** 2) / max(np.sum(r ** 2), 1e-300)))
    return cos, rel


def check(name, g, r, per_head_axis=None):
    cos, rel = metrics(g, r)
    print("%s cos %.7f rel_rms %.3e" % (name, cos, rel), flush=True)
    assert cos >= COS_MIN, (name, cos)
    assert rel <= REL_RMS_MAX, (name, rel)
    if per_head_axis is not None:
        for h in range(g.shape[per_head_axis]):
            gh, rh = np.take(g, h, per_head_axis), np.take(r, h, per_head_axis)
            if np.any(rh != 0):
                c, _ = metrics(gh, rh)
                assert c >= COS_MIN, (name, h, c)


SMALL = [
    # (B, H, Hkv, N, D)
    (1, 1, 1, 128, 64),     # one key tile, two query blocks
    (1, 2, 2, 96, 64),      # ragged tile and ragged query block
    (2, 4, 2, 352, 128),    # 3 key tiles (last ragged), GQA group of 2
    (1, 3, 1, 544, 128),    # N = 4*128 + 32, three query heads on one KV head
    (1, 2, 1, 1024, 64),
    (1, 2, 1, 32, 128),     # the smallest N: part of one query block and one key tile
]


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "noncausal"])
@pytest.mark.parametrize("shape", SMALL, ids=["x".join(map(str, s)) for s in SMALL])
def test_backward_small_all_elements(orc, shape, causal):
    dev = require_gpu()
    B, H, Hkv, N, D = shape
    print("bwd case", shape, "causal", causal, flush=True)
    x = attention_inputs(B, H, Hkv, N, D, seed=100 + sum(shape), with_do=True)
    fwd = orc.causal_forward(x["q"], x["k"], x["v"], KB=64) if causal else \
        orc.directp_forward(x["q"], x["k"], x["v"], KB=64)
    o16, lse = fwd["O_bf16"], fwd["lse"].astype(np.float32)
    dq, dk, dv = gpu_backward(x, o16, lse, causal, dev)
    ref = orc.causal_backward(x["q"], x["k"], x["v"], x["do"], o16, lse, causal=causal)
    check("dQ", dq.reshape(B, H, N, D), ref["dQ"], per_head_axis=1)
    check("dK", dk.reshape(B, Hkv, N, D), ref["dK"], per_head_axis=1)
    check("dV", dv.reshape(B, Hkv, N, D), ref["dV"], per_head_axis=1)


def test_backward_deterministic():
    import precision_attention_amd as pa  # noqa: F401

    dev = require_gpu()
    B, H, Hkv, N, D = 1, 4, 2, 384, 128
    x = attention_inputs(B, H, Hkv, N, D, seed=9, with_do=True)
    rng = np.random.default_rng(9)
    o16 = x["do"][..., ::-1].copy()  # any O works for determinism
    lse = (rng.standard_normal((B, H, N)) + 6.0).astype(np.float32)
    a = gpu_backward(x, o16, lse, True, dev)
    b = gpu_backward(x, o16, lse, True, dev)
    for u, w in zip(a, b):
        assert np.array_equal(u, w)


def test_backward_zero_do_gives_zero_gradients():
    """dO = 0: dP = 0 and Delta = 0, so every gradient is exactly zero."""
    dev = require_gpu()
    B, H, Hkv, N, D = 1, 2, 1, 256, 128
    x = attention_inputs(B, H, Hkv, N, D, seed=4, with_do=True)
    x["do"] = np.zeros_like(x["do"])
    lse = np.full((B, H, N), 4.0, np.float32)
    dq, dk, dv = gpu_backward(x, x["v"].repeat(H // Hkv, axis=1), lse, True, dev)
    assert not dq.any() and not dk.any() and not dv.any()


def _pad256(n):
    return (n + 255) // 256 * 256


@pytest.mark.parametrize("shape", [(1, 2, 1, 288, 128), (2, 3, 1, 160, 64)], ids=["1x2x1x288x128", "2x3x1x160x64"])
def test_backward_preprocessing_workspace(orc, shape):
    """The backward's first launch writes into the caller's workspace, in this order and each
    region padded to 256 bytes: -Delta (fp32 per row), -fp32(LSE log2 e) (fp32 per row), dO's
    MXFP8 codes and scales along D, and dO's MXFP8 codes and scales along the queries. This
    white-box check reads them back after a call: both views of dO must equal the oracle's MX
    quantization bit for bit, -fp32(LSE log2 e) is one fp32 product and must match exactly, and
    -Delta must equal -sum_d dO_id O_id (exact bf16 products, formed in binary64 here) within
    the fp32 summation bound (12 rounding levels, under 2e-6 of sum_d |dO_id O_id|)."""
    import precision_attention_amd as pa
    import torch

    dev = require_gpu()
    B, H, Hkv, N, D = shape
    print("bwd workspace case", shape, flush=True)
    x = attention_inputs(B, H, Hkv, N, D, seed=31 + N, with_do=True)
    rng = np.random.default_rng(N)
    o16 = x["q"][..., ::-1].copy()  # any O of the right shape
    lse = (rng.standard_normal((B, H, N)) * 2.0 + 6.0).astype(np.float32)
    q, k, v, do = (to_dev(x[n], dev) for n in ("q", "k", "v", "do"))
    nbytes = pa.bwd_workspace_bytes(B, H, Hkv, N, D)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
    pa.bwd(pa.quantize_mx(q, pa.MXFP4, pa.ALONG_D), pa.quantize_mx(k, pa.MXFP4, pa.ALONG_D),
           pa.quantize_mx(q, pa.MXFP8, pa.ALONG_SEQ), pa.quantize_mx(k, pa.MXFP8, pa.ALONG_SEQ),
           pa.quantize_mx(v, pa.MXFP8, pa.ALONG_D), to_dev(o16, dev), do,
           torch.from_numpy(lse).to(dev), causal=True, workspace=ws)
    torch.cuda.synchronize()
    w = ws.cpu().numpy()
    rows = B * H * N
    off_nl = _pad256(rows * 4)
    off_dod = 2 * _pad256(rows * 4)
    off_dods = off_dod + _pad256(rows * D)
    off_doq = off_dods + _pad256(rows * D // 32)
    off_doqs = off_doq + _pad256(rows * D)
    assert off_doqs + _pad256(rows * D // 32) == nbytes
    ndelta = w[:rows * 4].view(np.float32).reshape(B, H, N)
    nl = w[off_nl:off_nl + rows * 4].view(np.float32).reshape(B, H, N)
    assert np.array_equal(nl, -(lse * np.float32(1.44269504)))
    prod = orc.bf16_to_f64(x["do"]) * orc.bf16_to_f64(o16)
    ref = -prod.sum(axis=-1)
    err = np.abs(ndelta.astype(np.float64) - ref)
    bound = 2e-6 * np.abs(prod).sum(axis=-1) + 1e-30
    assert np.all(err <= bound), "Delta off by %.3e at %s" % (err.max(), np.unravel_index(np.argmax(err / bound), err.shape))
    for axis, oc_off, os_off in ((0, off_dod, off_dods), (1, off_doq, off_doqs)):
        codes = unpack_codes(w[oc_off:oc_off + rows * D], 2, axis, (B, H, N, D))
        scales = unpack_scales(w[os_off:os_off + rows * D // 32], axis, (B, H, N, D))
        oc, os_ = orc.mx_quantize(x["do"], 2, ("d", "seq")[axis])
        assert np.array_equal(scales, os_), ("scales", axis)
        assert np.array_equal(codes, oc), ("codes", axis, np.argwhere(codes != oc)[:5])
