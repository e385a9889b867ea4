"""Every route at seeded random shapes against the oracle, with the tolerances of the per-route
tests: B in {1, 2}, 1-2 KV heads with 1-4 query heads each, N any multiple of 32 up to 1248
(ragged against every tile and key block size), D in {64, 128}. The shape list is fixed by its
seed, so a failing case is named and repeatable.

Routes: Direct-P (running max and integer-log2 anchor), the noncausal FP8 P/V route, the causal
FP8 forward, the BF16-MFMA forward (noncausal and causal, against fp64 textbook attention), the
NVFP4-style Q/K forward, and the FP8 backward (causal and noncausal; cosine >= 0.999 and relative
RMS <= 5e-3 per gradient)."""
import numpy as np
import pytest

from precision_attention_amd.inputs import attention_inputs
from tests.gpuhelpers import assert_parity, bf16_to_np, oracle_o, parity, require_gpu, to_dev

pytestmark = pytest.mark.gpu


def _shapes(seed=20261203, count=16):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        D = int(rng.choice([64, 128]))
        Hkv = int(rng.integers(1, 3))
        G = int(rng.choice([1, 2, 3, 4]))
        B = int(rng.integers(1, 3))
        N = 32 * int(rng.integers(1, 40))
        out.append((B, Hkv * G, Hkv, N, D, int(rng.integers(0, 1 << 30))))
    return out


SHAPES = _shapes()
ROUTES = ["directp", "anchored", "fp8route", "causal", "bf16", "bf16_causal", "nvfp4", "bwd_causal", "bwd_noncausal"]


def _cos_rel(g, r):
    g = np.asarray(g, np.float64).ravel()
    r = np.asarray(r, np.float64).ravel()
    cos = float(g @ r / max(np.sqrt((g @ g) * (r @ r)), 1e-300))
    rel = float(np.sqrt(np.sum((g - r) ** 2) / max(np.sum(r ** 2), 1e-300)))
    return cos, rel


@pytest.mark.parametrize("route", ROUTES)
@pytest.mark.parametrize("shape", SHAPES, ids=["x".join(map(str, s[:5])) for s in SHAPES])
def test_route_at_random_shape(orc, shape, route):
    import precision_attention_amd as pa
    import torch

    from oracle import textbook

    dev = require_gpu()
    B, H, Hkv, N, D, seed = shape
    print("sweep case", route, (B, H, Hkv, N, D), "seed", seed, flush=True)
    x = attention_inputs(B, H, Hkv, N, D, seed=seed, with_do=route.startswith("bwd"))
    q, k, v = (to_dev(x[n], dev) for n in ("q", "k", "v"))
    if route in ("directp", "anchored", "fp8route", "causal"):
        causal = route == "causal"
        qm = pa.quantize_mx(q, pa.MXFP4, pa.ALONG_D)
        km = pa.quantize_mx(k, pa.MXFP4, pa.ALONG_D)
        vm = pa.quantize_mx(v, pa.MXFP8 if route in ("fp8route", "causal") else pa.MXFP4, pa.ALONG_SEQ)
        o, lse = pa.fwd(qm, km, vm, causal=causal, anchored=route == "anchored")
        torch.cuda.synchronize()
        if route == "directp":
            ref = orc.directp_forward(x["q"], x["k"], x["v"], KB=pa.key_block(D, False))
        elif route == "anchored":
            ref = orc.directp_anchored_forward(x["q"], x["k"], x["v"])
        else:
            ref = orc.fp8_forward(x["q"], x["k"], x["v"], KB=pa.key_block(D, causal), causal=causal)
        m = parity(bf16_to_np(o), oracle_o(ref), lse.cpu().numpy(), ref["lse"])
        print(m, flush=True)
        assert_parity(m, route)
    elif route.startswith("bf16"):
        causal = route == "bf16_causal"
        o, lse = pa.fwd_bf16(q, k, v.transpose(-1, -2).contiguous(), causal=causal)
        torch.cuda.synchronize()
        Q, K, V = (orc.bf16_to_f64(x[n]) for n in ("q", "k", "v"))
        O, L, _ = textbook.attention(Q, K, V, causal)
        m = parity(bf16_to_np(o), O, lse.cpu().numpy(), L)
        print(m, flush=True)
        assert_parity(m, route)
    elif route == "nvfp4":
        qn, kn = pa.quantize_nvfp4(q), pa.quantize_nvfp4(k)
        o, lse = pa.fwd_nvfp4(qn, kn, pa.quantize_mx(v, pa.MXFP4, pa.ALONG_SEQ))
        torch.cuda.synchronize()
        ref = orc.nvfp4_anchored_forward(x["q"], x["k"], x["v"])
        m = parity(bf16_to_np(o), oracle_o(ref), lse.cpu().numpy(), ref["lse"])
        print(m, flush=True)
        assert_parity(m, route)
    else:
        causal = route == "bwd_causal"
        fwd = orc.causal_forward(x["q"], x["k"], x["v"], KB=64) if causal else \
            orc.directp_forward(x["q"], x["k"], x["v"], KB=64)
        o16, lse32 = fwd["O_bf16"], fwd["lse"].astype(np.float32)
        o = to_dev(o16, dev)
        lse = torch.from_numpy(np.ascontiguousarray(lse32)).to(dev)
        qm = pa.quantize_mx(q, pa.MXFP4, pa.ALONG_D)
        km = pa.quantize_mx(k, pa.MXFP4, pa.ALONG_D)
        q8 = pa.quantize_mx(q, pa.MXFP8, pa.ALONG_SEQ)
        k8 = pa.quantize_mx(k, pa.MXFP8, pa.ALONG_SEQ)
        v8 = pa.quantize_mx(v, pa.MXFP8, pa.ALONG_D)
        dq, dk, dv = pa.bwd(qm, km, q8, k8, v8, o, to_dev(x["do"], dev), lse, causal=causal)
        torch.cuda.synchronize()
        ref = orc.causal_backward(x["q"], x["k"], x["v"], x["do"], o16, lse32, causal=causal)
        for name, g, r in (("dQ", dq, ref["dQ"]), ("dK", dk, ref["dK"]), ("dV", dv, ref["dV"])):
            cos, rel = _cos_rel(bf16_to_np(g), r)
            print("%s cos %.7f rel_rms %.3e" % (name, cos, rel), flush=True)
            assert cos >= 0.999 and rel <= 5e-3, (name, cos, rel)
