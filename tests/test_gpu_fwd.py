"""GPU forward (fp4attn_fwd) versus the oracle.

Tolerances (at unit-variance outputs): O and LSE max |err| <= 1e-2 and mean |err| <= 1e-3,
plus relative RMS of O <= 5e-3. On the outlier-channel workload the V channels scaled by 10
give outputs 10x larger, so there each channel's error is measured in units of its scale. Small shapes compare every element and
span several query tiles, several key blocks, ragged tails (N % 128 != 0 and N % 64 != 0) and
grouped-query heads. The full-size workloads are compared in tests/test_gpu_fullsize.py.
"""
import numpy as np
import pytest

from precision_attention_amd.inputs import attention_inputs, f32_to_bf16_bits
from tests.gpuhelpers import assert_parity, bf16_to_np, oracle_o, parity, require_gpu, to_dev

pytestmark = pytest.mark.gpu


def run_gpu(x, causal, dev, fp8=None):
    """fp8=None: the route's own V format (MXFP8 causal, MXFP4 Direct-P); fp8=True with
    causal=False: the noncausal FP8 P/V route."""
    import precision_attention_amd as pa
    import torch

    fp8 = causal if fp8 is None else fp8
    q, k, v = (to_dev(x[n], dev) for n in ("q", "k", "v"))
    qm = pa.quantize_mx(q, pa.MXFP4, pa.ALONG_D)
    km = pa.quantize_mx(k, pa.MXFP4, pa.ALONG_D)
    vm = pa.quantize_mx(v, pa.MXFP8 if fp8 else pa.MXFP4, pa.ALONG_SEQ)
    o, lse = pa.fwd(qm, km, vm, causal=causal)
    torch.cuda.synchronize()
    return bf16_to_np(o), lse.cpu().numpy()


def run_oracle(orc, x, causal, KB, rows=None, fp8=None):
    fp8 = causal if fp8 is None else fp8
    if fp8:
        return orc.fp8_forward(x["q"], x["k"], x["v"], KB=KB, causal=causal, rows=rows)
    return orc.directp_forward(x["q"], x["k"], x["v"], KB=KB, rows=rows)


SMALL = [
    # (B, H, Hkv, N, D)
    (1, 1, 1, 128, 64),      # the tiny configuration: one query tile, two key blocks
    (1, 2, 2, 96, 64),       # one ragged query tile, ragged key block
    (2, 4, 2, 352, 128),     # 3 query tiles (last ragged), 6 key blocks (last half), GQA
    (1, 3, 1, 544, 128),     # N = 4*128 + 32, three query heads on one KV head
    (1, 2, 1, 1024, 64),     # 16 key blocks, running max moves many times
    (1, 2, 1, 32, 128),      # the smallest N: one 32-key block, the rest of the key block masked
    (2, 1, 1, 32, 64),       # the same at D = 64, two batches
]


@pytest.mark.parametrize("causal", [False, True], ids=["directp", "causal_fp8"])
@pytest.mark.parametrize("shape", SMALL, ids=["x".join(map(str, s)) for s in SMALL])
def test_forward_small_all_elements(orc, shape, causal):
    import precision_attention_amd as pa

    dev = require_gpu()
    B, H, Hkv, N, D = shape
    print("fwd case", shape, "causal", causal, flush=True)
    x = attention_inputs(B, H, Hkv, N, D, seed=sum(shape))
    o, lse = run_gpu(x, causal, dev)
    ref = run_oracle(orc, x, causal, pa.key_block(D, causal))
    m = parity(o, oracle_o(ref), lse, ref["lse"])
    print(m, flush=True)
    assert_parity(m, str(shape))


@pytest.mark.parametrize("shape", SMALL, ids=["x".join(map(str, s)) for s in SMALL])
def test_forward_fp8_noncausal_small_all_elements(orc, shape):
    """The noncausal FP8 P/V route (MXFP8 V, E4M3 P, no mask) against the oracle."""
    import precision_attention_amd as pa

    dev = require_gpu()
    B, H, Hkv, N, D = shape
    print("fp8 noncausal case", shape, flush=True)
    x = attention_inputs(B, H, Hkv, N, D, seed=sum(shape) + 1)
    o, lse = run_gpu(x, False, dev, fp8=True)
    ref = run_oracle(orc, x, False, pa.key_block(D, False), fp8=True)
    m = parity(o, oracle_o(ref), lse, ref["lse"])
    print(m, flush=True)
    assert_parity(m, str(shape))


@pytest.mark.parametrize("causal", [False, True], ids=["directp", "causal_fp8"])
def test_consistent_normalization_v_ones(orc, causal):
    """V = 1 gives O = 1 exactly: numerator and denominator use the same represented P."""
    dev = require_gpu()
    x = attention_inputs(1, 2, 1, 352, 128, seed=3)
    x["v"] = np.full_like(x["v"], 0x3F80)
    o, _ = run_gpu(x, causal, dev)
    assert np.array_equal(o, np.ones_like(o))


def test_deterministic(orc):
    dev = require_gpu()
    x = attention_inputs(1, 4, 4, 512, 128, seed=5)
    o1, l1 = run_gpu(x, False, dev)
    o2, l2 = run_gpu(x, False, dev)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("D", [64, 128])
def test_large_logits(orc, D):
    """Scores far from zero (inputs x 8): the running max and the E8M0 clamp at -127, on Direct-P,
    the causal FP8 route and the noncausal FP8 P/V route."""
    import precision_attention_amd as pa

    dev = require_gpu()
    rng = np.random.default_rng(8)
    B, H, N = 1, 2, 256
    q = (rng.standard_normal((B, H, N, D)) * 8).astype(np.float32)
    k = (rng.standard_normal((B, H, N, D)) * 8).astype(np.float32)
    v = rng.standard_normal((B, H, N, D)).astype(np.float32)
    x = {"q": f32_to_bf16_bits(q), "k": f32_to_bf16_bits(k), "v": f32_to_bf16_bits(v)}
    for causal, fp8 in ((False, None), (True, None), (False, True)):
        o, lse = run_gpu(x, causal, dev, fp8=fp8)
        ref = run_oracle(orc, x, causal, pa.key_block(D, causal), fp8=fp8)
        m = parity(o, oracle_o(ref), lse, ref["lse"])
        print("large logits D", D, "causal", causal, "fp8", fp8, m, flush=True)
        assert m["o_over_bound"] == 0 and m["lse_max"] <= 1e-2, m
