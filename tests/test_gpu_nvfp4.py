"""GPU NVFP4-style Q/K route against the oracle: the block quantizer (fp4attn_quantize_nvfp4) bit for
bit, and the Direct-P forward on the integer-log2 anchor with S from the bf16 expansions
(fp4attn_fwd_nvfp4) within the tolerances of the other forward routes.

S = Q_hat K_hat^T is not exact in fp32 for NVFP4 operands (E4M3 block scales spread the products
over more bits than an fp32 sum keeps); the oracle takes the binary32 rounding of the exact sum, the
kernel the MFMA's fp32 accumulation, so a code whose u lies within an ulp or two of a step point can
differ. The O and LSE bounds cover that (a flipped code moves one score's weight by one E2M1 step).
"""
import numpy as np
import pytest

from precision_attention_amd.inputs import WORKLOADS, attention_inputs, f32_to_bf16_bits
from tests.gpuhelpers import assert_parity, bf16_to_np, channel_scale, oracle_o, parity, require_gpu, to_dev

pytestmark = pytest.mark.gpu


def _special(seed):
    """Gaussian rows plus rows holding the quantizer's edge cases, as bf16 bits [1, 2, 64, 128]."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((1, 2, 64, 128)).astype(np.float32)
    x[0, 0, 0] = 0.0                                      # all-zero blocks
    x[0, 0, 1, :16] = [6.375, -3.1875, 0.53125] + [0.0] * 13  # the scale tie (1.0625 -> 1.0)
    x[0, 0, 2] = -2.0 ** -20                              # blocks below the smallest scale
    x[0, 0, 3] = 6.0 * 448.0 * 3.0                        # the scale saturates at 448
    x[0, 0, 4] *= 1000.0
    x[0, 0, 5] *= 1e-3
    # elements on the E2M1 midpoints of a block whose scale is 1 (amax 6)
    x[0, 1, 0, :16] = [6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -0.75, -1.25, -1.75, -2.5, -3.5, -5.0, 0.1]
    return f32_to_bf16_bits(x)


@pytest.mark.parametrize("g", [0, -3, 5])
@pytest.mark.parametrize("case", ["special", "gaussian_h4_n352_d64"])
def test_nvfp4_quantizer_bit_exact(orc, case, g):
    import precision_attention_amd as pa
    import torch

    dev = require_gpu()
    x = _special(3) if case == "special" else attention_inputs(1, 4, 4, 352, 64, seed=5)["q"]
    if g:
        x = f32_to_bf16_bits((x.astype(np.uint32) << 16).view(np.float32) * np.float32(2.0 ** g))
    print("nvfp4 quantizer case", case, x.shape, "g", g, flush=True)
    out = pa.quantize_nvfp4(to_dev(x, dev), tensor_exp=g)
    torch.cuda.synchronize()
    raw = out.codes.cpu().numpy()
    codes = np.stack([raw & 15, raw >> 4], axis=-1).reshape(x.shape)
    oc, os_, oxh = orc.nvfp4_quantize(x, g)
    assert np.array_equal(out.scales.cpu().numpy(), os_), "scales differ"
    bad = np.argwhere(codes != oc)
    assert bad.size == 0, "codes differ at %s" % (bad[:5],)
    assert np.array_equal(bf16_to_np(out.xhat).astype(np.float64), oxh), "x_hat differs"


def gpu_nvfp4(x, dev):
    import precision_attention_amd as pa
    import torch

    q, k, v = (to_dev(x[n], dev) for n in ("q", "k", "v"))
    qn, kn = pa.quantize_nvfp4(q), pa.quantize_nvfp4(k)
    vm = pa.quantize_mx(v, pa.MXFP4, pa.ALONG_SEQ)
    o, lse = pa.fwd_nvfp4(qn, kn, vm)
    torch.cuda.synchronize()
    return bf16_to_np(o), lse.cpu().numpy()


SMALL = [
    (1, 1, 1, 128, 64),
    (1, 2, 2, 96, 64),
    (2, 4, 2, 352, 128),
    (1, 3, 1, 544, 128),
    (1, 2, 1, 32, 128),
]


@pytest.mark.parametrize("shape", SMALL, ids=["x".join(map(str, s)) for s in SMALL])
def test_nvfp4_forward_small_all_elements(orc, shape):
    dev = require_gpu()
    B, H, Hkv, N, D = shape
    print("nvfp4 forward case", shape, flush=True)
    x = attention_inputs(B, H, Hkv, N, D, seed=sum(shape) + 11)
    o, lse = gpu_nvfp4(x, dev)
    ref = orc.nvfp4_anchored_forward(x["q"], x["k"], x["v"])
    m = parity(o, oracle_o(ref), lse, ref["lse"])
    print(m, flush=True)
    assert_parity(m, str(shape))


def test_nvfp4_forward_v_ones(orc):
    dev = require_gpu()
    x = attention_inputs(1, 2, 1, 352, 128, seed=3)
    x["v"] = np.full_like(x["v"], 0x3F80)
    o, _ = gpu_nvfp4(x, dev)
    assert np.array_equal(o, np.ones_like(o))


def test_nvfp4_forward_headline_whole(orc):
    dev = require_gpu()
    x = attention_inputs(1, 16, 16, 4096, 128, seed=0)
    print("nvfp4 forward, B1 H16 N4096 D128, every element", flush=True)
    o, lse = gpu_nvfp4(x, dev)
    ref = orc.nvfp4_anchored_forward(x["q"], x["k"], x["v"])
    m = parity(o, oracle_o(ref), lse, ref["lse"])
    print(m, flush=True)
    assert_parity(m, "nvfp4 headline")


def test_nvfp4_forward_dit_two_heads_and_every_tile(orc):
    dev = require_gpu()
    w = WORKLOADS["dit_h24_n32768_d128_outliers"]
    B, H, N, D = w["B"], w["H"], w["N"], w["D"]
    print("nvfp4 forward, DiT shape", flush=True)
    x = attention_inputs(B, H, H, N, D, seed=0, outlier_frac=w["outlier_frac"])
    o, lse = gpu_nvfp4(x, dev)
    rng = np.random.default_rng(5)
    tiles = np.arange(0, N, 256)
    rows = [np.arange(0, N), np.arange((H - 1) * N, H * N)]
    rows += [h * N + tiles + rng.integers(0, 256, tiles.size) for h in range(1, H - 1)]
    rows = np.unique(np.concatenate(rows)).astype(np.int64)
    ref = orc.nvfp4_anchored_forward(x["q"], x["k"], x["v"], rows=rows)
    m = parity(o.reshape(-1, D)[rows], oracle_o(ref).reshape(-1, D), lse.reshape(-1)[rows], ref["lse"],
               scale=channel_scale(x, B, H, N, D, rows))
    print("nvfp4 dit", m, flush=True)
    assert_parity(m, "nvfp4 dit")


def test_nvfp4_range_guard_growing_keys(orc):
    """Key j scaled by 1 + 30 j / N (and Q by 4): the last key blocks' scores lie hundreds of
    binades above the first block's, so the anchor sampled on the first block must move several
    times (by exact powers of two), as in the MXFP4 anchored route's guard test."""
    dev = require_gpu()
    B, H, N, D = 1, 2, 1024, 128
    print("nvfp4 range-guard case", flush=True)
    x = attention_inputs(B, H, H, N, D, seed=17)
    f32 = lambda n: (x[n].astype(np.uint32) << 16).view(np.float32)
    x["q"] = f32_to_bf16_bits(f32("q") * np.float32(4.0))
    x["k"] = f32_to_bf16_bits(f32("k") * (1.0 + 30.0 * np.arange(N) / N).astype(np.float32)[None, None, :, None])
    ref = orc.nvfp4_anchored_forward(x["q"], x["k"], x["v"])
    assert np.all(np.isfinite(ref["O"])) and np.all(np.isfinite(ref["lse"]))
    o, lse = gpu_nvfp4(x, dev)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    m = parity(o, oracle_o(ref), lse, ref["lse"])
    # LSE is a few hundred here: compare it relative to its size as well (binary32 keeps 24 bits)
    rel_lse = float(np.max(np.abs(lse - ref["lse"]) / np.maximum(np.abs(ref["lse"]), 1.0)))
    print(m, "lse rel %.3g, largest lse %.0f" % (rel_lse, float(np.max(ref["lse"]))), flush=True)
    assert m["o_over_bound"] == 0 and m["o_mean"] <= 1e-3 and rel_lse <= 1e-6, m
