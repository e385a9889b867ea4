"""GPU Direct-P on the integer-log2 anchor (fp4attn_fwd_ex with FP4ATTN_FWD_ANCHORED) versus the
oracle's anchored mode (P_DIRECT_ANCHOR).

Tolerances are those of the running-max route (tests/gpuhelpers.py). Cases:
- small shapes compared on every element (several query tiles and key blocks, ragged tails, GQA);
- V = 1 gives O = 1 exactly (consistent normalization);
- the headline shape B1 H16 N4096 D128 on every element, and the DiT shape on two whole heads
  plus one row per 256-query tile;
- logits near 600 (the range the summary's range guard addresses), and key magnitudes growing
  along the sequence so that later key blocks lie far more than 64 binades above the anchor
  sampled from the first block: the guard must move the anchor, by exact powers of two;
- the code-flip rate, as for the running-max route (V the identity on a 128-key window).
"""
import numpy as np
import pytest

from precision_attention_amd.inputs import WORKLOADS, attention_inputs, f32_to_bf16_bits
from tests.gpuhelpers import assert_parity, bf16_to_np, channel_scale, oracle_o, parity, require_gpu, to_dev

pytestmark = pytest.mark.gpu


def gpu_anchored(x, dev):
    import precision_attention_amd as pa
    import torch

    q, k, v = (to_dev(x[n], dev) for n in ("q", "k", "v"))
    qm, km, vm = pa.quantize_mx_batch((q, k, v), (pa.MXFP4,) * 3, (pa.ALONG_D, pa.ALONG_D, pa.ALONG_SEQ))
    o, lse = pa.fwd(qm, km, vm, causal=False, anchored=True)
    torch.cuda.synchronize()
    return bf16_to_np(o), lse.cpu().numpy()


SMALL = [
    (1, 1, 1, 128, 64),
    (1, 2, 2, 96, 64),
    (2, 4, 2, 352, 128),
    (1, 3, 1, 544, 128),
    (1, 2, 1, 1024, 64),
    (1, 2, 1, 32, 128),
    (2, 1, 1, 32, 64),
]


@pytest.mark.parametrize("shape", SMALL, ids=["x".join(map(str, s)) for s in SMALL])
def test_anchored_small_all_elements(orc, shape):
    dev = require_gpu()
    B, H, Hkv, N, D = shape
    print("anchored case", shape, flush=True)
    x = attention_inputs(B, H, Hkv, N, D, seed=sum(shape) + 7)
    o, lse = gpu_anchored(x, dev)
    ref = orc.directp_anchored_forward(x["q"], x["k"], x["v"])
    m = parity(o, oracle_o(ref), lse, ref["lse"])
    print(m, flush=True)
    assert_parity(m, str(shape))


def test_anchored_v_ones(orc):
    dev = require_gpu()
    x = attention_inputs(1, 2, 1, 352, 128, seed=3)
    x["v"] = np.full_like(x["v"], 0x3F80)
    o, _ = gpu_anchored(x, dev)
    assert np.array_equal(o, np.ones_like(o))


def test_anchored_headline_whole(orc):
    dev = require_gpu()
    x = attention_inputs(1, 16, 16, 4096, 128, seed=0)
    print("anchored, B1 H16 N4096 D128, every element", flush=True)
    o, lse = gpu_anchored(x, dev)
    ref = orc.directp_anchored_forward(x["q"], x["k"], x["v"])
    m = parity(o, oracle_o(ref), lse, ref["lse"])
    print(m, flush=True)
    assert_parity(m, "anchored headline")


def test_anchored_dit_two_heads_and_every_tile(orc):
    dev = require_gpu()
    w = WORKLOADS["dit_h24_n32768_d128_outliers"]
    B, H, N, D = w["B"], w["H"], w["N"], w["D"]
    print("anchored, DiT shape", flush=True)
    x = attention_inputs(B, H, H, N, D, seed=0, outlier_frac=w["outlier_frac"])
    o, lse = gpu_anchored(x, dev)
    rng = np.random.default_rng(5)
    tiles = np.arange(0, N, 256)
    rows = [np.arange(0, N), np.arange((H - 1) * N, H * N)]
    rows += [h * N + tiles + rng.integers(0, 256, tiles.size) for h in range(1, H - 1)]
    rows = np.unique(np.concatenate(rows)).astype(np.int64)
    ref = orc.directp_anchored_forward(x["q"], x["k"], x["v"], rows=rows)
    m = parity(o.reshape(-1, D)[rows], oracle_o(ref).reshape(-1, D), lse.reshape(-1)[rows], ref["lse"],
               scale=channel_scale(x, B, H, N, D, rows))
    print("anchored dit", m, flush=True)
    assert_parity(m, "anchored dit")


def _scaled(x, n, f):
    return f32_to_bf16_bits((x[n].astype(np.uint32) << 16).view(np.float32) * f)


@pytest.mark.parametrize("case", ["logits_near_600", "growing_keys"])
def test_anchored_range_guard(orc, case):
    dev = require_gpu()
    B, H, N, D = 1, 2, 1024, 128
    x = attention_inputs(B, H, H, N, D, seed=17)
    if case == "logits_near_600":
        for n in ("q", "k"):
            x[n] = _scaled(x, n, np.float32(11.0))
    else:
        # key j scaled by 1 + 30 j / N: the last key blocks' scores reach hundreds of binades above
        # the first block's, so the anchor sampled there must move several times
        x["q"] = _scaled(x, "q", np.float32(4.0))
        f = (1.0 + 30.0 * np.arange(N) / N).astype(np.float32)[None, None, :, None]
        x["k"] = _scaled(x, "k", f)
    ref = orc.directp_anchored_forward(x["q"], x["k"], x["v"])
    # the oracle holds 2^(S c) in binary64, which covers logits up to about 700
    assert np.all(np.isfinite(ref["O"])) and np.all(np.isfinite(ref["lse"]))
    ops = ref["ops"]
    Qd = orc.mx_dequantize(*ops["q"], orc.FMT_E2M1, "d")
    Kd = orc.mx_dequantize(*ops["k"], orc.FMT_E2M1, "d")
    S = np.einsum("bhnd,bhmd->bhnm", Qd, Kd)
    c = float(orc.log2e_scale(D))
    first = np.floor(S[..., :128].max(-1) * c)
    rest = np.floor(S[..., 128:].max(-1) * c)
    print(case, "largest logit %.0f; rows whose later blocks exceed the first block by > 64 binades: %d" % (
        (S / np.sqrt(D)).max(), int(np.sum(rest - first > 64))), flush=True)
    if case == "logits_near_600":
        assert (S / np.sqrt(D)).max() > 500
    else:
        assert np.sum(rest - first > 64) > N
    o, lse = gpu_anchored(x, dev)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    m = parity(o, oracle_o(ref), lse, ref["lse"])
    # LSE is a few hundred here: compare it relative to its size as well (binary32 keeps 24 bits)
    rel_lse = float(np.max(np.abs(lse - ref["lse"]) / np.maximum(np.abs(ref["lse"]), 1.0)))
    print(case, m, "lse rel %.3g" % rel_lse, flush=True)
    assert m["o_over_bound"] == 0 and m["o_mean"] <= 1e-3 and rel_lse <= 1e-6, m


def test_anchored_code_flip_rate(orc):
    from tests.test_gpu_fullsize import FLIP_RATE_MAX, _window_identity_v, bf16_to_np_bits

    dev = require_gpu()
    B, H, N, D = 1, 16, 4096, 128
    x0 = attention_inputs(B, H, H, N, D, seed=0)
    observed = mism = 0
    for w0 in (0, 2048 + 512):
        print("anchored code-flip window at key %d" % w0, flush=True)
        x = dict(x0, v=_window_identity_v(x0["v"], w0))
        o, _ = gpu_anchored(x, dev)
        r = bf16_to_np_bits(orc.directp_anchored_forward(x["q"], x["k"], x["v"])["O_bf16"])
        big = np.maximum(np.abs(o), np.abs(r))
        bad = (np.abs(o - r) > 0.1 * big) & (big >= 2.0 ** -100)
        observed += o.size
        mism += int(bad.sum())
    print("anchored Direct-P code mismatches: %d of %d codes observed (bound %g)" % (mism, observed, FLIP_RATE_MAX),
          flush=True)
    assert mism / observed <= FLIP_RATE_MAX
