"""GPU BF16-MFMA forward (fp4attn_fwd_bf16) versus fp64 textbook attention on the same
bf16 inputs (its oracle is the plain definition: the variant quantizes nothing but P, which
it rounds to bf16 for the P.V product). Same O/LSE tolerances as the FP4 routes. The shapes
span one to 17 key blocks of 64 (odd and even counts, ragged against the 256-query tiles),
D 64 and 128, and grouped heads."""
import numpy as np
import pytest

from oracle import textbook
from precision_attention_amd.inputs import attention_inputs
from tests.gpuhelpers import assert_parity, bf16_to_np, parity, require_gpu, to_dev

pytestmark = pytest.mark.gpu

SHAPES = [(1, 1, 1, 128, 64), (2, 4, 2, 352, 128), (1, 3, 1, 544, 64), (1, 2, 2, 1024, 128), (1, 2, 1, 32, 128),
          (1, 2, 1, 1056, 64)]


@pytest.mark.parametrize("causal", [False, True], ids=["noncausal", "causal"])
@pytest.mark.parametrize("shape", SHAPES, ids=["x".join(map(str, s)) for s in SHAPES])
def test_bf16_forward(orc, shape, causal):
    import precision_attention_amd as pa
    import torch

    dev = require_gpu()
    B, H, Hkv, N, D = shape
    print("bf16 case", shape, causal, flush=True)
    x = attention_inputs(B, H, Hkv, N, D, seed=7 + N)
    q, k, v = (to_dev(x[n], dev) for n in ("q", "k", "v"))
    o, lse = pa.fwd_bf16(q, k, v.transpose(-1, -2).contiguous(), causal=causal)
    torch.cuda.synchronize()
    Q, K, V = (orc.bf16_to_f64(x[n]) for n in ("q", "k", "v"))
    O, L, _ = textbook.attention(Q, K, V, causal)
    m = parity(bf16_to_np(o), O, lse.cpu().numpy(), L)
    print(m, flush=True)
    assert_parity(m, str(shape))


@pytest.mark.parametrize("causal", [False, True], ids=["noncausal", "causal"])
def test_bf16_forward_growing_logits(orc, causal):
    """Keys whose magnitude steps up every 128 keys (x1, x2, ... x8), so that each row's max grows
    by far more than 2^8 in P several times along the sequence: the kernel's reference point and
    the rescale of O and l move mid-row, not only on the first block (on N(0,1) inputs they never
    do). Compared with fp64 textbook attention of the same bf16 inputs."""
    import precision_attention_amd as pa
    import torch

    from precision_attention_amd.inputs import f32_to_bf16_bits

    dev = require_gpu()
    B, H, Hkv, N, D = 1, 2, 1, 1024, 128
    print("bf16 growing-logits case", causal, flush=True)
    x = attention_inputs(B, H, Hkv, N, D, seed=23)
    kf = (x["k"].astype(np.uint32) << 16).view(np.float32)
    scale = (1.0 + np.arange(N) // 128).astype(np.float32)[None, None, :, None]
    x["k"] = f32_to_bf16_bits(kf * scale)
    q, k, v = (to_dev(x[n], dev) for n in ("q", "k", "v"))
    o, lse = pa.fwd_bf16(q, k, v.transpose(-1, -2).contiguous(), causal=causal)
    torch.cuda.synchronize()
    Q, K, V = (orc.bf16_to_f64(x[n]) for n in ("q", "k", "v"))
    O, L, _ = textbook.attention(Q, K, V, causal)
    m = parity(bf16_to_np(o), O, lse.cpu().numpy(), L)
    print(m, flush=True)
    assert_parity(m, "growing logits")
