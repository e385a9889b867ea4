"""GPU MX quantizer versus the oracle: codes and scales must be bit-identical."""
import numpy as np
import pytest

from precision_attention_amd.inputs import attention_inputs, f32_to_bf16_bits
from tests.gpuhelpers import require_gpu, to_dev
from tests.mxlayout import unpack_codes, unpack_scales

pytestmark = pytest.mark.gpu

ORC_FMT = {1: 1, 2: 2}  # library MXFP4/MXFP8 -> oracle E2M1/E4M3
AXES = {0: "d", 1: "seq"}


def special_tensor(B, H, N, D, seed):
    """Gaussian values plus the edge cases of the scale and rounding rules."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, H, N, D)).astype(np.float32)
    x[0, 0, :32, :] = 0.0                                   # all-zero blocks on both axes
    x[0, 0, 32:64, :32] = np.float32(2.0 ** -130) * x[0, 0, 32:64, :32]   # bf16 subnormals
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0], np.float32)
    x[0, 0, 64:96, :] = np.resize(ties, (32, D)) * np.float32(0.5)        # exact E2M1 ties
    x[0, 0, 96:128, :32] = np.float32(3e38) * np.sign(x[0, 0, 96:128, :32])  # near the bf16 max
    x[0, 0, 96:128, 32:64] = -0.0                                            # negative zeros
    if D > 64:
        x[0, 0, 96:128, 64:] *= np.float32(1e-30)                            # tiny normals
    if N > 128:
        x[0, 0, 128:, :] *= np.float32(1e-35)                                # mixed normal/subnormal
    return f32_to_bf16_bits(x)


CASES = [
    ("tiny_h1_n128_d64", lambda: attention_inputs(1, 1, 1, 128, 64, seed=0)["q"]),
    ("ragged_n96_d128", lambda: attention_inputs(2, 3, 3, 96, 128, seed=1)["k"]),
    ("special_n160_d64", lambda: special_tensor(1, 2, 160, 64, 2)),
    ("special_n256_d128", lambda: special_tensor(2, 1, 256, 128, 3)),
    # several sequence tiles with a ragged last one, and scale rows of 9 and 17 blocks (the
    # transposed scale rows then start at unaligned offsets as well as aligned ones)
    ("ragged_n288_d128", lambda: attention_inputs(1, 2, 2, 288, 128, seed=4)["v"]),
    ("ragged_n544_d64", lambda: special_tensor(1, 2, 544, 64, 5)),
    ("directp_h16_n4096_d128_q", lambda: attention_inputs(1, 16, 16, 4096, 128, seed=0)["q"]),
]


@pytest.mark.parametrize("name,make", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("fmt", [1, 2], ids=["mxfp4", "mxfp8"])
@pytest.mark.parametrize("axis", [0, 1], ids=["along_d", "along_seq"])
def test_quantizer_bit_exact(orc, name, make, fmt, axis):
    import precision_attention_amd as pa
    import torch

    dev = require_gpu()
    x = make()
    shape = x.shape
    print("quantizer case", name, shape, "fmt", fmt, "axis", axis, flush=True)
    mx = pa.quantize_mx(to_dev(x, dev), fmt, axis)
    torch.cuda.synchronize()
    codes = unpack_codes(mx.codes.cpu().numpy(), fmt, axis, shape)
    scales = unpack_scales(mx.scales.cpu().numpy(), axis, shape)
    oc, os_ = orc.mx_quantize(x, ORC_FMT[fmt], AXES[axis])
    assert np.array_equal(scales, os_), "scales differ at %s" % (np.argwhere(scales != os_)[:5],)
    bad = np.argwhere(codes != oc)
    assert bad.size == 0, "codes differ at %s: gpu %s oracle %s" % (bad[:5], codes[tuple(bad[0])], oc[tuple(bad[0])])


BATCH_CASES = [
    # (name, B, H, Hkv, N, D, formats, axes)
    ("fwd_qkv_gqa_h4kv2_n96_d128", 1, 4, 2, 96, 128, (1, 1, 1, 2), (0, 0, 1, 1)),
    ("bwd_views_h2kv1_n160_d64", 2, 2, 1, 160, 64, (2, 2, 2, 1), (1, 1, 0, 0)),
    ("directp_h16_n4096_d128", 1, 16, 16, 4096, 128, (1, 1, 1), (0, 0, 1)),
]


@pytest.mark.parametrize("case", BATCH_CASES, ids=[c[0] for c in BATCH_CASES])
def test_quantizer_batch_bit_exact(orc, case):
    """One launch over several tensors (Q and K heads differ under GQA; the fourth job carries the
    rule's edge cases) gives the oracle's codes and scales for every job."""
    import precision_attention_amd as pa
    import torch

    name, B, H, Hkv, N, D, fmts, axes = case
    dev = require_gpu()
    inp = attention_inputs(B, H, Hkv, N, D, seed=7)
    xs = [inp["q"], inp["k"], inp["v"]]
    if len(fmts) == 4:
        xs.append(special_tensor(B, Hkv, N, D, 4))
    print("quantizer batch", name, [x.shape for x in xs], fmts, axes, flush=True)
    outs = pa.quantize_mx_batch([to_dev(x, dev) for x in xs], fmts, axes)
    torch.cuda.synchronize()
    for i, (x, mx, fmt, axis) in enumerate(zip(xs, outs, fmts, axes)):
        codes = unpack_codes(mx.codes.cpu().numpy(), fmt, axis, x.shape)
        scales = unpack_scales(mx.scales.cpu().numpy(), axis, x.shape)
        oc, os_ = orc.mx_quantize(x, ORC_FMT[fmt], AXES[axis])
        assert np.array_equal(scales, os_), "job %d: scales differ at %s" % (i, np.argwhere(scales != os_)[:5])
        bad = np.argwhere(codes != oc)
        assert bad.size == 0, "job %d: codes differ at %s" % (i, bad[:5])
