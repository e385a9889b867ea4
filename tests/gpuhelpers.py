"""Helpers for the GPU parity tests: move seeded bf16 inputs to the device, read results
back, and the parity metrics with the tolerances the tests assert.

O is compared with the oracle's own output, which is bf16 like the kernel's (the oracle's
epilogue rounds O / l to bf16). Per element the bound is the larger of 1e-2 (in output units,
or per channel in units of that channel's scale) and one bf16 ulp of the reference value: where
|O| >= 4 one ulp (1/32 or more) exceeds 1e-2, so two correct bf16 roundings of values a few fp32
ulps apart may differ by more than 1e-2 there. Mean absolute error and relative RMS are bounded
as before."""
import numpy as np
import pytest

# Tolerances for O and LSE (output units, unit-variance inputs): max and mean absolute error.
O_MAX_ABS = 1e-2
O_MEAN_ABS = 1e-3
O_REL_RMS = 5e-3


def bf16_ulp(x):
    """Spacing of bfloat16 numbers at |x| (8 significant bits; subnormal spacing below 2^-126)."""
    a = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def oracle_o(ref):
    """The oracle's bf16 output O as float32 values."""
    return (np.asarray(ref["O_bf16"], np.uint16).astype(np.uint32) << 16).view(np.float32)


def require_gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a GPU")
    import precision_attention_amd as pa

    pa.lib()  # raises when the HIP library is missing: no fallback exists
    return torch.device("cuda:0")


def to_dev(bits: np.ndarray, dev):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(dev)


def bf16_to_np(t) -> np.ndarray:
    import torch

    u = t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return (u.astype(np.uint32) << 16).view(np.float32)


def channel_scale(x, B, H, N, D, rows=None):
    """Per-element output scale: 10 on the outlier channels of a head, 1 elsewhere. The
    tolerances hold for unit-variance outputs, so errors are compared in these units."""
    s = np.ones((B, H, N, D))
    for h, chans in enumerate(x.get("outlier_channels", [])):
        s[:, h, :, chans] = 10.0
    return s if rows is None else s.reshape(-1, D)[rows]


def parity(o_gpu, o_ref, lse_gpu, lse_ref, scale=None):
    og = np.asarray(o_gpu, np.float64)
    ref = np.asarray(o_ref, np.float64)
    sc = 1.0 if scale is None else np.asarray(scale, np.float64)
    do = np.abs(og - ref) / sc
    bound = np.maximum(O_MAX_ABS, bf16_ulp(ref) / sc)
    dl = np.abs(np.asarray(lse_gpu, np.float64) - np.asarray(lse_ref, np.float64))
    rel = float(np.sqrt(np.sum(do ** 2) / max(np.sum((ref / sc) ** 2), 1e-300)))
    worst = np.unravel_index(int(np.argmax(do / bound)), do.shape)
    return {"o_max": float(do.max()), "o_mean": float(do.mean()), "o_rel_rms": rel, "lse_max": float(dl.max()),
            "lse_mean": float(dl.mean()), "o_over_bound": int(np.sum(do > bound)),
            "o_bit_exact": float(np.mean(og == ref)), "o_worst_at": tuple(int(i) for i in worst),
            "o_worst_ref": float(ref[worst]), "o_worst_gpu": float(og[worst])}


def assert_parity(m, what=""):
    msg = "%s %s" % (what, m)
    assert m["o_over_bound"] == 0, msg
    assert m["o_mean"] <= O_MEAN_ABS, msg
    assert m["o_rel_rms"] <= O_REL_RMS, msg
    assert m["lse_max"] <= O_MAX_ABS, msg
    assert m["lse_mean"] <= O_MEAN_ABS, msg
