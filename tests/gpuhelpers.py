"""Helpers for the GPU parity tests: move seeded bf16 inputs to the device, read results
back, and the parity metrics with the tolerances the tests assert."""
import numpy as np
import pytest

# Tolerances for O and LSE (output units, unit-variance inputs): max and mean absolute error.
O_MAX_ABS = 1e-2
O_MEAN_ABS = 1e-3
O_REL_RMS = 5e-3


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
    do = np.abs(np.asarray(o_gpu, np.float64) - np.asarray(o_ref, np.float64))
    if scale is not None:
        do = do / scale
    dl = np.abs(np.asarray(lse_gpu, np.float64) - np.asarray(lse_ref, np.float64))
    ref = np.asarray(o_ref, np.float64)
    rel = float(np.sqrt(np.sum(do ** 2) / max(np.sum(ref ** 2), 1e-300)))
    return {"o_max": float(do.max()), "o_mean": float(do.mean()), "o_rel_rms": rel, "lse_max": float(dl.max()),
            "lse_mean": float(dl.mean())}


def assert_parity(m, what=""):
    msg = "%s %s" % (what, m)
    assert m["o_max"] <= O_MAX_ABS, msg
    assert m["o_mean"] <= O_MEAN_ABS, msg
    assert m["o_rel_rms"] <= O_REL_RMS, msg
    assert m["lse_max"] <= O_MAX_ABS, msg
    assert m["lse_mean"] <= O_MEAN_ABS, msg
