"""Host-side checks of the Python binding (no GPU needed).

The C ABI takes raw device pointers and cannot see buffer sizes, so the binding checks every
tensor before a call: an undersized workspace or MX buffer, a wrong shape, dtype or layout, or
mismatched head counts would otherwise become out-of-bounds device accesses. Each case below
breaks one rule and must raise ValueError before the library is called; a fully valid call on
CPU tensors is refused for its device.
"""
import pytest
import torch

import precision_attention_amd as pa

B, H, HKV, N, D = 1, 4, 2, 64, 128
CPU = torch.device("cpu")


def mx(heads, fmt, axis, n=N):
    return pa.mx_empty(B, heads, n, D, fmt, axis, CPU)


def fwd_args():
    return dict(q=mx(H, pa.MXFP4, pa.ALONG_D), k=mx(HKV, pa.MXFP4, pa.ALONG_D), v=mx(HKV, pa.MXFP4, pa.ALONG_SEQ),
                out=torch.empty(B, H, N, D, dtype=torch.bfloat16), lse=torch.empty(B, H, N))


def bwd_args():
    return dict(q=mx(H, pa.MXFP4, pa.ALONG_D), k=mx(HKV, pa.MXFP4, pa.ALONG_D), q8=mx(H, pa.MXFP8, pa.ALONG_SEQ),
                k8=mx(HKV, pa.MXFP8, pa.ALONG_SEQ), v8=mx(HKV, pa.MXFP8, pa.ALONG_D),
                o=torch.empty(B, H, N, D, dtype=torch.bfloat16), do=torch.empty(B, H, N, D, dtype=torch.bfloat16),
                lse=torch.empty(B, H, N),
                workspace=torch.empty(pa.bwd_workspace_bytes(B, H, HKV, N, D), dtype=torch.uint8))


def shrink(m: pa.MXTensor, what: str) -> pa.MXTensor:
    codes, scales = m.codes, m.scales
    if what == "codes":
        codes = codes[:-1]
    else:
        scales = scales[:-1]
    return pa.MXTensor(codes, scales, m.fmt, m.axis, m.shape)


FWD_BREAKS = {
    "k_other_n": lambda a: a.update(k=mx(HKV, pa.MXFP4, pa.ALONG_D, n=2 * N)),
    "v_other_n": lambda a: a.update(v=mx(HKV, pa.MXFP4, pa.ALONG_SEQ, n=N + 32)),
    "heads_not_multiple": lambda a: a.update(k=mx(3, pa.MXFP4, pa.ALONG_D), v=mx(3, pa.MXFP4, pa.ALONG_SEQ)),
    "q_codes_short": lambda a: a.update(q=shrink(a["q"], "codes")),
    "k_scales_short": lambda a: a.update(k=shrink(a["k"], "scales")),
    "v_along_d": lambda a: a.update(v=mx(HKV, pa.MXFP4, pa.ALONG_D)),
    "q_fp8": lambda a: a.update(q=mx(H, pa.MXFP8, pa.ALONG_D)),
    "out_shape": lambda a: a.update(out=torch.empty(B, H, N, D // 2, dtype=torch.bfloat16)),
    "out_dtype": lambda a: a.update(out=torch.empty(B, H, N, D, dtype=torch.float16)),
    "out_strided": lambda a: a.update(out=torch.empty(B, H, D, N, dtype=torch.bfloat16).transpose(2, 3)),
    "lse_shape": lambda a: a.update(lse=torch.empty(B, H, N + 1)),
    "lse_dtype": lambda a: a.update(lse=torch.empty(B, H, N, dtype=torch.float64)),
}


@pytest.mark.parametrize("case", sorted(FWD_BREAKS))
def test_fwd_rejects(case):
    a = fwd_args()
    FWD_BREAKS[case](a)
    with pytest.raises(ValueError):
        pa.fwd(a["q"], a["k"], a["v"], causal=False, out=a["out"], lse=a["lse"])


BWD_BREAKS = {
    "workspace_short": lambda a: a.update(workspace=a["workspace"][:-1]),
    "workspace_dtype": lambda a: a.update(workspace=torch.empty(a["workspace"].numel(), dtype=torch.int32)),
    "k_other_n": lambda a: a.update(k=mx(HKV, pa.MXFP4, pa.ALONG_D, n=2 * N)),
    "q8_along_d": lambda a: a.update(q8=mx(H, pa.MXFP8, pa.ALONG_D)),
    "k8_fp4": lambda a: a.update(k8=mx(HKV, pa.MXFP4, pa.ALONG_SEQ)),
    "v8_codes_short": lambda a: a.update(v8=shrink(a["v8"], "codes")),
    "o_shape": lambda a: a.update(o=torch.empty(B, HKV, N, D, dtype=torch.bfloat16)),
    "do_dtype": lambda a: a.update(do=torch.empty(B, H, N, D)),
    "lse_shape": lambda a: a.update(lse=torch.empty(B, HKV, N)),
    "heads_not_multiple": lambda a: a.update(k=mx(3, pa.MXFP4, pa.ALONG_D)),
}


@pytest.mark.parametrize("case", sorted(BWD_BREAKS))
def test_bwd_rejects(case):
    a = bwd_args()
    BWD_BREAKS[case](a)
    with pytest.raises(ValueError):
        pa.bwd(**a, causal=True)


def test_valid_calls_refused_off_gpu():
    a = fwd_args()
    with pytest.raises(ValueError, match="GPU"):
        pa.fwd(a["q"], a["k"], a["v"], causal=False, out=a["out"], lse=a["lse"])
    with pytest.raises(ValueError, match="GPU"):
        pa.bwd(**bwd_args(), causal=True)
    x = torch.empty(B, H, N, D, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        pa.quantize_mx(x, pa.MXFP4, pa.ALONG_D)


def test_quantize_rejects_wrong_output():
    x = torch.empty(B, H, N, D, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        pa.quantize_mx(x, pa.MXFP4, pa.ALONG_D, out=mx(H, pa.MXFP4, pa.ALONG_D, n=N // 2))
    with pytest.raises(ValueError):
        pa.quantize_mx(x, pa.MXFP4, pa.ALONG_D, out=shrink(mx(H, pa.MXFP4, pa.ALONG_D), "scales"))
    with pytest.raises(ValueError):
        pa.quantize_mx_batch((x, x), (pa.MXFP4, pa.MXFP4), (pa.ALONG_D, pa.ALONG_SEQ),
                             outs=(mx(H, pa.MXFP4, pa.ALONG_D), mx(H, pa.MXFP8, pa.ALONG_SEQ)))


def test_fwd_bf16_rejects():
    q = torch.empty(B, H, N, D, dtype=torch.bfloat16)
    k = torch.empty(B, HKV, N, D, dtype=torch.bfloat16)
    vt = torch.empty(B, HKV, D, N, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        pa.fwd_bf16(q, k, torch.empty(B, HKV, D, N + 32, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        pa.fwd_bf16(q, k, k)  # V not transposed
    with pytest.raises(ValueError):
        pa.fwd_bf16(q, k.float(), vt)
    with pytest.raises(ValueError):
        pa.fwd_bf16(q, k, vt)  # valid shapes, CPU tensors


def test_project_qkv_rejects():
    Dm = 256
    x = torch.empty(B, N, Dm, dtype=torch.bfloat16)
    w = torch.empty((H + 2 * HKV) * D, Dm, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="tile"):
        pa.project_qkv(x, w, H, HKV, D, tile=64)
    with pytest.raises(ValueError):
        pa.project_qkv(x, w[:-1], H, HKV, D)  # one weight row short
    with pytest.raises(ValueError):
        pa.project_qkv(x, w, H, HKV, D, v_fmt=3)
    for tile in (0, 128, 256):
        with pytest.raises(ValueError, match="GPU"):
            pa.project_qkv(x, w, H, HKV, D, tile=tile)  # valid shapes, CPU tensors
