"""The C ABI without a GPU: the library loads, exports every function that
include/fp4attn.h declares, and rejects invalid arguments on the host before any launch."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp4attn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp4attn_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def pa():
    import precision_attention_amd as pa

    if not os.path.exists(pa.library_path()):
        import precision_attention_amd.build as b

        b.build()
    return pa


def test_header_declares_the_abi():
    names = declared_functions()
    for n in ("fp4attn_quantize_mx", "fp4attn_fwd", "fp4attn_bwd", "fp4attn_fwd_bf16", "fp4attn_key_block"):
        assert n in names


def test_library_exports_every_declared_symbol(pa):
    out = subprocess.run(["nm", "-D", "--defined-only", pa.library_path()], stdout=subprocess.PIPE, text=True,
                         check=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if l.strip())
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    L = pa.lib()
    for n in declared_functions():
        getattr(L, n)
    assert sorted(pa.EXPORTED) == declared_functions()


def test_sizes_and_key_block(pa):
    L = pa.lib()
    assert L.fp4attn_mx_codes_bytes(pa.MXFP4, 1, 16, 4096, 128) == 16 * 4096 * 64
    assert L.fp4attn_mx_codes_bytes(pa.MXFP8, 1, 16, 4096, 128) == 16 * 4096 * 128
    assert L.fp4attn_mx_scales_bytes(1, 16, 4096, 128) == 16 * 4096 * 4
    assert L.fp4attn_mx_codes_bytes(7, 1, 1, 32, 64) == 0
    assert pa.key_block(128, False) == 128 and pa.key_block(64, True) == 64 and pa.key_block(64, False) == 64
    assert pa.key_block(128, True) == 128
    assert pa.key_block(96, False) == 0
    assert L.fp4attn_status_str(0) == b"ok"


def _mx(pa, fmt, axis, codes=16, scales=16):
    return pa._MX(fmt, axis, codes, scales)


def test_host_validation_errors(pa):
    L = pa.lib()
    ok4d = _mx(pa, pa.MXFP4, pa.ALONG_D)
    ok4s = _mx(pa, pa.MXFP4, pa.ALONG_SEQ)
    ok8s = _mx(pa, pa.MXFP8, pa.ALONG_SEQ)
    r = ctypes.byref
    # NULL pointers
    assert L.fp4attn_quantize_mx(None, r(ok4d), 1, 1, 128, 64, None) == 1
    assert L.fp4attn_fwd(None, r(ok4d), r(ok4s), 16, 16, 1, 1, 1, 128, 64, 0, None) == 1
    assert L.fp4attn_fwd(r(ok4d), r(ok4d), r(ok4s), None, 16, 1, 1, 1, 128, 64, 0, None) == 1
    assert L.fp4attn_fwd(r(_mx(pa, pa.MXFP4, pa.ALONG_D, 0, 16)), r(ok4d), r(ok4s), 16, 16, 1, 1, 1, 128, 64, 0,
                         None) == 1
    # shapes
    assert L.fp4attn_fwd(r(ok4d), r(ok4d), r(ok4s), 16, 16, 1, 4, 3, 128, 64, 0, None) == 2  # H % Hkv
    assert L.fp4attn_fwd(r(ok4d), r(ok4d), r(ok4s), 16, 16, 1, 1, 1, 100, 64, 0, None) == 2  # N % 32
    assert L.fp4attn_fwd(r(ok4d), r(ok4d), r(ok4s), 16, 16, -1, 1, 1, 128, 64, 0, None) == 2
    assert L.fp4attn_fwd(r(ok4d), r(ok4d), r(ok4s), 16, 16, 1, 1, 1, 128, 96, 0, None) == 3  # D
    assert L.fp4attn_quantize_mx(16, r(ok4d), 1, 1, 128, 256, None) == 3
    # alignment
    assert L.fp4attn_fwd(r(ok4d), r(ok4d), r(ok4s), 8, 16, 1, 1, 1, 128, 64, 0, None) == 4
    assert L.fp4attn_quantize_mx(24, r(ok4d), 1, 1, 128, 64, None) == 4
    # formats: V along the sequence, MXFP4 (Direct-P) or MXFP8 (the FP8 route) when noncausal,
    # MXFP8 when causal; Q and K MXFP4 along D
    assert L.fp4attn_fwd(r(ok4d), r(ok4d), r(ok4d), 16, 16, 1, 1, 1, 128, 64, 0, None) == 5
    assert L.fp4attn_fwd(r(ok4d), r(ok4d), r(ok4s), 16, 16, 1, 1, 1, 128, 64, 1, None) == 5
    assert L.fp4attn_fwd(r(ok4d), r(ok4d), r(_mx(pa, pa.MXFP8, pa.ALONG_D)), 16, 16, 1, 1, 1, 128, 64, 0, None) == 5
    assert L.fp4attn_fwd(r(ok4d), r(ok4d), r(_mx(pa, 3, pa.ALONG_SEQ)), 16, 16, 1, 1, 1, 128, 64, 0, None) == 5
    assert L.fp4attn_fwd(r(ok8s), r(ok4d), r(ok8s), 16, 16, 1, 1, 1, 128, 64, 0, None) == 5
    assert L.fp4attn_quantize_mx(16, r(_mx(pa, 3, 0)), 1, 1, 128, 64, None) == 5
    # empty work returns OK without launching anything
    assert L.fp4attn_fwd(r(ok4d), r(ok4d), r(ok4s), 16, 16, 0, 1, 1, 128, 64, 0, None) == 0
    assert L.fp4attn_fwd(r(ok4d), r(ok4d), r(ok4s), 16, 16, 1, 1, 1, 0, 64, 0, None) == 0
    assert L.fp4attn_quantize_mx(16, r(ok4d), 1, 1, 0, 64, None) == 0
    assert L.fp4attn_fwd_bf16(16, 16, 16, 16, 16, 0, 1, 1, 128, 64, 0, None) == 0
    assert L.fp4attn_fwd_bf16(16, 16, 16, 16, 16, 1, 1, 1, 128, 80, 0, None) == 3


def test_backward_workspace_and_validation(pa):
    L = pa.lib()
    rows = 1 * 32 * 8192
    # Delta and -LSE log2(e) (fp32 each) plus dO's two MXFP8 views (codes and scales)
    assert L.fp4attn_bwd_workspace_bytes(1, 32, 8, 8192, 128) == 2 * rows * 4 + 2 * (rows * 128 + rows * 4)
    assert L.fp4attn_bwd_workspace_bytes(1, 4, 3, 128, 64) == 0  # invalid sizes
    q4 = _mx(pa, pa.MXFP4, pa.ALONG_D)
    q8 = _mx(pa, pa.MXFP8, pa.ALONG_SEQ)
    v8 = _mx(pa, pa.MXFP8, pa.ALONG_D)
    r = ctypes.byref

    def bwd(q=q4, k=q4, qq=q8, kk=q8, vv=v8, ws=16, B=1, N=128, D=64, causal=1):
        return L.fp4attn_bwd(r(q), r(k), r(qq), r(kk), r(vv), 16, 16, 16, 16, 16, 16, ws, B, 2, 1, N, D, causal, None)

    assert bwd(ws=None) == 1
    assert bwd(N=100) == 2
    assert bwd(D=96) == 3
    assert bwd(causal=2) == 3
    assert bwd(ws=8) == 4
    assert bwd(vv=q8) == 5       # V must be MXFP8 along D
    assert bwd(qq=v8) == 5       # Q's FP8 view must be blocked along the sequence
    assert bwd(k=q8) == 5        # K must be the saved MXFP4 (along D)
    assert bwd(B=0) == 0 and bwd(N=0) == 0


def test_quantize_batch_validation(pa):
    """fp4attn_quantize_mx_batch rejects bad arguments on the host, before any launch."""
    L = pa.lib()

    def job(x=16, heads=2, fmt=pa.MXFP4, axis=pa.ALONG_D, codes=16, scales=16):
        j = pa._QuantJob()
        j.x_bf16, j.heads = x, heads
        j.out = pa._MX(fmt, axis, codes, scales)
        return j

    def run(jobs, count=None, B=1, N=128, D=64):
        arr = (pa._QuantJob * max(len(jobs), 1))(*jobs)
        return L.fp4attn_quantize_mx_batch(arr if jobs else None, len(jobs) if count is None else count, B, N, D, None)

    assert run([]) == 1                                   # no jobs array
    assert run([job()], count=0) == 2                     # count out of range
    assert run([job()] * 5) == 2
    assert run([job(), job(x=None)]) == 1                 # a NULL pointer in a job
    assert run([job(), job(heads=0)]) == 2
    assert run([job()], N=100) == 2
    assert run([job()], D=96) == 3
    assert run([job(), job(fmt=3)]) == 5
    assert run([job(), job(axis=2)]) == 5
    assert run([job(), job(codes=24)]) == 4
    assert run([job()] * 4, B=0) == 0 and run([job()], N=0) == 0
    assert pa.MAX_QUANT_JOBS == 4


def test_project_qkv_validation(pa):
    """fp4attn_project_qkv rejects bad arguments on the host, before any launch."""
    L = pa.lib()
    r = ctypes.byref
    q4 = _mx(pa, pa.MXFP4, pa.ALONG_D)
    v4 = _mx(pa, pa.MXFP4, pa.ALONG_SEQ)
    s8 = _mx(pa, pa.MXFP8, pa.ALONG_SEQ)
    d8 = _mx(pa, pa.MXFP8, pa.ALONG_D)

    def proj(x=16, w=16, q=q4, k=q4, v=v4, q8=None, k8=None, v8=None, B=1, N=256, Dm=256, H=2, Hkv=1, D=64):
        p = [None if t is None else r(t) for t in (q, k, v, q8, k8, v8)]
        return L.fp4attn_project_qkv(x, w, *p, B, N, Dm, H, Hkv, D, None)

    assert proj(x=None) == 1 and proj(w=None) == 1 and proj(v=None) == 1
    assert proj(N=100) == 2 and proj(N=0) == 2     # N a positive multiple of 32
    assert proj(Dm=96) == 2 and proj(Dm=0) == 2    # Dm a positive multiple of 64
    assert proj(H=3, Hkv=2) == 2
    assert proj(D=96) == 3
    assert proj(x=8) == 4 and proj(w=24) == 4
    assert proj(q=v4) == 5 and proj(k=d8) == 5      # Q, K MXFP4 along D
    assert proj(v=q4) == 5 and proj(v=_mx(pa, 3, pa.ALONG_SEQ)) == 5
    assert proj(q8=s8, k8=s8) == 5                  # all three FP8 views or none
    assert proj(q8=s8, k8=s8, v8=s8) == 5           # V's FP8 view runs along D
    assert proj(q8=d8, k8=s8, v8=d8) == 5
    assert proj(B=0) == 0 and proj(B=0, q8=s8, k8=s8, v8=d8, v=s8) == 0

    def proj_ex(tile, **kw):
        a = dict(x=16, w=16, B=0, N=256, Dm=256, H=2, Hkv=1, D=64)
        a.update(kw)
        p = [r(t) for t in (q4, q4, v4)] + [None] * 3
        return L.fp4attn_project_qkv_ex(a["x"], a["w"], *p, a["B"], a["N"], a["Dm"], a["H"], a["Hkv"], a["D"],
                                        tile, None)

    # fp4attn_project_qkv_ex: the tile is 0 (chosen by size), 128 or 256; the other checks as above
    assert proj_ex(0) == 0 and proj_ex(128) == 0 and proj_ex(256) == 0
    assert proj_ex(64) == 3 and proj_ex(-1) == 3 and proj_ex(512) == 3
    assert proj_ex(256, x=None) == 1 and proj_ex(256, N=100) == 2


def test_nvfp4_validation(pa):
    """fp4attn_quantize_nvfp4 and fp4attn_fwd_nvfp4 reject bad arguments on the host."""
    L = pa.lib()
    r = ctypes.byref
    v4 = _mx(pa, pa.MXFP4, pa.ALONG_SEQ)

    def quant(x=16, c=16, s=16, xh=16, g=0, B=1, heads=2, N=128, D=64):
        return L.fp4attn_quantize_nvfp4(x, c, s, xh, g, B, heads, N, D, None)

    assert quant(x=None) == 1 and quant(xh=None) == 1
    assert quant(N=100) == 2 and quant(g=101) == 2 and quant(g=-101) == 2
    assert quant(D=96) == 3
    assert quant(s=8) == 4
    assert quant(B=0) == 0

    def fwd(q=16, k=16, v=v4, o=16, lse=16, B=1, H=2, Hkv=1, N=128, D=64):
        return L.fp4attn_fwd_nvfp4(q, k, r(v), o, lse, B, H, Hkv, N, D, None, None, None)

    assert fwd(q=None) == 1 and fwd(lse=None) == 1
    assert fwd(H=3, Hkv=2) == 2 and fwd(N=96 + 8) == 2
    assert fwd(D=80) == 3
    assert fwd(o=24) == 4
    assert fwd(v=_mx(pa, pa.MXFP8, pa.ALONG_SEQ)) == 5 and fwd(v=_mx(pa, pa.MXFP4, pa.ALONG_D)) == 5
    assert fwd(B=0) == 0


def test_clock_probe_validation(pa):
    """fp4attn_clock_probe rejects NULL pointers and out-of-range sizes before any launch."""
    L = pa.lib()
    khz = ctypes.c_int32(0)
    dummy = ctypes.c_void_p(16)
    assert L.fp4attn_clock_probe(None, 512, 10, ctypes.byref(khz), None) == 1  # FP4ATTN_ERR_NULL
    assert L.fp4attn_clock_probe(dummy, 512, 10, None, None) == 1
    for nb, it in ((0, 10), (4097, 10), (512, 0), (512, (1 << 24) + 1)):
        assert L.fp4attn_clock_probe(dummy, nb, it, ctypes.byref(khz), None) == 2, (nb, it)  # FP4ATTN_ERR_SHAPE
