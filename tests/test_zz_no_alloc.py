"""fp4attn_bwd_noalloc (the backward without device allocation, its workspace in the library's
static scratch array) against fp4attn_bwd with a caller workspace, through the C ABI.

Both run the same kernels, which are deterministic, so the outputs must be identical bit for bit.
Two calls in a row, the second on smaller sizes (so it runs on the scratch the first call left
behind), and a call whose sizes need more than the scratch holds, which must be refused before
anything is enqueued."""
import ctypes

import numpy as np
import pytest

from precision_attention_amd.inputs import attention_inputs
from tests.gpuhelpers import require_gpu, to_dev

pytestmark = pytest.mark.gpu


def _operands(x, dev):
    import precision_attention_amd as pa

    q, k, v, do = (to_dev(x[n], dev) for n in ("q", "k", "v", "do"))
    return dict(q=pa.quantize_mx(q, pa.MXFP4, pa.ALONG_D), k=pa.quantize_mx(k, pa.MXFP4, pa.ALONG_D),
                q8=pa.quantize_mx(q, pa.MXFP8, pa.ALONG_SEQ), k8=pa.quantize_mx(k, pa.MXFP8, pa.ALONG_SEQ),
                v8=pa.quantize_mx(v, pa.MXFP8, pa.ALONG_D), do=do)


def _run_both(shape, seed, dev):
    import precision_attention_amd as pa
    import torch

    B, H, Hkv, N, D = shape
    x = attention_inputs(B, H, Hkv, N, D, seed=seed, with_do=True)
    ops = _operands(x, dev)
    o, lse = pa.fwd(ops["q"], ops["k"], pa.quantize_mx(to_dev(x["v"], dev), pa.MXFP8, pa.ALONG_SEQ), causal=True)
    ref = pa.bwd(ops["q"], ops["k"], ops["q8"], ops["k8"], ops["v8"], o, ops["do"], lse, causal=True)
    # the no-allocation entry point, called through the C ABI directly on preallocated outputs
    outs = [torch.full_like(t, float("nan")) for t in ref]
    L = pa.lib()
    structs = [ops[n].c_struct() for n in ("q", "k", "q8", "k8", "v8")]
    rc = L.fp4attn_bwd_noalloc(*[ctypes.byref(s) for s in structs], o.data_ptr(), ops["do"].data_ptr(),
                               lse.data_ptr(), outs[0].data_ptr(), outs[1].data_ptr(), outs[2].data_ptr(), B, H, Hkv,
                               N, D, 1, torch.cuda.current_stream(dev).cuda_stream)
    assert rc == 0, pa.lib().fp4attn_status_str(rc)
    torch.cuda.synchronize()
    return ref, outs


@pytest.mark.parametrize("first,second", [((1, 4, 2, 1024, 128), (1, 2, 1, 256, 64))], ids=["n1024_then_n256"])
def test_noalloc_matches_workspace_entry_point(first, second):
    dev = require_gpu()
    for i, shape in enumerate((first, second)):
        print("no-alloc backward call %d, shape %s" % (i + 1, shape), flush=True)
        ref, got = _run_both(shape, seed=40 + i, dev=dev)
        for name, r, g in zip(("dQ", "dK", "dV"), ref, got):
            import torch

            assert bool((r.view(torch.int16) == g.view(torch.int16)).all()), (shape, name)


def test_noalloc_refuses_sizes_beyond_the_scratch():
    import precision_attention_amd as pa

    require_gpu()
    L = pa.lib()
    B, H, Hkv, N, D = 1, 32, 8, 16384, 128  # needs about 136 MiB of workspace
    assert pa.bwd_workspace_bytes(B, H, Hkv, N, D) > pa.NOALLOC_SCRATCH_BYTES
    dummy = pa._MX(pa.MXFP4, pa.ALONG_D, 256, 256)
    rc = L.fp4attn_bwd_noalloc(*[ctypes.byref(dummy)] * 5, 256, 256, 256, 256, 256, 256, B, H, Hkv, N, D, 1, None)
    assert rc == 7, rc  # FP4ATTN_ERR_SCRATCH, before any pointer is used
    assert pa.bwd_workspace_bytes(1, 32, 8, 8192, 128) <= pa.NOALLOC_SCRATCH_BYTES
