"""GPU QKV projection with the MX quantization in its epilogue (fp4attn_project_qkv) against the
oracle's projection: binary64 products MX-quantized with no intermediate rounding.

- Grid inputs (X in multiples of 1/4 up to 2, W in multiples of 1/8 up to 1, Dm <= 4096): every
  fp32 partial sum is exact whatever the MFMA's summation order, so every code and scale must
  equal the oracle's bit for bit. The shapes cover D 64 and 128, token tails (N not a multiple of
  the kernel's 256-token tile), a feature count that is not a multiple of its 128-feature tile,
  heads of Q, K and V sharing one feature tile (D = 64), GQA, B = 2, one and several stages of
  the model dimension, V in MXFP4 and MXFP8, with and without the backward's FP8 views. Many
  values sit exactly on rounding midpoints, which checks the ties-to-even rule too. Each grid case
  runs with both workgroup tiles (256 x 128 and 256 x 256 features).
- Gaussian inputs, including the projection that feeds the headline attention (B1 N4096 Dm2048,
  H16 D128) and the 8B training shape (B1 N8192 Dm4096, H32 Hkv8, with the FP8 views), every
  code and scale compared: the fp32 sum and the binary64 sum may fall on the two sides of a
  rounding point. A difference is allowed only where the oracle's value lies within the fp32
  accumulation bound of that rounding point: (Dm/16 + 1) 2^-23 sum_k |x_k w_k| (one rounding per
  16-product MFMA step, each within 2^-23 of the partial sum, which is at most sum |x w|). A code
  may then differ only from a neighbouring code (or be +0 against -0, for a value within the
  bound of zero), and a block scale only by one with the block maximum within the bound of a power
  of two. The rate of such differences is printed and bounded by 1e-4 of the codes: with a bf16
  rounding point before the quantization the oracle's own codes would differ at 0.9 % (E2M1) and
  3.4 % (E4M3) of the elements of the headline projection.
- The two workgroup tiles against each other on Gaussian inputs: every code and scale byte equal
  (each fp32 sum takes the same MFMA steps in the same order), at ragged token and feature counts
  (F not a multiple of 256), D 64 and 128, B 2, and the 8B training shape, where the library's own
  choice is the wide tile.
"""
import numpy as np
import pytest

from precision_attention_amd.inputs import projection_inputs
from tests.gpuhelpers import require_gpu, to_dev
from tests.mxlayout import unpack_codes, unpack_scales

pytestmark = pytest.mark.gpu

RATE_MAX = 1e-4

# name -> (heads index into (q, k, v), format, axis); formats 1 = MXFP4, 2 = MXFP8
def _spec(v_fmt, views):
    s = {"q": (0, 1, 0), "k": (1, 1, 0), "v": (2, v_fmt, 1)}
    if views:
        s.update({"q8": (0, 2, 1), "k8": (1, 2, 1), "v8": (2, 2, 0)})
    return s


def run_gpu(x, B, N, Dm, H, Hkv, D, v_fmt, views, tile=0):
    import precision_attention_amd as pa
    import torch

    dev = require_gpu()
    out = pa.project_qkv(to_dev(x["x"], dev), to_dev(x["w"], dev), H, Hkv, D, v_fmt=v_fmt, fp8_views=views,
                         tile=tile)
    torch.cuda.synchronize()
    res = {}
    for name, (hi, fmt, axis) in _spec(v_fmt, views).items():
        shape = (B, (H, Hkv, Hkv)[hi], N, D)
        res[name] = (unpack_codes(out[name].codes.cpu().numpy(), fmt, axis, shape),
                     unpack_scales(out[name].scales.cpu().numpy(), axis, shape))
    return res


def _decode_table(orc, fmt):
    n = 16 if fmt == 1 else 256
    dec = orc.e2m1_decode if fmt == 1 else orc.e4m3_decode
    return np.array([dec(c) for c in range(n)], np.float64)


def compare_near_ties(orc, name, gpu, ref, vals, bound, fmt, axis):
    """Differences allowed only where the binary64 value lies within `bound` (per element, same
    units) of a rounding point; returns the count of differing codes."""
    gc, gs = gpu
    oc, os_ = ref
    # blocks along the last axis for axis "d"; along N for "seq": move the blocked axis last
    if axis == 1:
        gc, oc, vals, bound = (np.swapaxes(a, -1, -2) for a in (gc, oc, vals, bound))
        gs, os_ = (np.swapaxes(a, -1, -2) for a in (gs, os_))
    shp = vals.shape[:-1] + (vals.shape[-1] // 32, 32)
    v, bnd = vals.reshape(shp), bound.reshape(shp)
    gcb, ocb = gc.reshape(shp), oc.reshape(shp)
    sdiff = gs != os_
    if sdiff.any():
        d = np.abs(gs.astype(int) - os_.astype(int))[sdiff]
        vb, bb = np.abs(v[sdiff]), bnd[sdiff]
        i = np.argmax(vb, axis=-1)
        a = np.take_along_axis(vb, i[:, None], -1)[:, 0]
        ab = np.take_along_axis(bb, i[:, None], -1)[:, 0]
        near = np.abs(a - 2.0 ** np.round(np.log2(a))) <= ab
        assert np.all(d == 1) and np.all(near), "%s: scales differ away from a power of two" % name
    e = os_.astype(np.float64) - 127.0
    same = ~sdiff[..., None] & (gcb != ocb)
    n_bad = int(same.sum()) + 32 * int(sdiff.sum())
    if same.any():
        tab = _decode_table(orc, fmt)
        sc = 2.0 ** e[..., None]
        y, yb = (v / sc)[same], (bnd / sc)[same]
        g, o = gcb[same].astype(int), ocb[same].astype(int)
        sign = 8 if fmt == 1 else 128
        gm, om = g & (sign - 1), o & (sign - 1)
        # +0 against -0: a value within rounding of zero, whose sign the two sums disagree on
        zeros = (gm == 0) & (om == 0)
        assert np.all(np.abs(y[zeros]) <= yb[zeros]), "%s: the sign of a zero differs away from 0" % name
        step = ~zeros
        assert np.all((g[step] & sign) == (o[step] & sign)), "%s: a code differs in sign" % name
        assert np.all(np.abs(gm[step] - om[step]) == 1), "%s: codes differ by more than a step" % name
        mid = 0.5 * (tab[g[step]] + tab[o[step]])
        dist = np.abs(y[step] - mid)
        assert np.all(dist <= yb[step]), (
            "%s: a code differs away from a rounding point: %s > %s" % (name, dist.max(), yb[step][np.argmax(dist)]))
    return n_bad


GRID = [
    # (B, N, Dm, H, Hkv, D, v_fmt, views)
    (1, 256, 256, 2, 2, 128, 1, False),
    (2, 352, 128, 4, 2, 64, 2, True),
    (1, 96, 64, 1, 1, 64, 1, True),
    (1, 544, 192, 2, 1, 128, 2, True),
    (1, 1024, 512, 4, 4, 128, 1, False),
    (1, 288, 4096, 2, 1, 64, 1, True),
    (1, 800, 320, 3, 1, 128, 2, True),
]


@pytest.mark.parametrize("case", GRID, ids=["b%d_n%d_dm%d_h%d_kv%d_d%d_v%d_%s" % (c[:7] + ("views" if c[7] else "noviews",))
                                            for c in GRID])
def test_project_grid_bit_exact(orc, case):
    B, N, Dm, H, Hkv, D, v_fmt, views = case
    print("projection grid case", case, flush=True)
    x = projection_inputs(B, N, Dm, H, Hkv, D, seed=sum(case), grid=True)
    ref, _ = orc.project_qkv_views(x["x"], x["w"], H, Hkv, D, v_fmt=orc.FMT_E2M1 if v_fmt == 1 else orc.FMT_E4M3,
                                   fp8_views=views)
    for tile in (128, 256):
        print("  tile", tile, flush=True)
        gpu = run_gpu(x, B, N, Dm, H, Hkv, D, v_fmt, views, tile)
        for name in gpu:
            gc, gs = gpu[name]
            oc, os_ = ref[name]
            assert np.array_equal(gs, os_), "tile %d: %s scales differ at %s" % (tile, name, np.argwhere(gs != os_)[:5])
            bad = np.argwhere(gc != oc)
            assert bad.size == 0, "tile %d: %s codes differ at %s" % (tile, name, bad[:5])


GAUSS = [
    ("small_h2kv1_n544_dm256_d64", 1, 544, 256, 2, 1, 64, 1, True),
    ("directp_h16_n4096_dm2048_d128", 1, 4096, 2048, 16, 16, 128, 1, False),
    ("llama8b_h32kv8_n8192_dm4096_d128", 1, 8192, 4096, 32, 8, 128, 2, True),
]


@pytest.mark.parametrize("case", GAUSS, ids=[c[0] for c in GAUSS])
def test_project_gaussian_near_ties_only(orc, case):
    name, B, N, Dm, H, Hkv, D, v_fmt, views = case
    print("projection case", name, flush=True)
    x = projection_inputs(B, N, Dm, H, Hkv, D, seed=1)
    gpu = run_gpu(x, B, N, Dm, H, Hkv, D, v_fmt, views)
    ofmt = {1: orc.FMT_E2M1, 2: orc.FMT_E4M3}
    ref, qkv = orc.project_qkv_views(x["x"], x["w"], H, Hkv, D, v_fmt=ofmt[v_fmt], fp8_views=views)
    # the fp32 accumulation bound per element, in the layout of q, k, v
    ax = np.abs(orc.bf16_to_f64(x["x"]))
    aw = np.abs(orc.bf16_to_f64(x["w"]))
    sabs = np.matmul(ax, aw.T).reshape(B, N, H + 2 * Hkv, D).transpose(0, 2, 1, 3)
    bound = (Dm / 16 + 1) * 2.0 ** -23 * sabs
    bounds = (bound[:, :H], bound[:, H:H + Hkv], bound[:, H + Hkv:])
    total = bad = 0
    for vname, (hi, fmt, axis) in _spec(v_fmt, views).items():
        n = compare_near_ties(orc, vname, gpu[vname], ref[vname], qkv[hi], bounds[hi], fmt, axis)
        print("  %s: %d of %d codes differ at rounding points" % (vname, n, qkv[hi].size), flush=True)
        total += qkv[hi].size
        bad += n
    print("projection %s: rate %.3g (bound %g)" % (name, bad / total, RATE_MAX), flush=True)
    assert bad / total <= RATE_MAX


TILES = [
    # (B, N, Dm, H, Hkv, D, v_fmt, views)
    (1, 800, 320, 3, 1, 128, 2, True),      # 640 features: two and a half wide tiles
    (2, 1056, 1024, 5, 1, 64, 1, True),     # 448 features, D 64, B 2
    (1, 4128, 2048, 16, 16, 128, 1, False),
    (1, 8192, 4096, 32, 8, 128, 2, True),   # the 8B training shape
]


@pytest.mark.parametrize("case", TILES, ids=["b%d_n%d_dm%d_h%d_kv%d_d%d" % c[:6] for c in TILES])
def test_project_tiles_bit_identical(case):
    import precision_attention_amd as pa
    import torch

    dev = require_gpu()
    B, N, Dm, H, Hkv, D, v_fmt, views = case
    print("projection tiles case", case, flush=True)
    x = projection_inputs(B, N, Dm, H, Hkv, D, seed=7)
    xd, wd = to_dev(x["x"], dev), to_dev(x["w"], dev)
    outs = {}
    for tile in (128, 256, 0):
        o = pa.project_qkv(xd, wd, H, Hkv, D, v_fmt=v_fmt, fp8_views=views, tile=tile)
        torch.cuda.synchronize()
        outs[tile] = {n: (t.codes.cpu().numpy(), t.scales.cpu().numpy()) for n, t in o.items()}
    for tile in (256, 0):
        for n, (c, sc) in outs[128].items():
            c2, s2 = outs[tile][n]
            assert np.array_equal(s2, sc), "tile %d: %s scales differ at %s" % (tile, n, np.argwhere(s2 != sc)[:5])
            assert np.array_equal(c2, c), "tile %d: %s codes differ at %s" % (tile, n, np.argwhere(c2 != c)[:5])
