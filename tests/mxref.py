"""An independent MXFP4 (E2M1) quantizer for the oracle's pins: per row, blocks of 32 along the
last axis, OCP scale floor(log2 amax) - 2, nearest-even E2M1 codes, saturating. Written apart from
the oracle's own quantizer so that the pins compare two implementations of the written rule."""
import numpy as np


def mx_e2m1_rows(P):
    """Per row, blocks of 32 along the last axis: OCP scale from the block max, nearest-even
    E2M1 codes; written independently of the oracle's quantizer."""
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    mids = 0.5 * (grid[1:] + grid[:-1])
    R, n = P.shape
    out = np.zeros_like(P)
    for b0 in range(0, n, 32):
        blk = P[:, b0:b0 + 32]
        amax = blk.max(axis=1, keepdims=True)
        e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2, -127)
        e = np.maximum(e, -127)
        y = blk / 2.0 ** e
        idx = np.searchsorted(mids, y, side="left")  # y <= mid goes down ...
        at_mid = np.isin(y, mids)
        up_even = at_mid & (idx % 2 == 1)  # ... except ties whose upper neighbour is even
        idx = np.where(up_even, idx + 1, idx)
        idx = np.minimum(idx, 7)
        out[:, b0:b0 + 32] = grid[idx] * 2.0 ** e
    return out
