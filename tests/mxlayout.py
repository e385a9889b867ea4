"""Test helper: convert the library's physical MX layouts (include/fp4attn.h) to the
oracle's logical layout (one code per element, [B, heads, N, D]; scales [..., N, D/32] along
D or [..., N/32, D] along the sequence). Pure data movement, no arithmetic of the method."""
import numpy as np


def unpack_codes(raw: np.ndarray, fmt: int, axis: int, shape):
    B, H, N, D = shape
    raw = np.asarray(raw, np.uint8)
    if fmt == 1:  # two E2M1 codes per byte, lower index in the low nibble
        lo, hi = raw & 0x0F, raw >> 4
        flat = np.stack([lo, hi], axis=-1).reshape(-1)
    else:
        flat = raw.reshape(-1)
    if axis == 0:
        return flat.reshape(B, H, N, D)
    return np.ascontiguousarray(np.swapaxes(flat.reshape(B, H, D, N), -1, -2))


def unpack_scales(raw: np.ndarray, axis: int, shape):
    B, H, N, D = shape
    raw = np.asarray(raw, np.uint8)
    if axis == 0:
        return raw.reshape(B, H, N, D // 32)
    return np.ascontiguousarray(np.swapaxes(raw.reshape(B, H, D, N // 32), -1, -2))
