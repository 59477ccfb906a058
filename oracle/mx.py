"""MX-fp8 fake quantisation (e4m3 payload, one power-of-two scale per 32 values).

TEST INFRASTRUCTURE ONLY (see the package docstring).

KohakUwULLM README, "Key features" (native MXFP8 training): element values in
fp8 e4m3, a UE8M0 (pure power-of-two) scale shared by each block of 32
elements, applied to the routed experts' matmuls.  The pages do not say how
the block scale is chosen; the reading taken here is the smallest power of two
X for which every |v| / X fits the e4m3 range (amax / X <= 448), clamped to the
UE8M0 range [2^-127, 2^127], with X = 2^-127 for an all-zero block.  Nothing
then saturates.  e4m3 follows the OCP 8-bit floating point definition: bias 7,
largest finite 448, no infinities, subnormals k * 2^-9, round to nearest even.
"""

import numpy as np

E4M3_MAX = 448.0
BLOCK = 32


def e4m3_round(v):
    """Round float64 values to the nearest e4m3 value (ties to even mantissa),
    saturating at +-448."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    # exponent of the binade: a = m * 2^ex, m in [0.5, 1)  ->  floor(log2 a) = ex - 1
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    ebin = np.maximum(ex - 1, -6)                  # below 2^-6 the spacing is fixed
    step = np.ldexp(1.0, ebin - 3)                 # 3 mantissa bits
    q = np.round(a / step) * step                  # numpy rounds halves to even
    q = np.minimum(q, E4M3_MAX)
    return np.where(a > 0, np.copysign(q, v), 0.0 * v)


def mx_block_scale(amax):
    """Smallest power of two X with amax / X <= 448, as an integer exponent in
    [-127, 127]; amax == 0 gives -127."""
    amax = np.asarray(amax, dtype=np.float64)
    out = np.full(amax.shape, -127, dtype=np.int64)
    nz = amax > 0
    if np.any(nz):
        _, ex = np.frexp(amax[nz] / E4M3_MAX)
        e = ex.astype(np.int64)               # 2^(ex-1) <= amax/448 < 2^ex (up to the division's rounding)
        # settle the exponent with exact comparisons against 448 * 2^e
        lo = e - 1
        ok_lo = amax[nz] <= np.ldexp(E4M3_MAX, lo)
        e = np.where(ok_lo, lo, e)
        ok_e = amax[nz] <= np.ldexp(E4M3_MAX, e)
        e = np.where(ok_e, e, e + 1)
        out[nz] = np.clip(e, -127, 127)
    return out


def mx_fake_quant(a, axis):
    """Quantise and dequantise ``a`` in blocks of 32 along ``axis`` (the
    contraction axis of the GEMM that consumes it).  A partial last block is
    padded with zeros (padding never changes amax)."""
    a = np.asarray(a, dtype=np.float64)
    a = np.moveaxis(a, axis, -1)
    n = a.shape[-1]
    nb = -(-n // BLOCK)
    pad = nb * BLOCK - n
    if pad:
        a = np.concatenate([a, np.zeros(a.shape[:-1] + (pad,))], axis=-1)
    blk = a.reshape(a.shape[:-1] + (nb, BLOCK))
    ex = mx_block_scale(np.abs(blk).max(axis=-1))
    scale = np.ldexp(1.0, ex)[..., None]
    deq = e4m3_round(blk / scale) * scale
    out = deq.reshape(a.shape)[..., :n]
    return np.moveaxis(out, -1, axis)
