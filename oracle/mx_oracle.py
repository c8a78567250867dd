"""CPU oracle for the MXFP8 encoding (E4M3 elements, E8M0 block scales).

TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the CPU
baseline of the bench, never by the product path.  Shares no code with the HIP
library.

Source.  The Olmo-core 3 announcement ("Scaling and optimizing MoE training")
offers MXFP8 as a lower-precision format that pays when the savings exceed the
cost of converting between formats; it gives no detail of the format.  The
plain reading is the public OCP Microscaling Formats (MX) v1.0 specification,
FP8 E4M3 element type:

* a block is 32 consecutive elements along the quantisation axis (the GEMM's
  contraction axis); with segment offsets, blocks restart at each segment and
  the last block of a segment is zero-padded;
* the block scale is 2**e with e = floor(log2(max|v|)) - 8 (8 is the largest
  E4M3 exponent), clamped to [-127, 127]; an all-zero block gets e = -127; the
  scale is stored as the E8M0 byte e + 127;
* each element is v / 2**e rounded to the nearest E4M3 value, ties to the
  even code, magnitudes above 448 saturated to 448, sign kept (also on zero).

E4M3 (OCP): sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent
field 0 holds subnormals m * 2**-9; 0x7F and 0xFF are NaN; largest finite
value 448 = 2**8 * 1.75.

Pins: ``tests/test_oracle_pins.py`` checks the encoder against brute-force
nearest-even search, an exhaustive round trip over every finite code, values
derived by hand from the format definition and the scale invariant
256 * 2**e <= amax < 512 * 2**e.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
MX_BLOCK = 32
E4M3_EMAX = 8


def e4m3_decode(codes):
    """E4M3 byte -> value (fp64); NaN for 0x7F / 0xFF."""
    c = np.asarray(codes, np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    mf = c & 0x7
    sub = mf * 2.0 ** -9
    nor = np.ldexp(1.0 + mf / 8.0, ef - 7)
    val = sign * np.where(ef == 0, sub, nor)
    return np.where((ef == 15) & (mf == 7), np.nan, val)


_GRID = None


def _grid():
    """The 127 non-negative finite E4M3 values, ascending (codes 0x00..0x7E)."""
    global _GRID
    if _GRID is None:
        _GRID = e4m3_decode(np.arange(0x7F))
    return _GRID


def e4m3_encode(y):
    """Value (fp64, finite) -> E4M3 byte: round to nearest, ties to even, saturating."""
    y = np.asarray(y, np.float64)
    a = np.abs(y)
    _, ex = np.frexp(a)
    # Grid spacing: 2**(floor(log2 a) - 3) in the normal range, 2**-9 below 2**-6.
    quantum = np.ldexp(1.0, np.maximum(ex - 1, -6) - 3)
    r = np.minimum(np.round(a / quantum) * quantum, E4M3_MAX)  # np.round rounds half to even
    # r lies exactly on the E4M3 grid; its code is its index among the ascending values
    code = np.searchsorted(_grid(), r)
    code = np.where(np.signbit(y), code | 0x80, code)
    return code.astype(np.uint8)


def mx_block_exponent(amax):
    """Shared exponent e of a block from its max magnitude (int64 array)."""
    amax = np.asarray(amax, np.float64)
    _, ex = np.frexp(amax)
    e = (ex - 1) - E4M3_EMAX
    e = np.where(amax == 0.0, -127, e)
    return np.clip(e, -127, 127).astype(np.int64)


def _quantize_blocks(blocks):
    """blocks [nblk, 32] fp64 -> (codes uint8 [nblk, 32], scale bytes uint8 [nblk])."""
    amax = np.abs(blocks).max(axis=1)
    e = mx_block_exponent(amax)
    scaled = blocks / np.ldexp(1.0, e)[:, None]
    return e4m3_encode(scaled), (e + 127).astype(np.uint8)


def mx_quantize(v, axis=1, seg_offsets=None):
    """MX-quantise a 2-D array along ``axis`` (1: along columns, 0: along rows).

    Without segments the length along ``axis`` must be a multiple of 32.  With
    ``seg_offsets`` (axis 0 only: prefix offsets of row segments, length
    nseg+1) blocks restart at each segment and a segment's last block is
    zero-padded.

    Returns (q, scales):
      q       uint8 E4M3 codes, same shape as v (padding is not stored);
      scales  uint8 E8M0 bytes: [rows, cols/32] for axis 1,
              [num_row_blocks, cols] for axis 0 (blocks in segment order).
    """
    v = np.asarray(v, np.float64)
    rows, cols = v.shape
    if axis == 1:
        if seg_offsets is not None or cols % MX_BLOCK:
            raise ValueError("axis 1 needs cols % 32 == 0 and no segments")
        codes, sc = _quantize_blocks(v.reshape(rows * cols // MX_BLOCK, MX_BLOCK))
        return codes.reshape(rows, cols), sc.reshape(rows, cols // MX_BLOCK)
    if axis != 0:
        raise ValueError("axis must be 0 or 1")
    if seg_offsets is None:
        if rows % MX_BLOCK:
            raise ValueError("axis 0 without segments needs rows % 32 == 0")
        seg_offsets = [0, rows]
    seg = [int(s) for s in seg_offsets]
    q = np.zeros((rows, cols), np.uint8)
    scale_rows = []
    for s in range(len(seg) - 1):
        lo, hi = seg[s], seg[s + 1]
        n = hi - lo
        if n == 0:
            continue
        nb = (n + MX_BLOCK - 1) // MX_BLOCK
        padded = np.zeros((nb * MX_BLOCK, cols))
        padded[:n] = v[lo:hi]
        # blocks run down the rows: [nb, 32, cols] -> [nb*cols, 32]
        blk = padded.reshape(nb, MX_BLOCK, cols).transpose(0, 2, 1).reshape(nb * cols, MX_BLOCK)
        codes, sc = _quantize_blocks(blk)
        codes = codes.reshape(nb, cols, MX_BLOCK).transpose(0, 2, 1).reshape(nb * MX_BLOCK, cols)
        q[lo:hi] = codes[:n]
        scale_rows.append(sc.reshape(nb, cols))
    scales = np.concatenate(scale_rows, axis=0) if scale_rows else np.zeros((0, cols), np.uint8)
    return q, scales


def mx_dequantize(q, scales, axis=1, seg_offsets=None):
    """Inverse map for checking: value = 2**(scale-127) * E4M3(q), same layout as mx_quantize."""
    q = np.asarray(q)
    rows, cols = q.shape
    vals = e4m3_decode(q)
    sc = np.asarray(scales, np.int64)
    if axis == 1:
        f = np.ldexp(1.0, np.repeat(sc, MX_BLOCK, axis=1) - 127)
        return vals * f
    if seg_offsets is None:
        seg_offsets = [0, rows]
    out = np.zeros((rows, cols))
    b = 0
    for s in range(len(seg_offsets) - 1):
        lo, hi = int(seg_offsets[s]), int(seg_offsets[s + 1])
        for r0 in range(lo, hi, MX_BLOCK):
            r1 = min(r0 + MX_BLOCK, hi)
            out[r0:r1] = vals[r0:r1] * np.ldexp(1.0, sc[b] - 127)[None, :]
            b += 1
    return out
