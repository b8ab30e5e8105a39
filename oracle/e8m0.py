"""Power-of-two ("packed") block scales -- test infrastructure only.

The GB200 page ("Deploying DeepSeek on GB200 NVL72 with PD and Large Scale
EP (Part I)", section 方法实现细节 / method details) says the FP8 GEMM
library's new API quantises and packs the input scales, without defining
either.  This module is the reading used for that variant of the layer; the
rest of the layer (layout, GEMM definition, SiLU, combine) is oracle.moe
unchanged, fed with the scales below.

Readings (listed again in the design notes):
  R18 a block's scale is the smallest power of two not below
      fp32(amax / 448): s = 2^e, e = ceil(log2(fp32(amax / 448))); e = 0
      when amax == 0; e is kept in the E8M0 range [-127, 127] (a quotient
      that underflows to zero for amax > 0 takes the smallest, -127).
  R19 codes are E4M3_RNE(v / s) with v = fp32(value).  Dividing by a power
      of two is exact and |v / s| <= 448, so no saturation occurs.
  R20 packing: a scale is stored as its biased exponent byte e + 127
      (E8M0), four consecutive 128-wide blocks along K per 32-bit word,
      little-endian (byte j of word w belongs to block 4w + j); the bytes
      past the last block of a row are 127 (scale 1).
"""

import numpy as np

from .codec import e4m3_encode, E4M3_MAX
from .moe import BLOCK, silu_mul

E8M0_BIAS = 127


def scale_exponents(amax):
    """R18: e = ceil(log2(fp32(amax / 448))), 0 for amax == 0, clipped to
    [-127, 127] (-127 when the quotient underflows to zero).  With fp32(amax / 448) = m * 2^x, m in [0.5, 1) (frexp),
    the ceiling is x - 1 when m == 0.5 (an exact power of two) and x
    otherwise."""
    amax = np.asarray(amax, dtype=np.float32)
    sf = (amax / np.float32(E4M3_MAX)).astype(np.float32).astype(np.float64)
    m, x = np.frexp(sf)
    e = np.where(m == 0.5, x - 1, x)
    e = np.where(sf == 0, -E8M0_BIAS, e)     # quotient underflowed: smallest scale
    e = np.where(amax == 0, 0, e)
    return np.clip(e, -E8M0_BIAS, E8M0_BIAS).astype(np.int32)


def quantize_blocks(values, block_rows):
    """R18-R19 on a 2-D array in blocks of block_rows x 128.  Returns
    (codes uint8 [R, C], exponents int32 [R / block_rows, C / 128])."""
    v = np.asarray(values).astype(np.float32)
    R, C = v.shape
    assert R % block_rows == 0 and C % BLOCK == 0
    blk = v.reshape(R // block_rows, block_rows, C // BLOCK, BLOCK)
    e = scale_exponents(np.abs(blk).max(axis=(1, 3)))
    quot = np.ldexp(blk.astype(np.float64), -e[:, None, :, None])
    return e4m3_encode(quot).reshape(R, C), e


def scales(e):
    """fp32 scale values 2^e (exact for every E8M0 exponent)."""
    return np.ldexp(np.float32(1.0), np.asarray(e)).astype(np.float32)


def pack(e):
    """R20: exponents [..., nb] -> uint32 words [..., ceil(nb / 4)]."""
    e = np.asarray(e, dtype=np.int64)
    nb = e.shape[-1]
    nw = (nb + 3) // 4
    b = np.full(e.shape[:-1] + (nw * 4,), E8M0_BIAS, dtype=np.int64)
    b[..., :nb] = e + E8M0_BIAS
    b = b.reshape(e.shape[:-1] + (nw, 4))
    return (b[..., 0] | (b[..., 1] << 8) | (b[..., 2] << 16) | (b[..., 3] << 24)).astype(np.uint32)


def unpack(words, nb):
    """Inverse of pack: words [..., nw] -> exponents int32 [..., nb]."""
    w = np.asarray(words, dtype=np.uint32).astype(np.int64)
    b = np.stack([(w >> (8 * j)) & 0xFF for j in range(4)], axis=-1)
    b = b.reshape(w.shape[:-1] + (w.shape[-1] * 4,))[..., :nb]
    return (b - E8M0_BIAS).astype(np.int32)


def act_requant(h):
    """S6 with R18-R19: SiLU(gate) * up re-quantised in 1x128 blocks.
    Returns (codes [M, I], fp32 scales 2^e [M, I/128]) for oracle.moe.layer."""
    q, e = quantize_blocks(silu_mul(h), 1)
    return q, scales(e)
