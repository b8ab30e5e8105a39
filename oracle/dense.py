"""Brute-force per-token dense MoE (test infrastructure only).

A second, deliberately different formulation of the same layer, used to pin
oracle.moe on tiny inputs: no counting, no permutation, no grouped GEMM.  For
every token and every routed pick it runs the expert's two projections one
output element at a time as dot products over dequantised values, applies
SiLU(gate) * up and per-128-block re-quantisation element by element, and
accumulates the weighted rows in ascending k.  The rounding points are the
same as oracle.moe (bf16 for h, y and out; E4M3 round-to-nearest-even with
fp32 scales for q2), so the two must agree bit for bit.

Cost is O(T * K * (2I + H)) dot products; use only on tiny shapes.
"""

import math

import numpy as np

from .codec import e4m3_decode, e4m3_encode, bf16_round

_DECODE = e4m3_decode(np.arange(256, dtype=np.uint8))


def dequant_weight(codes, scales):
    """Dequantise one expert's [N, K] weight with its [N/128, K/128] scales,
    one 128x128 block at a time."""
    N, K = codes.shape
    out = np.empty((N, K))
    for nb in range(N // 128):
        for kb in range(K // 128):
            blk = codes[nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128]
            out[nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128] = \
                _DECODE[blk] * float(scales[nb, kb])
    return out


def _dequant_row(codes, scales):
    return np.array([_DECODE[int(c)] * float(scales[i // 128])
                     for i, c in enumerate(codes)])


def token_forward(x_codes, x_scale, picks, weights, w13d, w2d):
    """Dense MoE output row for one token.

    picks: local expert ids in k order (-1 = none); weights: matching top-k
    weights; w13d / w2d: per-expert dequantised weights from dequant_weight.
    Returns float64 [H] (bf16 values).
    """
    H = len(x_codes)
    I = w13d[0].shape[0] // 2
    xv = _dequant_row(x_codes, x_scale)
    acc = None
    for e, w in zip(picks, weights):
        if e < 0:
            continue
        h = np.array([bf16_round(float(np.dot(xv, w13d[e][n])))
                      for n in range(2 * I)])
        act = [float(h[j]) / (1.0 + math.exp(-float(h[j]))) * float(h[I + j])
               for j in range(I)]
        q = np.empty(I, dtype=np.uint8)
        qs = np.empty(I // 128, dtype=np.float32)
        for b in range(I // 128):
            # codes are decided in fp32: v, amax, s and v / s are fp32 values
            blk = [np.float32(v) for v in act[b * 128:(b + 1) * 128]]
            amax = max(abs(v) for v in blk)
            s = np.float32(amax / np.float32(448.0)) if amax != 0.0 else np.float32(1.0)
            qs[b] = s
            for i, v in enumerate(blk):
                q[b * 128 + i] = e4m3_encode(np.array([float(np.float32(v / s))]))[0]
        qv = _dequant_row(q, qs)
        y = np.array([bf16_round(float(np.dot(qv, w2d[e][n]))) for n in range(H)])
        term = float(w) * y
        acc = term if acc is None else acc + term
    if acc is None:
        return np.zeros(H)
    return bf16_round(acc)
