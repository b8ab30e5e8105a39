"""Test inputs: seeded draws (workloads.gen) quantised by the CPU oracle.

Every FP8 code and scale the GPU tests feed to the library comes from here,
so inputs flow oracle -> device, never the other way.  Results are cached per
process because the large configurations take tens of seconds to draw and
quantise.
"""

import functools
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from oracle import moe, e8m0
from workloads import CONFIGS, routing, activations, weights, bf16_to_f32

_THREADS = min(16, os.cpu_count() or 1)


def _quant_expert(cfg, e):
    w13b, w2b = weights(cfg, experts=[e])
    q13, s13 = moe.quantize_blocks(bf16_to_f32(w13b[0]), 128)
    q2, s2 = moe.quantize_blocks(bf16_to_f32(w2b[0]), 128)
    return q13, s13, q2, s2


@functools.lru_cache(maxsize=6)
def layer_inputs(cid, experts_needed_only=False):
    """Routing, quantised activations and weights of configuration `cid`.

    experts_needed_only: leave the weights of experts that receive no row as
    zero codes with unit scales (they are never read); used for the masked
    configuration, where a quarter of the experts is empty.
    """
    cfg = CONFIGS[cid]
    idx, w = routing(cfg)
    xb = activations(cfg)
    # quantise x in row chunks (bounded memory)
    x = np.empty((cfg.T, cfg.H), np.uint8)
    xs = np.empty((cfg.T, cfg.H // 128), np.float32)
    step = 4096

    def qx(r0):
        x[r0:r0 + step], xs[r0:r0 + step] = moe.quantize_blocks(
            bf16_to_f32(xb[r0:r0 + step]), 1)
    with ThreadPoolExecutor(_THREADS) as ex:
        list(ex.map(qx, range(0, cfg.T, step)))
    E, I, H = cfg.E, cfg.I, cfg.H
    w13 = np.zeros((E, 2 * I, H), np.uint8)
    s13 = np.ones((E, 2 * I // 128, H // 128), np.float32)
    w2 = np.zeros((E, H, I), np.uint8)
    s2 = np.ones((E, H // 128, I // 128), np.float32)
    used = np.unique(idx[idx >= 0])
    experts = used if experts_needed_only else range(E)

    def qe(e):
        w13[e], s13[e], w2[e], s2[e] = _quant_expert(cfg, e)
    with ThreadPoolExecutor(_THREADS) as ex:
        list(ex.map(qe, experts))
    return dict(cfg=cfg, idx=idx, w=w, x=x, xs=xs, w13=w13, s13=s13, w2=w2, s2=s2)


def rows_for(cfg, idx):
    """Buffer rows: M_cap = R + E*(align_m - 1) (contiguous) or C (masked)."""
    if cfg.layout == moe.LAYOUT_MASKED:
        return cfg.capacity
    R = int((idx >= 0).sum())
    return R + cfg.E * (cfg.align_m - 1)


def _quant_expert_e8m0(cfg, e):
    w13b, w2b = weights(cfg, experts=[e])
    q13, e13 = e8m0.quantize_blocks(bf16_to_f32(w13b[0]), 128)
    q2, e2 = e8m0.quantize_blocks(bf16_to_f32(w2b[0]), 128)
    return q13, e13, q2, e2


def as_words(p):
    """uint32 packed words as the int32 array the device tensors hold."""
    return np.ascontiguousarray(np.asarray(p, np.uint32).view(np.int32))


@functools.lru_cache(maxsize=6)
def layer_inputs_e8m0(cid, experts_needed_only=False):
    """layer_inputs with power-of-two scales (oracle.e8m0): for x, W13 and W2
    the codes, the exponents, the packed int32 words the device takes
    (xp [T, ceil(H/512)], p13 [E, 2I/128, ceil(H/512)], p2 [E, H/128,
    ceil(I/512)]) and the fp32 scale values 2^e the oracle takes."""
    cfg = CONFIGS[cid]
    idx, w = routing(cfg)
    xb = activations(cfg)
    x = np.empty((cfg.T, cfg.H), np.uint8)
    xe = np.empty((cfg.T, cfg.H // 128), np.int32)
    step = 4096

    def qx(r0):
        x[r0:r0 + step], xe[r0:r0 + step] = e8m0.quantize_blocks(
            bf16_to_f32(xb[r0:r0 + step]), 1)
    with ThreadPoolExecutor(_THREADS) as ex:
        list(ex.map(qx, range(0, cfg.T, step)))
    E, I, H = cfg.E, cfg.I, cfg.H
    w13 = np.zeros((E, 2 * I, H), np.uint8)
    e13 = np.zeros((E, 2 * I // 128, H // 128), np.int32)
    w2 = np.zeros((E, H, I), np.uint8)
    e2 = np.zeros((E, H // 128, I // 128), np.int32)
    used = np.unique(idx[idx >= 0])
    experts = used if experts_needed_only else range(E)

    def qe(e):
        w13[e], e13[e], w2[e], e2[e] = _quant_expert_e8m0(cfg, e)
    with ThreadPoolExecutor(_THREADS) as ex:
        list(ex.map(qe, experts))
    return dict(cfg=cfg, idx=idx, w=w, x=x, xe=xe, xs=e8m0.scales(xe), xp=as_words(e8m0.pack(xe)),
                w13=w13, e13=e13, s13=e8m0.scales(e13), p13=as_words(e8m0.pack(e13)),
                w2=w2, e2=e2, s2=e8m0.scales(e2), p2=as_words(e8m0.pack(e2)))
