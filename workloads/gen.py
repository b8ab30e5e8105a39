"""Seeded synthetic workloads for the routed-expert MoE layer.

This module only draws random numbers: routing (which local experts each
received token goes to, and its top-k weights) and raw bf16 activations and
weights.  It holds none of the layer's arithmetic; quantising the raw values
to E4M3 with block scales is done by whoever consumes them (the CPU oracle in
tests, the library's own quantiser in the benchmark).

The shapes stand in for the per-GPU shares of the deployments on the pages:
DeepSeek's 256 routed experts plus 32 redundant ones make a 288-expert pool
(H100-EP page, section EPLB); decode ran EP72 at 2K context and prefill EP32
at 4K context (H100-EP page, section 效果如何 / results); the GB200 decode
deployment used 12 decode nodes (GB200 page, section 实验环境 / setup), here
read as EP48.  H = 7168 and I = 2048 are DeepSeek-V3's hidden and routed-expert
intermediate sizes; top-k = 8 (DeepSeek-V3's routed top-8) is a reading: the
pages never state it.  No dataset, trace or trained weight is used: the
pages' real routing statistics are not available, so uniform, Zipf and
jittered per-expert loads stand in for them.

All randomness comes from numpy.random.default_rng([0, config_id, stream]).
"""

from dataclasses import dataclass

import numpy as np
import torch

LAYOUT_CONTIGUOUS = 0
LAYOUT_MASKED = 1

STREAM_COUNTS, STREAM_ROWS, STREAM_ASSIGN, STREAM_COLS, STREAM_W, STREAM_X, \
    STREAM_W13, STREAM_W2, STREAM_PICK = range(9)


@dataclass(frozen=True)
class Config:
    cid: int
    name: str
    E: int          # local experts
    H: int          # hidden size
    I: int          # expert intermediate size
    T: int          # source tokens
    K: int          # top-k columns
    layout: int
    capacity: int = 0      # masked layout: rows per expert
    align_m: int = 128     # contiguous layout: segment alignment


CONFIGS = {
    1: Config(1, "tiny", E=4, H=256, I=128, T=64, K=2, layout=LAYOUT_CONTIGUOUS),
    2: Config(2, "ep72_decode", E=4, H=7168, I=2048, T=1536, K=8,
              layout=LAYOUT_CONTIGUOUS),
    3: Config(3, "ep48_decode_zipf", E=6, H=7168, I=2048, T=4096, K=8,
              layout=LAYOUT_CONTIGUOUS),
    4: Config(4, "ep32_prefill_4k", E=9, H=7168, I=2048, T=65536, K=8,
              layout=LAYOUT_CONTIGUOUS),
    5: Config(5, "masked_decode", E=32, H=7168, I=2048, T=1024, K=8,
              layout=LAYOUT_MASKED, capacity=128),
}


def rng(cid, stream):
    return np.random.default_rng([0, cid, stream])


def largest_remainder(target_total, weights):
    """Integer counts proportional to `weights` that sum to target_total."""
    w = np.asarray(weights, dtype=np.float64)
    raw = w / w.sum() * target_total
    base = np.floor(raw).astype(np.int64)
    rem = target_total - int(base.sum())
    order = np.argsort(-(raw - base), kind="stable")
    base[order[:rem]] += 1
    return base


def expert_counts(cfg, zipf_s=1.0):
    """Per-expert routed-row counts for configs 2-5."""
    g = rng(cfg.cid, STREAM_COUNTS)
    if cfg.cid == 2:    # 2048 rows, uniform assignment
        return g.multinomial(2048, np.full(cfg.E, 1.0 / cfg.E)).astype(np.int64)
    if cfg.cid == 3:    # 6144 rows, Zipf(s) load over experts
        return largest_remainder(6144, 1.0 / np.arange(1, cfg.E + 1) ** zipf_s)
    if cfg.cid == 4:    # 14560 +- 20% per expert, total 131040
        c = 14560.0 * (1.0 + g.uniform(-0.2, 0.2, cfg.E))
        return largest_remainder(131040, c)
    if cfg.cid == 5:    # 25% empty, one full (C rows), the rest U{1..96}
        perm = g.permutation(cfg.E)
        n_empty = cfg.E // 4
        counts = np.zeros(cfg.E, dtype=np.int64)
        counts[perm[n_empty]] = cfg.capacity
        rest = perm[n_empty + 1:]
        counts[rest] = g.integers(1, 97, size=len(rest))
        return counts
    raise ValueError(cfg.cid)


def _assign(cfg, counts):
    """Turn per-expert counts into distinct (token, expert) pairs.

    Every token gets one row; the remaining rows go to random tokens, each
    token holding at most min(K, E) rows.  The expert multiset is shuffled
    onto the token rows and duplicate (token, expert) pairs are repaired by
    swapping with another row.
    """
    T, E, K = cfg.T, cfg.E, cfg.K
    R = int(counts.sum())
    cap = min(K, E)
    assert T <= R <= T * cap
    g = rng(cfg.cid, STREAM_ROWS)
    per_tok = np.ones(T, dtype=np.int64)
    extra = R - T
    while extra > 0:
        cand = g.integers(0, T, size=extra)
        for t in cand:
            if extra == 0:
                break
            if per_tok[t] < cap:
                per_tok[t] += 1
                extra -= 1
    tok_of_row = np.repeat(np.arange(T), per_tok)
    g2 = rng(cfg.cid, STREAM_ASSIGN)
    ex = g2.permutation(np.repeat(np.arange(E), counts))
    # repair duplicates: rows of one token are contiguous in tok_of_row
    starts = np.concatenate([[0], np.cumsum(per_tok)])
    for it in range(100):
        bad = []
        for t in range(T):
            s, e = starts[t], starts[t + 1]
            if e - s > 1:
                seen = set()
                for r in range(s, e):
                    if ex[r] in seen:
                        bad.append(r)
                    seen.add(ex[r])
        if not bad:
            break
        for r in bad:
            t = tok_of_row[r]
            mine = set(ex[starts[t]:starts[t + 1]])
            for _ in range(1000):
                o = int(g2.integers(0, R))
                to = tok_of_row[o]
                theirs = set(ex[starts[to]:starts[to + 1]])
                if ex[o] not in mine and ex[r] not in theirs and to != t:
                    ex[r], ex[o] = ex[o], ex[r]
                    break
    else:
        raise RuntimeError("could not repair duplicate token-expert pairs")
    return tok_of_row, ex, per_tok


def routing(cfg, zipf_s=1.0):
    """topk_idx [T, K] int32 (local expert id or -1) and topk_w [T, K] fp32."""
    T, E, K = cfg.T, cfg.E, cfg.K
    if cfg.cid == 1:
        # each token picks 2 distinct experts uniformly; weights are the
        # softmax of N(0,1) logits over its two picks
        g = rng(cfg.cid, STREAM_PICK)
        idx = np.stack([g.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
        logits = rng(cfg.cid, STREAM_W).standard_normal((T, K))
        w = np.exp(logits - logits.max(axis=1, keepdims=True))
        w = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
        return idx, w
    counts = expert_counts(cfg, zipf_s)
    tok_of_row, ex, per_tok = _assign(cfg, counts)
    idx = np.full((T, K), -1, dtype=np.int32)
    gc = rng(cfg.cid, STREAM_COLS)
    starts = np.concatenate([[0], np.cumsum(per_tok)])
    for t in range(T):
        cols = gc.permutation(K)[:per_tok[t]]
        idx[t, cols] = ex[starts[t]:starts[t + 1]]
    # weights U(0,1) over the local picks, normalised per token
    u = rng(cfg.cid, STREAM_W).uniform(0.0, 1.0, (T, K))
    u = np.where(idx >= 0, u, 0.0)
    w = (u / u.sum(axis=1, keepdims=True)).astype(np.float32)
    return idx, w


def _bf16(a):
    """float array -> bf16 bit patterns (uint16) via torch's RNE cast."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def activations(cfg, first_rows=None):
    """x ~ N(0, 1) as bf16 bits [T, H] (or only its first `first_rows` rows,
    which are the same values: the stream is drawn row by row)."""
    g = rng(cfg.cid, STREAM_X)
    n = cfg.T if first_rows is None else min(int(first_rows), cfg.T)
    return _bf16(g.standard_normal((n, cfg.H), dtype=np.float32))


def weights(cfg, experts=None):
    """W13 [E, 2I, H] and W2 [E, H, I] ~ N(0, 0.02) as bf16 bits.

    `experts` restricts the draw to a subset (still the same values those
    experts get in the full draw: each expert has its own sub-stream)."""
    E = cfg.E
    experts = range(E) if experts is None else experts
    w13 = np.empty((len(experts), 2 * cfg.I, cfg.H), dtype=np.uint16)
    w2 = np.empty((len(experts), cfg.H, cfg.I), dtype=np.uint16)
    for i, e in enumerate(experts):
        g13 = np.random.default_rng([0, cfg.cid, STREAM_W13, e])
        w13[i] = _bf16(g13.standard_normal((2 * cfg.I, cfg.H), dtype=np.float32) * 0.02)
        g2 = np.random.default_rng([0, cfg.cid, STREAM_W2, e])
        w2[i] = _bf16(g2.standard_normal((cfg.H, cfg.I), dtype=np.float32) * 0.02)
    return w13, w2


def bf16_to_f32(bits):
    """bf16 bit patterns -> float32 values (exact widening)."""
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32)

