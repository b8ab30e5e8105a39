"""GPU parity of the dense block-scaled FP8 GEMM (moe_gemm_fp8) against the
oracle's definition of the same product (oracle.moe.gemm_rows): the general
GEMM for linears outside the MoE block ("Deploying DeepSeek with PD
Disaggregation and Large-Scale Expert Parallelism on 96 H100 GPUs", section
大规模专家并行 > DeepGEMM 集成)."""

import numpy as np
import pytest
import torch

import fp8_routed_expert_amd as fre
from oracle import moe
from oracle.codec import e4m3_encode, bf16_decode
from tests.gpu_util import dev, host, check_close, log

pytestmark = pytest.mark.gpu


def _run_dense(a, sa_rows, w, sw):
    """Upload, run moe_gemm_fp8, return bf16 bits [M, N]."""
    M, _ = a.shape
    N = w.shape[0]
    c = torch.zeros(M, N, dtype=torch.bfloat16, device="cuda")
    fre.moe_gemm_fp8(dev(a), dev(np.ascontiguousarray(sa_rows.T)), dev(w), dev(sw), c)
    torch.cuda.synchronize()
    return host(c)


def _operands(g, M, N, K):
    x = g.standard_normal((M, K)) * np.exp(g.uniform(-2, 2, (M, 1)))
    wv = g.standard_normal((N, K)) * 0.02
    a, sa = moe.quantize_blocks(x, 1)
    w, sw = moe.quantize_blocks(wv, 128)
    return a, sa, w, sw


def test_dense_exact_integers_pow2_scales(gpu):
    """Small-integer codes and power-of-two scales keep every sum exact, so
    the result must equal the oracle's bit for bit (codes in [-4, 4], scales
    2^[-2, 2]: every partial sum is a multiple of 2^-4 below 2^17, exact in
    fp32 in any order); M is ragged (not a multiple of any tile) so the last
    tile is partly outside the matrix."""
    g = np.random.default_rng(41)
    M, N, K = 300, 384, 512
    a = e4m3_encode(g.integers(-4, 5, (M, K)).astype(np.float64))
    w = e4m3_encode(g.integers(-4, 5, (N, K)).astype(np.float64))
    sa = np.ldexp(1.0, g.integers(-2, 3, (M, K // 128))).astype(np.float32)
    sw = np.ldexp(1.0, g.integers(-2, 3, (N // 128, K // 128))).astype(np.float32)
    got = _run_dense(a, sa, w, sw)
    ref = moe.gemm_rows(a, sa, w, sw)
    assert np.array_equal(bf16_decode(got), ref)


# (M, N, K): a single row, ragged tails, the small tile configuration, and a
# shape large enough for the 256 x 256 configuration (checked on sampled rows)
DENSE_SHAPES = [(1, 128, 128), (257, 384, 640), (1000, 2048, 7168), (8192, 7168, 2048)]


@pytest.mark.parametrize("shape", DENSE_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_dense_parity(gpu, shape):
    M, N, K = shape
    g = np.random.default_rng(M + N + K)
    a, sa, w, sw = _operands(g, M, N, K)
    log(f"dense gemm M={M} N={N} K={K}")
    got = _run_dense(a, sa, w, sw)
    rows = np.arange(M) if M <= 1024 else np.unique(
        np.concatenate([g.choice(M, 384, replace=False), [0, M - 1]]))
    ref = moe.gemm_rows(a[rows], sa[rows], w, sw)
    check_close(bf16_decode(got[rows]), ref, f"dense gemm {M}x{N}x{K} ({len(rows)} rows)")


def test_dense_matches_grouped_single_expert(gpu):
    """The dense call is the grouped kernel with one expert whose segment is
    the whole buffer: both must give identical bits."""
    g = np.random.default_rng(7)
    M, N, K = 515, 512, 1024
    a, sa, w, sw = _operands(g, M, N, K)
    dense = _run_dense(a, sa, w, sw)
    c = torch.zeros(M, N, dtype=torch.bfloat16, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    fre.moe_grouped_gemm_fp8(dev(a), dev(np.ascontiguousarray(sa.T)), dev(w[None]),
                             dev(sw[None]), dev(np.array([0, M], np.int32)),
                             dev(np.array([M], np.int32)), c, st)
    torch.cuda.synchronize()
    assert np.array_equal(host(c), dense)


def test_dense_zero_rows_is_a_no_op(gpu):
    c = torch.full((0, 128), 1.0, dtype=torch.bfloat16, device="cuda")
    a = torch.zeros(0, 128, dtype=torch.uint8, device="cuda")
    sa = torch.zeros(1, 0, dtype=torch.float32, device="cuda")
    w = torch.zeros(128, 128, dtype=torch.uint8, device="cuda")
    sw = torch.ones(1, 1, dtype=torch.float32, device="cuda")
    fre.moe_gemm_fp8(a, sa, w, sw, c)
    torch.cuda.synchronize()
