"""CPU checks of the C-ABI library: it loads, exports every function that
include/moe_fp8.h declares, and rejects bad host-side arguments before any
launch (nothing here touches a GPU)."""

import ctypes
import os
import shutil
import subprocess

import pytest

from fp8_routed_expert_amd import _lib


def test_library_exports_every_header_function():
    lib = _lib.load()
    names = _lib.header_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.SIGNATURES), "binding and header disagree"


@pytest.mark.parametrize("lang,std", [("c", "-std=c99"), ("c++", "-std=c++11")])
def test_header_is_plain_c(lang, std):
    """The boundary header compiles on its own as C99 and as C++11 with
    warnings as errors: plain types and pointers only, nothing from HIP or
    torch."""
    cc = shutil.which("gcc" if lang == "c" else "g++")
    if cc is None:
        pytest.skip("no host compiler")
    hdr = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                       "include", "moe_fp8.h")
    subprocess.run([cc, "-fsyntax-only", "-Wall", "-Wextra", "-Werror", std, "-x", lang, hdr],
                   check=True, capture_output=True)


def test_version_and_status_strings():
    lib = _lib.load()
    assert lib.moe_abi_version() == _lib.ABI_VERSION
    for s in range(4):
        assert lib.moe_status_string(s)
    assert lib.moe_status_string(99) == b"unknown status"


def test_workspace_bytes():
    lib = _lib.load()
    # one int32 histogram and one int32 base per (chunk of 1024 entries, expert)
    assert lib.moe_layout_workspace_bytes(65536, 8, 9) == 2 * 512 * 9 * 4
    assert lib.moe_layout_workspace_bytes(129, 8, 9) == 2 * 2 * 9 * 4
    assert lib.moe_layout_workspace_bytes(1, 1, 4) == 2 * 1 * 4 * 4
    assert lib.moe_layout_workspace_bytes(0, 8, 4) == 2 * 1 * 4 * 4
    assert lib.moe_layout_workspace_bytes(-1, 8, 4) == 0


N = None


def test_host_argument_errors_launch_nothing():
    lib = _lib.load()
    fake = ctypes.c_void_p(4096)     # never dereferenced: validation fails first
    # grouped GEMM: N not a multiple of 128 -> UNSUPPORTED_SHAPE
    assert lib.moe_grouped_gemm_fp8(fake, fake, fake, fake, fake, fake, 2, 256, 100, 256,
                                    fake, fake, N) == 2
    # negative rows -> INVALID_ARG
    assert lib.moe_grouped_gemm_fp8(fake, fake, fake, fake, fake, fake, 2, -1, 128, 256,
                                    fake, fake, N) == 1
    # null offsets -> INVALID_ARG
    assert lib.moe_grouped_gemm_fp8(fake, fake, fake, fake, N, fake, 2, 256, 128, 256,
                                    fake, fake, N) == 1
    # misaligned A -> UNSUPPORTED_SHAPE
    assert lib.moe_grouped_gemm_fp8(ctypes.c_void_p(4097), fake, fake, fake, fake, fake, 2,
                                    256, 128, 256, fake, fake, N) == 2
    # dense GEMM: K not a multiple of 128, negative M, null scale, M = 0 is a no-op
    assert lib.moe_gemm_fp8(fake, fake, fake, fake, 64, 128, 100, fake, N) == 2
    assert lib.moe_gemm_fp8(fake, fake, fake, fake, -1, 128, 128, fake, N) == 1
    assert lib.moe_gemm_fp8(fake, N, fake, fake, 64, 128, 128, fake, N) == 1
    assert lib.moe_gemm_fp8(fake, fake, fake, fake, 0, 128, 128, fake, N) == 0
    # act: I not a multiple of 128
    assert lib.moe_act_requant(fake, fake, fake, 2, 16, 100, fake, fake, fake, N) == 2
    # fused gate/up + act: I or H not a multiple of 128, one expert's W13 of
    # 2 GB or more, null offsets, misaligned q2, rows_total = 0 is a no-op
    for f in (lib.moe_gate_up_act_fp8, lib.moe_gate_up_act_fp8_e8m0):
        assert f(fake, fake, fake, fake, fake, fake, 2, 256, 100, 256, fake, fake, fake, N) == 2
        assert f(fake, fake, fake, fake, fake, fake, 2, 256, 128, 200, fake, fake, fake, N) == 2
        assert f(fake, fake, fake, fake, fake, fake, 2, 256, 65536, 16384, fake, fake, fake,
                 N) == 2
        assert f(fake, fake, fake, fake, N, fake, 2, 256, 128, 256, fake, fake, fake, N) == 1
        assert f(fake, fake, fake, fake, fake, fake, 2, 256, 128, 256, ctypes.c_void_p(4097),
                 fake, fake, N) == 2
        assert f(fake, fake, fake, fake, fake, fake, 2, 0, 128, 256, fake, fake, fake, N) == 0
    # combine: K too large / H not a multiple of 128
    assert lib.moe_combine(fake, 16, fake, fake, 4, 65, 128, fake, fake, N) == 1
    assert lib.moe_combine(fake, 16, fake, fake, 4, 8, 100, fake, fake, N) == 2
    # quantize: bad block size, bad dtype flag, rows not a multiple of 128
    assert lib.moe_quantize_fp8(fake, 0, 128, 128, 2, fake, fake, N) == 1
    assert lib.moe_quantize_fp8(fake, 2, 128, 128, 1, fake, fake, N) == 1
    assert lib.moe_quantize_fp8(fake, 0, 100, 128, 128, fake, fake, N) == 2
    # layout: bad layout enum, E too large, workspace too small, H % 128
    args = [fake, fake, fake, 16, 2, 4, 256, 5, 128, 512, fake, fake, fake, fake, fake,
            fake, fake, fake, 1 << 20, fake, N]
    assert lib.moe_dispatch_layout(*args) == 1
    a2 = list(args); a2[7] = 0; a2[5] = 2000
    assert lib.moe_dispatch_layout(*a2) == 1
    a3 = list(args); a3[7] = 0; a3[18] = 8
    assert lib.moe_dispatch_layout(*a3) == 1
    a4 = list(args); a4[7] = 0; a4[6] = 200
    assert lib.moe_dispatch_layout(*a4) == 2
    a5 = list(args); a5[7] = 0; a5[8] = 0
    assert lib.moe_dispatch_layout(*a5) == 1


def test_row_scale_span_limit():
    """The row scales are addressed with 32-bit offsets: a call whose scale
    array reaches 0x7ffff000 bytes is refused (MOE_UNSUPPORTED_SHAPE) before
    any launch, in every GEMM entry point; one row less passes the check
    and then fails on the null pointer it is given (INVALID_ARG)."""
    lib = _lib.load()
    fake = ctypes.c_void_p(4096)
    K = 7168                                     # 56 scale blocks, 14 packed words
    lim = 0x7ffff000
    rows_f32 = lim // (56 * 4) + 1               # first row count over the limit
    rows_e8 = lim // (14 * 4) + 1
    assert lib.moe_grouped_gemm_fp8(fake, fake, fake, fake, fake, fake, 4, rows_f32, 4096, K,
                                    fake, fake, N) == 2
    assert lib.moe_grouped_gemm_fp8(fake, fake, fake, fake, N, fake, 4, rows_f32 - 1, 4096, K,
                                    fake, fake, N) == 1
    assert lib.moe_grouped_gemm_fp8_e8m0(fake, fake, fake, fake, fake, fake, 4, rows_e8, 4096,
                                         K, fake, fake, N) == 2
    assert lib.moe_grouped_gemm_fp8_e8m0(fake, fake, fake, fake, N, fake, 4, rows_e8 - 1,
                                         4096, K, fake, fake, N) == 1
    assert lib.moe_gate_up_act_fp8(fake, fake, fake, fake, fake, fake, 4, rows_f32, 2048, K,
                                   fake, fake, fake, N) == 2
    assert lib.moe_gate_up_act_fp8(fake, fake, fake, fake, N, fake, 4, rows_f32 - 1, 2048, K,
                                   fake, fake, fake, N) == 1
    assert lib.moe_gate_up_act_fp8_e8m0(fake, fake, fake, fake, fake, fake, 4, rows_e8, 2048,
                                        K, fake, fake, fake, N) == 2
    assert lib.moe_gemm_fp8(fake, fake, fake, fake, rows_f32, 4096, K, fake, N) == 2
    assert lib.moe_gemm_fp8(fake, N, fake, fake, rows_f32 - 1, 4096, K, fake, N) == 1


def test_binding_refuses_host_tensors():
    import torch
    import fp8_routed_expert_amd as fre
    with pytest.raises(ValueError):
        fre.moe_combine(torch.zeros(4, 128, dtype=torch.bfloat16),
                        torch.zeros(2, 2, dtype=torch.int32), torch.zeros(2, 2),
                        torch.zeros(2, 128, dtype=torch.bfloat16),
                        torch.zeros(1, dtype=torch.int32))


def test_gemm_tile_rule():
    """The host-side tile choice that the layer's fuse rule relies on."""
    lib = _lib.load()
    f = lib.moe_gemm_large_tiles
    assert f(132183, 4096, 9) == 1      # prefill EP32 share, gate/up
    assert f(132183, 7168, 9) == 1      # and down
    assert f(2556, 4096, 4) == 1        # EP72 decode share: 144 large tiles
    assert f(6906, 4096, 6) == 1        # EP48 decode share
    assert f(4096, 4096, 32) == 0       # masked, capacity 128: segments < 256 rows
    assert f(636, 256, 4) == 0          # tiny
    assert f(131072, 384, 1) == 0       # N not a multiple of 256
    assert f(8192, 4096, 1) == 1        # dense, 32 x 16 large tiles
    assert f(2048, 4096, 1) == 0        # dense, 8 x 16 = 128: not more than half the CUs
    assert f(0, 4096, 1) == -1 and f(256, 0, 1) == -1 and f(256, 256, 0) == -1
    rows = lib.moe_gemm_tile_rows
    H, I = 7168, 2048
    assert rows(132183, 2 * I, H, 9, 1) == 320   # prefill share, packed scales
    assert rows(132183, H, I, 9, 1) == 320
    assert rows(132183, 2 * I, H, 9, 0) == 256   # fp32 scales keep 256 x 256
    assert rows(6906, 2 * I, H, 6, 1) == 256     # decode: segments under 4096 rows
    assert rows(13135, 2048, 384, 3, 1) == 320   # the synthetic 320-row test shape
    # masked layout, capacity 128: 64-row tiles for gate/up, 128 for down
    assert rows(4096, 2 * I, H, 32, 1) == 64 and rows(4096, 2 * I, H, 32, 0) == 64
    assert rows(4096, H, I, 32, 1) == 128 and rows(4096, H, I, 32, 0) == 128
    assert rows(636, 256, 256, 4, 0) == 128      # tiny: 159 rows per expert
    # one round either way: EP72 decode gate/up (10 x 16 tiles of 256 rows,
    # 13 x 16 of 192) takes 192 rows; its down projection (N = 7168: 280
    # tiles of 256) and the EP48 share (432 tiles) keep 256
    assert rows(2556, 2 * I, H, 4, 0) == 192 and rows(2556, 2 * I, H, 4, 1) == 192
    assert rows(2556, H, I, 4, 0) == 256
    assert rows(2556, H, I, 4, 1) == 256   # packed too (320 rows measured slower there)
    assert rows(6906, 2 * I, H, 6, 0) == 256
    assert rows(0, 4096, H, 1, 1) == -1 and rows(256, 4096, 0, 1, 1) == -1


def test_gather_argument_checks():
    """The *_gather calls refuse a missing row_src, a negative source-row
    count, a null x with rows to read (MOE_INVALID_ARG) and an x beyond one
    buffer descriptor's 32-bit range (MOE_UNSUPPORTED_SHAPE) before any
    launch; with valid arguments but a null output they fail on that
    (INVALID_ARG), so the gather checks come first."""
    lib = _lib.load()
    fake = ctypes.c_void_p(4096)
    H, I, N2 = 7168, 2048, 4096
    big_T = 0x7ffff000 // H + 1
    for f in (lib.moe_grouped_gemm_fp8_gather, lib.moe_grouped_gemm_fp8_gather_e8m0):
        #        x     T      row_src a_scale w  w_scale offs  counts E rows   N   K  c  st  stream
        assert f(fake, 100, N, fake, fake, fake, fake, fake, 4, 256, N2, H, fake, fake, N) == 1
        assert f(fake, -1, fake, fake, fake, fake, fake, fake, 4, 256, N2, H, fake, fake, N) == 1
        assert f(N, 100, fake, fake, fake, fake, fake, fake, 4, 256, N2, H, fake, fake, N) == 1
        assert f(fake, big_T, fake, fake, fake, fake, fake, fake, 4, 256, N2, H, fake, fake,
                 N) == 2
        assert f(fake, big_T - 1, fake, fake, fake, fake, fake, fake, 4, 256, N2, H, N, fake,
                 N) == 1
    for f in (lib.moe_gate_up_act_fp8_gather, lib.moe_gate_up_act_fp8_gather_e8m0):
        #        x     T    row_src a_scale w13 w13_s offs  counts E rows  I  H  q2  q2s   st  stream
        assert f(fake, 100, N, fake, fake, fake, fake, fake, 4, 256, I, H, fake, fake, fake,
                 N) == 1
        assert f(fake, big_T, fake, fake, fake, fake, fake, fake, 4, 256, I, H, fake, fake,
                 fake, N) == 2
        assert f(fake, big_T - 1, fake, fake, fake, fake, fake, fake, 4, 256, I, H, N, fake,
                 fake, N) == 1
