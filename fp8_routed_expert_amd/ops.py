"""Python binding of libmoe_fp8: one function per C entry point, same names.

Each function checks shapes, dtypes, devices and contiguity of the torch
tensors it is given, then passes their device pointers and the current HIP
stream to the library.  Nothing is computed here.  FP8 tensors are
torch.uint8 (or torch.float8_e4m3fn, passed as bytes); bf16 tensors are
torch.bfloat16; scales float32; indices int32.
"""

import torch

from ._lib import load, check

LAYOUT_CONTIGUOUS = 0
LAYOUT_MASKED = 1
ERR_BAD_EXPERT = 1
ERR_OVERFLOW = 2
ERR_BAD_INDEX = 4


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t, dtypes, name, shape=None):
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    return t.data_ptr()


_U8 = (torch.uint8, torch.float8_e4m3fn)
_BF16 = (torch.bfloat16,)
_F32 = (torch.float32,)
_I32 = (torch.int32,)


def moe_layout_workspace_bytes(T, K, E):
    return int(load().moe_layout_workspace_bytes(T, K, E))


def moe_gemm_large_tiles(rows_total, N, E):
    """1 if the GEMM calls run this size with large tiles, 0 if with the
    small tiles, -1 for non-positive sizes (the library's host-side rule)."""
    return int(load().moe_gemm_large_tiles(int(rows_total), int(N), int(E)))


def moe_gemm_tile_rows(rows_total, N, K, E, packed_scales=False):
    """Row height (320, 256, 192, 128 or 64) of the output tiles the
    grouped GEMM calls use for N outputs over K inputs at this size;
    packed_scales for the *_e8m0 calls.  -1 for non-positive sizes."""
    return int(load().moe_gemm_tile_rows(int(rows_total), int(N), int(K), int(E),
                                         int(bool(packed_scales))))


def moe_dispatch_layout(topk_idx, x, x_scale, E, layout, align_m, rows, counts,
                        offsets, slot_of, row_src, row_expert, a, a_scale,
                        workspace, status, stream=None):
    """Count / prefix-sum / stably rank / permute the routed rows.

    rows is M_cap (contiguous) or the per-expert capacity C (masked);
    a is [rows_total, H], a_scale [H/128, rows_total] (K-block-major).
    a=None: the rows are not copied (for the *_gather GEMM calls)."""
    T, K = topk_idx.shape
    H = x.shape[1]
    rows_total = E * rows if layout == LAYOUT_MASKED else rows
    lib = load()
    st = lib.moe_dispatch_layout(
        _ptr(topk_idx, _I32, "topk_idx", (T, K)), _ptr(x, _U8, "x", (T, H)),
        _ptr(x_scale, _F32, "x_scale", (T, H // 128)), T, K, E, H, layout,
        align_m, rows, _ptr(counts, _I32, "counts", (E,)),
        _ptr(offsets, _I32, "offsets", (E + 1,)),
        _ptr(slot_of, _I32, "slot_of", (T, K)),
        _ptr(row_src, _I32, "row_src", (rows_total,)),
        _ptr(row_expert, _I32, "row_expert", (rows_total,)),
        None if a is None else _ptr(a, _U8, "a", (rows_total, H)),
        _ptr(a_scale, _F32, "a_scale", (H // 128, rows_total)),
        _ptr(workspace, (torch.uint8,), "workspace"), workspace.numel(),
        _ptr(status, _I32, "status", (1,)), _stream(stream))
    check(st, "moe_dispatch_layout")


def moe_dispatch_layout_noalloc(topk_idx, x, x_scale, E, layout, align_m, rows, counts,
                                offsets, slot_of, row_src, row_expert, a, a_scale, status,
                                stream=None):
    """moe_dispatch_layout without a workspace: the library's fixed device
    scratch holds the per-chunk histograms (nothing is allocated; calls that
    overlap on one GPU race).  Raises on MOE_SCRATCH_LIMIT."""
    T, K = topk_idx.shape
    H = x.shape[1]
    rows_total = E * rows if layout == LAYOUT_MASKED else rows
    lib = load()
    st = lib.moe_dispatch_layout_noalloc(
        _ptr(topk_idx, _I32, "topk_idx", (T, K)), _ptr(x, _U8, "x", (T, H)),
        _ptr(x_scale, _F32, "x_scale", (T, H // 128)), T, K, E, H, layout,
        align_m, rows, _ptr(counts, _I32, "counts", (E,)),
        _ptr(offsets, _I32, "offsets", (E + 1,)),
        _ptr(slot_of, _I32, "slot_of", (T, K)),
        _ptr(row_src, _I32, "row_src", (rows_total,)),
        _ptr(row_expert, _I32, "row_expert", (rows_total,)),
        None if a is None else _ptr(a, _U8, "a", (rows_total, H)),
        _ptr(a_scale, _F32, "a_scale", (H // 128, rows_total)),
        _ptr(status, _I32, "status", (1,)), _stream(stream))
    check(st, "moe_dispatch_layout_noalloc")


def moe_grouped_gemm_fp8(a, a_scale, w, w_scale, offsets, counts, c, status,
                         stream=None):
    """c[valid rows] = block-scaled FP8 grouped GEMM of a with w[expert]."""
    E, N, K = w.shape
    rows_total = a.shape[0]
    lib = load()
    st = lib.moe_grouped_gemm_fp8(
        _ptr(a, _U8, "a", (rows_total, K)),
        _ptr(a_scale, _F32, "a_scale", (K // 128, rows_total)),
        _ptr(w, _U8, "w", (E, N, K)),
        _ptr(w_scale, _F32, "w_scale", (E, N // 128, K // 128)),
        _ptr(offsets, _I32, "offsets", (E + 1,)), _ptr(counts, _I32, "counts", (E,)),
        E, rows_total, N, K, _ptr(c, _BF16, "c", (rows_total, N)),
        _ptr(status, _I32, "status", (1,)), _stream(stream))
    check(st, "moe_grouped_gemm_fp8")


def moe_gemm_fp8(a, a_scale, w, w_scale, c, stream=None):
    """c = dense block-scaled FP8 product of a [M, K] with w [N, K]
    (a_scale [K/128, M], w_scale [N/128, K/128])."""
    M, K = a.shape
    N = w.shape[0]
    lib = load()
    st = lib.moe_gemm_fp8(
        _ptr(a, _U8, "a", (M, K)), _ptr(a_scale, _F32, "a_scale", (K // 128, M)),
        _ptr(w, _U8, "w", (N, K)), _ptr(w_scale, _F32, "w_scale", (N // 128, K // 128)),
        M, N, K, _ptr(c, _BF16, "c", (M, N)), _stream(stream))
    check(st, "moe_gemm_fp8")


def _gate_up_act(name, a, a_scale, w13, w13_scale, offsets, counts, q2, q2_scale, status,
                 stream, packed):
    E, I2, H = w13.shape
    I = I2 // 2
    rows_total = a.shape[0]
    sdt = _I32 if packed else _F32
    hw = _words(H // 128) if packed else H // 128
    iw = _words(I // 128) if packed else I // 128
    lib = load()
    st = getattr(lib, name)(
        _ptr(a, _U8, "a", (rows_total, H)), _ptr(a_scale, sdt, "a_scale", (hw, rows_total)),
        _ptr(w13, _U8, "w13", (E, I2, H)), _ptr(w13_scale, sdt, "w13_scale", (E, I2 // 128, hw)),
        _ptr(offsets, _I32, "offsets", (E + 1,)), _ptr(counts, _I32, "counts", (E,)),
        E, rows_total, I, H, _ptr(q2, _U8, "q2", (rows_total, I)),
        _ptr(q2_scale, sdt, "q2_scale", (iw, rows_total)),
        _ptr(status, _I32, "status", (1,)), _stream(stream))
    check(st, name)


def moe_gate_up_act_fp8(a, a_scale, w13, w13_scale, offsets, counts, q2, q2_scale, status,
                        stream=None):
    """q2, q2_scale = moe_act_requant(moe_grouped_gemm_fp8(a, w13)) in one kernel:
    w13 [E, 2I, H] e4m3 (gate rows first), w13_scale [E, 2I/128, H/128] f32,
    q2 [rows_total, I] e4m3, q2_scale [I/128, rows_total] f32."""
    _gate_up_act("moe_gate_up_act_fp8", a, a_scale, w13, w13_scale, offsets, counts, q2,
                 q2_scale, status, stream, False)


def moe_gate_up_act_fp8_e8m0(a, a_scale, w13, w13_scale, offsets, counts, q2, q2_scale,
                             status, stream=None):
    """moe_gate_up_act_fp8 with packed scales (int32 words of four E8M0 bytes):
    a_scale [ceil(H/512), rows_total], w13_scale [E, 2I/128, ceil(H/512)],
    q2_scale [ceil(I/512), rows_total]."""
    _gate_up_act("moe_gate_up_act_fp8_e8m0", a, a_scale, w13, w13_scale, offsets, counts, q2,
                 q2_scale, status, stream, True)


def _grouped_gemm_gather(name, x, row_src, a_scale, w, w_scale, offsets, counts, c, status,
                         stream, packed):
    E, N, K = w.shape
    T = x.shape[0]
    rows_total = row_src.numel()
    kw = _words(K // 128) if packed else K // 128
    sdt = _I32 if packed else _F32
    lib = load()
    st = getattr(lib, name)(
        _ptr(x, _U8, "x", (T, K)), T, _ptr(row_src, _I32, "row_src", (rows_total,)),
        _ptr(a_scale, sdt, "a_scale", (kw, rows_total)), _ptr(w, _U8, "w", (E, N, K)),
        _ptr(w_scale, sdt, "w_scale", (E, N // 128, kw)),
        _ptr(offsets, _I32, "offsets", (E + 1,)), _ptr(counts, _I32, "counts", (E,)),
        E, rows_total, N, K, _ptr(c, _BF16, "c", (rows_total, N)),
        _ptr(status, _I32, "status", (1,)), _stream(stream))
    check(st, name)


def moe_grouped_gemm_fp8_gather(x, row_src, a_scale, w, w_scale, offsets, counts, c, status,
                                stream=None):
    """moe_grouped_gemm_fp8 reading buffer row r from x[row_src[r]] (x [T, K]
    e4m3; a row without a source reads zero) instead of a permuted buffer."""
    _grouped_gemm_gather("moe_grouped_gemm_fp8_gather", x, row_src, a_scale, w, w_scale,
                         offsets, counts, c, status, stream, False)


def moe_grouped_gemm_fp8_gather_e8m0(x, row_src, a_scale, w, w_scale, offsets, counts, c,
                                     status, stream=None):
    """moe_grouped_gemm_fp8_gather with packed scales."""
    _grouped_gemm_gather("moe_grouped_gemm_fp8_gather_e8m0", x, row_src, a_scale, w, w_scale,
                         offsets, counts, c, status, stream, True)


def _gate_up_act_gather(name, x, row_src, a_scale, w13, w13_scale, offsets, counts, q2,
                        q2_scale, status, stream, packed):
    E, I2, H = w13.shape
    I = I2 // 2
    T = x.shape[0]
    rows_total = row_src.numel()
    sdt = _I32 if packed else _F32
    hw = _words(H // 128) if packed else H // 128
    iw = _words(I // 128) if packed else I // 128
    lib = load()
    st = getattr(lib, name)(
        _ptr(x, _U8, "x", (T, H)), T, _ptr(row_src, _I32, "row_src", (rows_total,)),
        _ptr(a_scale, sdt, "a_scale", (hw, rows_total)),
        _ptr(w13, _U8, "w13", (E, I2, H)), _ptr(w13_scale, sdt, "w13_scale", (E, I2 // 128, hw)),
        _ptr(offsets, _I32, "offsets", (E + 1,)), _ptr(counts, _I32, "counts", (E,)),
        E, rows_total, I, H, _ptr(q2, _U8, "q2", (rows_total, I)),
        _ptr(q2_scale, sdt, "q2_scale", (iw, rows_total)),
        _ptr(status, _I32, "status", (1,)), _stream(stream))
    check(st, name)


def moe_gate_up_act_fp8_gather(x, row_src, a_scale, w13, w13_scale, offsets, counts, q2,
                               q2_scale, status, stream=None):
    """moe_gate_up_act_fp8 reading buffer row r from x[row_src[r]]."""
    _gate_up_act_gather("moe_gate_up_act_fp8_gather", x, row_src, a_scale, w13, w13_scale,
                        offsets, counts, q2, q2_scale, status, stream, False)


def moe_gate_up_act_fp8_gather_e8m0(x, row_src, a_scale, w13, w13_scale, offsets, counts, q2,
                                    q2_scale, status, stream=None):
    """moe_gate_up_act_fp8_gather with packed scales."""
    _gate_up_act_gather("moe_gate_up_act_fp8_gather_e8m0", x, row_src, a_scale, w13,
                        w13_scale, offsets, counts, q2, q2_scale, status, stream, True)


def moe_act_requant(h, offsets, counts, q, q_scale, status, stream=None):
    """q, q_scale = E4M3 1x128 requantisation of silu(h[:, :I]) * h[:, I:]."""
    rows_total, I2 = h.shape
    I = I2 // 2
    E = counts.numel()
    lib = load()
    st = lib.moe_act_requant(
        _ptr(h, _BF16, "h"), _ptr(offsets, _I32, "offsets", (E + 1,)),
        _ptr(counts, _I32, "counts", (E,)), E, rows_total, I,
        _ptr(q, _U8, "q", (rows_total, I)),
        _ptr(q_scale, _F32, "q_scale", (I // 128, rows_total)),
        _ptr(status, _I32, "status", (1,)), _stream(stream))
    check(st, "moe_act_requant")


def moe_combine(y, slot_of, topk_w, out, status, stream=None):
    """out[t] = sum_k topk_w[t,k] * y[slot_of[t,k]] (bf16, fp32 accumulation)."""
    rows_total, H = y.shape
    T, K = slot_of.shape
    lib = load()
    st = lib.moe_combine(
        _ptr(y, _BF16, "y"), rows_total, _ptr(slot_of, _I32, "slot_of"),
        _ptr(topk_w, _F32, "topk_w", (T, K)), T, K, H,
        _ptr(out, _BF16, "out", (T, H)), _ptr(status, _I32, "status", (1,)),
        _stream(stream))
    check(st, "moe_combine")


def moe_quantize_fp8(x, block_rows, q, scale, stream=None):
    """E4M3 block quantisation of a bf16 or fp32 [rows, cols] tensor (or a
    stacked [E, N, K] weight, taken as rows = E*N) with 1x128 or 128x128
    blocks."""
    cols = x.shape[-1]
    rows = x.numel() // cols
    is_f32 = x.dtype == torch.float32
    if q.numel() != x.numel() or scale.numel() != rows // block_rows * (cols // 128):
        raise ValueError("moe_quantize_fp8: q / scale sizes do not match x")
    lib = load()
    st = lib.moe_quantize_fp8(
        _ptr(x, _BF16 + _F32, "x"), 1 if is_f32 else 0, rows, cols, block_rows,
        _ptr(q, _U8, "q"), _ptr(scale, _F32, "scale"), _stream(stream))
    check(st, "moe_quantize_fp8")


# ---- packed power-of-two (E8M0) scales: four 128-wide blocks per 32-bit
# word, held in int32 tensors; see moe_fp8.h for the layouts.
def _words(nb):
    return (nb + 3) // 4


def moe_quantize_fp8_e8m0(x, block_rows, q, scale, stream=None):
    """moe_quantize_fp8 with packed E8M0 scales: scale int32
    [rows / block_rows, ceil(cols / 512)]."""
    cols = x.shape[-1]
    rows = x.numel() // cols
    is_f32 = x.dtype == torch.float32
    if q.numel() != x.numel() or scale.numel() != rows // block_rows * _words(cols // 128):
        raise ValueError("moe_quantize_fp8_e8m0: q / scale sizes do not match x")
    lib = load()
    st = lib.moe_quantize_fp8_e8m0(
        _ptr(x, _BF16 + _F32, "x"), 1 if is_f32 else 0, rows, cols, block_rows,
        _ptr(q, _U8, "q"), _ptr(scale, _I32, "scale"), _stream(stream))
    check(st, "moe_quantize_fp8_e8m0")


def moe_dispatch_layout_e8m0(topk_idx, x, x_scale, E, layout, align_m, rows, counts,
                             offsets, slot_of, row_src, row_expert, a, a_scale,
                             workspace, status, stream=None):
    """moe_dispatch_layout with packed scales: x_scale int32 [T, ceil(H/512)],
    a_scale int32 [ceil(H/512), rows_total]."""
    T, K = topk_idx.shape
    H = x.shape[1]
    hw = _words(H // 128)
    rows_total = E * rows if layout == LAYOUT_MASKED else rows
    lib = load()
    st = lib.moe_dispatch_layout_e8m0(
        _ptr(topk_idx, _I32, "topk_idx", (T, K)), _ptr(x, _U8, "x", (T, H)),
        _ptr(x_scale, _I32, "x_scale", (T, hw)), T, K, E, H, layout,
        align_m, rows, _ptr(counts, _I32, "counts", (E,)),
        _ptr(offsets, _I32, "offsets", (E + 1,)),
        _ptr(slot_of, _I32, "slot_of", (T, K)),
        _ptr(row_src, _I32, "row_src", (rows_total,)),
        _ptr(row_expert, _I32, "row_expert", (rows_total,)),
        None if a is None else _ptr(a, _U8, "a", (rows_total, H)),
        _ptr(a_scale, _I32, "a_scale", (hw, rows_total)),
        _ptr(workspace, (torch.uint8,), "workspace"), workspace.numel(),
        _ptr(status, _I32, "status", (1,)), _stream(stream))
    check(st, "moe_dispatch_layout_e8m0")


def moe_grouped_gemm_fp8_e8m0(a, a_scale, w, w_scale, offsets, counts, c, status,
                              stream=None):
    """moe_grouped_gemm_fp8 with packed scales: a_scale int32
    [ceil(K/512), rows_total], w_scale int32 [E, N/128, ceil(K/512)]."""
    E, N, K = w.shape
    rows_total = a.shape[0]
    kw = _words(K // 128)
    lib = load()
    st = lib.moe_grouped_gemm_fp8_e8m0(
        _ptr(a, _U8, "a", (rows_total, K)),
        _ptr(a_scale, _I32, "a_scale", (kw, rows_total)),
        _ptr(w, _U8, "w", (E, N, K)),
        _ptr(w_scale, _I32, "w_scale", (E, N // 128, kw)),
        _ptr(offsets, _I32, "offsets", (E + 1,)), _ptr(counts, _I32, "counts", (E,)),
        E, rows_total, N, K, _ptr(c, _BF16, "c", (rows_total, N)),
        _ptr(status, _I32, "status", (1,)), _stream(stream))
    check(st, "moe_grouped_gemm_fp8_e8m0")


def moe_act_requant_e8m0(h, offsets, counts, q, q_scale, status, stream=None):
    """moe_act_requant with packed scales: q_scale int32 [ceil(I/512), rows_total]."""
    rows_total, I2 = h.shape
    I = I2 // 2
    E = counts.numel()
    lib = load()
    st = lib.moe_act_requant_e8m0(
        _ptr(h, _BF16, "h"), _ptr(offsets, _I32, "offsets", (E + 1,)),
        _ptr(counts, _I32, "counts", (E,)), E, rows_total, I,
        _ptr(q, _U8, "q", (rows_total, I)),
        _ptr(q_scale, _I32, "q_scale", (_words(I // 128), rows_total)),
        _ptr(status, _I32, "status", (1,)), _stream(stream))
    check(st, "moe_act_requant_e8m0")


def moe_ceiling_copy(src, dst, stream=None):
    """Copy src to dst (same byte size) with the library's plain copy kernel
    (a measurement helper: HBM ceiling)."""
    if src.numel() * src.element_size() != dst.numel() * dst.element_size():
        raise ValueError("src and dst sizes differ")
    n = src.numel() * src.element_size()
    check(load().moe_ceiling_copy(_ptr(src, (src.dtype,), "src"), _ptr(dst, (dst.dtype,), "dst"),
                                  n, _stream(stream)), "moe_ceiling_copy")


def moe_ceiling_mfma_fp8(workgroups, iters, sink, stream=None):
    """Launch the register-only FP8 MFMA chain; returns its flop count (a
    measurement helper: matrix-core ceiling).  sink: float32 [workgroups]."""
    import ctypes
    fl = ctypes.c_double(0.0)
    check(load().moe_ceiling_mfma_fp8(int(workgroups), int(iters),
                                      _ptr(sink, _F32, "sink", (workgroups,)),
                                      ctypes.byref(fl), _stream(stream)), "moe_ceiling_mfma_fp8")
    return fl.value
