"""ctypes loader for libmoe_fp8.so (argument marshalling only).

The library is built in-tree (fp8_routed_expert_amd/libmoe_fp8.so) by
fp8_routed_expert_amd.build.  There is no fallback: if the library is missing
or cannot be loaded, every call raises.
"""

import ctypes
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_fp8.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "moe_fp8.h")

_c_int = ctypes.c_int
_i32p = ctypes.c_void_p
_vp = ctypes.c_void_p
_size = ctypes.c_size_t

# name -> (restype, argtypes), mirroring include/moe_fp8.h
SIGNATURES = {
    "moe_abi_version": (_c_int, []),
    "moe_status_string": (ctypes.c_char_p, [ctypes.c_int32]),
    "moe_layout_workspace_bytes": (_size, [_c_int, _c_int, _c_int]),
    "moe_gemm_large_tiles": (_c_int, [ctypes.c_longlong, _c_int, _c_int]),
    "moe_gemm_tile_rows": (_c_int, [ctypes.c_longlong, _c_int, _c_int, _c_int, _c_int]),
    "moe_dispatch_layout": (ctypes.c_int32, [
        _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
        _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _size, _vp, _vp]),
    "moe_dispatch_layout_noalloc": (ctypes.c_int32, [
        _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
        _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "moe_grouped_gemm_fp8": (ctypes.c_int32, [
        _vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp]),
    "moe_quantize_fp8_e8m0": (ctypes.c_int32, [
        _vp, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp]),
    "moe_dispatch_layout_e8m0": (ctypes.c_int32, [
        _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
        _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _size, _vp, _vp]),
    "moe_grouped_gemm_fp8_e8m0": (ctypes.c_int32, [
        _vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp]),
    "moe_act_requant_e8m0": (ctypes.c_int32, [
        _vp, _vp, _vp, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp]),
    "moe_gemm_fp8": (ctypes.c_int32, [
        _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _vp, _vp]),
    "moe_gate_up_act_fp8": (ctypes.c_int32, [
        _vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp]),
    "moe_gate_up_act_fp8_e8m0": (ctypes.c_int32, [
        _vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp]),
    "moe_act_requant": (ctypes.c_int32, [
        _vp, _vp, _vp, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp]),
    "moe_combine": (ctypes.c_int32, [
        _vp, _c_int, _vp, _vp, _c_int, _c_int, _c_int, _vp, _vp, _vp]),
    "moe_quantize_fp8": (ctypes.c_int32, [
        _vp, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp]),
    "moe_grouped_gemm_fp8_gather": (ctypes.c_int32, [
        _vp, _c_int, _vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _vp, _vp,
        _vp]),
    "moe_grouped_gemm_fp8_gather_e8m0": (ctypes.c_int32, [
        _vp, _c_int, _vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _vp, _vp,
        _vp]),
    "moe_gate_up_act_fp8_gather": (ctypes.c_int32, [
        _vp, _c_int, _vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _vp, _vp,
        _vp, _vp]),
    "moe_gate_up_act_fp8_gather_e8m0": (ctypes.c_int32, [
        _vp, _c_int, _vp, _vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _vp, _vp,
        _vp, _vp]),
    "moe_ceiling_copy": (ctypes.c_int32, [_vp, _vp, _size, _vp]),
    "moe_ceiling_mfma_fp8": (ctypes.c_int32, [_c_int, _c_int, _vp, _vp, _vp]),
}

ABI_VERSION = 9

_lib = None


class MoeError(RuntimeError):
    pass


def header_functions(path=HEADER):
    """Names of the functions declared in include/moe_fp8.h."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def load():
    """Load the library once and attach the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise MoeError(
            f"{LIB_PATH} is not built; run `python -m fp8_routed_expert_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.moe_abi_version() != ABI_VERSION:
        raise MoeError("libmoe_fp8.so ABI version does not match the binding")
    _lib = lib
    return lib


def check(status, what):
    if status != 0:
        msg = load().moe_status_string(status).decode()
        raise MoeError(f"{what} failed: status {status} ({msg})")
