"""Helpers for the GPU parity tests: host<->device copies and the acceptance
checks (exact for integer/byte work; FP8 code agreement >= 99.9%; outputs with
relative L2 error <= 2e-3 and per-element |err| <= 0.02 * max|ref|)."""

import sys
import time

import numpy as np
import torch

from oracle.codec import bf16_decode, e4m3_decode

REL_L2_TOL = 2e-3
MAX_ERR_FRAC = 0.02
CODE_AGREE_MIN = 0.999


def log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def dev(a, dtype=None):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    t = torch.from_numpy(a).cuda()
    return t if dtype is None else t.to(dtype)


def host(t):
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bf16_vals(t):
    return bf16_decode(host(t))


def check_close(got, ref, what, rel_l2_tol=REL_L2_TOL):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    d = got - ref
    nref = np.linalg.norm(ref)
    rel = np.linalg.norm(d) / nref if nref > 0 else np.linalg.norm(d)
    maxerr = np.abs(d).max() if d.size else 0.0
    bound = MAX_ERR_FRAC * (np.abs(ref).max() if ref.size else 0.0)
    log(f"{what}: rel_l2={rel:.3e} max_err={maxerr:.3e} bound={bound:.3e} n={ref.size}")
    assert rel <= rel_l2_tol, f"{what}: relative L2 {rel:.3e} > {rel_l2_tol}"
    assert maxerr <= bound, f"{what}: max |err| {maxerr:.3e} > {bound:.3e}"
    return rel


def code_agreement(got, ref, what, minimum=CODE_AGREE_MIN):
    """Fraction of E4M3 codes that decode to the same value (+0 == -0)."""
    g = e4m3_decode(np.asarray(got))
    r = e4m3_decode(np.asarray(ref))
    same = (g == r) | (np.isnan(g) & np.isnan(r))
    frac = same.mean() if same.size else 1.0
    log(f"{what}: code agreement {frac:.7f} ({(~same).sum()} differ of {same.size})")
    assert frac >= minimum, f"{what}: code agreement {frac} < {minimum}"
    return frac
