"""Helpers of the GPU parity tests: storage <-> device tensors and the
tolerance check.  Nothing here computes anything the oracle or the kernels
compute."""

from __future__ import annotations

import sys

import numpy as np
import torch

import paged_kv_cache_slots_amd as pkv

DEV = "cuda:0"

# Tolerances of attention outputs: |gpu - ref| <= atol + rtol * |ref| (torch
# allclose convention).
TOL = {"f32": (1e-5, 0.0), "bf16": (2e-2, 2e-2), "fp8": (6e-2, 6e-2)}
# The LSE is a log-domain value: an absolute error e scales every merge weight
# built from it by exp(e), whatever the LSE's size, so it is held to the
# absolute part of the tolerance alone (no term that grows with |lse|).
LSE_ATOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 6e-2}


def note(msg: str) -> None:
    """Name the case on stdout before a GPU step (flushed, so a fault still shows it)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(a).to(DEV)


def from_dev(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def as_f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def pool_to_dev(p) -> pkv.Pool:
    ks = None if p.k_scale is None else to_dev(p.k_scale)
    vs = None if p.v_scale is None else to_dev(p.v_scale)
    return pkv.Pool(to_dev(p.k), to_dev(p.v), ks, vs)


def assert_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = "") -> float:
    """Elementwise tolerance check; infinities must match exactly."""
    atol, rtol = TOL[dtype]
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    inf = np.isinf(ref)
    assert np.array_equal(np.isinf(got), inf) and np.array_equal(got[inf], ref[inf]), f"{what}: infinities differ"
    assert not np.any(np.isnan(got)), f"{what}: NaN in GPU result"
    g, r = got[~inf], ref[~inf]
    err = np.abs(g - r)
    bound = atol + rtol * np.abs(r)
    bad = err > bound
    if np.any(bad):
        i = int(np.argmax(err - bound))
        raise AssertionError(f"{what}: {int(bad.sum())} of {err.size} outside tolerance; worst |{g[i]} - {r[i]}| "
                             f"= {err[i]:.3g} > {bound[i]:.3g}")
    return float(err.max()) if err.size else 0.0


def assert_lse_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = "") -> float:
    """|lse_gpu - lse_ref| <= LSE_ATOL[dtype] elementwise; -inf (empty key
    sets, padding rows) must match exactly."""
    atol = LSE_ATOL[dtype]
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    inf = np.isinf(ref)
    assert np.array_equal(np.isinf(got), inf) and np.array_equal(got[inf], ref[inf]), f"{what}: infinities differ"
    assert not np.any(np.isnan(got)), f"{what}: NaN in GPU LSE"
    err = np.abs(got[~inf] - ref[~inf])
    if err.size and err.max() > atol:
        i = int(np.argmax(err))
        raise AssertionError(f"{what}: {int((err > atol).sum())} of {err.size} LSE values off by more than {atol}; "
                             f"worst |{got[~inf][i]} - {ref[~inf][i]}| = {err[i]:.3g}")
    return float(err.max()) if err.size else 0.0
