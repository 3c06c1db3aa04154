"""GPU parity of the exact-window commit operations: page-table row rotation
and the pool-to-pool slot copy, bit-exact against the oracle over whole
buffers (bytes outside the rotated rows or copied slots included)."""

import numpy as np
import pytest
import torch

import oracle as orc
import paged_kv_cache_slots_amd as pkv
from gpu_util import DEV, note

pytestmark = pytest.mark.gpu

DTYPES = {1: (torch.uint8, np.uint8), 2: (torch.int16, np.int16), 4: (torch.int32, np.int32),
          8: (torch.int64, np.int64), 16: (torch.complex128, np.complex128)}


def _rand(rng, shape, np_dtype):
    raw = rng.integers(0, 256, size=tuple(shape) + (np.dtype(np_dtype).itemsize,), dtype=np.uint8)
    return raw.view(np_dtype).reshape(shape)


def _bytes(a):
    return np.ascontiguousarray(a).view(np.uint8)


@pytest.mark.parametrize("esize", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("shape,pad,shift", [
    ((1, 5), 0, 2), ((3, 8), 0, -3), ((7, 129), 5, 1000003), ((64, 256), 0, 255),
    ((3, 9000), 3, 4321),        # rows past the LDS-staged size for 4+ byte elements: three reversals
    ((2, 40000), 0, -17),
    ((70000, 4), 0, 1),          # more rows than one grid dimension
    ((5, 33), 2, -(10 ** 12) - 7),
])
def test_rotate_rows_matches_oracle(esize, shape, pad, shift):
    tdt, ndt = DTYPES[esize]
    rows, cols = shape
    note(f"rotate esize={esize} shape={shape} pad={pad} shift={shift}")
    rng = np.random.default_rng(rows * 31 + cols + esize)
    full = _rand(rng, (rows, cols + pad), ndt)
    dev = torch.from_numpy(full.copy()).to(DEV)
    view = dev[:, :cols]
    pkv.pkv_rotate_rows(view, shift)
    torch.cuda.synchronize()
    got = dev.cpu().numpy()
    expect = full.copy()
    expect[:, :cols] = orc.rotate_rows(full[:, :cols], shift)
    assert np.array_equal(_bytes(got), _bytes(expect))


@pytest.mark.parametrize("shape", [(3, 0), (0, 4), (6, 1)])
def test_rotate_rows_empty_is_noop(shape):
    note(f"rotate empty {shape}")
    x = torch.arange(shape[0] * shape[1], dtype=torch.int32, device=DEV).view(shape)
    before = x.clone()
    pkv.pkv_rotate_rows(x, 3)
    torch.cuda.synchronize()
    assert torch.equal(x, before)


def test_rotate_rows_one_dimensional_page_table_row():
    note("rotate 1-D row")
    x = torch.arange(10, 30, dtype=torch.int32, device=DEV)
    pkv.pkv_rotate_rows(x, 6)
    torch.cuda.synchronize()
    assert x.cpu().numpy().tolist() == orc.rotate_rows(np.arange(10, 30, dtype=np.int32)[None], 6)[0].tolist()


@pytest.mark.parametrize("dtype,hkv,d,layers,page_size", [
    ("bf16", 8, 128, 3, 32), ("f32", 4, 64, 1, 16), ("fp8", 8, 128, 2, 32), ("bf16", 2, 64, 4, 64)])
def test_copy_slots_matches_oracle(dtype, hkv, d, layers, page_size):
    note(f"copy_slots {dtype} hkv={hkv} d={d} layers={layers} ps={page_size}")
    rng = np.random.default_rng(hkv * d + layers)
    n_pages = 40
    ndt = {"bf16": np.uint16, "f32": np.float32, "fp8": np.uint8}[dtype]
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32, "fp8": torch.uint8}[dtype]
    shape = (layers, n_pages, page_size, hkv, d)
    k = _rand(rng, shape, ndt)
    v = _rand(rng, shape, ndt)
    n_slots = n_pages * page_size
    perm = rng.permutation(n_slots)
    src = perm[:60].astype(np.int64)
    dst = perm[60:120].astype(np.int64)          # disjoint from every source
    src[[3, 17]] = -1                            # sentinel sources
    dst[[5, 41]] = -9                            # sentinel destinations
    def to_dev(a):
        t = torch.from_numpy(a.view(np.int16) if ndt == np.uint16 else a)
        return t.to(DEV).view(tdt) if ndt == np.uint16 else t.to(DEV)
    kd, vd = to_dev(k), to_dev(v)
    # layer 0; further layers sit layer_stride elements later (fp8 pools carry scales, which the copy ignores)
    scales = torch.ones((n_pages, hkv), dtype=torch.float32, device=DEV) if dtype == "fp8" else None
    pool = pkv.Pool(kd[0], vd[0], scales, scales)
    layer_stride = n_pages * page_size * hkv * d
    pkv.pkv_copy_slots(pool, torch.from_numpy(src).to(DEV), torch.from_numpy(dst).to(DEV), layers, layer_stride)
    torch.cuda.synchronize()
    def from_dev(t):
        t = t.cpu()
        return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()
    assert np.array_equal(_bytes(from_dev(kd)), _bytes(orc.copy_slots(k, src, dst)))
    assert np.array_equal(_bytes(from_dev(vd)), _bytes(orc.copy_slots(v, src, dst)))
