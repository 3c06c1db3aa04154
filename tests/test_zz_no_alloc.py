"""The no-allocation decode entry point against the workspace one.

``pkv_attn_decode_noalloc`` runs the same kernels as ``pkv_attn_decode`` with
a workspace, its cross-workgroup state in the library's per-device array.  Two
calls in a row (the second on a smaller input, so the array holds the first
call's state when the second starts) must equal the workspace call bit for
bit and the oracle within the bf16 / fp8 tolerances.  A call whose state does
not fit the array is refused before any launch.
"""

import math

import numpy as np
import pytest
import torch

import oracle as orc
import paged_kv_cache_slots_amd as pkv
import workloads as W
from gpu_util import DEV, as_f64, assert_close, assert_lse_close, from_dev, note, pool_to_dev, to_dev

pytestmark = pytest.mark.gpu


def _both(case):
    """Decode ``case`` through the no-allocation entry point, then through the
    workspace entry point; returns both (out, lse) pairs as numpy."""
    pool = pool_to_dev(case.pool)
    if case.slots is not None:
        pkv.pkv_scatter_slots(pool, to_dev(case.new_k), to_dev(case.new_v), to_dev(case.slots))
    q, tables, lens = to_dev(case.q), to_dev(case.tables), to_dev(case.kv_lens)
    t, n, hq, d = q.shape
    res = []
    for mode in ("noalloc", "workspace"):
        out = torch.full((t, n, hq, d), float("nan"), dtype=torch.bfloat16, device=DEV)
        lse = torch.full((t, n, hq), float("nan"), dtype=torch.float32, device=DEV)
        if mode == "noalloc":
            pkv.pkv_attn_decode_noalloc(pool, q, tables, lens, case.max_kv_len, case.sm_scale, out, lse)
        else:
            nb = pkv.pkv_attn_decode_workspace_bytes(t, n, hq, case.pool.num_kv_heads, d, case.max_kv_len)
            ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=DEV)
            pkv.pkv_attn_decode(pool, q, tables, lens, case.max_kv_len, case.sm_scale, out, lse, ws)
        torch.cuda.synchronize()
        res.append((from_dev(out), from_dev(lse)))
    return res


def _oracle(case):
    kp, vp = case.pool.k, case.pool.v
    if case.slots is not None:
        kp = orc.scatter_slots(kp, case.new_k, case.slots)
        vp = orc.scatter_slots(vp, case.new_v, case.slots)
    return orc.attn_decode(kp, vp, case.q, case.tables, case.kv_lens, case.sm_scale, kv_dtype=case.pool.dtype,
                           q_dtype=case.q_dtype, k_scale=case.pool.k_scale, v_scale=case.pool.v_scale)


def _check(case, tol):
    (o1, l1), (o2, l2) = _both(case)
    assert np.array_equal(o1.view(np.uint16), o2.view(np.uint16)), "outputs differ from the workspace call"
    assert np.array_equal(l1.view(np.uint32), l2.view(np.uint32)), "LSE differ from the workspace call"
    ref, ref_lse = _oracle(case)
    assert_close(as_f64(o1), ref, tol, f"{case.name} noalloc out")
    assert_lse_close(l1.astype(np.float64), ref_lse, tol, f"{case.name} noalloc lse")


def test_noalloc_two_calls_in_a_row_second_smaller():
    """The bf16 GQA workload (64 sequences, head-parallel workers), then a
    smaller fp8 decode (20 sequences, some empty, 12 q / 3 kv heads: one wave
    per worker) on the same array."""
    big = W.gqa_bf16_decode()
    note("noalloc decode 1: bf16 GQA workload (64 sequences)")
    _check(big, "bf16")
    lens = [0, 1, 31, 33, 700, 1025, 90, 0, 2048, 17, 5, 400, 512, 513, 64, 3, 1500, 250, 999, 12]
    small = W.make_decode_case("noalloc_small", 44, 1044, len(lens), 12, 3, 128, 32, lens, kv_dtype="fp8",
                               new_per_seq=0, num_pool_pages=sum(math.ceil(L / 32) for L in lens) + 4)
    note("noalloc decode 2: fp8, 12/3 heads, 20 sequences")
    _check(small, "fp8")


def test_noalloc_refuses_a_call_whose_state_does_not_fit():
    """More than 8192 table rows with long keys need fixed key splits whose
    partial states (here ~1.2 GB) exceed the array: PKV_ERR_SCRATCH, and
    nothing is launched (the output keeps its sentinel bytes)."""
    t, hq, hkv, d, ps, max_len = 9000, 32, 8, 128, 32, 4096
    pool = pkv.Pool(torch.zeros((8, ps, hkv, d), dtype=torch.bfloat16, device=DEV),
                    torch.zeros((8, ps, hkv, d), dtype=torch.bfloat16, device=DEV))
    q = torch.zeros((t, 1, hq, d), dtype=torch.bfloat16, device=DEV)
    tables = torch.zeros((t, max_len // ps), dtype=torch.int32, device=DEV)
    lens = torch.zeros(t, dtype=torch.int32, device=DEV)
    out = torch.full((t, 1, hq, d), 7.0, dtype=torch.bfloat16, device=DEV)
    note("noalloc decode 3: refused (state beyond the array)")
    with pytest.raises(pkv.PkvError) as e:
        pkv.pkv_attn_decode_noalloc(pool, q, tables, lens, max_len, 0.1, out)
    assert e.value.status == 7
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
