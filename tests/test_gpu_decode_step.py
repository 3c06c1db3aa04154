"""GPU parity of the multi-token decode step (speculative verification): the
step's q_len tokens are scattered into the pool as the last keys of each row,
then attended causally among themselves, through all three decode paths
(stream-K, key splits, unsplit) and the fp32 vector path, against the oracle."""

import math

import numpy as np
import pytest
import torch

import oracle as orc
import paged_kv_cache_slots_amd as pkv
import workloads as W
from gpu_util import assert_lse_close, DEV, as_f64, assert_close, from_dev, note, pool_to_dev, to_dev
from test_gpu_decode import split_only_bytes

pytestmark = pytest.mark.gpu


def run_step(case, use_ws="sk", out_dtype=torch.bfloat16, entry=None):
    pool = pool_to_dev(case.pool)
    if case.slots is not None:
        pkv.pkv_scatter_slots(pool, to_dev(case.new_k), to_dev(case.new_v), to_dev(case.slots))
    q = to_dev(case.q)
    t, n, hq, d = q.shape
    out = torch.full((t, n, hq, d), float("nan"), dtype=out_dtype, device=DEV)
    lse = torch.full((t, n, hq), float("nan"), dtype=torch.float32, device=DEV)
    ws = None
    if use_ws == "sk":
        nb = pkv.pkv_attn_decode_workspace_bytes(t, n, hq, case.pool.num_kv_heads, d, case.max_kv_len)
        ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=DEV)
    elif use_ws == "split":
        ws = torch.empty(max(split_only_bytes(t, n, hq, d, case.max_kv_len), 16), dtype=torch.uint8, device=DEV)
    (entry or pkv.pkv_attn_decode_step)(pool, q, to_dev(case.tables), to_dev(case.kv_lens), case.max_kv_len,
                                        case.sm_scale, out, lse, ws)
    torch.cuda.synchronize()
    return as_f64(from_dev(out)), from_dev(lse).astype(np.float64)


STEP_CASES = [
    # name, lens, Hq, Hkv, D, ps, q_len, kv dtype
    ("k8_verify_gqa4_d128", [9, 10, 40, 511, 512, 513, 1300], 32, 8, 128, 32, 9, "bf16"),
    ("q16_gqa8_d128", [16, 17, 700, 2048], 16, 2, 128, 32, 16, "bf16"),      # 128 rows per table row
    ("q4_mha_d64_ps16", [4, 5, 33, 600], 4, 4, 64, 16, 4, "bf16"),
    ("rows_shorter_than_step", [0, 1, 3, 5, 6, 70], 8, 2, 128, 32, 5, "bf16"),
    ("q2_fp8_gqa8", [2, 100, 1500], 64, 8, 128, 32, 2, "fp8"),
    ("q3_fp32_query", [3, 50, 70, 600], 4, 2, 64, 32, 3, "f32"),
]


@pytest.mark.parametrize("use_ws", ["sk", "split", "none"])
@pytest.mark.parametrize("case", STEP_CASES, ids=[c[0] for c in STEP_CASES])
def test_decode_step_parity(case, use_ws):
    name, lens, hq, hkv, d, ps, n, kv = case
    c = W.make_decode_case(name, 41, 1041, len(lens), hq, hkv, d, ps, lens, kv_dtype=kv, rows_per_table=n,
                           new_per_seq=0 if kv == "fp8" else n, extra_table_cols=2,
                           num_pool_pages=sum(math.ceil(L / ps) for L in lens) + 9)
    note(f"decode step {name} lens={lens} q_len={n} Hq={hq} Hkv={hkv} D={d} ps={ps} kv={kv} ws={use_ws}")
    out_dtype = torch.float32 if kv == "f32" else torch.bfloat16
    got, got_lse = run_step(c, use_ws, out_dtype)
    kp, vp = c.pool.k, c.pool.v
    if c.slots is not None:
        kp, vp = orc.scatter_slots(kp, c.new_k, c.slots), orc.scatter_slots(vp, c.new_v, c.slots)
    ref, ref_lse = orc.attn_decode_step(kp, vp, c.q, c.tables, c.kv_lens, c.sm_scale, kv_dtype=kv,
                                        q_dtype=c.q_dtype, k_scale=c.pool.k_scale, v_scale=c.pool.v_scale)
    tol = kv if kv != "f32" else "f32"
    assert_close(got, ref, tol, f"{name} out")
    assert_lse_close(got_lse, ref_lse, tol, f"{name} lse")
    assert np.all(np.isfinite(got))


def test_decode_step_of_one_token_equals_decode_bit_for_bit():
    c = W.make_decode_case("one_token", 42, 1042, 5, 32, 8, 128, 32, [1, 33, 600, 1300, 2000], rows_per_table=1,
                           new_per_seq=1, extra_table_cols=1)
    note("decode step q_len=1 against pkv_attn_decode")
    a = run_step(c, "sk")
    b = run_step(c, "sk", entry=pkv.pkv_attn_decode)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
