"""GPU parity of pkv_attn_decode_shared_prefix_append: an n-sample step that
writes its tokens' K/V into the tails' last q_len keys and runs the fused
prefix + tail + merge step, in one call.  The pool after the call must equal
the oracle's scatter of the same tokens byte for byte, and the output the
oracle's n-sample step over that pool.  The cases cover tail workgroups of one
row block (the wave that walks a token's tile writes it), of two and four row
blocks (the workgroup writes, then meets at a barrier), samples whose rows
need several tail workgroups (scatter first), tokens across a tile boundary,
tails shorter than the step, 16-key pages (a tile's halves on two pages),
tails longer than one 64-tile window of page ids, and fp8 pools."""

import numpy as np
import pytest
import torch

import oracle as orc
import paged_kv_cache_slots_amd as pkv
import workloads as W
from gpu_util import DEV, as_f64, assert_close, assert_lse_close, from_dev, note, pool_to_dev, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    # name, groups, samples, q_len, prefix lens, tail lens (or (lo, hi) drawn), Hq, Hkv, D, ps, kv
    ("one_token_gqa4", 3, 4, 1, [640, 1500, 32], (1, 200), 32, 8, 128, 32, "bf16"),
    ("q4_tokens_across_tiles", 1, 6, 4, [700], [4, 31, 33, 34, 35, 66], 32, 8, 128, 32, "bf16"),
    ("q8_two_row_blocks", 2, 3, 8, [900, 2100], (8, 300), 16, 4, 128, 32, "bf16"),
    ("q16_four_row_blocks_lds", 2, 2, 16, [300, 1100], (16, 90), 16, 4, 128, 32, "bf16"),
    ("q16_d64_four_row_blocks", 2, 2, 16, [0, 700], (16, 90), 16, 4, 64, 16, "bf16"),
    ("q16_gqa8_scatter_first", 1, 3, 16, [500], (16, 200), 16, 2, 128, 32, "bf16"),
    ("tails_shorter_than_step", 1, 4, 5, [333], [1, 3, 5, 40], 8, 8, 128, 32, "bf16"),
    ("fp8_q4", 2, 4, 4, [1024, 100], (4, 260), 32, 8, 128, 32, "fp8"),
    ("fp8_q9_two_row_blocks", 1, 3, 9, [400], (9, 120), 8, 4, 128, 32, "fp8"),
    ("q2_d64_ps16_half_tiles", 2, 3, 2, [300, 90], (2, 100), 8, 4, 64, 16, "bf16"),
    ("tails_past_one_window", 1, 2, 1, [100], [9000, 8300], 32, 8, 128, 32, "bf16"),
]


def step_tokens(c):
    """The step's token rows [rows * q_len, Hkv, D] (token j of sample r is
    tail key len - q_len + j), their slots (-1 where the key is negative) and
    the pools to start from.  bf16 cases take the rows the case generator
    moved out of the pool (their slots hold poison); fp8 cases take the pool's
    own codes and poison their slots here, so that only the call restores them."""
    ps, n = c.pool.page_size, c.q_len
    hkv, d = c.pool.num_kv_heads, c.pool.head_dim
    rows = len(c.tail_lens)
    flat_k, flat_v = c.pool.k.reshape(-1, hkv, d), c.pool.v.reshape(-1, hkv, d)
    new_k = np.zeros((rows * n, hkv, d), dtype=flat_k.dtype)
    new_v = np.zeros_like(new_k)
    slots = np.full(rows * n, -1, dtype=np.int64)
    src = {} if c.slots is None else {int(s): i for i, s in enumerate(c.slots)}
    for r, L in enumerate(c.tail_lens):
        for j in range(n):
            key = int(L) - n + j
            if key < 0:
                continue
            s = int(c.tail_tables[r][key // ps]) * ps + key % ps
            slots[r * n + j] = s
            if s in src:
                new_k[r * n + j], new_v[r * n + j] = c.new_k[src[s]], c.new_v[src[s]]
            else:
                new_k[r * n + j], new_v[r * n + j] = flat_k[s], flat_v[s]
    if c.slots is None:   # fp8: poison the step's slots of the device copy
        pk, pv = flat_k.copy(), flat_v.copy()
        live = slots[slots >= 0]
        pk[live] = W.POISON[c.pool.dtype]
        pv[live] = W.POISON[c.pool.dtype]
        return new_k, new_v, slots, pk.reshape(c.pool.k.shape), pv.reshape(c.pool.v.shape)
    return new_k, new_v, slots, c.pool.k, c.pool.v


def run_append(c, new_k, new_v, k_start, v_start, out_dtype=torch.bfloat16):
    pool = pool_to_dev(W.Pool(k_start, v_start, c.pool.dtype, c.pool.k_scale, c.pool.v_scale))
    q = to_dev(c.q)
    rows, n, hq, d = q.shape
    out = torch.full((rows, n, hq, d), float("nan"), dtype=out_dtype, device=DEV)
    lse = torch.full((rows, n, hq), float("nan"), dtype=torch.float32, device=DEV)
    mp, mt = int(c.prefix_lens.max()), int(c.tail_lens.max())
    nb = pkv.pkv_attn_decode_shared_prefix_workspace_bytes(rows // c.samples, c.samples, n, hq, d, mp)
    ws = torch.full((nb,), 0xFF, dtype=torch.uint8, device=DEV)        # NaN bytes: contents must not matter
    pkv.pkv_attn_decode_shared_prefix_append(pool, to_dev(new_k), to_dev(new_v), q, c.samples,
                                             to_dev(c.prefix_tables), to_dev(c.prefix_lens), mp,
                                             to_dev(c.tail_tables), to_dev(c.tail_lens), mt, c.sm_scale, out, ws, lse)
    torch.cuda.synchronize()
    return pool, out, lse


def check_append(c, out_dtype=torch.bfloat16):
    note(f"shared append {c.name} groups={len(c.prefix_lens)} samples={c.samples} q_len={c.q_len} "
         f"prefix={list(c.prefix_lens)} tails={list(c.tail_lens)[:8]} kv={c.pool.dtype}")
    new_k, new_v, slots, k_start, v_start = step_tokens(c)
    pool, out, lse = run_append(c, new_k, new_v, k_start, v_start, out_dtype)
    live = slots >= 0
    kp = orc.scatter_slots(k_start, new_k, slots[live], src_idx=np.nonzero(live)[0])
    vp = orc.scatter_slots(v_start, new_v, slots[live], src_idx=np.nonzero(live)[0])
    assert np.array_equal(from_dev(pool.k).view(np.uint8), kp.view(np.uint8)), "K pool differs from the scatter"
    assert np.array_equal(from_dev(pool.v).view(np.uint8), vp.view(np.uint8)), "V pool differs from the scatter"
    ref, ref_lse = orc.attn_decode_shared_prefix(kp, vp, c.q, c.samples, c.prefix_tables, c.prefix_lens,
                                                 c.tail_tables, c.tail_lens, c.sm_scale, kv_dtype=c.pool.dtype,
                                                 q_dtype="bf16", k_scale=c.pool.k_scale, v_scale=c.pool.v_scale)
    got, got_lse = as_f64(from_dev(out)), from_dev(lse).astype(np.float64)
    tol = "fp8" if c.pool.dtype == "fp8" else "bf16"
    assert np.all(np.isfinite(got))
    assert_close(got, ref, tol, f"{c.name} out")
    assert_lse_close(got_lse, ref_lse, tol, f"{c.name} lse")


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_shared_append_parity(case):
    name, groups, samples, n, pl, tl, hq, hkv, d, ps, kv = case
    if isinstance(tl, tuple):
        tl = np.random.default_rng(len(name)).integers(tl[0], tl[1], size=groups * samples, endpoint=True)
    c = W.make_shared_step_case(name, 61, 1061, groups, samples, n, pl, tl, hq, hkv, d, ps, kv_dtype=kv)
    check_append(c)


def test_shared_append_equals_scatter_then_step_bit_for_bit():
    """One call against pkv_scatter_slots + pkv_attn_decode_shared_prefix on the
    n-sample workload's shape (8 prompts x 16 samples, 2048 shared keys, tails
    U[1, 512], 32/8 heads x 128): the same output bits and pool bytes."""
    tl = np.random.default_rng(4).integers(1, 512, size=128, endpoint=True)
    c = W.make_shared_step_case("workload", 52, 1052, 8, 16, 1, [2048] * 8, tl, 32, 8, 128, 32)
    note("shared append against scatter + shared step, n-sample workload shape")
    new_k, new_v, _, _, _ = step_tokens(c)
    results = []
    for fused in (True, False):
        if fused:
            pool, out, lse = run_append(c, new_k, new_v, c.pool.k, c.pool.v)
        else:
            pool = pool_to_dev(c.pool)
            pkv.pkv_scatter_slots(pool, to_dev(c.new_k), to_dev(c.new_v), to_dev(c.slots))
            q = to_dev(c.q)
            rows, n, hq, d = q.shape
            out = torch.empty((rows, n, hq, d), dtype=torch.bfloat16, device=DEV)
            lse = torch.empty((rows, n, hq), dtype=torch.float32, device=DEV)
            mp, mt = int(c.prefix_lens.max()), int(c.tail_lens.max())
            nb = pkv.pkv_attn_decode_shared_prefix_workspace_bytes(rows // c.samples, c.samples, n, hq, d, mp)
            ws = torch.empty((nb,), dtype=torch.uint8, device=DEV)
            pkv.pkv_attn_decode_shared_prefix(pool, q, c.samples, to_dev(c.prefix_tables), to_dev(c.prefix_lens), mp,
                                              to_dev(c.tail_tables), to_dev(c.tail_lens), mt, c.sm_scale, out, ws,
                                              lse)
            torch.cuda.synchronize()
        results.append((from_dev(out), from_dev(lse), from_dev(pool.k), from_dev(pool.v)))
    for a, b in zip(*results):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


def test_shared_append_fp32_output_and_single_sample_groups():
    """fp32 outputs, groups of one sample each (every tail its own group), and an empty prefix."""
    tl = [7, 33, 64, 100, 1]
    c = W.make_shared_step_case("fp32_out_single", 62, 1062, 5, 1, 1, [0, 40, 300, 64, 1000], tl, 16, 4, 128, 32)
    check_append(c, out_dtype=torch.float32)
