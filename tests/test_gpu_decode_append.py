"""GPU parity of pkv_attn_decode_append: a step's K/V written into the last
q_len keys of every row, then attended causally, in one call.  The pool after
the call must equal the oracle's scatter of the same tokens byte for byte, and
the output the oracle's step attention over that pool.  The cases cover the
path where the head-parallel stream-K kernel writes the tokens itself (kv
heads in quads, one 16-row block per row) and the paths that scatter first
(more rows, other head counts, key splits, no workspace, fp32 queries)."""

import math

import numpy as np
import pytest
import torch

import oracle as orc
import paged_kv_cache_slots_amd as pkv
import workloads as W
from gpu_util import DEV, as_f64, assert_close, assert_lse_close, from_dev, note, pool_to_dev, to_dev
from test_gpu_decode import split_only_bytes

pytestmark = pytest.mark.gpu

CASES = [
    # name, lens, Hq, Hkv, D, page size, q_len, kv dtype
    ("gqa4_q1", [1, 33, 600, 1300, 4096], 32, 8, 128, 32, 1, "bf16"),
    ("gqa4_q3_tokens_across_tiles", [3, 31, 32, 33, 64, 65, 97, 700], 32, 8, 128, 32, 3, "bf16"),
    ("mha_q4_d64_ps16", [4, 5, 33, 600], 4, 4, 64, 16, 4, "bf16"),
    ("rows_shorter_than_step", [0, 1, 3, 5, 6, 70], 8, 4, 128, 32, 5, "bf16"),
    ("q16_gqa8_more_rows", [16, 17, 700, 2048], 16, 2, 128, 32, 16, "bf16"),
    ("hkv2_not_quads", [5, 600, 1000], 8, 2, 128, 32, 1, "bf16"),
    ("fp8_gqa8_q2", [2, 100, 1500], 64, 8, 128, 32, 2, "fp8"),
    ("fp32_query", [3, 50, 70, 600], 4, 4, 64, 32, 3, "f32"),
]


def step_tokens(c, n):
    """The step's token rows [T * n, Hkv, D] (token j of row t is key len - n + j)
    and their slots (-1 where the key is negative), in the pool's storage type.
    bf16 / f32 cases take the rows the case generator moved out of the pool
    (their slots hold poison); fp8 cases take the pool's own codes and poison
    their slots here, so that only the call can restore them."""
    ps = c.pool.page_size
    hkv, d = c.pool.num_kv_heads, c.pool.head_dim
    t_rows = len(c.kv_lens)
    flat_k = c.pool.k.reshape(-1, hkv, d)
    flat_v = c.pool.v.reshape(-1, hkv, d)
    new_k = np.zeros((t_rows * n, hkv, d), dtype=flat_k.dtype)
    new_v = np.zeros_like(new_k)
    slots = np.full(t_rows * n, -1, dtype=np.int64)
    src = {}
    if c.slots is not None:
        src = {int(s): i for i, s in enumerate(c.slots)}
    for t, L in enumerate(c.kv_lens):
        for j in range(n):
            key = int(L) - n + j
            if key < 0:
                continue
            s = int(c.tables[t][key // ps]) * ps + key % ps
            slots[t * n + j] = s
            if s in src:
                new_k[t * n + j], new_v[t * n + j] = c.new_k[src[s]], c.new_v[src[s]]
            else:
                new_k[t * n + j], new_v[t * n + j] = flat_k[s], flat_v[s]
    if c.slots is None:   # fp8: poison the step's slots of the device copy
        poisoned_k, poisoned_v = flat_k.copy(), flat_v.copy()
        live = slots[slots >= 0]
        poisoned_k[live] = W.POISON["fp8"]
        poisoned_v[live] = W.POISON["fp8"]
        return new_k, new_v, slots, poisoned_k.reshape(c.pool.k.shape), poisoned_v.reshape(c.pool.v.shape)
    return new_k, new_v, slots, c.pool.k, c.pool.v


@pytest.mark.parametrize("use_ws", ["sk", "split", "none"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_decode_append_parity(case, use_ws):
    name, lens, hq, hkv, d, ps, n, kv = case
    c = W.make_decode_case(name, 43, 1043, len(lens), hq, hkv, d, ps, lens, kv_dtype=kv, rows_per_table=n,
                           new_per_seq=0 if kv == "fp8" else n, extra_table_cols=2,
                           num_pool_pages=sum(math.ceil(L / ps) for L in lens) + 9)
    note(f"decode append {name} lens={lens} q_len={n} Hq={hq} Hkv={hkv} D={d} ps={ps} kv={kv} ws={use_ws}")
    new_k, new_v, slots, k_start, v_start = step_tokens(c, n)
    pool = pool_to_dev(W.Pool(k_start, v_start, c.pool.dtype, c.pool.k_scale, c.pool.v_scale) if c.slots is None
                       else c.pool)
    q = to_dev(c.q)
    t, _, _, _ = q.shape
    out_dtype = torch.float32 if kv == "f32" else torch.bfloat16
    out = torch.full((t, n, hq, d), float("nan"), dtype=out_dtype, device=DEV)
    lse = torch.full((t, n, hq), float("nan"), dtype=torch.float32, device=DEV)
    ws = None
    if use_ws == "sk":
        nb = pkv.pkv_attn_decode_workspace_bytes(t, n, hq, hkv, d, c.max_kv_len)
        ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=DEV)
    elif use_ws == "split":
        ws = torch.empty(max(split_only_bytes(t, n, hq, d, c.max_kv_len), 16), dtype=torch.uint8, device=DEV)
    pkv.pkv_attn_decode_append(pool, to_dev(new_k), to_dev(new_v), q, to_dev(c.tables), to_dev(c.kv_lens),
                               c.max_kv_len, c.sm_scale, out, lse, ws)
    torch.cuda.synchronize()
    # the pool: byte-identical to the oracle's scatter of the live tokens
    live = slots >= 0
    kp = orc.scatter_slots(k_start, new_k, slots[live], src_idx=np.nonzero(live)[0])
    vp = orc.scatter_slots(v_start, new_v, slots[live], src_idx=np.nonzero(live)[0])
    assert np.array_equal(from_dev(pool.k).view(np.uint8), kp.view(np.uint8)), "K pool differs from the scatter"
    assert np.array_equal(from_dev(pool.v).view(np.uint8), vp.view(np.uint8)), "V pool differs from the scatter"
    ref, ref_lse = orc.attn_decode_step(kp, vp, c.q, c.tables, c.kv_lens, c.sm_scale, kv_dtype=kv,
                                        q_dtype=c.q_dtype, k_scale=c.pool.k_scale, v_scale=c.pool.v_scale)
    got, got_lse = as_f64(from_dev(out)), from_dev(lse).astype(np.float64)
    assert_close(got, ref, kv, f"{name} out")
    assert_lse_close(got_lse, ref_lse, kv, f"{name} lse")
    assert np.all(np.isfinite(got))


def test_decode_append_equals_scatter_then_decode_bit_for_bit():
    """One call against pkv_scatter_slots + pkv_attn_decode on the headline shape
    (64 rows of 512-4096 keys, 32 / 8 heads): the same output bits and pool bytes."""
    c = W.gqa_bf16_decode()
    note("decode append against scatter + decode, headline shape")
    new_k, new_v, slots, _, _ = step_tokens(c, 1)
    t, n, hq, d = c.q.shape
    hkv = c.pool.num_kv_heads
    results = []
    for fused in (True, False):
        pool = pool_to_dev(c.pool)
        q = to_dev(c.q)
        out = torch.empty((t, n, hq, d), dtype=torch.bfloat16, device=DEV)
        lse = torch.empty((t, n, hq), dtype=torch.float32, device=DEV)
        ws = torch.empty(pkv.pkv_attn_decode_workspace_bytes(t, n, hq, hkv, d, c.max_kv_len), dtype=torch.uint8,
                         device=DEV)
        if fused:
            pkv.pkv_attn_decode_append(pool, to_dev(new_k), to_dev(new_v), q, to_dev(c.tables), to_dev(c.kv_lens),
                                       c.max_kv_len, c.sm_scale, out, lse, ws)
        else:
            pkv.pkv_scatter_slots(pool, to_dev(c.new_k), to_dev(c.new_v), to_dev(c.slots))
            pkv.pkv_attn_decode(pool, q, to_dev(c.tables), to_dev(c.kv_lens), c.max_kv_len, c.sm_scale, out, lse,
                                ws)
        torch.cuda.synchronize()
        results.append((from_dev(out), from_dev(lse), from_dev(pool.k), from_dev(pool.v)))
    for a, b in zip(*results):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


@pytest.mark.parametrize("layout", ["packed_qkv_slice", "misaligned_by_one_element"])
def test_decode_append_strided_token_rows(layout):
    """The step's K/V as views: the K and V slices of a packed [T * q_len, Hq + 2 Hkv, D] projection (token
    stride (Hq + 2 Hkv) D, 16-byte aligned: the kernel writes them itself), and rows that start one element
    off a 16-byte boundary (the call scatters them first, 2 bytes at a time)."""
    lens = [3, 31, 32, 33, 600, 1300]
    hq, hkv, d, ps, n = 32, 8, 128, 32, 3
    c = W.make_decode_case("strided_" + layout, 44, 1044, len(lens), hq, hkv, d, ps, lens, rows_per_table=n,
                           new_per_seq=n, extra_table_cols=2,
                           num_pool_pages=sum(math.ceil(L / ps) for L in lens) + 9)
    note(f"decode append strided {layout} lens={lens} q_len={n}")
    new_k, new_v, slots, k_start, v_start = step_tokens(c, n)
    rows = new_k.shape[0]
    if layout == "packed_qkv_slice":
        packed = torch.zeros((rows, hq + 2 * hkv, d), dtype=torch.bfloat16, device=DEV)
        packed[:, hq:hq + hkv] = to_dev(new_k)
        packed[:, hq + hkv:] = to_dev(new_v)
        dk, dv = packed[:, hq:hq + hkv], packed[:, hq + hkv:]
        assert dk.stride() == ((hq + 2 * hkv) * d, d, 1)
    else:
        flat = torch.zeros(2 * rows * hkv * d + 2, dtype=torch.bfloat16, device=DEV)
        dk = flat[1:1 + rows * hkv * d].view(rows, hkv, d)
        dv = flat[1 + rows * hkv * d:1 + 2 * rows * hkv * d].view(rows, hkv, d)
        dk.copy_(to_dev(new_k))
        dv.copy_(to_dev(new_v))
        assert dk.data_ptr() % 16 != 0
    pool = pool_to_dev(c.pool)
    q = to_dev(c.q)
    t = q.shape[0]
    out = torch.full((t, n, hq, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((t, n, hq), float("nan"), dtype=torch.float32, device=DEV)
    ws = torch.empty(pkv.pkv_attn_decode_workspace_bytes(t, n, hq, hkv, d, c.max_kv_len), dtype=torch.uint8,
                     device=DEV)
    pkv.pkv_attn_decode_append(pool, dk, dv, q, to_dev(c.tables), to_dev(c.kv_lens), c.max_kv_len, c.sm_scale,
                               out, lse, ws)
    torch.cuda.synchronize()
    live = slots >= 0
    kp = orc.scatter_slots(k_start, new_k, slots[live], src_idx=np.nonzero(live)[0])
    vp = orc.scatter_slots(v_start, new_v, slots[live], src_idx=np.nonzero(live)[0])
    assert np.array_equal(from_dev(pool.k).view(np.uint8), kp.view(np.uint8)), "K pool differs from the scatter"
    assert np.array_equal(from_dev(pool.v).view(np.uint8), vp.view(np.uint8)), "V pool differs from the scatter"
    ref, ref_lse = orc.attn_decode_step(kp, vp, c.q, c.tables, c.kv_lens, c.sm_scale, kv_dtype="bf16",
                                        q_dtype=c.q_dtype)
    assert_close(as_f64(from_dev(out)), ref, "bf16", f"{layout} out")
    assert_lse_close(from_dev(lse).astype(np.float64), ref_lse, "bf16", f"{layout} lse")


def test_decode_append_graph_replays():
    """The call captured in a HIP graph (it allocates nothing and records no memset): every replay, with eager
    work and synchronisations between them, gives the eager call's output bits and pool bytes."""
    lens = [5, 40, 600, 1300]
    hq, hkv, d, ps, n = 32, 8, 128, 32, 1
    c = W.make_decode_case("graph", 45, 1045, len(lens), hq, hkv, d, ps, lens, rows_per_table=n, new_per_seq=n,
                           extra_table_cols=2, num_pool_pages=sum(math.ceil(L / ps) for L in lens) + 9)
    note(f"decode append graph replays lens={lens}")
    new_k, new_v, _, _, _ = step_tokens(c, n)
    pool = pool_to_dev(c.pool)
    q, tables, kv_lens, nk, nv = to_dev(c.q), to_dev(c.tables), to_dev(c.kv_lens), to_dev(new_k), to_dev(new_v)
    t = q.shape[0]
    out = torch.zeros((t, n, hq, d), dtype=torch.bfloat16, device=DEV)
    lse = torch.zeros((t, n, hq), dtype=torch.float32, device=DEV)
    ws = torch.empty(pkv.pkv_attn_decode_workspace_bytes(t, n, hq, hkv, d, c.max_kv_len), dtype=torch.uint8,
                     device=DEV)

    def call(stream=None):
        pkv.pkv_attn_decode_append(pool, nk, nv, q, tables, kv_lens, c.max_kv_len, c.sm_scale, out, lse, ws,
                                   stream=stream)
    call()
    torch.cuda.synchronize()
    ref_out, ref_lse = out.clone(), lse.clone()
    ref_k, ref_v = pool.k.clone(), pool.v.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(torch.cuda.current_stream())
    for _ in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
        assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32))
        assert torch.equal(pool.k.view(torch.uint8), ref_k.view(torch.uint8))
        assert torch.equal(pool.v.view(torch.uint8), ref_v.view(torch.uint8))
