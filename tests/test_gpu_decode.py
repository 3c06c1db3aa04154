"""GPU parity of the slot scatter and the paged decode against the oracle.

Every comparison is element by element on the same seeded inputs: scatter is
compared bit for bit over the whole pool (untouched bytes included), decode
outputs and LSE within the stated tolerance (fp32 1e-5 abs, bf16 2e-2 abs/rel,
fp8 K/V 6e-2).  Poison (NaN) fills every pool slot no sequence owns, the dead
rows of partial last pages and the table entries past each row's last page, so
a kernel that reads one key too many returns NaN and fails.
"""

import math

import numpy as np
import pytest
import torch

import oracle as orc
import paged_kv_cache_slots_amd as pkv
import workloads as W
from gpu_util import assert_lse_close, DEV, as_f64, assert_close, from_dev, note, pool_to_dev, to_dev

pytestmark = pytest.mark.gpu


def _oracle_pools(case):
    kp, vp = case.pool.k, case.pool.v
    if case.slots is not None:
        kp = orc.scatter_slots(kp, case.new_k, case.slots)
        vp = orc.scatter_slots(vp, case.new_v, case.slots)
    return kp, vp


def split_only_bytes(t, n, hq, d, max_len):
    """Workspace that holds the key-split partials but not the stream-K state
    (splits: chunks of >= 512 tokens, at most 16), so the split kernel runs."""
    splits = min(16, max(1, -(-max_len // 512)))
    return splits * t * n * hq * (d + 1) * 4 if splits > 1 else 0


def run_decode(case, out_dtype=torch.bfloat16, use_ws="sk", q_override=None):
    """Scatter the case's new tokens, then decode; returns (out, lse) numpy and the device pool.
    use_ws: "sk" (full workspace: stream-K), "split" (key-split partials only) or "none"."""
    pool = pool_to_dev(case.pool)
    if case.slots is not None:
        pkv.pkv_scatter_slots(pool, to_dev(case.new_k), to_dev(case.new_v), to_dev(case.slots))
    q = to_dev(case.q if q_override is None else q_override)
    t, n, hq, d = q.shape
    out = torch.full((t, n, hq, d), float("nan"), dtype=out_dtype, device=DEV)
    lse = torch.full((t, n, hq), float("nan"), dtype=torch.float32, device=DEV)
    ws = None
    if use_ws in ("sk", True):
        nb = pkv.pkv_attn_decode_workspace_bytes(t, n, hq, case.pool.num_kv_heads, d, case.max_kv_len)
        ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=DEV)
    elif use_ws == "split":
        ws = torch.empty(max(split_only_bytes(t, n, hq, d, case.max_kv_len), 16), dtype=torch.uint8, device=DEV)
    pkv.pkv_attn_decode(pool, q, to_dev(case.tables), to_dev(case.kv_lens), case.max_kv_len, case.sm_scale, out, lse,
                        ws)
    torch.cuda.synchronize()
    return as_f64(from_dev(out)), from_dev(lse).astype(np.float64), pool


def check_decode(case, out_dtype=torch.bfloat16, use_ws="sk", subset=None, q_override=None):
    note(f"decode {case.name} T={len(case.kv_lens)} n={case.rows_per_table} Hq={case.num_q_heads} "
         f"Hkv={case.pool.num_kv_heads} D={case.pool.head_dim} ps={case.pool.page_size} kv={case.pool.dtype} "
         f"max_len={case.max_kv_len} ws={use_ws} out={out_dtype}")
    got, got_lse, _ = run_decode(case, out_dtype, use_ws, q_override)
    kp, vp = _oracle_pools(case)
    q = case.q if q_override is None else q_override
    ref, ref_lse = orc.attn_decode(kp, vp, q, case.tables, case.kv_lens, case.sm_scale, kv_dtype=case.pool.dtype,
                                   q_dtype=case.q_dtype, k_scale=case.pool.k_scale, v_scale=case.pool.v_scale,
                                   tables_subset=subset)
    rows = slice(None) if subset is None else list(subset)
    tol = case.pool.dtype if case.pool.dtype != "f32" else ("f32" if out_dtype == torch.float32 else "bf16")
    err = assert_close(got[rows], ref[rows], tol, f"{case.name} out")
    assert_lse_close(got_lse[rows], ref_lse[rows], tol, f"{case.name} lse")
    assert np.all(np.isfinite(got)), "NaN/inf leaked into outputs"
    return err


# --------------------------------------------------------------------------- scatter


def test_tiny_fp32_scatter_is_bit_exact_then_fp32_decode():
    c = W.tiny_fp32_decode()
    note("tiny_fp32_decode scatter + fp32 decode")
    got, got_lse, pool = run_decode(c, out_dtype=torch.float32)
    kp, vp = _oracle_pools(c)
    assert np.array_equal(from_dev(pool.k).view(np.uint32), kp.view(np.uint32))
    assert np.array_equal(from_dev(pool.v).view(np.uint32), vp.view(np.uint32))
    ref, ref_lse = orc.attn_decode(kp, vp, c.q, c.tables, c.kv_lens, c.sm_scale, kv_dtype="f32")
    assert_close(got, ref, "f32", "tiny_fp32_decode out")
    assert_lse_close(got_lse, ref_lse, "f32", "tiny_fp32_decode lse")


@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8"])
@pytest.mark.parametrize("variant", ["plain", "strided_idx_two_dest", "misaligned"])
def test_scatter_variants_bit_exact(dtype, variant):
    rng = np.random.default_rng(21)
    n_pages, ps, hkv, d = 12, 16, 3, 40
    npd = W.STORAGE_NP[dtype]
    pool_k = rng.integers(0, 255, size=(n_pages, ps, hkv, d * np.dtype(npd).itemsize), dtype=np.uint8).view(npd)
    pool_v = rng.integers(0, 255, size=pool_k.view(np.uint8).shape, dtype=np.uint8).view(npd)
    n_src = 30
    packed = rng.integers(0, 255, size=(n_src, 2 * hkv + 5, d * np.dtype(npd).itemsize), dtype=np.uint8).view(npd)
    src_k, src_v = packed[:, 5:5 + hkv], packed[:, 5 + hkv:]
    n_tok = 20
    perm = rng.permutation(n_pages * ps)
    slots = perm[:n_tok].astype(np.int64)
    slots[[2, 9]] = -1
    slots2 = src_idx = None
    if variant != "plain":
        slots2 = perm[n_tok:2 * n_tok].astype(np.int64)
        slots2[[0, 4]] = -3
        src_idx = rng.permutation(n_src)[:n_tok].astype(np.int64)
    note(f"scatter {dtype} {variant}")
    dk, dv = to_dev(pool_k), to_dev(pool_v)
    pk = to_dev(packed)
    if variant == "misaligned":
        # a pool that starts one element into its allocation forces narrow accesses
        flat_k = torch.zeros(dk.numel() + 1, dtype=dk.dtype, device=DEV)
        flat_v = torch.zeros(dv.numel() + 1, dtype=dv.dtype, device=DEV)
        flat_k[1:] = dk.reshape(-1)
        flat_v[1:] = dv.reshape(-1)
        dk = flat_k[1:].view(dk.shape)
        dv = flat_v[1:].view(dv.shape)
    pool = pkv.Pool(dk, dv, torch.ones(1, device=DEV), torch.ones(1, device=DEV)) if dtype == "fp8" else pkv.Pool(dk, dv)
    pkv.pkv_scatter_slots(pool, pk[:, 5:5 + hkv], pk[:, 5 + hkv:], to_dev(slots),
                          None if src_idx is None else to_dev(src_idx), None if slots2 is None else to_dev(slots2))
    torch.cuda.synchronize()
    ref_k = orc.scatter_slots(pool_k, src_k, slots, src_idx=src_idx, slots2=slots2)
    ref_v = orc.scatter_slots(pool_v, src_v, slots, src_idx=src_idx, slots2=slots2)
    assert np.array_equal(from_dev(dk).view(np.uint8), ref_k.view(np.uint8))
    assert np.array_equal(from_dev(dv).view(np.uint8), ref_v.view(np.uint8))


def test_scatter_empty_is_noop():
    c = W.tiny_fp32_decode()
    pool = pool_to_dev(c.pool)
    before = from_dev(pool.k).copy()
    pkv.pkv_scatter_slots(pool, to_dev(c.new_k), to_dev(c.new_v), to_dev(c.slots[:0]))
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(pool.k).view(np.uint32), before.view(np.uint32))


# --------------------------------------------------------------------------- decode parity


EDGE_LENS = [0, 1, 15, 16, 17, 31, 32, 33, 511, 512, 513, 700, 1300]

DECODE_CASES = [
    # name, (T-lens), Hq, Hkv, D, ps, n, kv dtype
    ("gqa4_d128_ps32", EDGE_LENS, 32, 8, 128, 32, 1, "bf16"),
    ("mha_d64_ps16", EDGE_LENS, 4, 4, 64, 16, 1, "bf16"),
    ("gqa8_d128_ps64", [1, 40, 64, 65, 900], 16, 2, 128, 64, 1, "bf16"),
    ("rows32_ps32", [5, 100, 600], 8, 2, 128, 32, 8, "bf16"),     # R = 32: two row blocks
    ("rows64_ps32", [2048, 77], 32, 8, 128, 32, 16, "bf16"),      # R = 64: shared-prefix shape
    ("rows80_ps32", [300, 1025], 8, 2, 64, 32, 20, "bf16"),       # R = 80: row groups
    ("fp8_gqa8_d128", EDGE_LENS, 64, 8, 128, 32, 1, "fp8"),
    ("fp8_d64_ps16", [1, 17, 33, 700], 8, 4, 64, 16, 1, "fp8"),
    ("gqa4_ps128", [1, 127, 128, 129, 1000], 32, 8, 128, 128, 1, "bf16"),
    ("fp8_ps256", [1, 255, 256, 257, 2000], 64, 8, 128, 256, 1, "fp8"),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
@pytest.mark.parametrize("use_ws", ["sk", "split", "none"])
def test_decode_parity(case, use_ws):
    name, lens, hq, hkv, d, ps, n, kv = case
    c = W.make_decode_case(name, 31, 1031, len(lens), hq, hkv, d, ps, lens, kv_dtype=kv, rows_per_table=n,
                           new_per_seq=0 if kv == "fp8" else 1, extra_table_cols=2,
                           num_pool_pages=sum(math.ceil(L / ps) for L in lens) + 9)
    check_decode(c, use_ws=use_ws)


@pytest.mark.parametrize("hq,hkv", [(8, 2), (32, 8), (24, 12)], ids=["per-unit", "head-quads2", "head-quads3"])
def test_decode_stream_k_many_rows_with_empty_ones(hq, hkv):
    """Hundreds of table rows (some empty) so that chunk boundaries cut many
    units and whole units fall inside one worker's chunk; with kv heads in
    quads the workers are head-parallel workgroups (2 or 3 quads per row)."""
    rng = np.random.default_rng(3)
    lens = rng.integers(0, 300, size=300)
    lens[::7] = 0
    lens[5] = 4000
    c = W.make_decode_case("many_rows", 81, 1081, len(lens), hq, hkv, 128, 32, lens, new_per_seq=1)
    check_decode(c, use_ws="sk")
    check_decode(c, out_dtype=torch.float32, use_ws="sk")


def _random_decode_case(seed):
    """A seeded random decode shape: pool dtype, head_dim, page size, GQA
    grouping (kv heads 1-12), rows per table 1-4 and lengths 0-1500 (some
    empty), so that head-parallel and per-unit stream-K workers, cut and whole
    units and every page-size path occur across the seeds."""
    rng = np.random.default_rng(900 + seed)
    kv = "fp8" if rng.random() < 0.3 else "bf16"
    d = 128 if (kv == "fp8" or rng.random() < 0.7) else 64
    ps = int(rng.choice([32, 64])) if kv == "fp8" else int(rng.choice([16, 32, 64]))
    hkv = int(rng.choice([1, 2, 4, 8, 12]))
    group = int(rng.choice([1, 2, 4, 8]))
    n = int(rng.integers(1, 5))
    t = int(rng.integers(1, 40))
    lens = rng.integers(0, 1500, size=t)
    lens[rng.random(t) < 0.1] = 0
    lens[0] = max(int(lens[0]), 1)
    return W.make_decode_case(f"rand{seed}", 700 + seed, 1700 + seed, t, hkv * group, hkv, d, ps, lens,
                              kv_dtype=kv, rows_per_table=n, new_per_seq=0 if kv == "fp8" else 1,
                              extra_table_cols=1, num_pool_pages=sum(math.ceil(int(L) / ps) for L in lens) + 5)


@pytest.mark.parametrize("seed", range(12))
def test_decode_random_shapes(seed):
    c = _random_decode_case(seed)
    check_decode(c, use_ws=["sk", "split", "none"][seed % 3])


def test_decode_fp32_out_and_fp32_query_paths():
    lens = [3, 64, 129, 700]
    c = W.make_decode_case("f32out", 41, 1041, len(lens), 8, 2, 128, 32, lens, kv_dtype="bf16", new_per_seq=1)
    check_decode(c, out_dtype=torch.float32)
    # q fp32 over a bf16 pool runs the vector-ALU kernel
    qf = W.to_storage(as_f64(c.q).astype(np.float32), "f32")
    note("decode fp32 query over bf16 pool")
    got, got_lse, _ = run_decode(c, out_dtype=torch.float32, q_override=qf)
    kp, vp = _oracle_pools(c)
    ref, ref_lse = orc.attn_decode(kp, vp, qf, c.tables, c.kv_lens, c.sm_scale, kv_dtype="bf16", q_dtype="f32")
    assert_close(got, ref, "f32", "valu out")
    assert_lse_close(got_lse, ref_lse, "f32", "valu lse")


@pytest.mark.parametrize("use_ws", ["sk", "split"])
def test_decode_page_permutation_gives_bit_identical_output(use_ws):
    lens = [1000, 37, 2048, 513]
    outs = []
    for perm_seed in (5, 6, 7):
        c = W.make_decode_case("perm", 51, perm_seed, len(lens), 32, 8, 128, 32, lens, num_pool_pages=400)
        note(f"page permutation seed {perm_seed} ws={use_ws}")
        got, got_lse, _ = run_decode(c, use_ws=use_ws)
        outs.append((got, got_lse))
    for got, got_lse in outs[1:]:
        assert np.array_equal(got, outs[0][0]) and np.array_equal(got_lse, outs[0][1])
    kp, vp = _oracle_pools(c)
    ref, _ = orc.attn_decode(kp, vp, c.q, c.tables, c.kv_lens, c.sm_scale)
    assert_close(outs[0][0], ref, "bf16", "perm out")


def test_decode_peaked_newest_key_dominates():
    """Every query row's newest key (the scattered one) scores far above the
    rest, so the output is that key's V row: a length off by one either way
    changes the result by O(1) (or to NaN)."""
    lens = [1, 32, 33, 400, 1055]
    c = W.make_decode_case("peaked", 61, 1061, len(lens), 8, 2, 128, 32, lens, new_per_seq=1)
    qf = as_f64(c.q).astype(np.float32)
    qf[:, :, :, :] = qf[:, :, :1, :]                       # all heads of a row share one query vector
    c.q = W.to_storage(qf, "bf16")
    qv = as_f64(c.q)[:, 0, 0, :]                           # [T, D] (bf16-rounded)
    newk = qv / np.linalg.norm(qv, axis=1, keepdims=True) * 6.0 * math.sqrt(128)
    c.new_k = np.repeat(W.to_storage(newk.astype(np.float32), "bf16")[:, None, :], 2, axis=1)
    check_decode(c)
    got, _, _ = run_decode(c)
    vnew = as_f64(c.new_v)                                 # [T, Hkv, D]
    for t in range(len(lens)):
        for h in range(8):
            np.testing.assert_allclose(got[t, 0, h], vnew[t, h // 4], atol=3e-2)


def test_full_size_gqa_bf16_decode():
    """The bf16 GQA workload at full size (64 sequences, lengths U[512, 4096],
    32/8 heads x 128, 16384-page pool): every output row and LSE against the
    oracle."""
    check_decode(W.gqa_bf16_decode())


_FP8_CHUNKS = 4


@pytest.fixture(scope="module")
def long_fp8_gpu():
    """The long fp8 workload (256 sequences, lengths log-uniform in [1024,
    32768], 64/8 heads, e4m3fn K/V) decoded once on the GPU; the tests below
    compare its rows with the oracle a quarter at a time."""
    c = W.long_fp8_decode()
    note(f"decode {c.name} T={len(c.kv_lens)} full size, stream-K workspace")
    got, got_lse, _ = run_decode(c, use_ws="sk")
    assert np.all(np.isfinite(got)), "NaN/inf leaked into outputs"
    return c, got, got_lse


@pytest.mark.parametrize("chunk", range(_FP8_CHUNKS))
def test_full_size_long_fp8_decode(long_fp8_gpu, chunk):
    """Every row of the long fp8 decode against the oracle (streamed one
    sequence at a time by the oracle itself), in four chunks of 64 sequences
    so that each test stays short; the longest sequence is in one of them."""
    c, got, got_lse = long_fp8_gpu
    rows = list(range(chunk * len(c.kv_lens) // _FP8_CHUNKS, (chunk + 1) * len(c.kv_lens) // _FP8_CHUNKS))
    ref, ref_lse = orc.attn_decode(c.pool.k, c.pool.v, c.q, c.tables, c.kv_lens, c.sm_scale, kv_dtype="fp8",
                                   q_dtype=c.q_dtype, k_scale=c.pool.k_scale, v_scale=c.pool.v_scale,
                                   tables_subset=rows)
    err = assert_close(got[rows], ref[rows], "fp8", f"{c.name} out rows {rows[0]}..{rows[-1]}")
    lerr = assert_lse_close(got_lse[rows], ref_lse[rows], "fp8", f"{c.name} lse rows {rows[0]}..{rows[-1]}")
    print(f"[fp8 decode] rows {rows[0]}..{rows[-1]}: max |out err| {err:.3g}, max |lse err| {lerr:.3g}")


@pytest.mark.parametrize("tables", [8192, 8193], ids=["stream_k_limit", "past_limit_split_path"])
def test_decode_table_count_at_and_past_the_stream_k_limit(tables):
    """8192 table rows is the most the stream-K kernel takes (its prefix sums
    of tiles per row live in LDS); one more row falls back to the key-split
    kernel with the same workspace.  Short and empty rows; sampled rows are
    checked, among them the first, the last and the longest."""
    rng = np.random.default_rng(tables)
    lens = rng.integers(0, 80, size=tables)
    lens[::11] = 0
    lens[tables // 2] = 700
    c = W.make_decode_case(f"tables{tables}", 83, 1083, tables, 8, 2, 64, 32, lens, new_per_seq=1)
    subset = sorted(set(rng.choice(tables, 12, replace=False).tolist()) | {0, tables - 1, tables // 2})
    check_decode(c, use_ws="sk", subset=subset)


def test_decode_fp32_query_rows_past_65535_blocks():
    """The fp32 kernel runs one workgroup per (query row, q head) and split:
    2100 tables x 32 q heads = 67,200 of them, more than a grid's y or z
    dimension holds, with one long row so the keys are split."""
    rng = np.random.default_rng(7)
    lens = rng.integers(0, 40, size=2100)
    lens[::13] = 0
    lens[1234] = 3000
    c = W.make_decode_case("fp32_many_rows", 84, 1084, len(lens), 32, 4, 64, 16, lens, kv_dtype="f32",
                           new_per_seq=1)
    subset = sorted(set(rng.choice(len(lens), 10, replace=False).tolist()) | {0, 1234, len(lens) - 1})
    check_decode(c, out_dtype=torch.float32, use_ws="split", subset=subset)


def test_decode_more_tables_than_65535_without_workspace():
    """Without a workspace the bf16 decode runs one workgroup per table row and
    kv head: 65,600 table rows take more blocks than a grid's y or z dimension
    holds."""
    rng = np.random.default_rng(8)
    lens = rng.integers(1, 17, size=65600)
    c = W.make_decode_case("bf16_many_tables", 85, 1085, len(lens), 2, 1, 64, 16, lens, new_per_seq=1)
    subset = sorted(set(rng.choice(len(lens), 10, replace=False).tolist()) | {0, 65535, len(lens) - 1})
    check_decode(c, use_ws="none", subset=subset)


def test_headline_decode_is_run_to_run_bit_identical():
    """Stream-K cut points depend only on the lengths and the CU count, and
    every partial state is merged in a fixed order, so two calls on the same
    inputs give the same bits (outputs and LSE)."""
    c = W.gqa_bf16_decode()
    note("gqa_bf16_decode twice, bitwise")
    out1, lse1, _ = run_decode(c)
    out2, lse2, _ = run_decode(c)
    assert np.array_equal(out1.view(np.uint64), out2.view(np.uint64))
    assert np.array_equal(lse1.view(np.uint64), lse2.view(np.uint64))


def test_timing_events_carry_the_decode_kernel_alone():
    """With the measurement hook on, the decode kernel is launched with the
    caller's start / stop events: they fall inside events recorded around the
    whole call (decode kernel + merge kernel), span less than it, and the
    output is unchanged.  Repeated over several calls, each call sets both
    events again."""
    c = W.gqa_bf16_decode()
    note("timing events hook on the bf16 GQA workload")
    ref_out, ref_lse, _ = run_decode(c)
    pool = pool_to_dev(c.pool)
    pkv.pkv_scatter_slots(pool, to_dev(c.new_k), to_dev(c.new_v), to_dev(c.slots))
    q = to_dev(c.q)
    t, n, hq, d = q.shape
    out = torch.empty((t, n, hq, d), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((t, n, hq), dtype=torch.float32, device=DEV)
    ws = torch.empty(pkv.pkv_attn_decode_workspace_bytes(t, n, hq, 8, d, c.max_kv_len), dtype=torch.uint8,
                     device=DEV)
    tables, lens = to_dev(c.tables), to_dev(c.kv_lens)
    for _ in range(3):
        a, ks, ke, b = (torch.cuda.Event(enable_timing=True) for _ in range(4))
        ks.record()     # creates the events; the launch sets them again
        ke.record()
        a.record()
        pkv.pkv_set_timing_events(ks, ke)
        try:
            pkv.pkv_attn_decode(pool, q, tables, lens, c.max_kv_len, c.sm_scale, out, lse, ws)
        finally:
            pkv.pkv_set_timing_events(None, None)
        b.record()
        torch.cuda.synchronize()
        kern, call = ks.elapsed_time(ke), a.elapsed_time(b)
        assert 0.0 < kern < call
        assert a.elapsed_time(ks) >= 0.0 and ke.elapsed_time(b) > 0.0
    assert np.array_equal(as_f64(from_dev(out)), ref_out) and np.array_equal(from_dev(lse).astype(np.float64),
                                                                             ref_lse)
