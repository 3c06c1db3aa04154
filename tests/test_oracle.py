"""Pins of the float64 oracle to things other than itself.

Library routines (torch casts, torch SDPA, index_copy_), closed forms,
hand-worked fixtures under tests/golden/ and invariants.  Each test is chosen
so that a plausible slip in the oracle (a dropped scale, a wrong sign, a wrong
GQA index, a transposed operand, an off-by-one length) fails it.
"""

import math
import os

import numpy as np
import pytest
import torch

import oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# --------------------------------------------------------------------------- storage


def test_e4m3fn_table_matches_torch_cast():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = orc.e4m3fn_table()
    assert np.array_equal(np.isnan(ref), np.isnan(mine))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], mine[ok])
    assert np.isnan(mine[0x7F]) and np.isnan(mine[0xFF])
    assert mine[0x7E] == 448.0 and mine[0x01] == 2.0 ** -9


def test_bf16_decode_matches_torch_view():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)   # every bf16 pattern
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    mine = orc.decode_bf16(bits)
    assert np.array_equal(np.isnan(ref), np.isnan(mine))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], mine[ok])


def test_fp8_scaled_decode_matches_torch():
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 256, size=(6, 4), dtype=np.uint8)
    codes[codes & 0x7F == 0x7F] = 0
    scale = rng.uniform(0.01, 2.0, size=(6, 1)).astype(np.float32)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy() * scale.astype(np.float64)
    assert np.array_equal(orc.decode_e4m3fn(codes, scale), ref)


# --------------------------------------------------------------------------- scatter


@pytest.mark.parametrize("np_dtype", [np.float32, np.uint16, np.uint8])
@pytest.mark.parametrize("with_idx", [False, True])
@pytest.mark.parametrize("with_second", [False, True])
def test_scatter_matches_index_copy(np_dtype, with_idx, with_second):
    rng = np.random.default_rng(2)
    pages, ps, hkv, d = 7, 8, 3, 16
    if np_dtype == np.float32:
        pool = rng.standard_normal((pages, ps, hkv, d)).astype(np.float32)
        src = rng.standard_normal((20, hkv, d)).astype(np.float32)
    else:
        info = np.iinfo(np_dtype)
        pool = rng.integers(0, info.max, size=(pages, ps, hkv, d)).astype(np_dtype)
        src = rng.integers(0, info.max, size=(20, hkv, d)).astype(np_dtype)
    n = 12
    perm = rng.permutation(pages * ps)
    slots = perm[:n].astype(np.int64)
    slots[[3, 7]] = -1                      # skipped tokens
    slots2 = perm[n:2 * n].astype(np.int64) if with_second else None
    if with_second:
        slots2[5] = -4
    src_idx = rng.permutation(20)[:n] if with_idx else None
    mine = orc.scatter_slots(pool, src, slots, src_idx=src_idx, slots2=slots2)

    as_t = lambda a: torch.from_numpy(a.view(np.int32) if a.dtype == np.float32 else a.astype(np.int32))
    flat = as_t(pool.copy()).reshape(pages * ps, hkv, d)
    srows = as_t(src)[torch.from_numpy(src_idx) if with_idx else torch.arange(20)[:n]]
    for dst in ([slots] if slots2 is None else [slots, slots2]):
        keep = torch.from_numpy(dst >= 0)
        flat.index_copy_(0, torch.from_numpy(dst)[keep], srows[keep])
    assert np.array_equal(as_t(mine).reshape(pages * ps, hkv, d).numpy(), flat.numpy())


# --------------------------------------------------------------------------- table translation


def test_gather_matches_hand_worked_slot_fixture():
    rows = _read_golden("slot_mapping.txt")
    ps = int(rows[0][1])
    table = np.array([int(x) for x in rows[1][1:]])
    length = int(rows[2][1])
    expect = np.array([[int(x) for x in r] for r in rows[3:]])
    pages = 8
    # every pool row carries its own slot id as its value
    pool = np.arange(pages * ps, dtype=np.int64).reshape(pages, ps, 1, 1)
    got = orc.gather_logical(pool, table, length)[:, 0, 0]
    assert got.tolist() == expect[:, 3].tolist()
    assert (got // ps).tolist() == expect[:, 1].tolist()
    assert (got % ps).tolist() == expect[:, 2].tolist()


def test_gather_is_page_permutation_invariant():
    rng = np.random.default_rng(3)
    ps, hkv, d, length = 4, 2, 3, 13
    logical = rng.standard_normal((length, hkv, d))
    n_pages = math.ceil(length / ps)
    for seed in range(3):
        order = np.random.default_rng(seed).permutation(10)[:n_pages]
        pool = np.full((10, ps, hkv, d), np.nan)
        for j, page in enumerate(order):           # page-wise placement, block copies
            chunk = logical[j * ps:(j + 1) * ps]
            pool[page, :len(chunk)] = chunk
        table = np.concatenate([order, [-12345]])  # trailing entry must never be read
        assert np.array_equal(orc.gather_logical(pool, table, length), logical)


# --------------------------------------------------------------------------- attention


def _sdpa(q, k, v, scale, mask=None, gqa=False):
    """torch SDPA in float64 on the CPU; q [..., R, D], k/v [..., L, D]."""
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=None if mask is None else torch.from_numpy(mask), scale=scale, enable_gqa=gqa)
    return out.numpy()


def test_attention_matches_torch_sdpa_and_logsumexp():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((5, 16))
    k = rng.standard_normal((37, 16))
    v = rng.standard_normal((37, 16))
    scale = 0.37
    o, lse = orc.attention_rows(q, k, v, scale)
    np.testing.assert_allclose(o, _sdpa(q, k, v, scale), rtol=0, atol=1e-12)
    ref_lse = torch.logsumexp(torch.from_numpy(scale * q @ k.T), dim=1).numpy()
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-12)


def test_attention_closed_forms():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 8))
    k = rng.standard_normal((2, 8))
    v = rng.standard_normal((2, 8))
    scale = 0.5
    # one key: the output is that value, the LSE its score
    o, lse = orc.attention_rows(q, k[:1], v[:1], scale)
    np.testing.assert_allclose(o[0], v[0], atol=1e-15)
    np.testing.assert_allclose(lse[0], scale * float(q[0] @ k[0]), atol=1e-15)
    # two keys: logistic weight of the score difference
    s0, s1 = scale * float(q[0] @ k[0]), scale * float(q[0] @ k[1])
    w0 = 1.0 / (1.0 + math.exp(s1 - s0))
    o, lse = orc.attention_rows(q, k, v, scale)
    np.testing.assert_allclose(o[0], w0 * v[0] + (1 - w0) * v[1], atol=1e-14)
    np.testing.assert_allclose(lse[0], math.log(math.exp(s0) + math.exp(s1)), atol=1e-14)
    # zero query: uniform weights, the output is the mean value and LSE = ln L
    o, lse = orc.attention_rows(np.zeros((1, 8)), k, v, scale)
    np.testing.assert_allclose(o[0], v.mean(axis=0), atol=1e-15)
    np.testing.assert_allclose(lse[0], math.log(2), atol=1e-15)
    # no keys: zero output, LSE -inf
    o, lse = orc.attention_rows(q, k[:0], v[:0], scale)
    assert np.all(o == 0) and np.isneginf(lse[0])


def test_attention_peaked_key_dominates():
    rng = np.random.default_rng(6)
    d, length = 16, 40
    k = rng.standard_normal((length, d)) * 0.1
    v = rng.standard_normal((length, d))
    q = np.zeros((1, d))
    q[0, 0] = 1.0
    k[23, 0] = 60.0   # score 60 * scale above the rest
    o, _ = orc.attention_rows(q, k, v, 1.0)
    np.testing.assert_allclose(o[0], v[23], atol=1e-20 + 1e-12)


def _paged_pool_from_logical(rng, logical_k, logical_v, ps, n_pool, poison=np.nan):
    """Place logical keys of each sequence on random pages, page by page."""
    n_t = len(logical_k)
    hkv, d = logical_k[0].shape[1:]
    perm = rng.permutation(n_pool)
    kp = np.full((n_pool, ps, hkv, d), poison)
    vp = np.full((n_pool, ps, hkv, d), poison)
    width = max(math.ceil(len(x) / ps) for x in logical_k) + 1
    tables = np.full((n_t, width), perm[-1], dtype=np.int64)
    at = 0
    for t in range(n_t):
        for j in range(math.ceil(len(logical_k[t]) / ps)):
            page = perm[at]
            at += 1
            tables[t, j] = page
            kc = logical_k[t][j * ps:(j + 1) * ps]
            kp[page, :len(kc)] = kc
            vp[page, :len(kc)] = logical_v[t][j * ps:(j + 1) * ps]
    return kp.astype(np.float32), vp.astype(np.float32), tables


@pytest.mark.parametrize("hq,hkv,n_rows", [(4, 4, 1), (4, 2, 1), (8, 2, 3)])
def test_decode_matches_sdpa_over_contiguous_keys(hq, hkv, n_rows):
    rng = np.random.default_rng(7)
    d, ps = 8, 4
    lens = [9, 1, 16, 0]
    lk = [rng.standard_normal((L, hkv, d)).astype(np.float32).astype(np.float64) for L in lens]
    lv = [rng.standard_normal((L, hkv, d)).astype(np.float32).astype(np.float64) for L in lens]
    kp, vp, tables = _paged_pool_from_logical(rng, lk, lv, ps, 16)
    q = rng.standard_normal((len(lens), n_rows, hq, d)).astype(np.float32)
    scale = 0.41
    out, lse = orc.attn_decode(kp, vp, q, tables, np.array(lens), scale, kv_dtype="f32")
    assert np.all(np.isfinite(out))              # poison is never read
    for t, L in enumerate(lens):
        if L == 0:
            assert np.all(out[t] == 0) and np.all(np.isneginf(lse[t]))
            continue
        qt = q[t].astype(np.float64).transpose(1, 0, 2)          # [Hq, n, D]
        kt = lk[t].transpose(1, 0, 2)                            # [Hkv, L, D]
        vt = lv[t].transpose(1, 0, 2)
        ref = _sdpa(qt, kt, vt, scale, gqa=(hq != hkv))          # [Hq, n, D]
        np.testing.assert_allclose(out[t].transpose(1, 0, 2), ref, atol=1e-12)


def test_decode_fp8_matches_torch_dequant():
    rng = np.random.default_rng(8)
    ps, hkv, d, hq = 4, 2, 8, 4
    n_pool = 6
    codes_k = rng.integers(0, 0x7E, size=(n_pool, ps, hkv, d), dtype=np.uint8)
    codes_v = rng.integers(0, 0x7E, size=(n_pool, ps, hkv, d), dtype=np.uint8)
    codes_k |= (rng.integers(0, 2, size=codes_k.shape, dtype=np.uint8) << 7)
    sk = rng.uniform(0.001, 0.02, size=(n_pool, hkv)).astype(np.float32)
    sv = rng.uniform(0.001, 0.02, size=(n_pool, hkv)).astype(np.float32)
    table = np.array([[4, 1, 3]])
    L = 10
    q = to_bf16_bits(rng.standard_normal((1, 1, hq, d)).astype(np.float32))
    out, lse = orc.attn_decode(codes_k, codes_v, q, table, [L], 0.3, kv_dtype="fp8", k_scale=sk, v_scale=sv)
    deq = lambda c, s: torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64).numpy() * \
        s.astype(np.float64)[:, None, :, None]
    kr = deq(codes_k, sk)[[4, 1, 3]].reshape(3 * ps, hkv, d)[:L]
    vr = deq(codes_v, sv)[[4, 1, 3]].reshape(3 * ps, hkv, d)[:L]
    qf = torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    ref = _sdpa(qf[0].transpose(1, 0, 2), kr.transpose(1, 0, 2), vr.transpose(1, 0, 2), 0.3, gqa=True)
    np.testing.assert_allclose(out[0].transpose(1, 0, 2), ref, atol=1e-12)


def to_bf16_bits(x):
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# --------------------------------------------------------------------------- prefill


def _visibility_cases():
    rows = _read_golden("prefill_visibility.txt")
    cases = []
    for i in range(0, len(rows), 2):
        _, n_ctx, seq_len, cbs, s_q = rows[i]
        cases.append((int(n_ctx), int(seq_len), int(cbs), int(s_q), [int(x) for x in rows[i + 1]]))
    return cases


@pytest.mark.parametrize("case", _visibility_cases())
def test_prefill_visibility_matches_hand_worked_fixture(case):
    n_ctx, seq_len, cbs, s_q, counts = case
    assert [orc.prefill_visible_keys(i, n_ctx, seq_len, cbs) for i in range(s_q)] == counts


@pytest.mark.parametrize("case", _visibility_cases())
def test_prefill_zero_query_one_hot_values_reveal_visible_set(case):
    """q = 0 makes every visible score equal, so with one-hot V rows the output
    is 1/count on each visible key's coordinate and 0 elsewhere."""
    n_ctx, seq_len, cbs, s_q, counts = case
    ps = 2
    total = n_ctx + seq_len
    d = max(total, 1)
    n_pages = math.ceil(total / ps)
    order = np.random.default_rng(9).permutation(n_pages + 3)[:n_pages]
    kp = np.full((n_pages + 3, ps, 1, d), np.nan, dtype=np.float32)
    vp = np.full((n_pages + 3, ps, 1, d), np.nan, dtype=np.float32)
    eye = np.eye(d, dtype=np.float32)
    for j, page in enumerate(order):
        for r in range(ps):
            p = j * ps + r
            if p < total:
                kp[page, r, 0] = 1.0
                vp[page, r, 0] = eye[p]
    table = np.concatenate([order, [order[0]]])[None]
    q = np.zeros((1, s_q, 1, d), dtype=np.float32)
    out, lse = orc.attn_prefill_block_causal(kp, vp, q, table, [n_ctx], [seq_len], cbs, 1.0, kv_dtype="f32")
    for i, c in enumerate(counts):
        expect = np.zeros(d)
        expect[:c] = 1.0 / c if c else 0.0
        np.testing.assert_allclose(out[0, i, 0], expect, atol=1e-15)
        if c == 0:
            assert np.isneginf(lse[0, i, 0])
        else:
            np.testing.assert_allclose(lse[0, i, 0], math.log(c), atol=1e-15)


def test_prefill_one_token_blocks_is_causal_sdpa():
    rng = np.random.default_rng(10)
    s, h, d, ps = 11, 2, 8, 4
    k = rng.standard_normal((s, h, d)).astype(np.float32)
    v = rng.standard_normal((s, h, d)).astype(np.float32)
    kp, vp, tables = _paged_pool_from_logical(rng, [k.astype(np.float64)], [v.astype(np.float64)], ps, 8)
    q = rng.standard_normal((1, s, h, d)).astype(np.float32)
    out, _ = orc.attn_prefill_block_causal(kp, vp, q, tables, [0], [s], 1, 0.3, kv_dtype="f32")
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q[0].transpose(1, 0, 2)).double(), torch.from_numpy(k.transpose(1, 0, 2)).double(),
        torch.from_numpy(v.transpose(1, 0, 2)).double(), is_causal=True, scale=0.3).numpy()
    np.testing.assert_allclose(out[0].transpose(1, 0, 2), ref, atol=1e-12)


def test_prefill_matches_masked_sdpa_with_context_and_gqa():
    rng = np.random.default_rng(11)
    n_ctx, seq_len, s_q, cbs, hq, hkv, d, ps = 6, 7, 9, 3, 4, 2, 8, 4
    total = n_ctx + seq_len
    k = rng.standard_normal((total, hkv, d)).astype(np.float32)
    v = rng.standard_normal((total, hkv, d)).astype(np.float32)
    kp, vp, tables = _paged_pool_from_logical(rng, [k.astype(np.float64)], [v.astype(np.float64)], ps, 8)
    q = rng.standard_normal((1, s_q, hq, d)).astype(np.float32)
    out, lse = orc.attn_prefill_block_causal(kp, vp, q, tables, [n_ctx], [seq_len], cbs, 0.25, kv_dtype="f32")
    counts = [9, 9, 9, 12, 12, 12, 13, 0, 0]  # by hand: n_ctx 6 + {3, 6, 7}; rows 7, 8 are padding
    mask = np.zeros((s_q, total), dtype=bool)
    for i, c in enumerate(counts):
        mask[i, :c] = True
    real = np.array([c > 0 for c in counts])
    ref = _sdpa(q[0].transpose(1, 0, 2)[:, real].astype(np.float64), k.transpose(1, 0, 2).astype(np.float64),
                v.transpose(1, 0, 2).astype(np.float64), 0.25, mask=mask[real], gqa=True)
    np.testing.assert_allclose(out[0, real].transpose(1, 0, 2), ref, atol=1e-12)
    assert np.all(out[0, ~real] == 0) and np.all(np.isneginf(lse[0, ~real]))


# --------------------------------------------------------------------------- merge


def test_merge_hand_worked_fixture():
    rows = {r[0]: [float(x) for x in r[1:]] for r in _read_golden("merge_two_states.txt")}
    o, lse = orc.merge_states(np.array([[rows["o1"]], [rows["o2"]]]), np.array([rows["lse1"], rows["lse2"]]))
    np.testing.assert_allclose(o[0], rows["o"], atol=1e-15)
    np.testing.assert_allclose(lse[0], rows["lse"][0], atol=1e-15)


@pytest.mark.parametrize("n_chunks", [1, 2, 5])
def test_merge_of_chunks_equals_whole(n_chunks):
    rng = np.random.default_rng(12 + n_chunks)
    q = rng.standard_normal((3, 8))
    k = rng.standard_normal((50, 8))
    v = rng.standard_normal((50, 8))
    cuts = np.sort(rng.choice(np.arange(1, 50), size=n_chunks - 1, replace=False))
    bounds = [0, *cuts.tolist(), 50]
    parts = [orc.attention_rows(q, k[a:b], v[a:b], 0.7) for a, b in zip(bounds[:-1], bounds[1:])]
    parts.append(orc.attention_rows(q, k[:0], v[:0], 0.7))          # an empty run is the identity
    o, lse = orc.merge_states(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    o_ref, lse_ref = orc.attention_rows(q, k, v, 0.7)
    np.testing.assert_allclose(o, o_ref, atol=1e-13)
    np.testing.assert_allclose(lse, lse_ref, atol=1e-13)


def test_merge_all_empty_is_zero_and_ignores_garbage():
    o_parts = np.full((3, 2, 4), np.nan)
    lse_parts = np.full((3, 2), -np.inf)
    o, lse = orc.merge_states(o_parts, lse_parts)
    assert np.all(o == 0) and np.all(np.isneginf(lse))
    # an empty state with garbage output next to a real one leaves the real one unchanged
    o_parts[0, 0] = [1, 2, 3, 4]
    lse_parts[0, 0] = 0.5
    o, lse = orc.merge_states(o_parts, lse_parts)
    np.testing.assert_allclose(o[0], [1, 2, 3, 4])
    assert lse[0] == 0.5


def test_prefix_tail_merge_equals_full_attention_through_tables():
    """Shared prefix read once, private tail per row, merged: equals decode over
    the concatenated table (the n-sample path of the FMHA page)."""
    rng = np.random.default_rng(13)
    ps, hq, hkv, d = 4, 4, 2, 8
    prefix_len, tails = 8, [3, 6, 1]
    lk_p = rng.standard_normal((prefix_len, hkv, d))
    lv_p = rng.standard_normal((prefix_len, hkv, d))
    lk_t = [rng.standard_normal((t, hkv, d)) for t in tails]
    lv_t = [rng.standard_normal((t, hkv, d)) for t in tails]
    kp, vp, tab = _paged_pool_from_logical(rng, [lk_p] + lk_t, [lv_p] + lv_t, ps, 16)
    n_pref_pages = prefix_len // ps
    q = rng.standard_normal((len(tails), 1, hq, d)).astype(np.float32)
    o_pre, l_pre = orc.attn_decode(kp, vp, q.reshape(1, len(tails), hq, d), tab[:1], [prefix_len], 0.3, "f32")
    o_tail, l_tail = orc.attn_decode(kp, vp, q, tab[1:], tails, 0.3, "f32")
    o, lse = orc.merge_states(np.stack([o_pre.reshape(len(tails), 1, hq, d), o_tail]),
                              np.stack([l_pre.reshape(len(tails), 1, hq), l_tail]))
    full = np.concatenate([np.repeat(tab[:1, :n_pref_pages], len(tails), 0), tab[1:]], axis=1)
    o_full, lse_full = orc.attn_decode(kp, vp, q, full, [prefix_len + t for t in tails], 0.3, "f32")
    np.testing.assert_allclose(o, o_full, atol=1e-13)
    np.testing.assert_allclose(lse, lse_full, atol=1e-13)


# --------------------------------------------------------------------------- exact-window commit ops


def test_rotate_rows_hand_worked_fixture():
    for line in open(os.path.join(GOLDEN, "rotate_rows.txt")).read().splitlines():
        if not line.strip() or line.startswith("#"):
            continue
        shift, before, after = (part.strip() for part in line.split("|"))
        row = np.array([[int(v) for v in before.split()]])
        assert orc.rotate_rows(row, int(shift)).tolist() == [[int(v) for v in after.split()]]


@pytest.mark.parametrize("shape", [(1, 5), (3, 8), (7, 33), (2, 1), (3, 0), (0, 4)])
@pytest.mark.parametrize("shift", [0, 1, 3, -2, 64, -1000003])
def test_rotate_rows_matches_numpy_roll(shape, shift):
    rng = np.random.default_rng(abs(shift) + shape[1])
    x = rng.integers(-(2 ** 31), 2 ** 31, size=shape, dtype=np.int64).astype(np.int32)
    expect = np.roll(x, -shift, axis=1) if shape[1] > 0 else x
    assert np.array_equal(orc.rotate_rows(x, shift), expect)


def test_rotate_rows_composes_and_inverts():
    x = np.arange(6 * 11, dtype=np.int32).reshape(6, 11)
    assert np.array_equal(orc.rotate_rows(orc.rotate_rows(x, 4), 9), orc.rotate_rows(x, 13))
    assert np.array_equal(orc.rotate_rows(orc.rotate_rows(x, 5), -5), x)
    assert np.array_equal(orc.rotate_rows(x, 11), x)


def test_copy_slots_matches_fancy_indexing_and_skips_sentinels():
    rng = np.random.default_rng(5)
    layers, pages, ps, h, d = 3, 12, 4, 2, 8
    pool = rng.integers(0, 65536, size=(layers, pages, ps, h, d), dtype=np.int64).astype(np.uint16)
    src = np.array([3, 7, -1, 20, 44, 5], dtype=np.int64)
    dst = np.array([30, 31, 9, -4, 2, 47], dtype=np.int64)
    got = orc.copy_slots(pool, src, dst)
    flat = pool.reshape(layers, pages * ps, h, d).copy()
    keep = (src >= 0) & (dst >= 0)
    flat[:, dst[keep]] = pool.reshape(layers, pages * ps, h, d)[:, src[keep]]
    assert np.array_equal(got, flat.reshape(pool.shape))
    # sentinel destinations and untouched slots keep their bytes
    untouched = np.setdiff1d(np.arange(pages * ps), dst[keep])
    assert np.array_equal(got.reshape(layers, -1, h, d)[:, untouched], pool.reshape(layers, -1, h, d)[:, untouched])


# --------------------------------------------------------------------------- exact-window layout

LAYOUT_KEYS = ("block_tables", "n_ctx", "seq_len", "stage_slots", "stage_slots2",
               "commit_src", "commit_dst", "current_src", "current_dst")


def _layout_cases():
    import json
    with open(os.path.join(GOLDEN, "causal_layout.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _layout_cases(), ids=lambda c: c["name"])
def test_causal_layout_hand_worked_fixtures(case):
    out = orc.causal_layout(case["table"], case["private_pages"], case["page_size"], case["pin"],
                            case["window"], case["committed"], case["evicted"], case["block_sizes"],
                            case["table_width"], case["list_stride"])
    for key in LAYOUT_KEYS:
        assert out[key].tolist() == np.asarray(case[key]).reshape(out[key].shape).tolist(), key


def _forward(pool, lay, committed, ps, block_sizes):
    """Drive a pool of logical positions with a layout's slot lists only, then
    read every block's keys back through its row; returns the key lists."""
    for s, d in zip(lay["commit_src"], lay["commit_dst"]):
        if s >= 0 and d >= 0:
            pool[d] = pool[s]
    for t, (s1, s2) in enumerate(zip(lay["stage_slots"], lay["stage_slots2"])):
        pool[s1] = committed + t
        if s2 >= 0:
            pool[s2] = committed + t
    for s, d in zip(lay["current_src"], lay["current_dst"]):
        if s >= 0 and d >= 0:
            pool[d] = pool[s]
    keys = []
    for b, size in enumerate(block_sizes):
        n = int(lay["n_ctx"][b]) + int(size)
        row = lay["block_tables"][b]
        keys.append([int(pool[int(row[j // ps]) * ps + j % ps]) for j in range(n)])
    return keys


def _check_window(keys, committed, block_sizes, pin, window):
    start = committed
    for b, size in enumerate(block_sizes):
        end = start + size
        want = set(range(min(pin, end))) | set(range(max(pin, start - window), end))
        got = keys[b]
        assert len(got) == len(set(got)), f"block {b}: a key is read twice"
        assert set(got) == want, f"block {b}: read {sorted(set(got) ^ want)} wrongly"
        assert got[len(got) - size:] == list(range(start, end)), f"block {b}: own keys not last"
        start = end


GEOMETRIES = [
    # page_size, pin, window, block_sizes, commit sizes
    (4, 6, 7, [2, 5], [7, 7, 2, 7, 7, 7]),
    (4, 4, 8, [4, 4], [8, 8, 8, 4, 8]),
    (8, 0, 19, [3, 3, 3], [9, 9, 9, 9, 9, 3, 9]),
    (16, 37, 50, [13, 13, 13], [39] * 6),
    (8, 8, 0, [5, 6], [11] * 5),
    (32, 96, 64, [32, 32], [64] * 5),
    (2, 3, 5, [1, 2, 1], [4, 4, 1, 4, 4, 4]),
    (16, 21, 200, [7, 30, 3], [40, 40, 40, 40, 40, 40]),
]


@pytest.mark.parametrize("geometry", GEOMETRIES, ids=lambda g: f"ps{g[0]}_pin{g[1]}_w{g[2]}")
def test_causal_layout_rollout_reads_exactly_the_window(geometry):
    """A rollout from an empty cache: forwards write only through the layout's
    slot lists, commits evict by rotating the rolling part of the table.  Every
    block must read its fixed region, its window and itself, each key once,
    its own keys last."""
    ps, pin, window, sizes, commits = geometry
    bounds = orc.causal_layout_bounds(ps, pin, window, sizes)
    n_fixed, n_roll, n_priv = bounds["fixed_pages"], bounds["rolling_pages"], bounds["private_pages"]
    rng = np.random.default_rng(ps * 1000 + pin)
    ids = rng.permutation(n_fixed + n_roll + len(sizes) * n_priv + 5)
    table = ids[:n_fixed + n_roll].copy()
    private = ids[n_fixed + n_roll:n_fixed + n_roll + len(sizes) * n_priv].reshape(len(sizes), n_priv)
    pool = np.full((len(ids) + 1) * ps, -1, np.int64)
    committed = evicted = 0
    for n in commits:
        lay = orc.causal_layout(table, private, ps, pin, window, committed, evicted, sizes,
                                bounds["table_width"], bounds["list_stride"])
        for _ in range(2):     # several denoising forwards between commits
            _check_window(_forward(pool, lay, committed, ps, sizes), committed, sizes, pin, window)
        committed += n
        new_evicted = orc.window_evicted_tokens(ps, pin, window, committed)
        shift = (new_evicted - evicted) // ps
        table = np.concatenate([table[:n_fixed], orc.rotate_rows(table[None, n_fixed:], shift)[0]])
        evicted = new_evicted


def test_causal_layout_read_back_catches_a_page_aligned_window():
    """The read-back check is strong enough to see the error the exact layout
    removes: a block that reads its window from the start of the window-start
    page sees keys outside its window."""
    case = _layout_cases()[0]
    lay = orc.causal_layout(case["table"], case["private_pages"], case["page_size"], case["pin"],
                            case["window"], case["committed"], case["evicted"], case["block_sizes"],
                            case["table_width"], case["list_stride"])
    ps = case["page_size"]
    pool = np.full(64 * ps, -1, np.int64)
    # committed keys already sit at their own slots
    table = case["table"]
    for x in range(case["committed"]):
        if x < case["pin"]:
            pool[table[x // ps] * ps + x % ps] = x
        elif x - case["pin"] >= case["evicted"]:
            r = x - case["pin"] - case["evicted"]
            pool[table[2 + r // ps] * ps + r % ps] = x
    keys = _forward(pool.copy(), lay, case["committed"], ps, case["block_sizes"])
    _check_window(keys, case["committed"], case["block_sizes"], case["pin"], case["window"])
    # Block 0 reading the whole window-start page (id 10) instead of its piece.
    bad = dict(lay)
    bad["block_tables"] = lay["block_tables"].copy()
    bad["block_tables"][0, :3] = [7, 10, 11]
    bad["n_ctx"] = lay["n_ctx"].copy()
    bad["n_ctx"][0] = 12
    keys = _forward(pool.copy(), bad, case["committed"], ps, case["block_sizes"])
    with pytest.raises(AssertionError):
        _check_window(keys, case["committed"], case["block_sizes"], case["pin"], case["window"])


def test_causal_layout_bounds_hold_and_lists_split_by_commit_point():
    rng = np.random.default_rng(5)
    for _ in range(200):
        ps = int(2 ** rng.integers(0, 6))
        pin = int(rng.integers(0, 4 * ps + 3))
        window = int(rng.integers(0, 6 * ps + 3))
        sizes = [int(v) for v in rng.integers(1, 3 * ps + 2, size=int(rng.integers(1, 5)))]
        committed = int(rng.integers(0, pin + window + 10 * ps))
        evicted = orc.window_evicted_tokens(ps, pin, window, committed)
        bounds = orc.causal_layout_bounds(ps, pin, window, sizes)
        n_tab = bounds["fixed_pages"] + bounds["rolling_pages"]
        table = np.arange(n_tab)
        private = n_tab + np.arange(len(sizes) * bounds["private_pages"]).reshape(len(sizes), -1)
        lay = orc.causal_layout(table, private, ps, pin, window, committed, evicted, sizes,
                                bounds["table_width"], bounds["list_stride"])
        # committed copies read committed keys only, current copies staged ones
        src_pos = {}
        for x in range(committed + sum(sizes)):
            if x < pin:
                src_pos[int(table[x // ps]) * ps + x % ps] = x
            elif x - pin >= evicted:
                r = x - pin - evicted
                src_pos[int(table[bounds["fixed_pages"] + r // ps]) * ps + r % ps] = x
        assert all(src_pos[s] < committed for s in lay["commit_src"] if s >= 0)
        assert all(src_pos[s] >= committed for s in lay["current_src"] if s >= 0)
        assert sorted(src_pos[s] for s in lay["stage_slots"]) == list(range(committed, committed + sum(sizes)))
        # destinations are private slots, each written once
        dst = [d for d in np.concatenate([lay["commit_dst"], lay["current_dst"], lay["stage_slots2"]]) if d >= 0]
        assert len(dst) == len(set(dst)) and all(d // ps >= n_tab for d in dst)


def test_causal_layout_rejects_what_it_cannot_lay_out():
    case = _layout_cases()[0]
    args = dict(table=case["table"], private_pages=case["private_pages"], page_size=4, pin=6, window=7,
                committed=19, evicted=4, block_sizes=[2, 5], table_width=6, list_stride=9)
    orc.causal_layout(**args)
    for change in (dict(page_size=3), dict(evicted=8), dict(evicted=2), dict(table_width=4),
                   dict(table=case["table"][:4]), dict(block_sizes=[2, 13])):
        with pytest.raises(ValueError):
            orc.causal_layout(**{**args, **change})


def test_fp8_prefill_equals_prefill_over_torch_dequantised_pool():
    """An e4m3fn pool with a scale per (page, kv head) attends exactly like an
    fp32 pool holding torch's dequantisation code -> f32 x scale."""
    rng = np.random.default_rng(21)
    n_pages, ps, hkv, d = 9, 16, 2, 32
    codes_k = rng.integers(0, 256, size=(n_pages, ps, hkv, d), dtype=np.uint8)
    codes_v = rng.integers(0, 256, size=(n_pages, ps, hkv, d), dtype=np.uint8)
    for c in (codes_k, codes_v):                         # no NaN codes (0x7F, 0xFF)
        c[(c & 0x7F) == 0x7F] = 0x3C
    # power-of-two scales: code x scale is exact in float32, so both pools hold
    # the same values; a wrong page or head of a scale still changes them
    ks = np.exp2(rng.integers(-9, -2, size=(n_pages, hkv))).astype(np.float32)
    vs = np.exp2(rng.integers(-9, -2, size=(n_pages, hkv))).astype(np.float32)

    def deq(codes, sc):
        f = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32)
        return (f * torch.from_numpy(sc)[:, None, :, None]).numpy()

    tables = np.array([[4, 1, 7, 0, 2, 8]], dtype=np.int32)
    q = rng.standard_normal((1, 40, 4, d)).astype(np.float32)
    qb = torch.from_numpy(q).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    n_ctx, seq = np.array([50], np.int32), np.array([37], np.int32)
    a, la = orc.attn_prefill_block_causal(codes_k, codes_v, qb, tables, n_ctx, seq, 10, 0.2, kv_dtype="fp8",
                                          q_dtype="bf16", k_scale=ks, v_scale=vs)
    b, lb = orc.attn_prefill_block_causal(deq(codes_k, ks), deq(codes_v, vs), qb, tables, n_ctx, seq, 10, 0.2,
                                          kv_dtype="f32", q_dtype="bf16")
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(la, lb, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------- multi-token decode step

def test_decode_step_matches_masked_sdpa_and_empty_rows():
    """Token j of an n-token step attends keys [0, len - (n - 1 - j)): torch
    SDPA with that boolean mask (GQA by repeating kv heads); rows left with no
    key give 0 and -inf."""
    rng = np.random.default_rng(31)
    n_pages, ps, hkv, hq, d, n = 12, 16, 2, 4, 32, 5
    kpool = rng.standard_normal((n_pages, ps, hkv, d)).astype(np.float32)
    vpool = rng.standard_normal((n_pages, ps, hkv, d)).astype(np.float32)
    tables = np.array([[3, 7, 1, 0], [5, 9, 2, 11], [4, 6, 8, 10]], dtype=np.int32)
    lens = np.array([41, 3, 64], dtype=np.int32)          # row 1: fewer keys than step tokens
    q = rng.standard_normal((3, n, hq, d)).astype(np.float32)
    out, lse = orc.attn_decode_step(kpool, vpool, q, tables, lens, 0.3, kv_dtype="f32")
    for t in range(3):
        L = int(lens[t])
        k = np.concatenate([kpool[p] for p in tables[t]])[:L]        # [L, hkv, d]
        v = np.concatenate([vpool[p] for p in tables[t]])[:L]
        kt = torch.from_numpy(np.repeat(k, hq // hkv, axis=1)).permute(1, 0, 2).double()   # [hq, L, d]
        vt = torch.from_numpy(np.repeat(v, hq // hkv, axis=1)).permute(1, 0, 2).double()
        qt = torch.from_numpy(q[t]).permute(1, 0, 2).double()                             # [hq, n, d]
        lim = np.array([L - (n - 1 - j) for j in range(n)])
        mask = torch.from_numpy(np.arange(L)[None, :] < lim[:, None])                   # [n, L]
        live = lim > 0
        if live.any():
            ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=0.3)
            scores = (qt @ kt.transpose(1, 2)) * 0.3
            ref_lse = torch.logsumexp(scores.masked_fill(~mask, float("-inf")), dim=-1)
            np.testing.assert_allclose(out[t][live], ref.permute(1, 0, 2).numpy()[live], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(lse[t][live], ref_lse.permute(1, 0).numpy()[live], rtol=1e-12, atol=1e-12)
        assert np.all(out[t][~live] == 0) and np.all(np.isneginf(lse[t][~live]))
    assert (~(np.array([int(lens[1]) - (n - 1 - j) for j in range(n)]) > 0)).sum() == 2


def test_decode_step_of_one_token_is_plain_decode():
    rng = np.random.default_rng(32)
    kpool = rng.standard_normal((6, 16, 1, 32)).astype(np.float32)
    vpool = rng.standard_normal((6, 16, 1, 32)).astype(np.float32)
    tables = np.array([[2, 0, 5], [1, 3, 4]], dtype=np.int32)
    lens = np.array([40, 17], dtype=np.int32)
    q = rng.standard_normal((2, 1, 2, 32)).astype(np.float32)
    a = orc.attn_decode_step(kpool, vpool, q, tables, lens, 0.2, kv_dtype="f32")
    b = orc.attn_decode(kpool, vpool, q, tables, lens, 0.2, kv_dtype="f32")
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_shared_prefix_step_equals_step_over_joined_tables():
    """Prefix keys then tail keys: with whole-page prefixes, a step over the
    concatenated table row (prefix pages, then tail pages) gives the same
    attention, token by token (the mathematics of the prefix / tail split)."""
    rng = np.random.default_rng(33)
    ps, hkv, hq, d, n, samples = 8, 2, 4, 16, 3, 2
    kpool = rng.standard_normal((30, ps, hkv, d)).astype(np.float32)
    vpool = rng.standard_normal((30, ps, hkv, d)).astype(np.float32)
    prefix_tables = np.array([[3, 9, 14], [20, 1, 7]], dtype=np.int32)
    prefix_lens = np.array([24, 8], dtype=np.int32)              # whole pages
    tail_tables = np.array([[0, 2], [4, 5], [6, 8], [10, 11]], dtype=np.int32)
    tail_lens = np.array([9, 3, 16, 4], dtype=np.int32)           # every tail holds the step's n tokens
    q = rng.standard_normal((4, n, hq, d)).astype(np.float32)
    out, lse = orc.attn_decode_shared_prefix(kpool, vpool, q, samples, prefix_tables, prefix_lens, tail_tables,
                                             tail_lens, 0.25, kv_dtype="f32")
    full = np.zeros((4, 5), dtype=np.int32)
    for r in range(4):
        pp = prefix_tables[r // samples][:prefix_lens[r // samples] // ps]
        row = np.concatenate([pp, tail_tables[r]])
        full[r, :len(row)] = row
    ref, ref_lse = orc.attn_decode_step(kpool, vpool, q, full, prefix_lens[np.arange(4) // samples] + tail_lens,
                                        0.25, kv_dtype="f32")
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------- brute force on tiny inputs


def _walk_keys(pool, table_row, length):
    """Logical keys 0..length-1 of one row, found by walking the table page by
    page and row by row in plain Python (no fancy indexing, no shifts)."""
    page_size = pool.shape[1]
    keys = []
    page_index, offset = 0, 0
    for _ in range(length):
        keys.append(pool[int(table_row[page_index]), offset])
        offset += 1
        if offset == page_size:
            page_index, offset = page_index + 1, 0
    return keys


def _brute_attention(q, keys, vals, scale):
    """Softmax attention by its definition in plain Python floats: weights
    exp(scale q.k_j) summed exactly with math.fsum, no max subtraction (the
    tiny inputs keep every exponent small)."""
    if not keys:
        return [0.0] * len(q), -math.inf
    w = [math.exp(scale * math.fsum(a * b for a, b in zip(q, k))) for k in keys]
    total = math.fsum(w)
    out = [math.fsum(wj * v[d] for wj, v in zip(w, vals)) / total for d in range(len(q))]
    return out, math.log(total)


@pytest.mark.parametrize("seed", range(4))
def test_decode_and_prefill_equal_brute_force_on_tiny_inputs(seed):
    """Tiny pools (D <= 8, lengths <= 40, pages of 4) through random tables:
    the oracle's decode and block-causal prefill equal plain-Python attention
    over keys found by walking the table slot by slot, to 1e-12."""
    rng = np.random.default_rng(4000 + seed)
    ps, hkv, group, d = 4, 2, 2, int(rng.choice([4, 8]))
    hq = hkv * group
    n_pages = 30
    kp = rng.standard_normal((n_pages, ps, hkv, d)).astype(np.float32)
    vp = rng.standard_normal((n_pages, ps, hkv, d)).astype(np.float32)
    lens = [int(x) for x in rng.integers(0, 41, size=3)]
    tables = np.stack([rng.permutation(n_pages)[:10] for _ in lens]).astype(np.int32)
    q = rng.standard_normal((3, 1, hq, d)).astype(np.float32)
    out, lse = orc.attn_decode(kp, vp, q, tables, lens, 0.4, kv_dtype="f32")
    for t, L in enumerate(lens):
        keys, vals = _walk_keys(kp, tables[t], L), _walk_keys(vp, tables[t], L)
        for h in range(hq):
            g = h // group
            o, s = _brute_attention([float(x) for x in q[t, 0, h]], [[float(x) for x in k[g]] for k in keys],
                                    [[float(x) for x in v[g]] for v in vals], 0.4)
            np.testing.assert_allclose(out[t, 0, h], o, rtol=0, atol=1e-12)
            assert (lse[t, 0, h] == s) if s == -math.inf else abs(lse[t, 0, h] - s) < 1e-12
    # block-causal prefill: 9 queries in blocks of 4 over 13 cached keys (one padding row)
    s_q, seq, n_ctx, cbs = 10, 9, 13, 4
    qp = rng.standard_normal((1, s_q, hq, d)).astype(np.float32)
    pout, plse = orc.attn_prefill_block_causal(kp, vp, qp, tables[:1], [n_ctx], [seq], cbs, 0.3, kv_dtype="f32")
    for i in range(s_q):
        count = n_ctx + min((i // cbs + 1) * cbs, seq) if i < seq else 0
        keys, vals = _walk_keys(kp, tables[0], count), _walk_keys(vp, tables[0], count)
        for h in range(hq):
            g = h // group
            o, s = _brute_attention([float(x) for x in qp[0, i, h]], [[float(x) for x in k[g]] for k in keys],
                                    [[float(x) for x in v[g]] for v in vals], 0.3)
            np.testing.assert_allclose(pout[0, i, h], o, rtol=0, atol=1e-12)
            assert (plse[0, i, h] == s) if s == -math.inf else abs(plse[0, i, h] - s) < 1e-12


def test_merge_over_every_subset_split_equals_whole():
    """For a set of 10 keys, every one of the 2^10 ways to split it into a key
    subset and its complement (either side possibly empty) merges back to the
    attention over the whole set."""
    rng = np.random.default_rng(77)
    d, n = 6, 10
    q = rng.standard_normal((2, d))
    k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, d))
    whole, whole_lse = orc.attention_rows(q, k, v, 0.7)
    for mask in range(1 << n):
        a = [j for j in range(n) if mask >> j & 1]
        b = [j for j in range(n) if not mask >> j & 1]
        oa, la = orc.attention_rows(q, k[a], v[a], 0.7)
        ob, lb = orc.attention_rows(q, k[b], v[b], 0.7)
        o, lse = orc.merge_states(np.stack([oa, ob]), np.stack([la, lb]))
        np.testing.assert_allclose(o, whole, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, whole_lse, rtol=0, atol=1e-12)
