"""Plain float64 reference for the paged K/V-cache attention path.

TEST INFRASTRUCTURE ONLY: used by ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py``; the HIP library never imports or calls it.

Every function is the plain definition of what the paged path computes, in
numpy float64, with no blocking, splitting or fusion beyond what the definition
states.  Sources (page titles and sections):

* [P1] "Paged causal K/V cache and cached attention for VisualGen":
  Description / Cache (one pool and one page table for all layers; the chunk
  K/V write that puts each token into one or two pool slots; frame-causal
  blocks that need no mask), Description / Attention (real-token ``seq_len``:
  padding rows are neither written nor attended and come back zero), and the
  review thread that fixes the int64 slot id as ``view_page * tokens_per_page
  + slot``.
* [P5] "Support shared-prefix attention for n-sample requests in FMHA":
  commit messages on the FA4 tail (prefix and tail states joined by one merge
  kernel, natural-log LSE), on small-batch splits (an empty run has LSE -inf)
  and on grouping (block-table entries past a row's last page are ignored).

Readings where the pages are silent (softmax scale is an argument; GQA maps
query head h to kv head h // (Hq / Hkv); LSE is natural log; e4m3 is the OCP
e4m3fn format with a float scale per (page, kv head)) are listed in the
design notes of the repository.

Storage conventions (the oracle works on raw storage, never on the GPU's
decoded values):

* fp32 pools / tensors: ``np.float32``;
* bf16: ``np.uint16`` bit patterns;
* fp8 e4m3fn: ``np.uint8`` codes, with ``np.float32`` scales ``[num_pages, Hkv]``.

A pool is ``[num_pages, page_size, Hkv, D]``; slot ``s`` is row ``s % page_size``
of page ``s // page_size``.

Parity pins: every function here is pinned in ``tests/test_oracle.py`` against
library routines, closed forms, hand-listed fixtures or invariants.
"""

from __future__ import annotations

import math

import numpy as np

E4M3FN_MAX = 448.0


# ----------------------------------------------------------------------------
# Storage decoding
# ----------------------------------------------------------------------------

def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64.

    A bfloat16 value is the upper half of an IEEE binary32 word, so the value
    is the binary32 whose high 16 bits are the pattern and low bits zero.
    """
    bits = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def e4m3fn_table() -> np.ndarray:
    """Value of every OCP e4m3fn code, as float64 (NaN for the two NaN codes).

    Format: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent
    field 0 is subnormal (0.m * 2^-6); no infinities; S.1111.111 is NaN; the
    largest finite magnitude is 1.75 * 2^8 = 448.
    """
    table = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        exponent = (code >> 3) & 0xF
        mantissa = code & 0x7
        if exponent == 0xF and mantissa == 0x7:
            table[code] = math.nan
        elif exponent == 0:
            table[code] = sign * (mantissa / 8.0) * 2.0 ** (1 - 7)
        else:
            table[code] = sign * (1.0 + mantissa / 8.0) * 2.0 ** (exponent - 7)
    return table


_E4M3FN = e4m3fn_table()


def decode_e4m3fn(codes: np.ndarray, scale=None) -> np.ndarray:
    """fp8 e4m3fn codes -> float64, times ``scale`` (broadcast) when given.

    The real value of a stored fp8 K/V element is its code value times the
    float scale of its (page, kv head).
    """
    vals = _E4M3FN[np.asarray(codes, dtype=np.uint8)]
    if scale is not None:
        vals = vals * np.asarray(scale, dtype=np.float64)
    return vals


def _decode(raw: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return decode_bf16(raw)
    raise ValueError(f"no plain decoding for {dtype!r} without scales")


# ----------------------------------------------------------------------------
# Slot scatter  [P1] Description / Cache, chunk K/V write; slot-id review thread
# ----------------------------------------------------------------------------

def scatter_slots(pool: np.ndarray, src: np.ndarray, slots, src_idx=None, slots2=None) -> np.ndarray:
    """Return a copy of ``pool`` with source tokens written to their slots.

    ``pool`` is ``[num_pages, page_size, Hkv, D]`` raw storage; ``src`` is
    ``[n_src, Hkv, D]`` of the same storage type.  Token ``i`` (the source row
    ``src_idx[i]``, or ``i`` when no indices are given) is written whole, all
    kv heads, to slot ``slots[i]`` and, when a second list is given, also to
    ``slots2[i]``.  A negative slot is skipped.  The bytes are copied as they
    are: no conversion happens, so fp8 codes stay fp8 codes.
    """
    out = np.array(pool, copy=True)
    page_size = out.shape[1]
    slots = np.asarray(slots, dtype=np.int64)
    n_tokens = slots.shape[0]
    lists = [slots] if slots2 is None else [slots, np.asarray(slots2, dtype=np.int64)]
    for i in range(n_tokens):
        row = i if src_idx is None else int(src_idx[i])
        for dst_list in lists:
            dst = int(dst_list[i])
            if dst < 0:
                continue
            page, offset = divmod(dst, page_size)
            out[page, offset] = src[row]
    return out


# ----------------------------------------------------------------------------
# Block-table translation
# ----------------------------------------------------------------------------

def gather_logical(pool: np.ndarray, table_row, length: int) -> np.ndarray:
    """Logical keys ``0..length-1`` of one sequence, ``[length, Hkv, D]`` raw.

    Logical position p lives on page ``table_row[p // page_size]`` at row
    ``p % page_size``.  Only the entries ``table_row[0 .. ceil(length /
    page_size) - 1]`` are read; later entries are never looked at ([P5] grouping
    commit message).
    """
    page_size = pool.shape[1]
    positions = np.arange(int(length), dtype=np.int64)
    pages = np.asarray(table_row, dtype=np.int64)[positions // page_size]
    rows = positions % page_size
    return pool[pages, rows]


def _gather_real(pool, table_row, length, dtype, scale):
    """Gathered logical keys decoded to float64 ``[length, Hkv, D]``."""
    raw = gather_logical(pool, table_row, length)
    if dtype == "fp8":
        page_size = pool.shape[1]
        positions = np.arange(int(length), dtype=np.int64)
        pages = np.asarray(table_row, dtype=np.int64)[positions // page_size]
        per_key_scale = np.asarray(scale, dtype=np.float64)[pages]  # [length, Hkv]
        return decode_e4m3fn(raw, per_key_scale[:, :, None])
    return _decode(raw, dtype)


# ----------------------------------------------------------------------------
# Softmax attention over a visible key set
# ----------------------------------------------------------------------------

def attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, sm_scale: float):
    """Softmax attention of query rows over one key set, float64.

    ``q`` is ``[R, D]``, ``k`` and ``v`` are ``[L, D]``.  For each row:
    ``s = sm_scale * k @ q``, ``m = max s``, ``l = sum exp(s - m)``,
    ``o = sum exp(s - m) v / l`` and ``lse = m + ln l`` (natural log of
    ``sum exp(s)``).  An empty key set gives ``o = 0`` and ``lse = -inf``
    ([P5] small-batch split commit: an empty run has LSE -inf).
    Returns ``(o [R, D], lse [R])``.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n_rows, head_dim = q.shape
    if k.shape[0] == 0:
        return np.zeros((n_rows, v.shape[1] if v.ndim == 2 else head_dim)), np.full(n_rows, -np.inf)
    s = sm_scale * (q @ k.T)                      # [R, L]
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    o = (e @ v) / l
    lse = (m + np.log(l))[:, 0]
    return o, lse


# ----------------------------------------------------------------------------
# Paged decode  (one or several query rows per block-table row)
# ----------------------------------------------------------------------------

def attn_decode(k_pool, v_pool, q, tables, kv_lens, sm_scale, kv_dtype="bf16", q_dtype=None,
                k_scale=None, v_scale=None, tables_subset=None):
    """Paged decode attention.

    ``q`` is ``[T, n, Hq, D]`` raw storage (``q_dtype``, default the K/V dtype,
    or ``"bf16"`` for fp8 K/V): ``n`` query rows share the block-table row
    ``tables[t]`` and its length ``kv_lens[t]`` (n > 1 is the shared-prefix
    pass of an n-sample group, [P5] FA4 prefix/tail commits).  Query head h
    reads kv head ``h // (Hq // Hkv)``.  Keys are logical positions
    ``0 .. kv_lens[t]-1`` of the table row.

    Returns ``(out [T, n, Hq, D], lse [T, n, Hq])`` in float64.  Only the rows
    in ``tables_subset`` (all when None) are computed; the others stay NaN.
    """
    if q_dtype is None:
        q_dtype = "bf16" if kv_dtype == "fp8" else kv_dtype
    qf = _decode(q, q_dtype)
    n_t, n_rows, n_qh, head_dim = qf.shape
    n_kvh = k_pool.shape[2]
    group = n_qh // n_kvh
    out = np.full((n_t, n_rows, n_qh, head_dim), np.nan)
    lse = np.full((n_t, n_rows, n_qh), np.nan)
    todo = range(n_t) if tables_subset is None else tables_subset
    for t in todo:
        length = int(kv_lens[t])
        keys = _gather_real(k_pool, tables[t], length, kv_dtype, k_scale)
        vals = _gather_real(v_pool, tables[t], length, kv_dtype, v_scale)
        for h in range(n_qh):
            g = h // group
            o, s = attention_rows(qf[t, :, h, :], keys[:, g, :], vals[:, g, :], sm_scale)
            out[t, :, h, :] = o
            lse[t, :, h] = s
    return out, lse


# ----------------------------------------------------------------------------
# Block-causal paged prefill  [P1] Description / Cache and / Attention
# ----------------------------------------------------------------------------

def prefill_visible_keys(i: int, n_ctx: int, seq_len: int, causal_block_size: int) -> int:
    """Number of logical keys query ``i`` sees (0 for a padding row).

    The real tokens of a forward are cut into consecutive causal blocks of
    ``causal_block_size`` tokens (0: one block holding all real tokens).  A
    query sees every cached key (the pinned prefix and the history, ``n_ctx``
    of them) and the new tokens of its own block and all earlier blocks: full
    attention inside a block, causal across blocks, no mask otherwise.  Rows at
    or past ``seq_len`` are padding: neither attended nor attending.
    """
    if i >= seq_len:
        return 0
    cbs = seq_len if causal_block_size <= 0 else causal_block_size
    block = i // cbs
    return n_ctx + min((block + 1) * cbs, seq_len)


def attn_prefill_block_causal(k_pool, v_pool, q, tables, n_ctx, seq_len, causal_block_size, sm_scale,
                              kv_dtype="bf16", q_dtype=None, k_scale=None, v_scale=None, rows_subset=None):
    """Block-causal prefill over a paged pool.

    ``q`` is ``[B, S_q, Hq, D]`` raw storage.  Query row i of batch b attends
    the first ``prefill_visible_keys(i, n_ctx[b], seq_len[b], cbs)`` logical
    keys of ``tables[b]``; padding rows get ``o = 0`` and ``lse = -inf``.
    Returns ``(out [B, S_q, Hq, D], lse [B, S_q, Hq])`` float64.  When
    ``rows_subset`` (a list of (b, i)) is given only those rows are computed.
    """
    if q_dtype is None:
        q_dtype = "bf16" if kv_dtype == "fp8" else kv_dtype
    qf = _decode(q, q_dtype)
    n_b, s_q, n_qh, head_dim = qf.shape
    n_kvh = k_pool.shape[2]
    group = n_qh // n_kvh
    out = np.full((n_b, s_q, n_qh, head_dim), np.nan)
    lse = np.full((n_b, s_q, n_qh), np.nan)
    for b in range(n_b):
        wanted = range(s_q) if rows_subset is None else sorted(i for (bb, i) in rows_subset if bb == b)
        by_count: dict[int, list[int]] = {}
        for i in wanted:
            by_count.setdefault(prefill_visible_keys(i, int(n_ctx[b]), int(seq_len[b]), causal_block_size),
                                []).append(i)
        if not by_count:
            continue
        longest = max(by_count)
        keys = _gather_real(k_pool, tables[b], longest, kv_dtype, k_scale)
        vals = _gather_real(v_pool, tables[b], longest, kv_dtype, v_scale)
        for count, rows in by_count.items():
            rows = np.asarray(rows)
            if count == 0:
                out[b, rows] = 0.0
                lse[b, rows] = -np.inf
                continue
            for h in range(n_qh):
                g = h // group
                o, s = attention_rows(qf[b, rows, h, :], keys[:count, g, :], vals[:count, g, :], sm_scale)
                out[b, rows, h, :] = o
                lse[b, rows, h] = s
    return out, lse


# ----------------------------------------------------------------------------
# Attention-state merge  [P5] FA4 tail commit (natural-log LSE, one merge)
# ----------------------------------------------------------------------------

def merge_states(o_parts: np.ndarray, lse_parts: np.ndarray):
    """Join attention states computed over disjoint key sets.

    ``o_parts`` is ``[N, ..., D]`` (each normalised over its own key set) and
    ``lse_parts`` is ``[N, ...]`` (natural-log sum of exp scores).  With
    ``m = max_i lse_i`` and ``w_i = exp(lse_i - m)``: ``o = sum w_i o_i /
    sum w_i`` and ``lse = m + ln sum w_i``.  When every state is empty (all
    LSE -inf) the result is ``o = 0`` and ``lse = -inf``.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    m = lse_parts.max(axis=0)
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    w = np.exp(lse_parts - m_safe[None])           # exp(-inf) = 0 for empty parts
    w_sum = w.sum(axis=0)
    w_sum_safe = np.where(empty, 1.0, w_sum)
    # A weight of zero must not let a NaN/garbage partial of an empty state in.
    contrib = np.where((w > 0)[..., None], w[..., None] * o_parts, 0.0)
    o = contrib.sum(axis=0) / w_sum_safe[..., None]
    o = np.where(empty[..., None], 0.0, o)
    lse = np.where(empty, -np.inf, m_safe + np.log(w_sum_safe))
    return o, lse


# ----------------------------------------------------------------------------
# Exact-window commit operations  [P1] Description / Cache (eviction is an
# in-place rotation of the page table; commit fills the private pages with one
# pool-to-pool copy whose table carries sentinel entries)
# ----------------------------------------------------------------------------

def rotate_rows(rows: np.ndarray, shift: int) -> np.ndarray:
    """In-place rotation of every row of a 2-D array, returned as a new array.

    Element ``c`` of a row takes the old element ``(c + shift) mod cols``: the
    first ``shift`` entries (the oldest window pages) move to the end of the
    row.  Any integer shift is allowed (negative or larger than the row); rows
    of at most one element and empty arrays are unchanged.
    """
    rows = np.asarray(rows)
    out = rows.copy()
    n_rows, cols = rows.shape
    if n_rows == 0 or cols <= 1:
        return out
    s = shift % cols
    for r in range(n_rows):
        for c in range(cols):
            out[r, c] = rows[r, (c + s) % cols]
    return out


def copy_slots(pool: np.ndarray, src_slots, dst_slots) -> np.ndarray:
    """Pool-to-pool copy of whole key rows, returned as a new pool.

    ``pool`` is ``[layers, num_pages, page_size, H, D]`` raw storage (one of K
    or V).  Entry i copies slot ``src_slots[i]`` to slot ``dst_slots[i]`` in
    every layer (slot = page * page_size + row, all heads, all dims).  An
    entry with a negative source or destination is a sentinel and is skipped.
    Entries are applied in order, reading the pool as it was before the call
    (a destination that is another entry's source is not defined by the op;
    callers keep them disjoint).
    """
    pool = np.asarray(pool)
    out = pool.copy()
    layers, n_pages, page_size = pool.shape[:3]
    flat_in = pool.reshape(layers, n_pages * page_size, *pool.shape[3:])
    flat_out = out.reshape(layers, n_pages * page_size, *pool.shape[3:])
    for s, d in zip(np.asarray(src_slots).tolist(), np.asarray(dst_slots).tolist()):
        if s < 0 or d < 0:
            continue
        flat_out[:, d] = flat_in[:, s]
    return out
