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


def attn_decode_step(k_pool, v_pool, q, tables, kv_lens, sm_scale, kv_dtype="bf16", q_dtype=None,
                     k_scale=None, v_scale=None):
    """Paged decode of a multi-token step ([P5] n-sample commit with CUDA
    graphs: up to 16 query tokens per row, the K draft tokens + 1 of a
    verification step; FA4 tail commit: the step's K/V is in the row's pages
    and is attended causally).

    ``q`` is ``[T, n, Hq, D]``: the n tokens of row t are its last n keys, so
    token j attends logical keys ``0 .. kv_lens[t] - (n - 1 - j) - 1`` (none,
    giving ``o = 0`` and ``lse = -inf``, when that count is not positive).
    Returns ``(out [T, n, Hq, D], lse [T, n, Hq])`` in float64.
    """
    if q_dtype is None:
        q_dtype = "bf16" if kv_dtype == "fp8" else kv_dtype
    qf = _decode(q, q_dtype)
    n_t, n_rows, n_qh, head_dim = qf.shape
    group = n_qh // k_pool.shape[2]
    out = np.full((n_t, n_rows, n_qh, head_dim), np.nan)
    lse = np.full((n_t, n_rows, n_qh), np.nan)
    for t in range(n_t):
        length = int(kv_lens[t])
        keys = _gather_real(k_pool, tables[t], length, kv_dtype, k_scale)
        vals = _gather_real(v_pool, tables[t], length, kv_dtype, v_scale)
        for j in range(n_rows):
            seen = max(0, length - (n_rows - 1 - j))
            for h in range(n_qh):
                o, s_ = attention_rows(qf[t, j:j + 1, h, :], keys[:seen, h // group, :], vals[:seen, h // group, :],
                                       sm_scale)
                out[t, j, h, :] = o[0]
                lse[t, j, h] = s_[0]
    return out, lse


def attn_decode_shared_prefix(k_pool, v_pool, q, samples, prefix_tables, prefix_lens, tail_tables, tail_lens,
                              sm_scale, kv_dtype="bf16", q_dtype=None, k_scale=None, v_scale=None):
    """One n-sample decode step ([P5] n-sample commits: a group's shared
    pages are read once and merged with each row's private tail, for up to 16
    query tokens per row; FA4 tail commit: the step's tokens are attended
    causally in the tail).

    ``q`` is ``[G * samples, n, Hq, D]``; token j of sample r attends the
    ``prefix_lens[r // samples]`` keys of its group's prefix table followed by
    the first ``tail_lens[r] - (n - 1 - j)`` keys of its tail table.
    Returns ``(out [G * samples, n, Hq, D], lse [G * samples, n, Hq])`` float64.
    """
    if q_dtype is None:
        q_dtype = "bf16" if kv_dtype == "fp8" else kv_dtype
    qf = _decode(q, q_dtype)
    n_r, n_tok, n_qh, head_dim = qf.shape
    group = n_qh // k_pool.shape[2]
    out = np.full((n_r, n_tok, n_qh, head_dim), np.nan)
    lse = np.full((n_r, n_tok, n_qh), np.nan)
    for r in range(n_r):
        g = r // samples
        pk = _gather_real(k_pool, prefix_tables[g], int(prefix_lens[g]), kv_dtype, k_scale)
        pv = _gather_real(v_pool, prefix_tables[g], int(prefix_lens[g]), kv_dtype, v_scale)
        tk = _gather_real(k_pool, tail_tables[r], int(tail_lens[r]), kv_dtype, k_scale)
        tv = _gather_real(v_pool, tail_tables[r], int(tail_lens[r]), kv_dtype, v_scale)
        for j in range(n_tok):
            seen = max(0, int(tail_lens[r]) - (n_tok - 1 - j))
            keys = np.concatenate([pk, tk[:seen]])
            vals = np.concatenate([pv, tv[:seen]])
            for h in range(n_qh):
                o, s_ = attention_rows(qf[r, j:j + 1, h, :], keys[:, h // group, :], vals[:, h // group, :],
                                       sm_scale)
                out[r, j, h, :] = o[0]
                lse[r, j, h] = s_[0]
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


# ----------------------------------------------------------------------------
# Exact-window layout  [P1] Description / Cache (the sequence is [fixed region |
# rolling history window | staged tokens]; a table row can start a key sequence
# only at a page boundary, so every causal block gets private pages at the end
# of its row holding the visible keys of the partly visible pages, then the
# block's own tokens, which stay the last keys of the row) and the review thread
# on the private-page regions (committed_private is copied at commit,
# current_private every forward; bounds 3 (page_size - 1) and 2 (page_size - 1)).
#
# Readings (the pages give the regions, not formulas):
# * a causal block whose first key is at logical position s sees the fixed
#   region [0, pin), the ``window`` positions just before s, and itself;
# * the fixed region owns ceil(pin / page_size) pages; the rolling region
#   (positions >= pin) starts on a page of its own, so rolling position x sits
#   at offset (x - pin) of the rolling pages, of which the first ``evicted``
#   tokens' pages have been rotated out;
# * the table row of the sequence is [fixed pages | rolling pages], entry
#   F + j holding rolling page (evicted / page_size + j);
# * a block's row is its fully visible pages (all keys visible and before the
#   block), in logical order, then private pages that hold, packed in logical
#   order, every other visible key before the block and then the block's own
#   keys; a block with no such keys whose first key starts a rolling page reads
#   its own keys from their own pages instead and needs no private copy.
# ----------------------------------------------------------------------------

def window_evicted_tokens(page_size: int, pin: int, window: int, committed: int) -> int:
    """Rolling tokens before the first page any later block can see.

    After ``committed`` tokens, the next block starts at ``committed`` and its
    window at max(pin, committed - window); whole rolling pages before that
    start are never read again.
    """
    first_needed = max(0, committed - window - pin)
    return (first_needed // page_size) * page_size


def visible_keys(start: int, end: int, pin: int, window: int) -> list:
    """Logical positions a causal block [start, end) attends to, ascending."""
    window_start = max(pin, start - window)
    return [x for x in range(end) if x < pin or x >= window_start]


def causal_layout_bounds(page_size: int, pin: int, window: int, block_sizes) -> dict:
    """Sizes a geometry needs: fixed and rolling table pages, private pages per
    block, per-block row width and piece-list capacity per block."""
    ps = page_size
    total = int(sum(block_sizes))
    biggest = int(max(block_sizes)) if len(block_sizes) else 0
    pieces = 3 * (ps - 1)
    return {
        "fixed_pages": -(-pin // ps),
        "rolling_pages": -(-(window + ps - 1 + total) // ps),
        "private_pages": -(-(pieces + biggest) // ps),
        "table_width": pin // ps + window // ps + -(-(pieces + biggest) // ps),
        "list_stride": pieces,
    }


def causal_layout(table, private_pages, page_size: int, pin: int, window: int, committed: int,
                  evicted: int, block_sizes, table_width: int, list_stride: int) -> dict:
    """Per-block rows and slot lists for exact-window block-causal attention.

    table          page ids of the sequence, [fixed pages | rolling pages].
    private_pages  [num_blocks, P] page ids owned by each block.
    committed      tokens already history (C); staged token t is position C + t.
    evicted        rolling tokens rotated out of the table (multiple of
                   page_size, at most window_evicted_tokens(...)).
    block_sizes    staged tokens of each causal block, in order.

    Returns int32 ``block_tables`` [nb, table_width] (unused entries -1),
    ``n_ctx`` [nb] (keys before the block's own tokens) and ``seq_len`` [nb];
    int64 ``stage_slots`` / ``stage_slots2`` [T] (the staged token's own slot
    and its copy in its block's private pages, -1 if none); and int64
    ``commit_src`` / ``commit_dst`` and ``current_src`` / ``current_dst``
    [nb * list_stride] (block b's entries at b * list_stride, padded with -1):
    copies of committed keys, made at commit, and of earlier blocks' staged
    keys, made after every forward's scatter.
    """
    ps = int(page_size)
    if ps < 1 or ps & (ps - 1):
        raise ValueError("page_size must be a power of two")
    if min(pin, window, committed, evicted) < 0 or evicted % ps:
        raise ValueError("negative size or unaligned eviction")
    if evicted > window_evicted_tokens(ps, pin, window, committed):
        raise ValueError("eviction reaches into the next block's window")
    table = [int(t) for t in np.asarray(table).reshape(-1)]
    private_pages = np.asarray(private_pages).reshape(len(block_sizes), -1)
    n_fixed = -(-pin // ps)
    n_roll = len(table) - n_fixed
    total = int(sum(block_sizes))
    last = committed + total - 1
    if n_roll < 0 or (last >= pin and (last - pin - evicted) // ps >= n_roll):
        raise ValueError("table too short for the staged tokens")

    def slot_of(x):
        if x < pin:
            return table[x // ps] * ps + x % ps
        r = x - pin - evicted
        return table[n_fixed + r // ps] * ps + r % ps

    # Every page of the table with the logical positions it holds.
    pages = []
    for p in range(n_fixed):
        pages.append((table[p], list(range(p * ps, min((p + 1) * ps, pin)))))
    for j in range(n_roll):
        q = evicted // ps + j
        pages.append((table[n_fixed + j], list(range(pin + q * ps, pin + (q + 1) * ps))))

    nb = len(block_sizes)
    out = {
        "block_tables": np.full((nb, table_width), -1, np.int32),
        "n_ctx": np.zeros(nb, np.int32),
        "seq_len": np.asarray(block_sizes, np.int32).copy(),
        "stage_slots": np.zeros(total, np.int64),
        "stage_slots2": np.full(total, -1, np.int64),
    }
    for name in ("commit_src", "commit_dst", "current_src", "current_dst"):
        out[name] = np.full(nb * list_stride, -1, np.int64)

    start = committed
    for b, size in enumerate(block_sizes):
        end = start + int(size)
        seen = set(visible_keys(start, end, pin, window))
        full = [pid for pid, pos in pages
                if len(pos) == ps and all(x in seen and x < start for x in pos)]
        on_full = {x for pid, pos in pages if pid in full for x in pos}
        pieces = [x for x in sorted(seen) if x < start and x not in on_full]
        direct = not pieces and start >= pin and (start - pin) % ps == 0
        if direct:
            own_pages = [pid for pid, pos in pages if pos and start <= pos[0] < end]
            row = full + own_pages
        else:
            n_priv = -(-(len(pieces) + int(size)) // ps)
            if n_priv > private_pages.shape[1]:
                raise ValueError("too few private pages")
            row = full + [int(p) for p in private_pages[b, :n_priv]]
        if len(row) > table_width:
            raise ValueError("table_width too small")
        out["block_tables"][b, :len(row)] = row
        out["n_ctx"][b] = len(full) * ps + len(pieces)

        def private_slot(k):
            return int(private_pages[b, k // ps]) * ps + k % ps

        committed_pieces = [(k, x) for k, x in enumerate(pieces) if x < committed]
        current_pieces = [(k, x) for k, x in enumerate(pieces) if x >= committed]
        for lists, chosen in ((("commit_src", "commit_dst"), committed_pieces),
                              (("current_src", "current_dst"), current_pieces)):
            if len(chosen) > list_stride:
                raise ValueError("list_stride too small")
            for i, (k, x) in enumerate(chosen):
                out[lists[0]][b * list_stride + i] = slot_of(x)
                out[lists[1]][b * list_stride + i] = private_slot(k)
        for i in range(int(size)):
            t = start - committed + i
            out["stage_slots"][t] = slot_of(start + i)
            if not direct:
                out["stage_slots2"][t] = private_slot(len(pieces) + i)
        start = end
    return out
