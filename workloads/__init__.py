"""Seeded synthetic inputs for the paged K/V-cache path.

This package is shared by the tests, the benchmark and the smoke check; it
holds no attention, merge or scatter arithmetic.  It only lays out synthetic
scenarios: random N(0, 1) values stored as fp32 / bf16 / fp8 e4m3fn, page
permutations, block tables, sequence lengths, poison in every pool slot that no
sequence owns, and the pool slot where each newly written token belongs
(written with the slot-id convention ``page * page_size + row``).

Random numbers come from numpy's PCG64 with the seed given; value conversion
to bf16 / e4m3fn uses torch's CPU casts (round to nearest even).

The five named workloads follow the shapes of the paged-attention use cases
on the source pages (one video-generation causal block over a pinned prefix
and a rolling history; GQA decode; n-sample decode with a shared prompt; long
fp8 decode).
"""

from __future__ import annotations

import math
import os
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

STORAGE_NP = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}
# Poison patterns: quiet NaN in each storage type (0x7F is an e4m3fn NaN).
POISON = {"f32": np.float32(np.nan), "bf16": np.uint16(0x7FC0), "fp8": np.uint8(0x7F)}
E4M3FN_MAX = 448.0


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 values -> raw storage of ``dtype`` ("f32" or "bf16")."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    raise ValueError(dtype)


def quantize_e4m3fn(x: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """float32 values / scale -> e4m3fn codes (torch cast, round to nearest even)."""
    y = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)) / torch.from_numpy(
        np.ascontiguousarray(scale, dtype=np.float32))
    return y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _normal_pages(seed: int, n_pages: int, page_shape, chunk_elems: int = 1 << 22) -> np.ndarray:
    """N(0,1) float32 of shape [n_pages, *page_shape], drawn chunk by chunk.

    Each chunk of pages has its own child seed, so the values do not depend on
    how the work is spread over threads (numpy releases the GIL while drawing).
    """
    out = np.empty((n_pages, *page_shape), dtype=np.float32)
    per_page = int(np.prod(page_shape))
    chunk_pages = max(1, chunk_elems // max(per_page, 1))
    n_chunks = max(1, math.ceil(n_pages / chunk_pages))
    children = np.random.SeedSequence(seed).spawn(n_chunks)

    def fill(c):
        lo, hi = c * chunk_pages, min(n_pages, (c + 1) * chunk_pages)
        if lo < hi:
            out[lo:hi] = np.random.Generator(np.random.PCG64(children[c])).standard_normal(
                (hi - lo, *page_shape), dtype=np.float32)

    workers = min(16, n_chunks, len(os.sched_getaffinity(0)))
    if workers > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(fill, range(n_chunks)))
    else:
        for c in range(n_chunks):
            fill(c)
    return out


# ----------------------------------------------------------------------------
# Pools
# ----------------------------------------------------------------------------

@dataclass
class Pool:
    """K and V pools ``[num_pages, page_size, Hkv, D]`` in raw storage."""
    k: np.ndarray
    v: np.ndarray
    dtype: str
    k_scale: Optional[np.ndarray] = None   # [num_pages, Hkv] float32, fp8 only
    v_scale: Optional[np.ndarray] = None

    @property
    def num_pages(self):
        return self.k.shape[0]

    @property
    def page_size(self):
        return self.k.shape[1]

    @property
    def num_kv_heads(self):
        return self.k.shape[2]

    @property
    def head_dim(self):
        return self.k.shape[3]


def _fill_pool(seed, num_pages, page_size, n_kvh, head_dim, dtype, owned_pages, valid_rows):
    """Pool full of poison except rows ``< valid_rows[j]`` of page ``owned_pages[j]``.

    Valid rows hold N(0,1) data (K from ``seed``, V from ``seed + 1``); for fp8
    the scale of a (page, kv head) is the largest magnitude of its valid rows
    over 448 (1 for a page with no valid rows), so every code is finite.
    """
    shape = (num_pages, page_size, n_kvh, head_dim)
    owned_pages = np.asarray(owned_pages, dtype=np.int64)
    valid_rows = np.asarray(valid_rows, dtype=np.int64)
    row_ok = np.arange(page_size)[None, :] < valid_rows[:, None]          # [n_owned, ps]
    pools = []
    scales = []
    for which in range(2):
        vals = _normal_pages(seed + which, len(owned_pages), (page_size, n_kvh, head_dim))
        pool = np.full(shape, POISON[dtype], dtype=STORAGE_NP[dtype])
        if dtype == "fp8":
            ok_t = torch.from_numpy(row_ok)[:, :, None, None]
            mags = torch.where(ok_t, torch.from_numpy(vals).abs(), 0.0).amax(dim=(1, 3)).numpy()  # [n_owned, Hkv]
            sc_owned = np.where(mags > 0, mags / E4M3FN_MAX, 1.0).astype(np.float32)
            codes = quantize_e4m3fn(vals, sc_owned[:, None, :, None])
            codes = np.where(row_ok[:, :, None, None], codes, POISON["fp8"])
            pool[owned_pages] = codes
            scale = np.ones((num_pages, n_kvh), dtype=np.float32)
            scale[owned_pages] = sc_owned
            scales.append(scale)
        else:
            stored = to_storage(vals, dtype)
            pool[owned_pages] = np.where(row_ok[:, :, None, None], stored, POISON[dtype])
        pools.append(pool)
    if dtype == "fp8":
        return Pool(pools[0], pools[1], dtype, scales[0], scales[1])
    return Pool(pools[0], pools[1], dtype)


def _assign_pages(perm_seed, num_pool_pages, pages_per_seq):
    """Give each sequence its pages in the order of one random pool permutation.

    Returns (list of page arrays, poison page index, permutation)."""
    perm = np.random.Generator(np.random.PCG64(perm_seed)).permutation(num_pool_pages)
    need = int(np.sum(pages_per_seq)) + 1
    if need > num_pool_pages:
        raise ValueError(f"pool of {num_pool_pages} pages cannot hold {need}")
    out, at = [], 0
    for n in pages_per_seq:
        out.append(perm[at:at + n].astype(np.int32))
        at += n
    return out, int(perm[at]), perm


def _table(page_lists, width, poison_page):
    """Block table [rows, width]: each row's pages, then the poison page."""
    t = np.full((len(page_lists), width), poison_page, dtype=np.int32)
    for r, pages in enumerate(page_lists):
        t[r, :len(pages)] = pages
    return t


def _slot(table_row, position, page_size):
    """Pool slot id of a logical position: ``page * page_size + row``."""
    return int(table_row[position // page_size]) * page_size + position % page_size


# ----------------------------------------------------------------------------
# Decode
# ----------------------------------------------------------------------------

@dataclass
class DecodeCase:
    name: str
    pool: Pool                  # state BEFORE the new tokens are scattered
    q: np.ndarray               # [T, n, Hq, D] raw storage (q_dtype)
    q_dtype: str
    tables: np.ndarray          # int32 [T, width]
    kv_lens: np.ndarray         # int32 [T]
    rows_per_table: int
    num_q_heads: int
    sm_scale: float
    new_k: Optional[np.ndarray] = None   # [n_new, Hkv, D] raw storage
    new_v: Optional[np.ndarray] = None
    slots: Optional[np.ndarray] = None   # int64 [n_new]
    poison_page: int = -1
    meta: dict = field(default_factory=dict)

    @property
    def max_kv_len(self):
        return int(self.kv_lens.max()) if len(self.kv_lens) else 0


def make_decode_case(name, seed, perm_seed, num_tables, num_q_heads, num_kv_heads, head_dim, page_size,
                     kv_lens, num_pool_pages=None, kv_dtype="bf16", q_dtype=None, rows_per_table=1,
                     new_per_seq=1, table_width=None, extra_table_cols=0):
    """A decode batch over a permuted paged pool.

    Sequence t holds ``kv_lens[t]`` logical keys; its last ``new_per_seq`` keys
    are the step's new tokens: their pool slots hold poison until they are
    scattered from ``new_k`` / ``new_v`` at ``slots``.  Dead rows of a last
    page, unowned pages and table entries past a row's last page (which point
    at the poison page) are all NaN.
    """
    if q_dtype is None:
        q_dtype = "bf16" if kv_dtype == "fp8" else kv_dtype
    kv_lens = np.asarray(kv_lens, dtype=np.int32)
    pages_per_seq = [math.ceil(int(L) / page_size) for L in kv_lens]
    if num_pool_pages is None:
        num_pool_pages = int(sum(pages_per_seq)) + 1
    page_lists, poison_page, _ = _assign_pages(perm_seed, num_pool_pages, pages_per_seq)
    width = table_width or (max(pages_per_seq + [1]) + extra_table_cols)
    tables = _table(page_lists, width, poison_page)

    owned = np.concatenate(page_lists) if page_lists else np.zeros(0, np.int32)
    valid = []
    for L, pages in zip(kv_lens, page_lists):
        for j in range(len(pages)):
            valid.append(min(page_size, int(L) - j * page_size))
    pool = _fill_pool(seed, num_pool_pages, page_size, num_kv_heads, head_dim, kv_dtype, owned, valid)

    new_k = new_v = slots = None
    if new_per_seq > 0 and kv_dtype != "fp8":
        slot_list = []
        for t, L in enumerate(kv_lens):
            for p in range(max(0, int(L) - new_per_seq), int(L)):
                slot_list.append(_slot(tables[t], p, page_size))
        slots = np.asarray(slot_list, dtype=np.int64)
        flat_k = pool.k.reshape(-1, num_kv_heads, head_dim)
        flat_v = pool.v.reshape(-1, num_kv_heads, head_dim)
        new_k = flat_k[slots].copy()
        new_v = flat_v[slots].copy()
        flat_k[slots] = POISON[kv_dtype]
        flat_v[slots] = POISON[kv_dtype]

    rng = np.random.Generator(np.random.PCG64(seed + 7))
    qf = rng.standard_normal((len(kv_lens), rows_per_table, num_q_heads, head_dim), dtype=np.float32)
    q = to_storage(qf, q_dtype)
    return DecodeCase(name, pool, q, q_dtype, tables, kv_lens, rows_per_table, num_q_heads,
                      1.0 / math.sqrt(head_dim), new_k, new_v, slots, poison_page)


def tiny_fp32_decode(seed=1):
    """Tiny fp32 decode: 2 sequences of 256 keys (254 resident + 2 new), 4/4
    heads of 64, 32-token pages, a 32-page pool randomly permuted."""
    return make_decode_case("tiny_fp32_decode", seed, 1000 + seed, 2, 4, 4, 64, 32, [256, 256],
                            num_pool_pages=32, kv_dtype="f32", new_per_seq=2, extra_table_cols=2)


def gqa_bf16_decode(seed=2, batch=64, len_range=(512, 4096), num_pool_pages=16384):
    """bf16 GQA decode: 64 sequences, lengths uniform in [512, 4096], 32 q /
    8 kv heads of 128, 32-token pages shuffled across a 16k-page pool, one new
    token per sequence scattered before attention."""
    lens = np.random.Generator(np.random.PCG64(seed + 100)).integers(
        len_range[0], len_range[1], size=batch, endpoint=True)
    return make_decode_case("bf16_gqa_decode", seed, 1000 + seed, batch, 32, 8, 128, 32, lens,
                            num_pool_pages=num_pool_pages, kv_dtype="bf16", new_per_seq=1)


def long_fp8_decode(seed=5, batch=256, len_range=(1024, 32768)):
    """Large fp8 decode: 256 sequences, lengths log-uniform in [1024, 32768],
    64 q / 8 kv heads of 128, e4m3fn K/V with a float scale per (page, kv
    head), bf16 queries and outputs, pages randomly permuted."""
    u = np.random.Generator(np.random.PCG64(seed + 100)).uniform(
        math.log(len_range[0]), math.log(len_range[1]), size=batch)
    lens = np.rint(np.exp(u)).astype(np.int64)
    return make_decode_case("fp8_long_decode", seed, 1000 + seed, batch, 64, 8, 128, 32, lens,
                            kv_dtype="fp8", q_dtype="bf16", new_per_seq=0)


# ----------------------------------------------------------------------------
# Shared-prefix n-sample decode
# ----------------------------------------------------------------------------

@dataclass
class SharedPrefixCase:
    name: str
    pool: Pool                     # state before the new tokens are scattered
    q: np.ndarray                  # [groups * n, 1, Hq, D] bf16 bits (= [groups, n, Hq, D])
    num_groups: int
    samples: int
    num_q_heads: int
    sm_scale: float
    prefix_tables: np.ndarray      # [groups, prefix_pages]
    prefix_lens: np.ndarray        # [groups]
    tail_tables: np.ndarray        # [groups * n, tail_width]
    tail_lens: np.ndarray          # [groups * n]
    full_tables: np.ndarray        # [groups * n, prefix_pages + tail_width]
    full_lens: np.ndarray
    new_k: np.ndarray
    new_v: np.ndarray
    slots: np.ndarray
    poison_page: int


def make_shared_prefix_case(name, seed, perm_seed, groups, samples, prefix_len, tail_range, num_q_heads,
                            num_kv_heads, head_dim, page_size, num_pool_pages):
    """n-sample decode: each group of ``samples`` rows shares ``prefix_len``
    keys (whole pages, held once in the pool) and each row owns a private tail
    of uniform length in ``tail_range`` on fresh pages.  The last tail token of
    each row is the step's new token."""
    if prefix_len % page_size:
        raise ValueError("the shared prefix must be whole pages")
    rng = np.random.Generator(np.random.PCG64(seed + 100))
    n_rows = groups * samples
    tails = rng.integers(tail_range[0], tail_range[1], size=n_rows, endpoint=True)
    prefix_pages = prefix_len // page_size
    tail_pages = [math.ceil(int(t) / page_size) for t in tails]
    page_lists, poison_page, _ = _assign_pages(perm_seed, num_pool_pages, [prefix_pages] * groups + tail_pages)
    prefix_lists, tail_lists = page_lists[:groups], page_lists[groups:]
    tail_width = math.ceil(tail_range[1] / page_size)
    prefix_tables = _table(prefix_lists, prefix_pages, poison_page)
    tail_tables = _table(tail_lists, tail_width, poison_page)
    full_lists = [np.concatenate([prefix_lists[r // samples], tail_lists[r]]) for r in range(n_rows)]
    full_tables = _table(full_lists, prefix_pages + tail_width, poison_page)

    owned = np.concatenate(page_lists)
    valid = [page_size] * (groups * prefix_pages)
    for t, pages in zip(tails, tail_lists):
        valid += [min(page_size, int(t) - j * page_size) for j in range(len(pages))]
    pool = _fill_pool(seed, num_pool_pages, page_size, num_kv_heads, head_dim, "bf16", owned, valid)

    slots = np.asarray([_slot(tail_tables[r], int(tails[r]) - 1, page_size) for r in range(n_rows)], np.int64)
    flat_k = pool.k.reshape(-1, num_kv_heads, head_dim)
    flat_v = pool.v.reshape(-1, num_kv_heads, head_dim)
    new_k, new_v = flat_k[slots].copy(), flat_v[slots].copy()
    flat_k[slots] = POISON["bf16"]
    flat_v[slots] = POISON["bf16"]

    qf = np.random.Generator(np.random.PCG64(seed + 7)).standard_normal(
        (n_rows, 1, num_q_heads, head_dim), dtype=np.float32)
    return SharedPrefixCase(name, pool, to_storage(qf, "bf16"), groups, samples, num_q_heads,
                            1.0 / math.sqrt(head_dim), prefix_tables,
                            np.full(groups, prefix_len, np.int32), tail_tables, tails.astype(np.int32),
                            full_tables, (tails + prefix_len).astype(np.int32), new_k, new_v, slots, poison_page)


def shared_prefix_decode(seed=4, groups=8, samples=16, prefix_len=2048, tail_range=(1, 512), num_pool_pages=4096):
    """Shared-prefix n-sample decode: 8 prompts x 16 samples, 2048 shared
    prefix tokens per prompt, private tails uniform in [1, 512], 32 q / 8 kv
    heads of 128, bf16, 32-token pages in a 4096-page pool."""
    return make_shared_prefix_case("shared_prefix_decode", seed, 1000 + seed, groups, samples, prefix_len,
                                   tail_range, 32, 8, 128, 32, num_pool_pages)


# ----------------------------------------------------------------------------
# Block-causal prefill
# ----------------------------------------------------------------------------

@dataclass
class PrefillCase:
    name: str
    pool: Pool                 # before the current block is scattered
    qkv: np.ndarray            # [B, S_q, Hq + 2 Hkv, D] raw (packed projection)
    num_q_heads: int
    num_kv_heads: int
    tables: np.ndarray         # [B, width]
    n_ctx: np.ndarray          # [B] cached keys (pinned prefix + history)
    seq_len: np.ndarray        # [B] real query tokens (<= S_q)
    causal_block_size: int
    sm_scale: float
    slots: np.ndarray          # [B * S_q] int64: slot of real token, -1 for padding
    poison_page: int

    @property
    def s_q(self):
        return self.qkv.shape[1]

    @property
    def q(self):
        return self.qkv[:, :, :self.num_q_heads]

    @property
    def new_k(self):
        return self.qkv[:, :, self.num_q_heads:self.num_q_heads + self.num_kv_heads]

    @property
    def new_v(self):
        return self.qkv[:, :, self.num_q_heads + self.num_kv_heads:]

    @property
    def max_keys(self):
        return int((self.n_ctx + self.seq_len).max())


def make_prefill_case(name, seed, perm_seed, batch, s_q, seq_lens, n_ctxs, num_q_heads, num_kv_heads,
                      head_dim, page_size, causal_block_size, num_pool_pages=None, kv_dtype="bf16",
                      extra_table_cols=1):
    """Prefill over a cache: batch b holds ``n_ctx[b]`` cached keys (pinned
    prefix + history) and writes its ``seq_len[b]`` real tokens right after
    them; rows ``seq_len[b] .. s_q-1`` of the packed projection are padding
    (random values, never written, never attended).  Dead rows of the last
    page are poison."""
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    n_ctxs = np.asarray(n_ctxs, dtype=np.int64)
    totals = n_ctxs + seq_lens
    pages_per_seq = [math.ceil(int(t) / page_size) for t in totals]
    if num_pool_pages is None:
        num_pool_pages = int(sum(pages_per_seq)) + 1
    page_lists, poison_page, _ = _assign_pages(perm_seed, num_pool_pages, pages_per_seq)
    tables = _table(page_lists, max(pages_per_seq) + extra_table_cols, poison_page)
    owned = np.concatenate(page_lists)
    valid = []
    for c, pages in zip(n_ctxs, page_lists):
        # only the cached keys are resident; the current block's rows are poison until scattered
        valid += [max(0, min(page_size, int(c) - j * page_size)) for j in range(len(pages))]
    pool = _fill_pool(seed, num_pool_pages, page_size, num_kv_heads, head_dim, kv_dtype, owned, valid)

    rng = np.random.Generator(np.random.PCG64(seed + 7))
    qkv_f = rng.standard_normal((batch, s_q, num_q_heads + 2 * num_kv_heads, head_dim), dtype=np.float32)
    qkv = to_storage(qkv_f, kv_dtype)
    slots = np.full(batch * s_q, -1, dtype=np.int64)
    for b in range(batch):
        for i in range(int(seq_lens[b])):
            slots[b * s_q + i] = _slot(tables[b], int(n_ctxs[b]) + i, page_size)
    return PrefillCase(name, pool, qkv, num_q_heads, num_kv_heads, tables, n_ctxs.astype(np.int32),
                       seq_lens.astype(np.int32), causal_block_size, 1.0 / math.sqrt(head_dim), slots,
                       poison_page)


def make_fp8_prefill_case(name, seed, perm_seed, batch, s_q, seq_lens, n_ctxs, num_q_heads, num_kv_heads,
                          head_dim, page_size, causal_block_size, num_pool_pages=None, extra_table_cols=1,
                          zero_scale_pages=0, q_outlier=1.0):
    """Prefill over an fp8 e4m3fn K/V pool: every key, the current block's
    included, is resident (quantised with a scale per (page, kv head)); Q is
    bf16, rows ``seq_len[b] ..`` are padding; dead rows of the last page are
    NaN codes.  ``zero_scale_pages`` owned pages get K and V scales of 0.
    ``q_outlier`` multiplies one dim of every Q row (dim = row % head_dim), so
    the rest of the row is small next to the row's largest entry."""
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    n_ctxs = np.asarray(n_ctxs, dtype=np.int64)
    totals = n_ctxs + seq_lens
    pages_per_seq = [math.ceil(int(t) / page_size) for t in totals]
    if num_pool_pages is None:
        num_pool_pages = int(sum(pages_per_seq)) + 1
    page_lists, poison_page, _ = _assign_pages(perm_seed, num_pool_pages, pages_per_seq)
    tables = _table(page_lists, max(pages_per_seq) + extra_table_cols, poison_page)
    owned = np.concatenate(page_lists)
    valid = []
    for t, pages in zip(totals, page_lists):
        valid += [max(0, min(page_size, int(t) - j * page_size)) for j in range(len(pages))]
    pool = _fill_pool(seed, num_pool_pages, page_size, num_kv_heads, head_dim, "fp8", owned, valid)
    if zero_scale_pages:
        pick = np.random.Generator(np.random.PCG64(seed + 11)).choice(owned, zero_scale_pages, replace=False)
        pool.k_scale[pick] = 0.0
        pool.v_scale[pick] = 0.0
    rng = np.random.Generator(np.random.PCG64(seed + 7))
    qkv_f = rng.standard_normal((batch, s_q, num_q_heads + 2 * num_kv_heads, head_dim), dtype=np.float32)
    if q_outlier != 1.0:
        rows = np.arange(s_q)
        qkv_f[:, rows, :num_q_heads, rows % head_dim] *= np.float32(q_outlier)
    slots = np.full(batch * s_q, -1, dtype=np.int64)
    return PrefillCase(name, pool, to_storage(qkv_f, "bf16"), num_q_heads, num_kv_heads, tables,
                       n_ctxs.astype(np.int32), seq_lens.astype(np.int32), causal_block_size,
                       1.0 / math.sqrt(head_dim), slots, poison_page)


def block_causal_prefill(seed=3, causal_block_size=1560):
    """bf16 block-causal prefill (video-generation style): 24 heads of 128,
    32-token pages, pinned prefix 1024 + rolling history 4096 + a current block
    of 1560 real queries padded to 1568 rows; every query sees the prefix, the
    history and its whole block; the last page is 24/32 full; 512-page pool."""
    return make_prefill_case("bf16_block_causal_prefill", seed, 1000 + seed, 1, 1568, [1560], [1024 + 4096],
                             24, 24, 128, 32, causal_block_size, num_pool_pages=512)


@dataclass
class SharedStepCase:
    name: str
    pool: Pool
    q: np.ndarray                # [groups * samples, q_len, Hq, D] bf16 bits
    samples: int
    num_q_heads: int
    sm_scale: float
    prefix_tables: np.ndarray    # [groups, width] int32
    prefix_lens: np.ndarray      # [groups] int32
    tail_tables: np.ndarray      # [groups * samples, width] int32
    tail_lens: np.ndarray        # [groups * samples] int32
    new_k: Optional[np.ndarray]  # the step's tokens, scattered before attention (bf16 pools)
    new_v: Optional[np.ndarray]
    slots: Optional[np.ndarray]

    @property
    def q_len(self):
        return self.q.shape[1]


def make_shared_step_case(name, seed, perm_seed, groups, samples, q_len, prefix_lens, tail_lens, num_q_heads,
                          num_kv_heads, head_dim, page_size, kv_dtype="bf16", extra_cols=1):
    """n-sample decode step over a permuted pool: group g's shared prefix of
    ``prefix_lens[g]`` keys and each sample's private tail of ``tail_lens[r]``
    keys sit on pages of their own (the tails on fresh pages); the step's
    ``q_len`` tokens are the tail's last keys.  bf16 pools: those tokens are
    poison until scattered from ``new_k`` / ``new_v`` at ``slots``; fp8 pools:
    every key is resident.  Dead rows, unowned pages and table padding are
    poison."""
    prefix_lens = np.asarray(prefix_lens, dtype=np.int32)
    tail_lens = np.asarray(tail_lens, dtype=np.int32)
    n_rows = groups * samples
    p_pages = [math.ceil(int(x) / page_size) for x in prefix_lens]
    t_pages = [math.ceil(int(x) / page_size) for x in tail_lens]
    num_pool_pages = sum(p_pages) + sum(t_pages) + 3
    page_lists, poison_page, _ = _assign_pages(perm_seed, num_pool_pages, p_pages + t_pages)
    prefix_tables = _table(page_lists[:groups], max(p_pages + [1]) + extra_cols, poison_page)
    tail_tables = _table(page_lists[groups:], max(t_pages + [1]) + extra_cols, poison_page)
    owned = np.concatenate([pl for pl in page_lists if len(pl)])
    valid = []
    for L, pages in zip(list(prefix_lens) + list(tail_lens), page_lists):
        valid += [min(page_size, int(L) - j * page_size) for j in range(len(pages))]
    pool = _fill_pool(seed, num_pool_pages, page_size, num_kv_heads, head_dim, kv_dtype, owned, valid)
    new_k = new_v = slots = None
    if kv_dtype != "fp8":
        slot_list = [_slot(tail_tables[r], p, page_size)
                     for r in range(n_rows) for p in range(max(0, int(tail_lens[r]) - q_len), int(tail_lens[r]))]
        slots = np.asarray(slot_list, dtype=np.int64)
        flat_k = pool.k.reshape(-1, num_kv_heads, head_dim)
        flat_v = pool.v.reshape(-1, num_kv_heads, head_dim)
        new_k, new_v = flat_k[slots].copy(), flat_v[slots].copy()
        flat_k[slots] = POISON[kv_dtype]
        flat_v[slots] = POISON[kv_dtype]
    qf = np.random.Generator(np.random.PCG64(seed + 7)).standard_normal(
        (n_rows, q_len, num_q_heads, head_dim), dtype=np.float32)
    return SharedStepCase(name, pool, to_storage(qf, "bf16"), samples, num_q_heads, 1.0 / math.sqrt(head_dim),
                          prefix_tables, prefix_lens, tail_tables, tail_lens, new_k, new_v, slots)
