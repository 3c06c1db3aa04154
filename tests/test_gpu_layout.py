"""GPU parity of the exact-window layout, and the exact window end to end.

The layout kernel is compared bit-exactly with the oracle (every output,
padding included).  The end-to-end rollouts drive a poisoned pool only
through the library: each commit rotates the rolling part of the page table,
lays out the causal blocks and fills their private pages; each forward
scatters the staged tokens, copies earlier blocks' keys and runs the
block-causal prefill over the per-block rows.  Every forward is compared with
float64 attention over each block's visible keys (fixed region, window,
itself), and a zero-query, one-hot-V forward shows the visible key set
exactly."""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as orc
import paged_kv_cache_slots_amd as pkv
from gpu_util import DEV, as_f64, assert_close, from_dev, note, to_dev
from workloads import POISON, to_storage

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
KEYS = ("block_tables", "n_ctx", "seq_len", "stage_slots", "stage_slots2",
        "commit_src", "commit_dst", "current_src", "current_dst")


def _layout(table, priv, ps, pin, window, committed, evicted, sizes, width=None, list_stride=None):
    lay = pkv.CausalLayout(ps, pin, window, sizes, device=DEV)
    if width is not None:      # caller-sized (larger) buffers
        lay.block_tables = torch.empty((len(sizes), width), dtype=torch.int32, device=DEV)
    if list_stride is not None:
        lay.bounds = dict(lay.bounds, list_stride=list_stride)
        for name in ("commit_src", "commit_dst", "current_src", "current_dst"):
            setattr(lay, name, torch.empty(len(sizes) * list_stride, dtype=torch.int64, device=DEV))
    for name in KEYS:          # poison: every entry must be written
        getattr(lay, name).fill_(12345)
    t = torch.tensor(np.asarray(table, np.int32), device=DEV)
    p = torch.tensor(np.asarray(priv, np.int32), device=DEV)
    pkv.pkv_causal_layout(lay, t, p, committed, evicted)
    torch.cuda.synchronize()
    return lay


def _compare(lay, want):
    for name in KEYS:
        got = getattr(lay, name).cpu().numpy()
        exp = np.asarray(want[name]).reshape(got.shape)
        assert np.array_equal(got, exp), f"{name}: {got.tolist()} != {exp.tolist()}"


def _cases():
    with open(os.path.join(GOLDEN, "causal_layout.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_layout_hand_worked_fixtures(case):
    note(f"causal_layout fixture {case['name']}")
    lay = _layout(case["table"], case["private_pages"], case["page_size"], case["pin"], case["window"],
                  case["committed"], case["evicted"], case["block_sizes"])
    _compare(lay, case)


def _random_geometry(rng, max_blocks=6):
    ps = int(2 ** rng.integers(0, 7))
    pin = int(rng.integers(0, 5 * ps + 3))
    window = int(rng.integers(0, 8 * ps + 3))
    sizes = [int(v) for v in rng.integers(1, 3 * ps + 3, size=int(rng.integers(1, max_blocks + 1)))]
    committed = int(rng.integers(0, pin + window + 12 * ps))
    evicted = orc.window_evicted_tokens(ps, pin, window, committed)
    if rng.random() < 0.3:
        evicted = int(rng.integers(0, evicted // ps + 1)) * ps
    bounds = orc.causal_layout_bounds(ps, pin, window, sizes)
    last = committed + sum(sizes) - 1
    n_roll = 0 if last < pin else (last - pin - evicted) // ps + 1       # as few rolling pages as allowed
    n_tab = bounds["fixed_pages"] + n_roll
    ids = rng.permutation(n_tab + len(sizes) * bounds["private_pages"] + 3).astype(np.int32)
    table = ids[:n_tab]
    priv = ids[n_tab:n_tab + len(sizes) * bounds["private_pages"]].reshape(len(sizes), -1)
    return ps, pin, window, sizes, committed, evicted, table, priv, bounds


@pytest.mark.parametrize("seed", range(8))
def test_layout_matches_oracle_random_geometries(seed):
    rng = np.random.default_rng(100 + seed)
    for i in range(25):
        ps, pin, window, sizes, committed, evicted, table, priv, b = _random_geometry(rng)
        note(f"causal_layout seed={seed} i={i} ps={ps} pin={pin} window={window} sizes={sizes} "
             f"committed={committed} evicted={evicted}")
        lay = _layout(table, priv, ps, pin, window, committed, evicted, sizes)
        _compare(lay, orc.causal_layout(table, priv, ps, pin, window, committed, evicted, sizes,
                                        b["table_width"], b["list_stride"]))


def test_layout_many_blocks_long_rows_and_wide_buffers():
    """64 causal blocks (the limit), rows and lists longer than a workgroup,
    and output buffers wider than needed (their padding is written too)."""
    rng = np.random.default_rng(7)
    ps, pin, window = 64, 1000, 20000
    sizes = [int(v) for v in rng.integers(1, 700, size=64)]
    committed = 50000
    evicted = orc.window_evicted_tokens(ps, pin, window, committed)
    b = orc.causal_layout_bounds(ps, pin, window, sizes)
    n_tab = b["fixed_pages"] + b["rolling_pages"]
    ids = rng.permutation(n_tab + 64 * b["private_pages"]).astype(np.int32)
    table, priv = ids[:n_tab], ids[n_tab:].reshape(64, -1)
    width, ls = b["table_width"] + 37, b["list_stride"] + 300
    note(f"causal_layout 64 blocks width={width} list_stride={ls}")
    lay = _layout(table, priv, ps, pin, window, committed, evicted, sizes, width=width, list_stride=ls)
    _compare(lay, orc.causal_layout(table, priv, ps, pin, window, committed, evicted, sizes, width, ls))


# --------------------------------------------------------------------------- end to end

class Rollout:
    """A sequence driven through the library: pool, page table, private pages."""

    def __init__(self, seed, ps, pin, window, sizes, hq, hkv, d):
        self.ps, self.pin, self.window, self.sizes = ps, pin, window, list(sizes)
        self.hq, self.hkv, self.d = hq, hkv, d
        self.lay = pkv.CausalLayout(ps, pin, window, sizes, device=DEV)
        b = self.lay.bounds
        self.n_fixed = b["fixed_pages"]
        n_tab = b["fixed_pages"] + b["rolling_pages"]
        n_pages = n_tab + len(sizes) * b["private_pages"] + 4
        ids = np.random.default_rng(seed).permutation(n_pages).astype(np.int32)
        self.table = torch.tensor(ids[:n_tab], device=DEV)
        self.priv = torch.tensor(ids[n_tab:n_tab + len(sizes) * b["private_pages"]].reshape(len(sizes), -1),
                                 device=DEV)
        shape = (n_pages, ps, hkv, d)
        k = torch.from_numpy(np.full(shape, POISON["bf16"], np.uint16).view(np.int16)).to(DEV)
        self.pool = pkv.Pool(k.view(torch.bfloat16), k.clone().view(torch.bfloat16))
        self.committed = self.evicted = 0

    def commit_layout(self):
        pkv.pkv_causal_layout(self.lay, self.table, self.priv, self.committed, self.evicted)
        pkv.pkv_copy_slots(self.pool, self.lay.commit_src, self.lay.commit_dst)

    def forward(self, k_new, v_new, q, out=None, ragged=False):
        """k_new / v_new [T, Hkv, D] and q [T, Hq, D] bf16 on the device.
        Equal blocks run the padded prefill ([nb, cbs, Hq, D] output); with
        ``ragged`` (any block sizes) the ragged one ([T, Hq, D] output, block b
        at rows offsets[b] ..)."""
        lay = self.lay
        pkv.pkv_scatter_slots(self.pool, k_new, v_new, lay.stage_slots, slots2=lay.stage_slots2)
        pkv.pkv_copy_slots(self.pool, lay.current_src, lay.current_dst)
        if ragged:
            total = sum(self.sizes)
            offs = torch.tensor(np.concatenate([[0], np.cumsum(self.sizes)]).astype(np.int32), device=DEV)
            if out is None:
                out = torch.empty((total, self.hq, self.d), dtype=torch.float32, device=DEV)
            max_keys = self.pin + self.window + max(self.sizes)
            pkv.pkv_attn_prefill_block_causal_ragged(self.pool, q, offs, lay.block_tables, lay.n_ctx, lay.seq_len, 0,
                                                     max(self.sizes), max_keys, 1.0 / math.sqrt(self.d), out)
            return out
        nb, cbs = len(self.sizes), self.sizes[0]
        if out is None:
            out = torch.empty((nb, cbs, self.hq, self.d), dtype=torch.float32, device=DEV)
        max_keys = self.pin + self.window + cbs
        pkv.pkv_attn_prefill_block_causal(self.pool, q.view(nb, cbs, self.hq, self.d), lay.block_tables,
                                          lay.n_ctx, lay.seq_len, 0, max_keys, 1.0 / math.sqrt(self.d), out)
        return out

    def commit(self, n):
        self.committed += n
        new_evicted = pkv.pkv_window_evicted_tokens(self.ps, self.pin, self.window, self.committed)
        shift = (new_evicted - self.evicted) // self.ps
        pkv.pkv_rotate_rows(self.table[self.n_fixed:], shift)
        self.evicted = new_evicted
        self.commit_layout()


def _dense_reference(keys_all, vals_all, q, start, sizes, pin, window, hq, hkv):
    """float64 attention of each block's queries over its visible keys."""
    group = hq // hkv
    out = []
    s = start
    for size in sizes:
        vis = orc.visible_keys(s, s + size, pin, window)
        o = np.zeros((size, hq, q.shape[-1]))
        for h in range(hq):
            o[:, h], _ = orc.attention_rows(q[s - start:s - start + size, h], keys_all[vis, h // group],
                                            vals_all[vis, h // group], 1.0 / math.sqrt(q.shape[-1]))
        out.append(o)
        s += size
    return np.stack(out) if len(set(sizes)) == 1 else np.concatenate(out)


@pytest.mark.parametrize("geom", [
    # ps, pin, window, causal block size, blocks, commits, Hq, Hkv, D
    (32, 40, 100, 24, 3, [72, 72, 72, 72, 72], 4, 2, 128),
    (16, 16, 64, 16, 2, [32, 32, 32, 32, 16, 32], 8, 2, 64),
    (32, 0, 300, 40, 4, [160, 160, 160], 2, 1, 128),
    (16, 37, 0, 20, 2, [40, 40, 40], 4, 4, 128),
], ids=lambda g: f"ps{g[0]}_pin{g[1]}_w{g[2]}_cbs{g[3]}x{g[4]}")
def test_exact_window_rollout_attention(geom):
    ps, pin, window, cbs, nb, commits, hq, hkv, d = geom
    sizes = [cbs] * nb
    total = nb * cbs
    rng = np.random.default_rng(ps + pin + window)
    n_keys = sum(commits) + total
    keys = to_storage(rng.standard_normal((n_keys, hkv, d)).astype(np.float32), "bf16")
    vals = to_storage(rng.standard_normal((n_keys, hkv, d)).astype(np.float32), "bf16")
    ro = Rollout(11, ps, pin, window, sizes, hq, hkv, d)
    ro.commit_layout()
    for step, n in enumerate(commits + [0]):
        c = ro.committed
        q = to_storage(rng.standard_normal((total, hq, d)).astype(np.float32), "bf16")
        note(f"exact window geom={geom} step={step} committed={c} evicted={ro.evicted}")
        out = ro.forward(to_dev(keys[c:c + total]), to_dev(vals[c:c + total]), to_dev(q))
        torch.cuda.synchronize()
        ref = _dense_reference(as_f64(keys), as_f64(vals), as_f64(q), c, sizes, pin, window, hq, hkv)
        assert_close(from_dev(out), ref, "bf16", f"step {step}")
        if n:
            ro.commit(n)


@pytest.mark.parametrize("geom", [
    # ps, pin, window, block sizes, commits, Hq, Hkv, D
    (32, 40, 100, [24, 17, 40], [81, 81, 81, 81], 4, 2, 128),
    (16, 16, 64, [5, 33], [38, 38, 38, 38, 20], 8, 2, 64),
    (32, 0, 300, [1, 64, 31, 64], [160, 160, 160], 2, 1, 128),
    (16, 37, 0, [20, 3, 9], [32, 32, 32], 4, 4, 128),
    (32, 40, 100, [24, 24, 24], [72, 72, 72], 4, 2, 128),
], ids=lambda g: f"ps{g[0]}_pin{g[1]}_w{g[2]}_blocks{'-'.join(map(str, g[3]))}")
def test_exact_window_rollout_with_unequal_causal_blocks(geom):
    """Causal blocks of different sizes in one forward, run as one ragged
    batch over the layout's per-block tables (no padding copy), against
    float64 attention of each block over its visible keys, across commits."""
    ps, pin, window, sizes, commits, hq, hkv, d = geom
    total = sum(sizes)
    rng = np.random.default_rng(ps + pin + window + total)
    n_keys = sum(commits) + total
    keys = to_storage(rng.standard_normal((n_keys, hkv, d)).astype(np.float32), "bf16")
    vals = to_storage(rng.standard_normal((n_keys, hkv, d)).astype(np.float32), "bf16")
    ro = Rollout(13, ps, pin, window, sizes, hq, hkv, d)
    ro.commit_layout()
    for step, n in enumerate(commits + [0]):
        c = ro.committed
        q = to_storage(rng.standard_normal((total, hq, d)).astype(np.float32), "bf16")
        note(f"exact window ragged geom={geom} step={step} committed={c} evicted={ro.evicted}")
        out = ro.forward(to_dev(keys[c:c + total]), to_dev(vals[c:c + total]), to_dev(q), ragged=True)
        torch.cuda.synchronize()
        ref = _dense_reference(as_f64(keys), as_f64(vals), as_f64(q), c, sizes, pin, window, hq, hkv)
        assert_close(from_dev(out), ref.reshape(total, hq, d), "bf16", f"step {step}")
        if n:
            ro.commit(n)


def test_exact_window_zero_query_one_hot_values_show_the_visible_keys():
    """q = 0 gives every visible key the same weight; V of key x is the unit
    vector e_x, so output d is 1/|visible| exactly when key d is visible."""
    ps, pin, window, cbs, nb, d = 16, 10, 30, 8, 2, 128
    sizes = [cbs] * nb
    ro = Rollout(5, ps, pin, window, sizes, 2, 1, d)
    keys = to_storage(np.random.default_rng(3).standard_normal((d, 1, d)).astype(np.float32), "bf16")
    one_hot = np.zeros((d, 1, d), dtype=np.float32)       # fresh array: same strides as the keys
    one_hot[np.arange(d), 0, np.arange(d)] = 1.0
    vals = to_storage(one_hot, "bf16")
    q = torch.zeros((nb * cbs, 2, d), dtype=torch.bfloat16, device=DEV)
    ro.commit_layout()
    while ro.committed + nb * cbs <= d:
        c = ro.committed
        note(f"exact window one-hot committed={c}")
        out = ro.forward(to_dev(keys[c:c + nb * cbs]), to_dev(vals[c:c + nb * cbs]), q)
        torch.cuda.synchronize()
        got = from_dev(out)
        for b in range(nb):
            s = c + b * cbs
            vis = orc.visible_keys(s, s + cbs, pin, window)
            want = np.zeros(d)
            want[vis] = 1.0 / len(vis)
            for i in range(cbs):
                for h in range(2):
                    seen = set(np.nonzero(got[b, i, h] > 0.5 / len(vis))[0].tolist())
                    assert seen == set(vis), f"committed {c} block {b}: {sorted(seen ^ set(vis))}"
                    np.testing.assert_allclose(got[b, i, h], want, rtol=1e-2, atol=1e-6)
        ro.commit(cbs)


def test_exact_window_forward_graph_replays_across_commits():
    """The forward (scatter, current copies, per-block prefill) reads only
    device tensors that each commit rewrites in place, so one captured graph
    serves every commit: capture once, then per commit run the commit eagerly,
    refill the static inputs, replay and compare with float64 attention."""
    ps, pin, window, cbs, nb, hq, hkv, d = 32, 40, 100, 24, 3, 4, 2, 128
    sizes, total = [cbs] * nb, cbs * nb
    rng = np.random.default_rng(77)
    n_keys = 6 * total
    keys = to_storage(rng.standard_normal((n_keys, hkv, d)).astype(np.float32), "bf16")
    vals = to_storage(rng.standard_normal((n_keys, hkv, d)).astype(np.float32), "bf16")
    qs = to_storage(rng.standard_normal((6, total, hq, d)).astype(np.float32), "bf16")
    ro = Rollout(21, ps, pin, window, sizes, hq, hkv, d)
    ro.commit_layout()
    kbuf = torch.empty((total, hkv, d), dtype=torch.bfloat16, device=DEV)
    vbuf, qbuf = torch.empty_like(kbuf), torch.empty((total, hq, d), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((nb, cbs, hq, d), dtype=torch.float32, device=DEV)

    def fill(step):
        c = ro.committed
        kbuf.copy_(to_dev(keys[c:c + total]))
        vbuf.copy_(to_dev(vals[c:c + total]))
        qbuf.copy_(to_dev(qs[step]))
        torch.cuda.synchronize()

    def check(step, what):
        c = ro.committed
        ref = _dense_reference(as_f64(keys), as_f64(vals), as_f64(qs[step]), c, sizes, pin, window, hq, hkv)
        assert_close(from_dev(out), ref, "bf16", f"{what} step {step} (committed {c})")

    note("exact window graph: eager forward, then capture")
    fill(0)
    ro.forward(kbuf, vbuf, qbuf, out=out)
    torch.cuda.synchronize()
    check(0, "eager")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ro.forward(kbuf, vbuf, qbuf, out=out)
    torch.cuda.synchronize()
    for step in range(1, 6):
        ro.commit(total)                      # eager: rotate, lay out, fill private pages
        fill(step)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        note(f"exact window graph replay step {step} committed={ro.committed} evicted={ro.evicted}")
        graph.replay()
        torch.cuda.synchronize()
        check(step, "replay")
