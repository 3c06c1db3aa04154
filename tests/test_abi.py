"""The C ABI on the CPU: the library loads, exports every symbol include/pkv.h
declares, and refuses bad arguments on the host before any HIP call (so these
tests need no GPU; no call here reaches a kernel launch)."""

import ctypes
import os
import re

import pytest

import paged_kv_cache_slots_amd as pkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
A = 0x10000      # a fake 64 KiB-aligned device address: never dereferenced by the host checks


def _declared():
    text = open(os.path.join(ROOT, "include", "pkv.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\*]+\s+\**(pkv_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    lib = pkv.load_library()
    names = _declared()
    assert set(names) == set(pkv.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version():
    lib = pkv.load_library()
    assert lib.pkv_abi_version() == 2
    for code in range(8):
        assert lib.pkv_status_string(code)
    assert b"scratch" in lib.pkv_status_string(7)


def _pool(**kw):
    d = dict(k=A, v=2 * A, page_stride=32 * 8 * 128, num_pages=100, page_size=32, num_kv_heads=8, head_dim=128,
             dtype=pkv.PKV_BF16, k_scale=None, v_scale=None)
    d.update(kw)
    return pkv.PkvPoolStruct(**d)


def _decode(pool, **kw):
    a = dict(q=A, q_dtype=pkv.PKV_BF16, T=4, n=1, hq=32, table=A, tstride=128, lens=A, maxlen=4096, scale=0.1,
             out=A, out_dtype=pkv.PKV_BF16, lse=None, ws=None, wsb=0)
    a.update(kw)
    return pkv.load_library().pkv_attn_decode(ctypes.byref(pool), a["q"], a["q_dtype"], a["T"], a["n"], a["hq"],
                                              a["table"], a["tstride"], a["lens"], a["maxlen"], a["scale"],
                                              a["out"], a["out_dtype"], a["lse"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("pool_kw,call_kw,expect", [
    ({"k": None}, {}, 1),
    ({}, {"q": None}, 1),
    ({}, {"lens": None}, 1),
    ({"dtype": pkv.PKV_FP8_E4M3FN}, {}, 1),                 # fp8 without scales
    ({"page_size": 24}, {}, 2),                             # not a power of two
    ({}, {"hq": 30}, 2),                                    # Hq % Hkv != 0
    ({}, {"maxlen": 128 * 32 + 1}, 2),                      # beyond the table's capacity
    ({"page_stride": 100}, {}, 2),
    ({}, {"q_dtype": 7}, 3),
    ({"head_dim": 96, "page_stride": 32 * 8 * 96}, {}, 4),
    ({"page_size": 8}, {"tstride": 1024}, 4),
    ({}, {"out_dtype": pkv.PKV_FP8_E4M3FN}, 4),
    ({"k": A + 2}, {}, 6),
    ({}, {"T": 0}, 0),                                      # empty batch: OK, nothing launched
])
def test_decode_argument_checks(pool_kw, call_kw, expect):
    assert _decode(_pool(**pool_kw), **call_kw) == expect


def test_scatter_argument_checks():
    lib = pkv.load_library()
    p = _pool()
    assert lib.pkv_scatter_slots(ctypes.byref(p), None, A, 0, 0, None, A, None, 4, None) == 1
    assert lib.pkv_scatter_slots(ctypes.byref(p), A, A, 0, 0, None, None, None, 4, None) == 1
    assert lib.pkv_scatter_slots(ctypes.byref(p), A, A, 0, 0, None, A, None, -1, None) == 2
    assert lib.pkv_scatter_slots(ctypes.byref(p), A, A, -5, 0, None, A, None, 4, None) == 2
    assert lib.pkv_scatter_slots(ctypes.byref(p), A, A, 1024, 128, None, A, None, 0, None) == 0
    bad = _pool(page_size=48)
    assert lib.pkv_scatter_slots(ctypes.byref(bad), A, A, 1024, 128, None, A, None, 4, None) == 2


def test_prefill_argument_checks():
    lib = pkv.load_library()

    def call(pool, **kw):
        a = dict(q=A, q_dtype=pkv.PKV_BF16, qt=72 * 128, qh=128, b=1, s_q=1568, hq=8, table=A, ts=256, n_ctx=A,
                 seq=A, cbs=0, maxk=6680, out=A, od=pkv.PKV_BF16)
        a.update(kw)
        return lib.pkv_attn_prefill_block_causal(ctypes.byref(pool), a["q"], a["q_dtype"], a["qt"], a["qh"], a["b"],
                                                 a["s_q"], a["hq"], a["table"], a["ts"], a["n_ctx"], a["seq"],
                                                 a["cbs"], a["maxk"], 0.1, a["out"], a["od"], None, None, 0, None)
    p = _pool()
    assert call(p, seq=None) == 1
    assert call(p, cbs=-1) == 2
    assert call(p, hq=12) == 2
    assert call(p, maxk=256 * 32 + 1) == 2
    assert call(p, q_dtype=pkv.PKV_F32) == 4
    assert call(_pool(dtype=pkv.PKV_F32)) == 4
    assert call(p, qt=72 * 128 + 1) == 6
    assert call(p, s_q=0) == 0
    # fp8 K/V: scales required; head_dim 128 and pages of >= 32 tokens only
    assert call(_pool(dtype=pkv.PKV_FP8_E4M3FN)) == 1
    fp8 = dict(dtype=pkv.PKV_FP8_E4M3FN, k_scale=3 * A, v_scale=4 * A)
    assert call(_pool(page_size=16, page_stride=16 * 8 * 128, **fp8), maxk=4096) == 4
    assert call(_pool(head_dim=64, page_stride=32 * 8 * 64, **fp8)) == 4
    assert call(_pool(page_stride=32 * 8 * 128 + 8, **fp8)) == 6


def test_merge_argument_checks():
    lib = pkv.load_library()
    assert lib.pkv_merge_states(None, A, 2, 10, 4, 128, A, 0, None, None) == 1
    assert lib.pkv_merge_states(None, None, 2, 0, 4, 128, None, 0, None, None) == 0
    assert lib.pkv_merge_states(A, A, 0, 10, 4, 128, A, 0, None, None) == 2
    assert lib.pkv_merge_states(A, A, 2, 10, 4, 126, A, 0, None, None) == 2
    assert lib.pkv_merge_states(A, A, 2, 10, 4, 128, A, 9, None, None) == 3
    assert lib.pkv_merge_states(A, A, 2, 0, 4, 128, A, 0, None, None) == 0


def test_workspace_sizes():
    lib = pkv.load_library()
    # the larger of: key splits (8 x 64 rows x 32 heads x 129 floats) and the stream-K
    # state (table prefix sums + 2 slots x 16 rows for each of 4096 waves, outputs + LSE)
    sk = lambda t, d: ((4 * (t + 1) + 255) // 256 * 256) + 2 * 4096 * 16 * d * 4 + 2 * 4096 * 16 * 4
    assert lib.pkv_attn_decode_workspace_bytes(64, 1, 32, 8, 128, 4096) == max(8 * 64 * 32 * 129 * 4, sk(64, 128))
    assert lib.pkv_attn_decode_workspace_bytes(64, 1, 32, 8, 128, 512) == sk(64, 128)
    assert lib.pkv_attn_decode_workspace_bytes(256, 1, 64, 8, 128, 32768) == max(16 * 256 * 64 * 129 * 4,
                                                                                sk(256, 128))
    assert lib.pkv_attn_decode_workspace_bytes(0, 1, 64, 8, 128, 32768) == 0


def test_rotate_rows_argument_checks():
    lib = pkv.load_library()
    assert lib.pkv_rotate_rows(None, 4, 8, 8, 4, 3, None) == 1
    assert lib.pkv_rotate_rows(A, -1, 8, 8, 4, 3, None) == 2
    assert lib.pkv_rotate_rows(A, 4, 8, 7, 4, 3, None) == 2
    assert lib.pkv_rotate_rows(A, 4, 8, 8, 3, 3, None) == 4
    assert lib.pkv_rotate_rows(A + 2, 4, 8, 8, 4, 3, None) == 6
    # nothing moves: no launch, NULL allowed
    assert lib.pkv_rotate_rows(None, 0, 8, 8, 4, 3, None) == 0
    assert lib.pkv_rotate_rows(None, 4, 1, 1, 4, 3, None) == 0
    assert lib.pkv_rotate_rows(None, 4, 0, 0, 4, 3, None) == 0
    assert lib.pkv_rotate_rows(None, 4, 8, 8, 4, 16, None) == 0
    assert lib.pkv_rotate_rows(None, 4, 8, 8, 4, -8, None) == 0


def test_copy_slots_argument_checks():
    lib = pkv.load_library()
    p = _pool()
    assert lib.pkv_copy_slots(ctypes.byref(p), 1, 0, None, A, 4, None) == 1
    assert lib.pkv_copy_slots(ctypes.byref(p), 1, 0, A, A, -1, None) == 2
    assert lib.pkv_copy_slots(ctypes.byref(p), 0, 0, A, A, 4, None) == 2
    assert lib.pkv_copy_slots(ctypes.byref(p), 2, 5, A, A, 4, None) == 2
    assert lib.pkv_copy_slots(ctypes.byref(p), 1, 0, None, None, 0, None) == 0
    bad = _pool(page_size=48)
    assert lib.pkv_copy_slots(ctypes.byref(bad), 1, 0, A, A, 4, None) == 2


def test_causal_layout_host_sizes_match_the_oracle():
    import numpy as np
    import oracle as orc
    rng = np.random.default_rng(2)
    for _ in range(300):
        ps = int(2 ** rng.integers(0, 8))
        pin, window = int(rng.integers(0, 6 * ps + 5)), int(rng.integers(0, 9 * ps + 5))
        sizes = [int(v) for v in rng.integers(1, 4 * ps + 3, size=int(rng.integers(1, 65)))]
        assert pkv.pkv_causal_layout_bounds(ps, pin, window, sizes) == orc.causal_layout_bounds(ps, pin, window,
                                                                                                sizes)
        committed = int(rng.integers(0, 20 * ps + pin + window))
        assert pkv.pkv_window_evicted_tokens(ps, pin, window, committed) == orc.window_evicted_tokens(
            ps, pin, window, committed)
    lib = pkv.load_library()
    assert lib.pkv_window_evicted_tokens(24, 0, 0, 100) == -1
    assert lib.pkv_window_evicted_tokens(16, -1, 0, 100) == -1


def _layout_call(**kw):
    """pkv_causal_layout of the first hand-worked geometry (page size 4, pin 6,
    window 7, committed 19, evicted 4, blocks [2, 5]), fake device pointers."""
    a = dict(table=A, table_len=7, priv=A, priv_stride=4, ps=4, pin=6, window=7, committed=19, evicted=4,
             sizes=[2, 5], bt=A, width=6, n_ctx=A, seq_len=A, st=A, st2=A, cs=A, cd=A, us=A, ud=A, ls=9)
    a.update(kw)
    sizes = (ctypes.c_int32 * max(1, len(a["sizes"])))(*a["sizes"])
    return pkv.load_library().pkv_causal_layout(
        a["table"], a["table_len"], a["priv"], a["priv_stride"], a["ps"], a["pin"], a["window"], a["committed"],
        a["evicted"], sizes, len(a["sizes"]), a["bt"], a["width"], a["n_ctx"], a["seq_len"], a["st"], a["st2"],
        a["cs"], a["cd"], a["us"], a["ud"], a["ls"], None)


@pytest.mark.parametrize("kw,expect", [
    (dict(table=None), 1), (dict(priv=None), 1), (dict(cd=None), 1), (dict(st2=None), 1), (dict(us=None), 1),
    (dict(ps=6), 2), (dict(pin=-1), 2), (dict(evicted=2), 2), (dict(evicted=8), 2), (dict(committed=-1), 2),
    (dict(table_len=5), 2), (dict(table_len=1), 2), (dict(priv_stride=3), 2), (dict(width=5), 2), (dict(ls=8), 2),
    (dict(sizes=[]), 2), (dict(sizes=[2, 0]), 2), (dict(sizes=[1] * 65), 2), (dict(sizes=[2, 13]), 2),
    (dict(committed=2 ** 31 - 3, pin=0, window=2 ** 31), 2),
])
def test_causal_layout_argument_checks(kw, expect):
    assert _layout_call(**kw) == expect


def test_decode_step_argument_checks():
    lib = pkv.load_library()
    p = _pool()

    def call(pool, **kw):
        a = dict(q=A, qd=pkv.PKV_BF16, T=4, n=9, hq=32, table=A, ts=128, lens=A, maxlen=4096, scale=0.1, out=A,
                 od=pkv.PKV_BF16)
        a.update(kw)
        return lib.pkv_attn_decode_step(ctypes.byref(pool), a["q"], a["qd"], a["T"], a["n"], a["hq"], a["table"],
                                        a["ts"], a["lens"], a["maxlen"], a["scale"], a["out"], a["od"], None, None, 0,
                                        None)
    assert call(p, lens=None) == 1
    assert call(p, n=0) == 2
    assert call(p, hq=12) == 2
    assert call(p, maxlen=128 * 32 + 1) == 2
    assert call(p, scale=0.0) == 2
    assert call(p, qd=pkv.PKV_FP8_E4M3FN) == 4
    assert call(_pool(page_size=8, page_stride=8 * 8 * 128), maxlen=512) == 4
    assert call(p, T=0) == 0


def test_decode_shared_prefix_argument_checks():
    lib = pkv.load_library()
    p = _pool()

    def call(pool, **kw):
        a = dict(q=A, qd=pkv.PKV_BF16, G=8, S=16, n=1, hq=32, pt=A, ps=64, pl=A, mp=2048, tt=A, ts=16, tl=A, mt=512,
                 scale=0.1, out=A, od=pkv.PKV_BF16, ws=A, wsb=1 << 30)
        a.update(kw)
        return lib.pkv_attn_decode_shared_prefix(
            ctypes.byref(pool), a["q"], a["qd"], a["G"], a["S"], a["n"], a["hq"], a["pt"], a["ps"], a["pl"], a["mp"],
            a["tt"], a["ts"], a["tl"], a["mt"], a["scale"], a["out"], a["od"], None, a["ws"], a["wsb"], None)
    assert call(p, ws=None) == 1
    assert call(p, tl=None) == 1
    assert call(p, S=0) == 2
    assert call(p, n=0) == 2
    assert call(p, mp=64 * 32 + 1) == 2
    assert call(p, mt=16 * 32 + 1) == 2
    need = pkv.pkv_attn_decode_shared_prefix_workspace_bytes(8, 16, 1, 32, 128, 2048)
    assert need == 3 * 128 * 32 * 129 * 4   # 2048-key prefix in splits of >= 1024 keys, + the tail state
    assert call(p, wsb=need - 1) == 2
    assert call(p, qd=pkv.PKV_F32) == 4
    assert call(_pool(dtype=pkv.PKV_F32, page_stride=32 * 8 * 128)) == 4
    assert call(p, ws=A + 8) == 6
    assert call(p, G=0) == 0


def test_decode_append_argument_checks():
    lib = pkv.load_library()
    p = _pool()

    def call(pool, **kw):
        a = dict(nk=A, nv=A, ts=8 * 128, hs=128, q=A, qd=pkv.PKV_BF16, T=4, n=1, hq=32, table=A, tstride=128,
                 lens=A, maxlen=4096, scale=0.1, out=A, od=pkv.PKV_BF16)
        a.update(kw)
        return lib.pkv_attn_decode_append(ctypes.byref(pool), a["nk"], a["nv"], a["ts"], a["hs"], a["q"], a["qd"],
                                          a["T"], a["n"], a["hq"], a["table"], a["tstride"], a["lens"], a["maxlen"],
                                          a["scale"], a["out"], a["od"], None, None, 0, None)
    assert call(p, nk=None, nv=None) == 1
    assert call(p, nk=None) == 1
    assert call(p, nv=None) == 1
    assert call(_pool(k=None), nk=None, nv=None) == 1    # the pool is checked first
    assert call(p, ts=-1) == 2
    assert call(p, hs=-1) == 2
    assert call(p, hq=30) == 2
    assert call(p, maxlen=128 * 32 + 1) == 2
    assert call(p, qd=pkv.PKV_FP8_E4M3FN) == 4
    assert call(p, T=0, nk=None, nv=None) == 0           # empty batch: OK, nothing launched


def test_decode_shared_prefix_append_argument_checks():
    lib = pkv.load_library()
    p = _pool()

    def call(pool, **kw):
        a = dict(nk=A, nv=A, nts=8 * 128, nhs=128, q=A, qd=pkv.PKV_BF16, G=8, S=16, n=1, hq=32, pt=A, ps=64, pl=A,
                 mp=2048, tt=A, ts=16, tl=A, mt=512, scale=0.1, out=A, od=pkv.PKV_BF16, ws=A, wsb=1 << 30)
        a.update(kw)
        return lib.pkv_attn_decode_shared_prefix_append(
            ctypes.byref(pool), a["nk"], a["nv"], a["nts"], a["nhs"], a["q"], a["qd"], a["G"], a["S"], a["n"],
            a["hq"], a["pt"], a["ps"], a["pl"], a["mp"], a["tt"], a["ts"], a["tl"], a["mt"], a["scale"], a["out"],
            a["od"], None, a["ws"], a["wsb"], None)
    assert call(p, nk=None, nv=None) == 1
    assert call(p, nv=None) == 1
    assert call(p, nts=-8) == 2
    assert call(p, ws=None) == 1
    assert call(p, mt=16 * 32 + 1) == 2
    assert call(p, qd=pkv.PKV_F32) == 4
    assert call(p, ws=A + 8) == 6
    assert call(p, G=0, nk=None, nv=None) == 0


def test_check_calls_argument_checks():
    lib = pkv.load_library()
    p = _pool()
    assert lib.pkv_check_slots(ctypes.byref(p), A, 10, None, None) == 1
    assert lib.pkv_check_slots(ctypes.byref(p), None, 10, A, None) == 1
    assert lib.pkv_check_slots(ctypes.byref(p), A, -1, A, None) == 2
    assert lib.pkv_check_tables(ctypes.byref(p), A, 0, A, 4, A, None) == 2
    assert lib.pkv_check_tables(ctypes.byref(p), A, 8, A, -1, A, None) == 2
    assert lib.pkv_check_tables(ctypes.byref(p), None, 8, A, 4, A, None) == 1
    bad = _pool(page_size=48)
    assert lib.pkv_check_tables(ctypes.byref(bad), A, 8, A, 4, A, None) == 2


def test_xcd_probe_argument_checks():
    """pkv_xcd_ids refuses bad launch shapes and pointers on the host (nothing
    launched); an empty probe is OK with a NULL pointer."""
    lib = pkv.load_library()
    assert lib.pkv_xcd_ids(None, 0, 64, None) == 0
    assert lib.pkv_xcd_ids(None, 8, 64, None) == 1
    assert lib.pkv_xcd_ids(A, -1, 64, None) == 2
    assert lib.pkv_xcd_ids(A, 8, 63, None) == 2
    assert lib.pkv_xcd_ids(A, 8, 96, None) == 2
    assert lib.pkv_xcd_ids(A, 8, 2048, None) == 2
    assert lib.pkv_xcd_ids(A + 2, 8, 64, None) == 6


def _decode_noalloc(pool, **kw):
    a = dict(q=A, q_dtype=pkv.PKV_BF16, T=4, n=1, hq=32, table=A, tstride=128, lens=A, maxlen=4096, scale=0.1,
             out=A, out_dtype=pkv.PKV_BF16, lse=None)
    a.update(kw)
    return pkv.load_library().pkv_attn_decode_noalloc(
        ctypes.byref(pool), a["q"], a["q_dtype"], a["T"], a["n"], a["hq"], a["table"], a["tstride"], a["lens"],
        a["maxlen"], a["scale"], a["out"], a["out_dtype"], a["lse"], None)


@pytest.mark.parametrize("pool_kw,call_kw,expect", [
    ({"k": None}, {}, 1),
    ({}, {"q": None}, 1),
    ({"dtype": pkv.PKV_FP8_E4M3FN}, {}, 1),                 # fp8 without scales
    ({"page_size": 24}, {}, 2),
    ({}, {"hq": 30}, 2),
    ({}, {"maxlen": 128 * 32 + 1}, 2),
    ({"head_dim": 96}, {}, 4),
    ({}, {"q": A + 8}, 6),                                  # misaligned q
    ({}, {"T": 0, "q": None, "out": None}, 0),              # empty: OK, nothing touched
])
def test_decode_noalloc_refuses_bad_arguments_on_the_host(pool_kw, call_kw, expect):
    """The no-allocation decode checks its arguments like pkv_attn_decode, on
    the host, before it looks up its device array or launches anything."""
    assert _decode_noalloc(_pool(**pool_kw), **call_kw) == expect


def _prefill_ragged(pool, **kw):
    a = dict(q=A, q_dtype=pkv.PKV_BF16, qts=8 * 128, qhs=128, B=3, max_rows=200, hq=8, offs=A, table=A, tstride=64,
             n_ctx=A, seq=A, cbs=0, max_keys=1000, scale=0.1, out=A, out_dtype=pkv.PKV_BF16, lse=None, ws=None,
             wsb=0)
    a.update(kw)
    return pkv.load_library().pkv_attn_prefill_block_causal_ragged(
        ctypes.byref(pool), a["q"], a["q_dtype"], a["qts"], a["qhs"], a["B"], a["max_rows"], a["hq"], a["offs"],
        a["table"], a["tstride"], a["n_ctx"], a["seq"], a["cbs"], a["max_keys"], a["scale"], a["out"],
        a["out_dtype"], a["lse"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("pool_kw,call_kw,expect", [
    ({}, {"offs": None}, 1),                                # the row offsets are required
    ({}, {"q": None}, 1),
    ({}, {"hq": 7}, 2),                                     # Hq % Hkv != 0
    ({}, {"max_keys": 64 * 32 + 1}, 2),                     # beyond the table's capacity
    ({"head_dim": 96}, {}, 4),
    ({}, {"offs": A + 2}, 6),                               # misaligned int32 offsets
    ({}, {"B": 0, "q": None, "offs": None}, 0),             # empty batch: OK, nothing touched
])
def test_prefill_ragged_refuses_bad_arguments_on_the_host(pool_kw, call_kw, expect):
    assert _prefill_ragged(_pool(**pool_kw), **call_kw) == expect


def test_prefill_workspace_size_without_a_device_is_the_largest_grid():
    """With no device to ask for its CU count the size covers the largest grid
    (512 workgroups x 2 partial states); a shape with no batch needs none."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is present: the size follows its CU count (checked by the GPU prefill tests)")
    lib = pkv.load_library()
    assert lib.pkv_attn_prefill_workspace_bytes(1, 1568, 24, 24, 128, 6680) == 2 * 512 * 66560
    assert lib.pkv_attn_prefill_workspace_bytes(0, 1568, 24, 24, 128, 6680) == 0
