"""GPU parity of the LSE state merge and of the shared-prefix n-sample flow
(prefix decode once per group + tail decode per row + merge) against the
oracle."""

import numpy as np
import pytest
import torch

import oracle as orc
import paged_kv_cache_slots_amd as pkv
import workloads as W
from gpu_util import assert_lse_close, DEV, as_f64, assert_close, from_dev, note, pool_to_dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_states", [1, 2, 5])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_merge_random_states(n_states, out_dtype):
    rng = np.random.default_rng(n_states)
    rows, hq, d = 37, 6, 128
    o = rng.standard_normal((n_states, rows, hq, d)).astype(np.float32)
    lse = (rng.standard_normal((n_states, rows, hq)) * 3).astype(np.float32)
    # some empty states (LSE -inf) with garbage outputs, and one row empty in every state
    empty = rng.random((n_states, rows, hq)) < 0.2
    lse[empty] = -np.inf
    o[empty] = np.nan
    lse[:, 3, :] = -np.inf
    note(f"merge N={n_states} out={out_dtype}")
    out = torch.empty((rows, hq, d), dtype=out_dtype, device=DEV)
    out_lse = torch.empty((rows, hq), dtype=torch.float32, device=DEV)
    pkv.pkv_merge_states(to_dev(o), to_dev(lse), out, out_lse)
    torch.cuda.synchronize()
    ref, ref_lse = orc.merge_states(o, lse)
    tol = "f32" if out_dtype == torch.float32 else "bf16"
    assert_close(as_f64(from_dev(out)), ref, tol, "merge out")
    assert_lse_close(from_dev(out_lse).astype(np.float64), ref_lse, "f32", "merge lse")
    assert np.all(as_f64(from_dev(out))[3] == 0)


def _shared_prefix_flow(c, check_unshared=True):
    """prefix decode (rows_per_table = samples) + tail decode + merge -> bf16."""
    pool = pool_to_dev(c.pool)
    pkv.pkv_scatter_slots(pool, to_dev(c.new_k), to_dev(c.new_v), to_dev(c.slots))
    n_rows, hq, d = c.q.shape[0], c.num_q_heads, c.pool.head_dim
    hkv = c.pool.num_kv_heads
    q = to_dev(c.q)                                            # [rows, 1, Hq, D]
    parts_o = torch.empty((2, n_rows, hq, d), dtype=torch.float32, device=DEV)
    parts_lse = torch.empty((2, n_rows, hq), dtype=torch.float32, device=DEV)
    g, s = c.num_groups, c.samples
    max_pre, max_tail = int(c.prefix_lens.max()), int(c.tail_lens.max())
    ws = torch.empty(max(16, pkv.pkv_attn_decode_workspace_bytes(g, s, hq, hkv, d, max_pre),
                         pkv.pkv_attn_decode_workspace_bytes(n_rows, 1, hq, hkv, d, max_tail)),
                     dtype=torch.uint8, device=DEV)
    pkv.pkv_attn_decode(pool, q.view(g, s, hq, d), to_dev(c.prefix_tables), to_dev(c.prefix_lens), max_pre,
                        c.sm_scale, parts_o[0].view(g, s, hq, d), parts_lse[0].view(g, s, hq), ws)
    pkv.pkv_attn_decode(pool, q, to_dev(c.tail_tables), to_dev(c.tail_lens), max_tail, c.sm_scale,
                        parts_o[1].view(n_rows, 1, hq, d), parts_lse[1].view(n_rows, 1, hq), ws)
    out = torch.empty((n_rows, hq, d), dtype=torch.bfloat16, device=DEV)
    out_lse = torch.empty((n_rows, hq), dtype=torch.float32, device=DEV)
    pkv.pkv_merge_states(parts_o, parts_lse, out, out_lse)
    unshared = None
    if check_unshared:
        unshared = torch.empty((n_rows, 1, hq, d), dtype=torch.bfloat16, device=DEV)
        max_full = int(c.full_lens.max())
        ws2 = torch.empty(max(16, pkv.pkv_attn_decode_workspace_bytes(n_rows, 1, hq, hkv, d, max_full)),
                          dtype=torch.uint8, device=DEV)
        pkv.pkv_attn_decode(pool, q, to_dev(c.full_tables), to_dev(c.full_lens), max_full, c.sm_scale, unshared,
                            None, ws2)
    torch.cuda.synchronize()
    return (as_f64(from_dev(out)), from_dev(out_lse).astype(np.float64),
            None if unshared is None else as_f64(from_dev(unshared))[:, 0])


@pytest.mark.parametrize("size", ["small", "shared_prefix_decode"])
def test_shared_prefix_merge_equals_full_attention(size):
    if size == "small":
        c = W.make_shared_prefix_case("sp_small", 71, 1071, 3, 5, 256, (1, 70), 16, 4, 128, 32, 128)
    else:
        c = W.shared_prefix_decode()
    note(f"shared prefix flow {size}")
    got, got_lse, unshared = _shared_prefix_flow(c)
    kp = orc.scatter_slots(c.pool.k, c.new_k, c.slots)
    vp = orc.scatter_slots(c.pool.v, c.new_v, c.slots)
    rows = list(range(c.q.shape[0]))          # every row, at both sizes
    ref, ref_lse = orc.attn_decode(kp, vp, c.q, c.full_tables, c.full_lens, c.sm_scale)
    assert_close(got[rows], ref[rows, 0], "bf16", "prefix+tail merged vs full attention")
    assert_lse_close(got_lse[rows], ref_lse[rows, 0], "bf16", "merged lse")
    assert_close(unshared[rows], ref[rows, 0], "bf16", "unshared decode")
