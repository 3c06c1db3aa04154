"""GPU parity of the fused n-sample step (shared prefix + private tails +
merge in two launches) against the oracle: one or several step tokens per
sample, bf16 and fp8 pools, uneven and empty prefixes, tails shorter than the
step, and the n-sample workload's full shape."""

import numpy as np
import pytest
import torch

import oracle as orc
import paged_kv_cache_slots_amd as pkv
import workloads as W
from gpu_util import assert_lse_close, DEV, as_f64, assert_close, from_dev, note, pool_to_dev, to_dev

pytestmark = pytest.mark.gpu


def run_shared(c, out_dtype=torch.bfloat16):
    pool = pool_to_dev(c.pool)
    if c.slots is not None:
        pkv.pkv_scatter_slots(pool, to_dev(c.new_k), to_dev(c.new_v), to_dev(c.slots))
    q = to_dev(c.q)
    rows, n, hq, d = q.shape
    out = torch.full((rows, n, hq, d), float("nan"), dtype=out_dtype, device=DEV)
    lse = torch.full((rows, n, hq), float("nan"), dtype=torch.float32, device=DEV)
    mp, mt = int(c.prefix_lens.max()), int(c.tail_lens.max())
    nb = pkv.pkv_attn_decode_shared_prefix_workspace_bytes(rows // c.samples, c.samples, n, hq, d, mp)
    ws = torch.full((nb,), 0xFF, dtype=torch.uint8, device=DEV)        # NaN bytes: contents must not matter
    pkv.pkv_attn_decode_shared_prefix(pool, q, c.samples, to_dev(c.prefix_tables), to_dev(c.prefix_lens), mp,
                                      to_dev(c.tail_tables), to_dev(c.tail_lens), mt, c.sm_scale, out, ws, lse)
    torch.cuda.synchronize()
    return as_f64(from_dev(out)), from_dev(lse).astype(np.float64)


def check_shared(c, out_dtype=torch.bfloat16):
    note(f"shared step {c.name} groups={len(c.prefix_lens)} samples={c.samples} q_len={c.q_len} "
         f"prefix={list(c.prefix_lens)} tails={list(c.tail_lens)[:8]} kv={c.pool.dtype}")
    got, got_lse = run_shared(c, out_dtype)
    kp, vp = c.pool.k, c.pool.v
    if c.slots is not None:
        kp, vp = orc.scatter_slots(kp, c.new_k, c.slots), orc.scatter_slots(vp, c.new_v, c.slots)
    ref, ref_lse = orc.attn_decode_shared_prefix(kp, vp, c.q, c.samples, c.prefix_tables, c.prefix_lens,
                                                 c.tail_tables, c.tail_lens, c.sm_scale, kv_dtype=c.pool.dtype,
                                                 q_dtype="bf16", k_scale=c.pool.k_scale, v_scale=c.pool.v_scale)
    tol = "fp8" if c.pool.dtype == "fp8" else "bf16"
    assert np.all(np.isfinite(got))
    assert_close(got, ref, tol, f"{c.name} out")
    assert_lse_close(got_lse, ref_lse, tol, f"{c.name} lse")


CASES = [
    # name, groups, samples, q_len, prefix lens, tail lens (or (lo, hi) drawn), Hq, Hkv, D, ps, kv
    ("one_token_gqa4", 3, 4, 1, [640, 1500, 32], (1, 200), 32, 8, 128, 32, "bf16"),
    ("k8_verify", 2, 3, 9, [900, 2100], (9, 300), 16, 4, 128, 32, "bf16"),
    ("q16_d64_ps16", 2, 2, 16, [0, 700], (16, 90), 8, 2, 64, 16, "bf16"),     # group 0: no shared prefix
    ("tails_shorter_than_step", 1, 4, 5, [333], [1, 3, 5, 40], 8, 8, 128, 32, "bf16"),
    ("fp8_q4", 2, 4, 4, [1024, 100], (4, 260), 32, 8, 128, 32, "fp8"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_shared_step_parity(case):
    name, groups, samples, n, pl, tl, hq, hkv, d, ps, kv = case
    if isinstance(tl, tuple):
        tl = np.random.default_rng(len(name)).integers(tl[0], tl[1], size=groups * samples, endpoint=True)
    c = W.make_shared_step_case(name, 51, 1051, groups, samples, n, pl, tl, hq, hkv, d, ps, kv_dtype=kv)
    check_shared(c)


def _random_shared_case(seed):
    """A seeded random n-sample step: groups, samples and step tokens, prefix
    lengths from empty to several splits, tails shorter and longer than the
    step, bf16 (128 or 64 dims) or fp8 pools and GQA groupings, so the prefix
    runs both as LDS-shared four-row-block workgroups and as the other forms."""
    rng = np.random.default_rng(500 + seed)
    kv = "fp8" if rng.random() < 0.3 else "bf16"
    d = 128 if (kv == "fp8" or rng.random() < 0.75) else 64
    ps = 32 if kv == "fp8" else int(rng.choice([16, 32]))
    hkv = int(rng.choice([2, 4, 8]))
    group = int(rng.choice([1, 2, 4]))
    groups = int(rng.integers(1, 4))
    samples = int(rng.integers(1, 17))
    n = int(rng.integers(1, 5))
    pl = rng.integers(0, 3000, size=groups)
    tl = rng.integers(1, 400, size=groups * samples)
    return W.make_shared_step_case(f"rand{seed}", 600 + seed, 1600 + seed, groups, samples, n, pl, tl,
                                   hkv * group, hkv, d, ps, kv_dtype=kv)


@pytest.mark.parametrize("seed", range(8))
def test_shared_step_random_shapes(seed):
    check_shared(_random_shared_case(seed))


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16], ids=["fp32_out", "bf16_out"])
def test_shared_step_workload_shape(out_dtype):
    """The n-sample workload: 8 prompts x 16 samples, 2048 shared keys, tails
    U[1, 512], 32/8 heads x 128, one new token per sample (bf16 output is the
    benchmarked form)."""
    tl = np.random.default_rng(4).integers(1, 512, size=128, endpoint=True)
    c = W.make_shared_step_case("workload", 52, 1052, 8, 16, 1, [2048] * 8, tl, 32, 8, 128, 32)
    check_shared(c, out_dtype)
