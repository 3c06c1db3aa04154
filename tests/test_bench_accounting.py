"""The benchmark's algorithmic byte and flop counts, which every roofline
figure rests on, checked against hand counts and brute force (CPU only)."""

import math

import numpy as np

import bench


def test_decode_bytes_hand_count():
    # Two sequences of 5 and 2 keys on 4-token pages (2 + 1 pages), 2 kv heads
    # of 8 dims in bf16, 3 query rows of 4 q heads in bf16, fp32 output, LSE.
    kv = 2 * (5 + 2) * 2 * 8 * 2           # K and V, every valid key once per kv head
    q_o = 3 * 4 * 8 * (2 + 4)
    lse = 3 * 4 * 4
    tables = 3 * 4 + 2 * 4                 # used table entries + lengths
    want = kv + q_o + lse + tables
    assert want == 448 + 576 + 48 + 20 == 1092
    assert bench.decode_bytes([5, 2], 4, 2, 8, 2, 3, 4, 2, 4, True, False) == want
    # fp8 scales: one fp32 scale per used page, kv head and K/V.
    assert bench.decode_bytes([5, 2], 4, 2, 8, 2, 3, 4, 2, 4, True, True) == want + 2 * 3 * 2 * 4


def test_decode_bytes_headline_batch():
    # 64 sequences with lengths uniform in [512, 4096] (PCG64 seed 102), 32-token
    # pages, 8 kv heads of 128 in bf16, one query row of 32 heads per sequence.
    lens = np.random.Generator(np.random.PCG64(102)).integers(512, 4096, size=64, endpoint=True)
    pages = sum(math.ceil(int(n) / 32) for n in lens)
    want = 2 * int(lens.sum()) * 8 * 128 * 2 + 64 * 32 * 128 * 4 + 4 * pages + 4 * 64
    assert bench.decode_bytes(lens, 32, 8, 128, 2, 64, 32, 2, 2, False, False) == want == 631229600


def _visible_keys_brute(seq_len, n_ctx, cbs):
    # Query i sees every context key and key j of the current chunk when j lies
    # in a causal block at or before its own.
    total = 0
    for i in range(seq_len):
        total += n_ctx + sum(1 for j in range(seq_len) if j // cbs <= i // cbs)
    return total


def test_prefill_flops_visibility():
    for seq_len, n_ctx, cbs in [(1560, 5120, 1560), (1560, 5120, 390), (100, 7, 33), (64, 0, 1)]:
        want = 4.0 * 128 * 24 * _visible_keys_brute(seq_len, n_ctx, cbs)
        assert bench.prefill_flops(seq_len, n_ctx, cbs, 128, 24) == want
    assert bench.prefill_flops(1560, 5120, 1560, 128, 24) == 128050790400
    # causal_block_size 0 means one block over the whole chunk.
    assert bench.prefill_flops(50, 3, 0, 64, 2) == bench.prefill_flops(50, 3, 50, 64, 2)


def test_parity_gate_accepts_within_and_rejects_outside_tolerance():
    """The bench's gate: outputs within atol + rtol |ref| pass and report the
    largest error; one element past it, a NaN or a shape mismatch fails; LSE is
    held to an absolute bound and -inf must match exactly."""
    import pytest
    ref = np.linspace(-3, 3, 50)
    got = ref + 0.5 * (2e-2 + 2e-2 * np.abs(ref))
    assert abs(bench.check_out(got, ref, "bf16", "x") - np.max(np.abs(got - ref))) < 1e-15
    bad = got.copy()
    bad[7] = ref[7] + 1.01 * (2e-2 + 2e-2 * abs(ref[7]))
    with pytest.raises(bench.ParityError):
        bench.check_out(bad, ref, "bf16", "x")
    with pytest.raises(bench.ParityError):
        bench.check_out(np.where(np.arange(50) == 3, np.nan, got), ref, "bf16", "x")
    with pytest.raises(bench.ParityError):
        bench.check_out(got[:49], ref, "bf16", "x")
    lse = np.array([300.0, -np.inf, 2.0])
    assert bench.check_lse(lse + np.array([0.019, 0.0, -0.019]), lse, "bf16", "l") < 0.02
    with pytest.raises(bench.ParityError):          # 0.03 on an LSE of 300 is out, however large the LSE
        bench.check_lse(lse + np.array([0.03, 0.0, 0.0]), lse, "bf16", "l")
    with pytest.raises(bench.ParityError):
        bench.check_lse(np.array([300.0, 5.0, 2.0]), lse, "bf16", "l")
