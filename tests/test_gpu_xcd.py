"""Where the dispatcher places workgroups.

The prefill's persistent schedule hands the kv heads of XCD x to workgroups
x, x + 8, x + 16, ... so that each K/V tile of a head is fetched once into that
XCD's L2 and reused by all the q-tiles there.  That assumes workgroup i runs on
XCD i mod 8.  The probe reads each workgroup's XCC_ID hardware register; these
tests check the assumption for the prefill's own launch shape (one 512-thread
workgroup per CU, rounded down to a multiple of 8) and for a grid many times
the CU count.  Correctness never depends on the placement; only the L2 reuse
does."""

import numpy as np
import pytest
import torch

import paged_kv_cache_slots_amd as pkv
from gpu_util import note

pytestmark = pytest.mark.gpu


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


@pytest.mark.parametrize("shape", ["prefill_grid", "many_small"])
def test_workgroup_i_runs_on_xcd_i_mod_8(shape):
    cus = _cus()
    if shape == "prefill_grid":
        n, threads = max(8, min(cus, 512) // 8 * 8), 512
    else:
        n, threads = 16 * cus, 64
    note(f"xcd probe: {n} workgroups x {threads} threads ({cus} CUs)")
    ids = pkv.pkv_xcd_ids(n, threads)
    torch.cuda.synchronize()
    xcd = ids.cpu().numpy() & 0xF
    want = np.arange(n) % 8
    # every die is used, and each workgroup sits on die (id mod 8)
    assert sorted(set(xcd.tolist())) == list(range(8)), f"dies seen: {sorted(set(xcd.tolist()))}"
    assert np.array_equal(xcd, want), f"{int((xcd != want).sum())} of {n} workgroups off their die"
