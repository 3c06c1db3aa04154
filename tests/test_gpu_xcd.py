"""Where the dispatcher places workgroups.

The prefill's persistent schedule gives the kv heads of group x to workgroups
x, x + 8, x + 16, ... so that each K/V tile of a head is fetched once into one
XCD's L2 and reused by all the q-tiles there.  That needs the workgroups whose
ids agree mod 8 to run on one XCD.  The dispatcher deals workgroups to the 8
XCDs round robin; which XCD receives workgroup 0 depends on the launches
before (seen on this chip: XCD 0 in a fresh process, XCD 7 after other
kernels), which the grouping does not care about.  The probe reads each
workgroup's XCC_ID hardware register; these tests check the grouping for the
prefill's own launch shape (one 512-thread workgroup per CU, rounded down to a
multiple of 8) and for a grid many times the CU count.  Correctness never
depends on the placement; only the L2 reuse does."""

import numpy as np
import pytest
import torch

import paged_kv_cache_slots_amd as pkv
from gpu_util import note

pytestmark = pytest.mark.gpu


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


@pytest.mark.parametrize("shape", ["prefill_grid", "many_small"])
def test_workgroups_agreeing_mod_8_share_an_xcd(shape):
    cus = _cus()
    if shape == "prefill_grid":
        n, threads = max(8, min(cus, 512) // 8 * 8), 512
    else:
        n, threads = 16 * cus, 64
    note(f"xcd probe: {n} workgroups x {threads} threads ({cus} CUs)")
    ids = pkv.pkv_xcd_ids(n, threads)
    torch.cuda.synchronize()
    xcd = ids.cpu().numpy() & 0xF
    # workgroups 0..7 land on 8 distinct dies, and every workgroup shares the
    # die of the one among 0..7 its id agrees with mod 8
    assert sorted(xcd[:8].tolist()) == list(range(8)), f"dies of workgroups 0..7: {xcd[:8].tolist()}"
    want = xcd[np.arange(n) % 8]
    assert np.array_equal(xcd, want), f"{int((xcd != want).sum())} of {n} workgroups off their group's die"
