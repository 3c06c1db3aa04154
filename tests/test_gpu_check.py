"""GPU tests of the device-side content checks: the counts of out-of-pool
slots and of table rows that would read outside the pool equal the counts
taken from the definition on the host.  The checks read only ids and
lengths, so bad entries are safe to plant."""

import numpy as np
import pytest
import torch

import paged_kv_cache_slots_amd as pkv
from gpu_util import DEV, note

pytestmark = pytest.mark.gpu


def _pool(num_pages=100, ps=32):
    k = torch.zeros((num_pages, ps, 2, 64), dtype=torch.bfloat16, device=DEV)
    return pkv.Pool(k, k.clone())


@pytest.mark.parametrize("n", [0, 1, 1000, 300001])
def test_check_slots_counts_out_of_pool_ids(n):
    note(f"check_slots n={n}")
    rng = np.random.default_rng(n + 1)
    cap = 100 * 32
    slots = rng.integers(-3, cap, size=n)
    bad_idx = rng.choice(n, size=min(n, 17), replace=False) if n else []
    slots[bad_idx] = cap + rng.integers(0, 1 << 40, size=len(bad_idx))
    got = pkv.pkv_check_slots(_pool(), torch.tensor(slots, dtype=torch.int64, device=DEV))
    torch.cuda.synchronize()
    assert int(got.item()) == int((slots >= cap).sum())


def test_check_tables_counts_rows_that_read_outside_the_pool():
    note("check_tables")
    rng = np.random.default_rng(9)
    rows, width, ps, n_pages = 3000, 8, 32, 100
    table = rng.integers(0, n_pages, size=(rows, width)).astype(np.int32)
    lens = rng.integers(0, width * ps + 1, size=rows).astype(np.int32)
    # plant bad rows: a used page out of range, a length past the row, a negative length,
    # and an out-of-range id past the used pages (which must not count)
    table[5, 0] = n_pages
    table[6, (int(lens[6]) - 1) // ps if lens[6] > 0 else 0] = -1
    lens[7] = width * ps + 1
    lens[8] = -4
    lens[9] = 33
    table[9, 2:] = 12345
    want = 0
    for r in range(rows):
        L = int(lens[r])
        if L < 0 or L > width * ps:
            want += 1
            continue
        used = table[r, :(L + ps - 1) // ps]
        want += int(np.any((used < 0) | (used >= n_pages)))
    got = pkv.pkv_check_tables(_pool(n_pages, ps), torch.tensor(table, device=DEV), torch.tensor(lens, device=DEV))
    torch.cuda.synchronize()
    assert int(got.item()) == want and want >= 3
