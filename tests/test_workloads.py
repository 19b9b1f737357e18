"""The seeded input generators (no GPU): row sampling per head covers every
32-row block across the heads, keeps the forced edge rows, and is
deterministic."""

import numpy as np
import pytest

import workloads


@pytest.mark.parametrize("name", ["flux_1024", "hunyuan_720p_129f"])
def test_rows_per_head_cover_every_block(name):
    c = workloads.CONFIGS[name]
    n, H = c["N"], c["H"]
    rows = workloads.sample_rows_per_head(c["config"], n, H, 256, c["n_text"])
    assert rows.shape == (H, 256)
    for h in range(H):
        r = rows[h]
        assert np.array_equal(r, np.unique(r)) and r.min() >= 0 and r.max() < n
        for forced in (0, n - 1, c["n_text"] - 1, c["n_text"], n - (n % 64 or 64)):
            assert forced in r
    covered = np.unique(np.concatenate([r // 32 for r in rows]))
    assert covered.size == -(-n // 32)
    # different heads draw different rows, and the draw is repeatable
    assert not np.array_equal(rows[0], rows[1])
    again = workloads.sample_rows_per_head(c["config"], n, H, 256, c["n_text"])
    assert np.array_equal(rows, again)


def test_rows_per_head_small_n():
    rows = workloads.sample_rows_per_head(1, 100, 3, 256)
    assert rows.shape == (3, 100)
    assert all(np.array_equal(r, np.arange(100)) for r in rows)
