"""Host-side checks of the workgroup-timeline summary (mask_aware_flashattention_amd.wg_timeline):
hand-made records with known answers."""

import numpy as np
import pytest

from mask_aware_flashattention_amd.wg_timeline import TICK_US, render, summarize


def rec(t0, t1, t2, t3, cu, xcc, tiles):
    return [t0, t1, t2, t3, (cu << 8) | (xcc << 32), tiles, 0, 0]


def test_summary_of_known_records():
    # XCD 0, CU 1: two workgroups back to back (gap 50 ticks), then a third beside the second;
    # XCD 1, CU 2: one workgroup without tiles (its rows fully masked)
    rows = np.array([
        rec(0, 400, 2400, 2600, 1, 0, 10),      # start 4 us, walk 20 us / 10 tiles, end 2 us
        rec(2650, 2950, 4950, 5150, 1, 0, 20),  # start 3 us, walk 20 us / 20 tiles
        rec(3000, 3300, 3900, 4000, 1, 0, 3),   # start 3 us, walk 6 us / 3 tiles
        rec(100, 0, 0, 300, 2, 1, 0),           # empty list: no walk
    ], dtype=np.int64)
    s = summarize(rows)
    assert s["workgroups"] == 4 and s["tiles"] == 33 and s["compute_units"] == 2
    assert s["span_us"] == pytest.approx(5150 * TICK_US)
    assert s["start_to_first_tile_us"] == pytest.approx((4 + 3 + 3) / 3)
    assert s["walk_per_tile_us"] == pytest.approx((20 + 20 + 6) / 33)
    assert s["walk_end_to_end_us"] == pytest.approx((2 + 2 + 1) / 3)
    assert [b[:3] for b in s["by_walk_length"]] == [(2, 5, 1), (10, 20, 1), (20, 40, 1)]
    # CU 1 from 0 to 5150: one workgroup 0-2600 and 2650-3000 and 4000-5150, none 2600-2650,
    # two 3000-4000; CU 2: none 0-100 and 300-5150, one 100-300
    occ = np.array([50 + 100 + 4850, 2600 + 350 + 1150 + 200, 1000, 0], dtype=float)
    assert np.allclose(s["residency"], occ / occ.sum())
    # refills: the second workgroup takes the first one's slot 50 ticks after it ended; the
    # third fills the compute unit's other slot (a first fill, not a refill)
    assert s["refill_gap_us"] == pytest.approx((0.5, 0.5))
    assert s["cu_end_us"][2] == pytest.approx(51.5)
    assert s["xcd_end_us"] == pytest.approx((3.0, 51.5))
    table = render("test", {"fwd": s})
    assert "| walk per tile | 1.394 |" in table and "forward" in table
