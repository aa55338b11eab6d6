"""The phase-timing summary (fp8_blockwise_quantized_amd/phase_timing.py) on
hand-made records: two CUs, one launch of four 512-thread workgroups and one
of two 256-thread workgroups sharing a CU, wall counter at 100 MHz."""
import numpy as np

from fp8_blockwise_quantized_amd.phase_timing import summarise


def rec(t0, t1, t2, t3, cu, grid, threads, clocks):
    hw = cu << 8                                    # CU id in HW_ID bits 8..11
    return [t0, t1, t2, t3, hw, grid | (threads << 32), 0, clocks]


def test_summary_of_one_launch():
    # CU 0 runs workgroups 0 and 2, CU 1 runs 1 and 3; 10 ns ticks
    r = np.array([rec(100, 110, 1110, 1160, 0, 4, 512, 2000),
                  rec(100, 120, 1120, 1170, 1, 4, 512, 2000),
                  rec(1200, 1210, 2210, 2260, 0, 4, 512, 2000),
                  rec(1170, 1180, 2180, 2230, 1, 4, 512, 2000)], dtype=np.uint64)
    (row,) = summarise(r, 100000.0, ksteps=10)
    assert row["grid"] == 4 and row["threads"] == 512 and row["complete"] and row["tiles"] == 4
    assert np.isclose(row["setup"], 0.1)             # 10 ticks
    assert np.isclose(row["loop"], 10.0) and np.isclose(row["step"], 1.0)
    assert np.isclose(row["epi"], 0.5)
    assert np.isclose(row["mhz"], 200.0)             # 2000 clocks over 10 us
    assert np.isclose(row["clk_step"], 200.0) and np.isclose(row["mfma_share"], 2048 / 200.0)
    assert np.isclose(row["span"], 21.6)             # 100 .. 2260
    # CU 0 busy 10.6 + 10.6 us, CU 1 10.7 + 10.6 us
    assert np.isclose(row["busy"], (21.2 + 21.3) / 2 / 21.6)
    assert np.isclose(row["gap"], np.median([0.4, 0.0]))
    assert np.isclose(row["tail"], (0.0 + 0.3) / 2)


def test_two_launches_and_overlapping_workgroups():
    big = [rec(100, 110, 1110, 1160, 0, 3, 512, 2000)]          # 1 of 3 records: incomplete
    small = [rec(2000, 2010, 2510, 2530, 0, 2, 256, 1000),     # two at once on one CU
             rec(2005, 2015, 2615, 2640, 0, 2, 256, 1200)]
    rows = summarise(np.array(big + small, dtype=np.uint64), 100000.0, ksteps=5)
    assert [r["grid"] for r in rows] == [3, 2]
    assert not rows[0]["complete"] and "span" not in rows[0]
    s = rows[1]
    assert s["complete"] and s["gap"] is None
    assert np.isclose(s["span"], 6.4)                # 2000 .. 2640
    assert np.isclose(s["busy"], 1.0)                # the CU holds one of them throughout
    assert np.isclose(s["mfma_share"], 512 / s["clk_step"])
