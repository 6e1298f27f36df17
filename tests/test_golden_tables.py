"""The GB/s convention of the benchmark against the timing tables printed on
the tuning page (no GPU): bandwidth = bytes / time with GB = 10^9 and MiB =
2^20, no (W-1)/W factor, and the size printed as 0 is 0.5 MiB."""
import os

import pytest

import bench

HERE = os.path.dirname(os.path.abspath(__file__))


def rows():
    out = []
    for line in open(os.path.join(HERE, "golden", "a2av_tables.txt")):
        if line.startswith("#") or not line.strip():
            continue
        table, mib, us, gbs = line.split()
        out.append((table, float(mib) or 0.5, float(us), float(gbs)))
    return out


def test_table_has_every_row():
    r = rows()
    assert len(r) == 28
    assert {t for t, *_ in r} == {"before", "after"}


@pytest.mark.parametrize("table,mib,us,gbs", rows())
def test_busbw_is_bytes_over_time(table, mib, us, gbs):
    got = bench.gbps(mib * (1 << 20), us * 1e-6)
    # printed values carry 2 decimals of time and bandwidth
    assert got == pytest.approx(gbs, rel=2e-3, abs=0.02)


def test_other_conventions_do_not_fit():
    """A (W-1)/W factor, GiB units or a 1 MiB first row would each miss the
    printed numbers, so the reading above is the only one of these that fits."""
    r = rows()
    ok = lambda f: all(abs(f(m, u) - g) <= max(2e-3 * g, 0.02) for _, m, u, g in r)
    assert ok(lambda m, u: bench.gbps(m * (1 << 20), u * 1e-6))
    assert not ok(lambda m, u: bench.gbps(m * (1 << 20), u * 1e-6) * 3 / 4)
    assert not ok(lambda m, u: m * (1 << 20) / (u * 1e-6) / (1 << 30))
    assert not ok(lambda m, u: bench.gbps((m if m >= 1 else 1) * (1 << 20), u * 1e-6))
