"""The payload kernels' last-line bounds check (``span_fits``), compiled for
the host from the very header the kernels include, against exact integer
arithmetic. The corrupt cases are the ones a check written as a sum lets
through: a row count or start whose sum with the other wraps past 2^64 (or
past 2^63 when read as signed) back below the capacity."""
import os
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "embeddings_a2av_virtual_amd", "csrc")
M64 = (1 << 64) - 1


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("bounds") / "bounds_driver")
    subprocess.run(["g++", "-O2", "-std=c++17", "-Wall", "-Werror", f"-I{CSRC}", "-o", exe,
                    os.path.join(ROOT, "tests", "bounds_driver.cpp")], check=True)
    return exe


def run(exe, triples):
    inp = "".join(f"{r0} {n} {cap}\n" for r0, n, cap in triples)
    out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
    return [int(x) for x in out.split()]


def exact(r0, n, cap):
    """Rows [r0, r0 + n) inside [0, cap), in exact arithmetic (r0 and n read
    as the unsigned 64-bit integers the kernels pass)."""
    return int(r0 + n <= cap)


def s64(x):
    """The unsigned 64-bit pattern of a signed value (a corrupt negative count)."""
    return x & M64


CORRUPT = [
    # (r0, n, cap): each passes "r0 + n <= cap" once the sum wraps
    (M64 - 4, 10, 100),            # r0 near 2^64: the sum wraps to 5
    (5, s64(-3), 100),             # a negative count: the sum is 2
    (s64(-1), 1, 0),               # r0 = -1, n = 1: the sum is 0
    (1 << 63, 1 << 63, 7),         # two halves of 2^64: the sum is 0
    (s64(-(1 << 62)), (1 << 62) + 3, 3),  # signed: the sum is 3 exactly
    (3, M64, 2),                   # n = 2^64 - 1: the sum is 2
    (M64, M64, 1 << 62),           # both maximal: the sum is 2^64 - 2, wraps to -2 signed
]


def test_corrupt_pairs_are_refused(driver):
    got = run(driver, CORRUPT)
    for (r0, n, cap), g in zip(CORRUPT, got):
        assert (r0 + n) % (1 << 64) <= cap or ((r0 + n) % (1 << 64)) >= (1 << 63), \
            "each corrupt case defeats a summed check (unsigned or signed)"
        assert exact(r0, n, cap) == 0
        assert g == 0, (r0, n, cap)


def test_exact_limits(driver):
    cases = []
    for cap in (0, 1, 2, 7, 1000, (1 << 62), (1 << 63) - 1):
        for r0 in {0, 1, cap // 2, cap - 1 if cap else 0, cap, cap + 1}:
            for n in {0, 1, cap - r0 if cap >= r0 else 0, cap - r0 + 1 if cap >= r0 else 1}:
                cases.append((r0 & M64, n & M64, cap))
    got = run(driver, cases)
    for c, g in zip(cases, got):
        assert g == exact(*c), c


def test_brute_force_small(driver):
    cases = [(r0, n, cap) for cap in range(9) for r0 in range(11) for n in range(11)]
    # and the same magnitudes as negative counts or starts
    cases += [(s64(-r0), n, cap) for cap in range(5) for r0 in range(1, 6) for n in range(8)]
    cases += [(r0, s64(-n), cap) for cap in range(5) for r0 in range(8) for n in range(1, 6)]
    got = run(driver, cases)
    assert got == [exact(*c) for c in cases]


def test_random_near_the_wrap_points(driver):
    g = np.random.default_rng(7)
    cases = []
    for _ in range(4000):
        cap = int(g.integers(0, 1 << 62)) * int(g.integers(1, 3))
        pick = g.integers(0, 4)
        base = [0, 1 << 63, 1 << 64, cap][pick]
        r0 = (base - int(g.integers(0, 1 << 20))) & M64
        n = (cap - r0 + int(g.integers(-4, 5))) & M64
        cases.append((r0, n, cap))
    got = run(driver, cases)
    assert got == [exact(*c) for c in cases]
