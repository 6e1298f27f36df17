"""The piece walk of the a2av copy for more than 8 ranks (wave_walk.h), run on
the host by a model of a 64-lane wave (tests/wave_walk_host.cpp) that executes
the kernel's own code with 64 threads in lockstep. The model stops on a
cross-lane operation that some lane does not reach, or lanes that reach
different ones, and on any load or copy outside its buffers. With offsets
from the oracle, the walk's outputs equal the oracle's a2av byte for byte and
every received byte is written exactly once; with corrupt offsets (which the
launch before the walk would refuse, but which it must survive) it stays
inside the buffers."""
import os
import subprocess

import numpy as np
import pytest

from embeddings_a2av_virtual_amd import inputs as I

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "embeddings_a2av_virtual_amd", "csrc")
SENT = 0xA5


@pytest.fixture(scope="module")
def model(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("walk") / "wave_walk_host")
    subprocess.run(["g++", "-O2", "-std=c++17", "-Wall", "-Werror", "-pthread", f"-I{CSRC}", "-o",
                    exe, os.path.join(ROOT, "tests", "wave_walk_host.cpp")], check=True)
    return exe


def run_model(exe, tmp_path, W, R, piece, waves, in_rows, cap, recv_off, send_off, X):
    case = tmp_path / "case.bin"
    out = tmp_path / "out.bin"
    with open(case, "wb") as f:
        np.array([W, R, piece, waves], dtype=np.int64).tofile(f)
        for a in (in_rows, cap, recv_off, send_off):
            np.ascontiguousarray(a, dtype=np.int64).tofile(f)
        for x in X:
            np.ascontiguousarray(x, dtype=np.uint8).tofile(f)
    p = subprocess.run([exe, str(case), str(out)], capture_output=True, text=True, timeout=600)
    if p.returncode != 0:
        raise AssertionError(f"wave model stopped ({p.returncode}): {p.stderr.strip()}")
    data = np.fromfile(out, dtype=np.uint8)
    total = int(np.sum(np.asarray(cap, dtype=np.int64))) * R
    ys, counts, o = [], [], 0
    for c in cap:
        ys.append(data[o:o + int(c) * R])
        counts.append(data[total + o: total + o + int(c) * R])
        o += int(c) * R
    return ys, counts


CASES = [
    # W, R, rows per source at most, fraction of zero splits, piece bytes, waves
    (9, 48, 40, 0.0, 4096, 5),
    (12, 24, 30, 0.3, 1000, 7),
    (16, 64, 25, 0.5, 4096, 3),
    (20, 8, 50, 0.2, 512, 11),
    (33, 48, 12, 0.3, 4096, 4),
    (64, 48, 10, 0.3, 4096, 9),
    (64, 16, 6, 0.8, 700, 13),
    (17, 8196, 3, 0.2, 32768, 2),
]


@pytest.mark.parametrize("W,R,max_rows,zero,piece,waves", CASES)
def test_walk_equals_the_oracle(ref, model, tmp_path, W, R, max_rows, zero, piece, waves):
    g = I.rng(W * 31 + R)
    S = I.random_splits(g, W, max_rows, zero)
    n = S.sum(axis=1) + g.integers(0, 3, size=W)    # some rows stay home
    cap = S.sum(axis=0) + g.integers(0, 3, size=W)  # some room left over
    X = [g.integers(0, 256, size=(int(n[s]), R), dtype=np.uint8) for s in range(W)]
    Y = [np.full((int(c), R), SENT, dtype=np.uint8) for c in cap]
    st, O, so, ro = ref.a2av(R, [x.reshape(-1) for x in X], n.astype(np.int64),
                             [y.reshape(-1) for y in Y], cap.astype(np.int64), S)
    assert st == 0
    ys, counts = run_model(model, tmp_path, W, R, piece, waves, n, cap, ro, so, X)
    for d in range(W):
        assert np.array_equal(ys[d], Y[d].reshape(-1)), f"destination {d}"
        got = int(ro[d, W]) * R
        assert (counts[d][:got] == 1).all(), f"destination {d}: a byte written other than once"
        assert (counts[d][got:] == 0).all(), f"destination {d}: written past its total"


def test_walk_degenerate(ref, model, tmp_path):
    """Every split zero, one destination takes everything, all on the diagonal."""
    W, R = 16, 40
    for name, S in (("zero", np.zeros((W, W), np.int64)),
                    ("to_one", np.tile(np.eye(W, dtype=np.int64)[5] * 7, (W, 1))),
                    ("diagonal", np.diag(np.arange(W, dtype=np.int64)))):
        n = S.sum(axis=1)
        cap = S.sum(axis=0)
        g = I.rng(7)
        X = [g.integers(0, 256, size=(int(n[s]), R), dtype=np.uint8) for s in range(W)]
        Y = [np.full((int(c), R), SENT, dtype=np.uint8) for c in cap]
        st, O, so, ro = ref.a2av(R, [x.reshape(-1) for x in X], n, [y.reshape(-1) for y in Y],
                                 cap, S)
        assert st == 0
        ys, counts = run_model(model, tmp_path, W, R, 4096, 3, n, cap, ro, so, X)
        for d in range(W):
            assert np.array_equal(ys[d], Y[d].reshape(-1)), f"{name}: destination {d}"
            assert (counts[d] == 1).all(), f"{name}: destination {d}"


CORRUPT = ["recv_row_wraps", "recv_negative", "send_huge", "send_negative", "recv_total_huge",
           "recv_descending"]


@pytest.mark.parametrize("how", CORRUPT)
def test_walk_stays_in_bounds_on_corrupt_offsets(ref, model, tmp_path, how):
    """Offsets the checking launch would refuse, fed to the walk anyway: every
    access must stay inside the caller's buffers (the model stops otherwise)."""
    W, R = 12, 32
    g = I.rng(40 + CORRUPT.index(how))
    S = I.random_splits(g, W, 20, 0.2)
    n = S.sum(axis=1)
    cap = S.sum(axis=0)
    X = [g.integers(0, 256, size=(int(n[s]), R), dtype=np.uint8) for s in range(W)]
    Y = [np.full((int(c), R), SENT, dtype=np.uint8) for c in cap]
    st, O, so, ro = ref.a2av(R, [x.reshape(-1) for x in X], n, [y.reshape(-1) for y in Y], cap, S)
    assert st == 0
    so, ro = so.copy(), ro.copy()
    big = np.int64(2 ** 63 - 5)
    if how == "recv_row_wraps":
        ro[3, 5] = -ro[3, 6] + 2          # the next entry minus this one wraps
    elif how == "recv_negative":
        ro[4, 2:] -= 1000
    elif how == "send_huge":
        so[:, 3] = big
    elif how == "send_negative":
        so[2, :] = -7
    elif how == "recv_total_huge":
        ro[1, W] = big
    else:
        ro[6, 1:W] = ro[6, 1:W][::-1]
    run_model(model, tmp_path, W, R, 1024, 5, n, cap, ro, so, X)


@pytest.mark.parametrize("plant", ["ballot_under_lane_branch", "readlane_under_lane_branch"])
def test_model_stops_on_a_divergent_cross_lane_operation(ref, tmp_path, plant):
    """The model is built against a copy of wave_walk.h with a planted mistake:
    a cross-lane operation only some lanes reach (the mistake that, on the
    GPU, lets a lane read a value no lane wrote). It must stop with code 4."""
    src = open(os.path.join(CSRC, "wave_walk.h")).read()
    if plant == "ballot_under_lane_branch":
        old = "const uint64_t mask_s = wv.ballot(5, lane < W && dbase + ro * R <= lo);"
        new = "uint64_t mask_s = 0;\n        if (lane < W) mask_s = wv.ballot(5, dbase + ro * R <= lo);"
    else:
        old = "const uint64_t nn = wv.readlane(6, n, s);"
        new = "const uint64_t nn = lane == W - 1 ? n : wv.readlane(6, n, s);"
    assert old in src
    planted = tmp_path / "planted"
    planted.mkdir()
    (planted / "wave_walk.h").write_text(src.replace(old, new))
    exe = str(tmp_path / "model_planted")
    subprocess.run(["g++", "-O2", "-std=c++17", "-pthread", f"-I{planted}", f"-I{CSRC}", "-o", exe,
                    os.path.join(ROOT, "tests", "wave_walk_host.cpp")], check=True)
    W, R = 12, 32
    g = I.rng(3)
    S = I.random_splits(g, W, 20, 0.2)
    n, cap = S.sum(axis=1), S.sum(axis=0)
    X = [g.integers(0, 256, size=(int(n[s]), R), dtype=np.uint8) for s in range(W)]
    Y = [np.full((int(c), R), SENT, dtype=np.uint8) for c in cap]
    st, O, so, ro = ref.a2av(R, [x.reshape(-1) for x in X], n, [y.reshape(-1) for y in Y], cap, S)
    with pytest.raises(AssertionError, match=r"stopped \(4\)"):
        run_model(exe, tmp_path, W, R, 1024, 3, n, cap, ro, so, X)
