"""Grids smaller than the work. The copy, scatter, gather and combine kernels
launch one wave per piece, row or slot and loop over the rest when the grid
does not cover them; by default only inputs of more than 2^22 workgroups'
worth (64 GiB of traffic in 4 KiB pieces) reach those later passes.
A2AV_MAX_GRID caps the grid, so that here every entry point runs them on
small inputs, with grids of 1, 3 and 7 workgroups, and gives the oracle's
bytes (the parity tests of each entry point, run under the cap), errors
included."""
import pytest
import torch

from embeddings_a2av_virtual_amd import _binding as B
from embeddings_a2av_virtual_amd import inputs as I
from gpu_util import assert_same, gpu_a2av, random_rows, ref_a2av

import test_gpu_a2av as TA
import test_gpu_ceilings as TG
import test_gpu_combine as TC
import test_gpu_keys as TK
import test_gpu_moe as TM
import test_gpu_pack_dispatch as TP
import test_gpu_regroup as TR

pytestmark = pytest.mark.gpu

GRIDS = ["1", "3", "7"]


@pytest.fixture(params=GRIDS, ids=[f"grid{g}" for g in GRIDS])
def small_grid(request, monkeypatch):
    monkeypatch.setenv("A2AV_MAX_GRID", request.param)
    print("A2AV_MAX_GRID", request.param, flush=True)
    return int(request.param)


@pytest.mark.parametrize("W,R,pad", [(4, 8192, 0), (8, 8196, 4), (12, 512, 0), (3, 24, 8),
                                     (20, 16, 0)])
@pytest.mark.parametrize("fused", [False, True], ids=["3call", "fused"])
def test_a2av(ref, small_grid, W, R, pad, fused):
    g = I.rng(7100 + W * 13 + R % 89 + small_grid)
    S = I.random_splits(g, W, max(2, 400_000 // (R * W)), 0.25)
    X = [random_rows(g, S[s].sum(), R) for s in range(W)]
    assert_same(gpu_a2av(R, X, S, in_pad=pad, out_pad=pad, fused=fused), ref_a2av(ref, R, X, S),
                f"grid={small_grid} W={W} R={R}")


@pytest.mark.parametrize("W,R", [(4, 16), (12, 24)])
@pytest.mark.parametrize("fused", [False, True], ids=["3call", "fused"])
def test_a2av_errors(ref, monkeypatch, small_grid, W, R, fused):
    TA.test_error_paths_match_oracle(ref, monkeypatch, fused, W, R, "wave")


def test_a2av_foreign_offsets(ref, monkeypatch, small_grid):
    TA.test_copy_rejects_foreign_offsets(ref, monkeypatch, 4, 16, "wave")


@pytest.mark.parametrize("nbytes", [4096 * 9 + 48, (1 << 20) + 4096 * 3 + 16])
def test_plain_copy_and_streams(small_grid, nbytes):
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda")
    dst = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    B.a2av_device_copy(dst, src, nbytes)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    TG.test_read_loads_every_vector(nbytes)
    TG.test_fill_writes_its_pattern_and_nothing_else(nbytes, True)


@pytest.mark.parametrize("case", [(8, 300, 8, 256, 1024, "zipf", 0),
                                  (4, 1500, 3, 12, 10, "uniform", 0),
                                  (2, 700, 2, 2, 16, "uniform", 4)])
def test_moe_pack_unpack(ref, small_grid, case):
    TM.test_moe_pack_round_trip_matches_oracle(ref, *case)


@pytest.mark.parametrize("case", [(8, 256, 1024, 3, 0, 0), (3, 12, 10, 50, 4, 1),
                                  (8, 64, 48, 9, 0, 1)])
def test_regroup(ref, small_grid, case):
    TR.test_regroup_matches_oracle(ref, *case)


@pytest.mark.parametrize("case", [(8, 256, 1024, 3, 0), (3, 12, 10, 50, 4)])
@pytest.mark.parametrize("direction", [0, 1])
def test_grouped(ref, small_grid, case, direction):
    TR.test_grouped_matches_oracle(ref, *case, direction)


@pytest.mark.parametrize("case", [(8, 26, 64, 0, 0), (3, 7, 100, 0, 4), (16, 300, 7, 0, 0),
                                  (33, 40, 3, 0, 0)])
def test_bucketize(ref, small_grid, case):
    TK.test_bucketize_matches_oracle(ref, *case)


@pytest.mark.parametrize("case", [(8, 26, 64, 0), (3, 7, 100, 4), (8, 65, 5, 0), (33, 50, 4, 0)])
def test_keys_exchange(ref, small_grid, case):
    TK.test_keys_exchange_matches_oracle(ref, *case)


@pytest.mark.parametrize("case", [TP.SHAPES[0], TP.SHAPES[2], TP.SHAPES[3]])
@pytest.mark.parametrize("layout", [0, 1])
def test_pack_dispatch_and_return(ref, small_grid, case, layout):
    TP.test_pack_dispatch_matches_oracle(ref, *case, layout)


@pytest.mark.parametrize("case", [TP.COMBINE_SHAPES[0], TP.COMBINE_SHAPES[2],
                                  TP.COMBINE_SHAPES[4]])
@pytest.mark.parametrize("layout", [0, 1])
def test_combine_return(ref, small_grid, case, layout):
    TP.test_combine_return_matches_oracle(ref, *case, layout)


@pytest.mark.parametrize("case", [(8, 40, 8, 7168, 0, True), (2, 50, 5, 77, 0, True),
                                  (3, 9, 70, 512, 0, True)])
def test_combine(ref, small_grid, case):
    TC.test_combine_matches_oracle(ref, *case)


@pytest.mark.parametrize("case", [(8, 30, 8, 256, 1000, 0, True, True),
                                  (4, 50, 3, 12, 77, 0, True, False)])
def test_combine_grouped(ref, small_grid, case):
    TC.test_combine_grouped_matches_oracle(ref, *case)

