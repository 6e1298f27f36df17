"""The payload kernels' tuning settings (piece size, loads in flight per
lane, LDS reserved to limit workgroups per CU) change only the schedule:
every setting gives the same bytes as the oracle, aligned and not, for the
one-call and the copy-only entries, with W <= 8 and W > 8."""
import numpy as np
import pytest

from embeddings_a2av_virtual_amd import inputs as I
from gpu_util import assert_same, gpu_a2av, random_rows, ref_a2av

pytestmark = pytest.mark.gpu

SETTINGS = [
    (4096, 4, 0), (4096, 4, 32768), (8192, 8, 0), (8192, 8, 32768), (32768, 16, 0),
    (4096, 16, 16384), (65536, 8, 0),
]


@pytest.mark.parametrize("piece,unroll,lds", SETTINGS)
@pytest.mark.parametrize("W,R,pad", [(4, 8192, 0), (8, 8196, 4), (16, 512, 0), (3, 24, 8)])
@pytest.mark.parametrize("fused", [False, True], ids=["3call", "fused"])
def test_settings_give_the_same_bytes(ref, monkeypatch, piece, unroll, lds, W, R, pad, fused):
    print("knobs", piece, unroll, lds, W, R, pad, fused, flush=True)
    monkeypatch.setenv("A2AV_WAVE_PIECE", str(piece))
    monkeypatch.setenv("A2AV_WAVE_UNROLL", str(unroll))
    monkeypatch.setenv("A2AV_WAVE_LDS", str(lds))
    g = I.rng(4000 + W * 7 + R % 97 + piece // 4096 + unroll + lds // 8192)
    S = I.random_splits(g, W, max(2, 600_000 // (R * W)), 0.25)
    X = [random_rows(g, S[s].sum(), R) for s in range(W)]
    assert_same(gpu_a2av(R, X, S, in_pad=pad, out_pad=pad, fused=fused), ref_a2av(ref, R, X, S),
                f"piece={piece} unroll={unroll} lds={lds} W={W} R={R}")
