"""Full-size a2av cases (1 and 4 GiB per rank) in the launch configuration the
benchmark times: split matrices and offsets compared whole against the
oracle, payload compared on sampled rows whose source the oracle computes one
by one (every chunk's first and last row plus random rows), and the round
trip with the transposed splits compared whole on the device."""
import numpy as np
import pytest
import torch

from embeddings_a2av_virtual_amd import inputs as I
from embeddings_a2av_virtual_amd.vranks import A2av

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _sample_rows(g, S, d, n_random=512):
    W = S.shape[0]
    tot = int(S[:, d].sum())
    if tot == 0:
        return []
    js = set(int(j) for j in g.integers(0, tot, size=n_random))
    start = 0
    for s in range(W):
        n = int(S[s, d])
        if n:
            js.update((start, start + n - 1))
        start += n
    return sorted(js)


def run_large(ref, W, mib, kind, seed, fused=True, R=8192):
    n = I.rows_for_mib(mib, R)
    g = I.rng(seed)
    S = I.uniform_splits(g, W, n) if kind == "uniform" else I.half_zero_splits(g, W, n)
    X = [I.payload_bytes(n, R, seed * 10 + s, device="cuda") for s in range(W)]
    cap = S.sum(axis=0)
    Y = [torch.empty((int(c), R), dtype=torch.uint8, device="cuda") for c in cap]
    st = A2av(W)
    st.set_splits(S)
    st(R, X, [n] * W, Y, [int(c) for c in cap], fused=fused)
    torch.cuda.synchronize()
    assert int(st.status.item()) == 0
    rst, rO = ref.exchange_splits(S)
    _, rso, rro = ref.offsets(S, rO)
    assert np.array_equal(st.O.cpu().numpy(), rO)
    assert np.array_equal(st.send_off.cpu().numpy(), rso)
    assert np.array_equal(st.recv_off.cpu().numpy(), rro)
    # sampled rows: the oracle names each sampled row's source
    for d in range(W):
        js = _sample_rows(g, S, d)
        src = [ref.source_of(S, d, j) for j in js]
        got = Y[d][torch.tensor(js, dtype=torch.int64, device="cuda")]
        for s in range(W):
            pick = [k for k, (ss, _) in enumerate(src) if ss == s]
            if not pick:
                continue
            rows = torch.tensor([src[k][1] for k in pick], dtype=torch.int64, device="cuda")
            want = X[s][rows]
            assert torch.equal(got[torch.tensor(pick, device="cuda")], want), \
                f"W={W} {mib} MiB {kind} R={R}: rank {d} rows from {s}"
    # round trip with the transposed splits, compared whole on the device
    back = [torch.empty((n, R), dtype=torch.uint8, device="cuda") for _ in range(W)]
    st2 = A2av(W)
    st2.S.copy_(st.O)
    st2(R, Y, [int(c) for c in cap], back, [n] * W)
    torch.cuda.synchronize()
    assert int(st2.status.item()) == 0
    for s in range(W):
        assert torch.equal(back[s], X[s]), f"round trip rank {s}"


@pytest.mark.parametrize("W", [4, 8])
def test_one_gib_per_rank(ref, W):
    _say("large", W, "1 GiB")
    run_large(ref, W, 1024, "uniform", 50 + W)


def test_one_gib_half_zero(ref):
    _say("large 4 1 GiB half zero")
    run_large(ref, 4, 1024, "half_zero", 60, fused=False)


def test_four_gib_per_rank(ref):
    _say("large 4 4 GiB")
    run_large(ref, 4, 4096, "uniform", 70)


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "3call"])
@pytest.mark.parametrize("W,mib,R,shape", [
    # rows 4 bytes past a multiple of 16: every source phase 0, 4, 8, 12
    (4, 160, 8196, "default"), (4, 160, 8196, "u16"),
    # 8-byte rows (keys): source phases 0 and 8
    (8, 80, 8, "default"), (8, 80, 8, "u16"),
    # more than 8 ranks: the prep workgroup, then the wave copy
    (12, 48, 8196, "default"),
])
def test_misaligned_rows_past_512_mib(ref, monkeypatch, W, mib, R, shape, fused):
    """More than 512 MiB on each side with rows that are not 16-byte
    multiples: chunks start at every 4-byte phase of the 16-byte grid and take
    the one-load misaligned path. In the default shapes, up to 8 ranks move
    4 KiB pieces with 4 vectors per lane in flight (every exchange of 64 MiB
    or more), and more ranks 32 KiB pieces with 16 in flight; "u16" sets the
    knobs so that up to 8 ranks take 32 KiB pieces with 16 in flight too."""
    if shape == "u16":
        monkeypatch.setenv("A2AV_WAVE_UNROLL", "16")
        monkeypatch.setenv("A2AV_WAVE_PIECE", "32768")
    _say("large misaligned", W, mib, R, shape, fused)
    run_large(ref, W, mib, "uniform", 90 + W + R % 7, fused=fused, R=R)
