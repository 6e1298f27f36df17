"""keys_exchange_noalloc (the library's fixed per-GPU scratch, no workspace)
against keys_exchange (a caller's workspace) on the same inputs, through the
C ABI: every output byte, split, offset and status word identical, on calls
in a row whose second is smaller than the first (the array keeps the first
call's contents), on an error case, against the oracle, and captured into a
HIP graph and replayed."""
import numpy as np
import pytest
import torch

from embeddings_a2av_virtual_amd import _binding as B
from embeddings_a2av_virtual_amd import inputs as I
from gpu_util import GuardedBuffer, SENT, upload_rows

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _inputs(W, NT, batch, seed, lam=20.0, cap=100):
    g = I.rng(seed)
    ranks = [I.emb_keys_rank(g, tables=NT, batch=batch, lam=lam, cap=cap) for _ in range(W)]
    return [r.lengths for r in ranks], [r.keys for r in ranks]


def _run(noalloc, W, NT, batch, lengths, keys, lcap, kcap):
    lin = [upload_rows(l.reshape(-1).view(np.uint8)) for l in lengths]
    kin = [upload_rows(k.view(np.uint8)) for k in keys]
    lout = [GuardedBuffer(int(c) * 4) for c in lcap]
    kout = [GuardedBuffer(int(c) * 8) for c in kcap]
    z = dict(dtype=torch.int64, device="cuda")
    sk = torch.full((W, W), -7, **z)
    sl = torch.full((W, W), -7, **z)
    ro = torch.full((W, W + 1), -7, **z)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    args = (W, NT, batch, [b.view for b in lin], [b.view for b in kin], [k.size for k in keys],
            [b.view for b in lout], list(lcap), [b.view for b in kout], list(kcap), sk, sl, ro)
    if noalloc:
        B.keys_exchange_noalloc(*args, status)
    else:
        ws = torch.empty(B.keys_exchange_workspace_bytes(W, NT), dtype=torch.uint8,
                         device="cuda")
        B.keys_exchange(*args, ws, status)
    torch.cuda.synchronize()
    assert all(b.guards_intact() for b in lin + kin + lout + kout)
    return (int(status.item()), [b.host() for b in lout], [b.host() for b in kout],
            sk.cpu().numpy(), sl.cpu().numpy(), ro.cpu().numpy())


def _same(a, b, what):
    assert a[0] == b[0], f"{what}: status {a[0]} != {b[0]}"
    for i in (3, 4, 5):
        assert np.array_equal(a[i], b[i]), f"{what}: matrix {i}"
    for i in (1, 2):
        for d, (x, y) in enumerate(zip(a[i], b[i])):
            assert np.array_equal(x, y), f"{what}: output {i} of rank {d}"


def _check_case(ref, W, NT, batch, seed, lcap=None, kcap=None, **kw):
    lengths, keys = _inputs(W, NT, batch, seed, **kw)
    want = ref.keys_exchange(W, NT, batch, lengths, keys)
    lcap = [x.size for x in want[1]] if lcap is None else lcap
    kcap = [x.size for x in want[2]] if kcap is None else kcap
    got = _run(True, W, NT, batch, lengths, keys, lcap, kcap)
    base = _run(False, W, NT, batch, lengths, keys, lcap, kcap)
    _same(got, base, f"W={W} NT={NT} batch={batch}")
    if got[0] == 0:
        for d in range(W):
            assert np.array_equal(got[1][d].view(np.int32), want[1][d])
            assert np.array_equal(got[2][d].view(np.int64), want[2][d])
    return got


def test_noalloc_equals_workspace_entry_twice_second_smaller(ref):
    _say("no-alloc: W=8 x 26 tables x 8192, then W=4 x 9 tables x 500")
    st = _check_case(ref, 8, 26, 8192, seed=501)
    assert st[0] == 0
    st = _check_case(ref, 4, 9, 500, seed=502, lam=6.0, cap=30)
    assert st[0] == 0


def test_noalloc_error_and_recovery(ref):
    """A receiver short of room for its keys: both entries give the same
    status and metadata and write no payload; the next call is whole again."""
    W, NT, batch = 5, 11, 300
    lengths, keys = _inputs(W, NT, batch, 503, lam=4.0, cap=20)
    want = ref.keys_exchange(W, NT, batch, lengths, keys)
    lcap = [x.size for x in want[1]]
    kcap = [x.size for x in want[2]]
    kcap[3] -= 1
    got = _run(True, W, NT, batch, lengths, keys, lcap, kcap)
    base = _run(False, W, NT, batch, lengths, keys, lcap, kcap)
    _same(got, base, "short receiver")
    assert got[0] == B.ST_RECV_OVERFLOW
    assert all((x == SENT).all() for x in got[1] + got[2])
    st = _check_case(ref, 3, 7, 100, seed=504, lam=3.0, cap=10)
    assert st[0] == 0


def test_noalloc_refuses_sizes_beyond_its_scratch():
    W, NT = 64, 4096
    assert B.keys_exchange_workspace_bytes(W, NT) > B.NOALLOC_SCRATCH_BYTES
    dummy = torch.zeros(8, dtype=torch.uint8, device="cuda")
    z = torch.zeros((W, W + 1), dtype=torch.int64, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(B.A2avError) as e:
        B.keys_exchange_noalloc(W, NT, 1, [dummy] * W, [dummy] * W, [0] * W, [dummy] * W,
                                [0] * W, [dummy] * W, [0] * W, z, z, z, status)
    assert e.value.code == B.EARG
    torch.cuda.synchronize()
    assert int(status.item()) == 0


def test_noalloc_under_graph_capture(ref):
    """The callers it is for include code under HIP graph capture: the entry
    captured once (after an eager call has looked up the scratch's address)
    and replayed four times, with unrelated eager work between replays, gives
    the workspace entry's bytes every time."""
    W, NT, batch = 8, 26, 256
    lengths, keys = _inputs(W, NT, batch, 31)
    rst, wlo, wko, wsk, wsl, wro = ref.keys_exchange(W, NT, batch, lengths, keys)
    assert rst == 0
    want = _run(False, W, NT, batch, lengths, keys, [x.size for x in wlo], [x.size for x in wko])
    assert want[0] == 0
    lin = [torch.from_numpy(l.reshape(-1)).cuda() for l in lengths]
    kin = [torch.from_numpy(k).cuda() for k in keys]
    lo = [torch.zeros(x.size, dtype=torch.int32, device="cuda") for x in wlo]
    ko = [torch.zeros(x.size, dtype=torch.int64, device="cuda") for x in wko]
    z = dict(dtype=torch.int64, device="cuda")
    sk, sl, ro = torch.zeros((W, W), **z), torch.zeros((W, W), **z), torch.zeros((W, W + 1), **z)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")

    def call():
        B.keys_exchange_noalloc(W, NT, batch, lin, kin, [k.size for k in keys], lo,
                                [x.size for x in wlo], ko, [x.size for x in wko], sk, sl, ro, status)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        call()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            call()
    torch.cuda.synchronize()
    for i in range(4):
        for x in lo + ko + [sk, sl, ro]:
            x.zero_()
        status.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _say("graph replay", i)
        got = (int(status.item()), [x.cpu().numpy().view(np.uint8) for x in lo],
               [x.cpu().numpy().view(np.uint8) for x in ko], sk.cpu().numpy(), sl.cpu().numpy(),
               ro.cpu().numpy())
        _same(got, want, f"replay {i}")
        x = torch.randn(1 << 20, device="cuda")
        (x * 2).sum().item()
        torch.cuda.synchronize()
