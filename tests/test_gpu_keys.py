"""GPU parity of the owner-order bucketing of jagged embedding keys
(keys_bucketize) against the CPU oracle, and the whole key exchange
(bucketing, then keys and lengths as two a2av calls) at full size."""
import numpy as np
import pytest
import torch

from embeddings_a2av_virtual_amd import _binding as B
from embeddings_a2av_virtual_amd import inputs as I
from embeddings_a2av_virtual_amd.vranks import A2av
from gpu_util import GuardedBuffer, SENT, assert_same, gpu_a2av, ref_a2av, upload_rows

pytestmark = pytest.mark.gpu

KSENT = np.frombuffer(bytes([SENT] * 8), dtype=np.int64)[0]
LSENT = np.frombuffer(bytes([SENT] * 4), dtype=np.int32)[0]


def _say(*a):
    print(*a, flush=True)


def gpu_bucketize(W, NT, batch, lengths, keys, n_keys=None, status_init=0, pad=0):
    """lengths: per-rank int32 [NT, batch]; keys: per-rank int64. Returns
    (status, [lengths_out], [keys_out], split_keys, split_lengths, guards)."""
    n_keys = [k.size for k in keys] if n_keys is None else list(n_keys)
    lin = [upload_rows(l.reshape(-1).view(np.uint8), pad=pad) for l in lengths]
    kin = [upload_rows(k.view(np.uint8), pad=pad) for k in keys]
    lout = [GuardedBuffer(NT * batch * 4, pad=pad) for _ in range(W)]
    kout = [GuardedBuffer(n * 8, pad=pad) for n in n_keys]
    sk = torch.full((W, W), -7, dtype=torch.int64, device="cuda")
    sl = torch.full((W, W), -7, dtype=torch.int64, device="cuda")
    ws = torch.empty(B.keys_bucketize_workspace_bytes(W, NT), dtype=torch.uint8, device="cuda")
    status = torch.full((1,), status_init, dtype=torch.int32, device="cuda")
    B.keys_bucketize(W, NT, batch, [b.view for b in lin], [b.view for b in kin], n_keys,
                     [b.view for b in lout], [b.view for b in kout], sk, sl, ws, status)
    torch.cuda.synchronize()
    guards = all(b.guards_intact() for b in lin + kin + lout + kout)
    return (int(status.item()), [b.host().view(np.int32) for b in lout],
            [b.host().view(np.int64) for b in kout], sk.cpu().numpy(), sl.cpu().numpy(), guards)


def _inputs(g, W, NT, batch, lam=5.0, cap=20, extra=0):
    ranks = [I.emb_keys_rank(g, tables=NT, batch=batch, lam=lam, cap=cap, key_range=1 << 40)
             for _ in range(W)]
    lengths = [r.lengths for r in ranks]
    keys = [np.concatenate([r.keys, g.integers(0, 1 << 40, size=extra, dtype=np.int64)])
            for r in ranks]
    return lengths, keys


def _compare(ref, W, NT, batch, lengths, keys, got, n_keys=None):
    st, lo, ko, sk, sl, guards = got
    assert guards
    n_keys = [k.size for k in keys] if n_keys is None else n_keys
    agg = 0
    want = []
    for r in range(W):
        rst, rlo, rko, rsk, rsl = ref.keys_bucketize(W, NT, batch, lengths[r], keys[r][:n_keys[r]])
        want.append((rlo, rko, rsk, rsl))
        agg |= rst
        if rst == 0:
            assert np.array_equal(sk[r], rsk) and np.array_equal(sl[r], rsl), f"splits rank {r}"
        else:
            assert (sk[r] == -7).all() and (sl[r] == -7).all()
        if rst == 0 and st == 0:
            assert np.array_equal(lo[r], rlo), f"lengths rank {r}"
            used = int(rsk.sum())
            assert np.array_equal(ko[r][:used], rko[:used]), f"keys rank {r}"
            assert (ko[r][used:] == KSENT).all(), f"keys past the total, rank {r}"
    assert st == agg
    if st:
        assert all((l == LSENT).all() for l in lo) and all((k == KSENT).all() for k in ko)
    return want


@pytest.mark.parametrize("W,NT,batch,extra,pad", [
    (8, 26, 64, 0, 0),     # the key workload's table count, short batch
    (8, 26, 333, 5, 0),    # spare keys past the lengths' total
    (3, 7, 100, 0, 4),     # misaligned bases
    (5, 2, 10, 0, 0),      # fewer tables than ranks
    (4, 0, 10, 0, 0),      # no tables
    (2, 3, 0, 0, 0),       # empty batch
    (1, 5, 33, 1, 0),      # one rank
    (16, 300, 7, 0, 0),    # many tables: search over 300 blocks
    (32, 50, 5, 0, 4),     # keys and lengths in one block copy over 2W = 64 ranks
    (33, 40, 3, 0, 0),     # above 32 ranks: two block copies
])
def test_bucketize_matches_oracle(ref, W, NT, batch, extra, pad):
    _say("bucketize", W, NT, batch, extra, pad)
    g = I.rng(W * 100 + NT + batch)
    lengths, keys = _inputs(g, W, NT, batch, extra=extra)
    got = gpu_bucketize(W, NT, batch, lengths, keys, pad=pad)
    assert got[0] == 0
    _compare(ref, W, NT, batch, lengths, keys, got)


@pytest.mark.parametrize("case", ["negative", "overrun", "mixed", "poisoned"])
def test_bucketize_errors(ref, case):
    W, NT, batch = 4, 9, 50
    g = I.rng(12)
    lengths, keys = _inputs(g, W, NT, batch)
    n_keys = [k.size for k in keys]
    init = 0
    if case == "negative":
        lengths[2][4, 7] = -1
    elif case == "overrun":
        n_keys[1] -= 1
    elif case == "mixed":
        lengths[0][0, 0] = -3
        n_keys[3] -= 2
    else:
        init = 16
    keys = [k[:n] for k, n in zip(keys, n_keys)]
    got = gpu_bucketize(W, NT, batch, lengths, keys, status_init=init)
    if case == "poisoned":
        st, lo, ko, sk, sl, guards = got
        assert guards and st == init and (sk == -7).all() and (sl == -7).all()
        assert all((l == LSENT).all() for l in lo) and all((k == KSENT).all() for k in ko)
        return
    assert got[0] != 0
    _compare(ref, W, NT, batch, lengths, keys, got)
    if case == "mixed":
        assert got[0] == B.ST_BAD_SPLIT | B.ST_SEND_OVERRUN


def test_embedding_key_exchange_full(ref):
    """W=8, 26 tables, batch 8192, lengths min(Poisson(20), 100), int64 keys:
    bucketing by owner on the GPU, then keys (8-byte rows) and lengths (4-byte
    rows) as two a2av calls; the oracle runs the same chain."""
    W, NT, batch = 8, 26, 8192
    g = I.rng(88)
    ranks = [I.emb_keys_rank(g) for _ in range(W)]
    lengths = [r.lengths for r in ranks]
    keys = [r.keys for r in ranks]
    got = gpu_bucketize(W, NT, batch, lengths, keys)
    assert got[0] == 0
    want = _compare(ref, W, NT, batch, lengths, keys, got)
    _, lo, ko, Sk, Sl, _ = got
    _say("emb keys per rank", [k.size for k in keys])
    gk = gpu_a2av(8, [k.view(np.uint8).reshape(-1, 8) for k in ko], Sk)
    gl = gpu_a2av(4, [l.view(np.uint8).reshape(-1, 4) for l in lo], Sl)
    # the oracle's chain starts from its own bucketing
    rSk = np.stack([w[2] for w in want])
    rSl = np.stack([w[3] for w in want])
    assert_same(gk, ref_a2av(ref, 8, [w[1].view(np.uint8).reshape(-1, 8) for w in want], rSk), "keys")
    assert_same(gl, ref_a2av(ref, 4, [w[0].view(np.uint8).reshape(-1, 4) for w in want], rSl),
                "lengths")
    # the two calls agree: each received lengths chunk sums to its keys chunk
    for d in range(W):
        lv = gl[4][d].reshape(-1).view(np.int32)
        for s in range(W):
            assert lv[gl[3][d, s]:gl[3][d, s + 1]].sum() == gk[1][d, s]
    # and rank d holds exactly the tables it owns, from every source in order
    for d in range(W):
        own = list(range(d, NT, W))
        want = np.concatenate([lengths[s][own].reshape(-1) for s in range(W)])
        assert np.array_equal(gl[4][d].reshape(-1).view(np.int32), want)


# ------------------------------------------------------------------ fused exchange
def gpu_keys_exchange(W, NT, batch, lengths, keys, lcap=None, kcap=None, status_init=0, pad=0,
                      ref=None):
    """keys_exchange on the GPU; capacities default to the oracle's (what each
    receiver gets). Returns (status, [lengths_out], [keys_out], split_keys,
    split_lengths, recv_off, guards)."""
    if lcap is None or kcap is None:
        _, lo, ko, _, _, _ = ref.keys_exchange(W, NT, batch, lengths, keys)
        lcap = [x.size for x in lo] if lcap is None else lcap
        kcap = [x.size for x in ko] if kcap is None else kcap
    lin = [upload_rows(l.reshape(-1).view(np.uint8), pad=pad) for l in lengths]
    kin = [upload_rows(k.view(np.uint8), pad=pad) for k in keys]
    lout = [GuardedBuffer(int(c) * 4, pad=pad) for c in lcap]
    kout = [GuardedBuffer(int(c) * 8, pad=pad) for c in kcap]
    sk = torch.full((W, W), -7, dtype=torch.int64, device="cuda")
    sl = torch.full((W, W), -7, dtype=torch.int64, device="cuda")
    ro = torch.full((W, W + 1), -7, dtype=torch.int64, device="cuda")
    ws = torch.empty(B.keys_exchange_workspace_bytes(W, NT), dtype=torch.uint8, device="cuda")
    status = torch.full((1,), status_init, dtype=torch.int32, device="cuda")
    B.keys_exchange(W, NT, batch, [b.view for b in lin], [b.view for b in kin],
                    [k.size for k in keys], [b.view for b in lout], list(lcap),
                    [b.view for b in kout], list(kcap), sk, sl, ro, ws, status)
    torch.cuda.synchronize()
    guards = all(b.guards_intact() for b in lin + kin + lout + kout)
    return (int(status.item()), [b.host().view(np.int32) for b in lout],
            [b.host().view(np.int64) for b in kout], sk.cpu().numpy(), sl.cpu().numpy(),
            ro.cpu().numpy(), guards)


def _compare_exchange(got, want, what=""):
    st, lo, ko, sk, sl, ro, guards = got
    rst, rlo, rko, rsk, rsl, rro = want
    assert guards, what
    assert st == rst, f"{what}: status {st} != oracle {rst}"
    assert np.array_equal(sk, rsk) and np.array_equal(sl, rsl), f"{what}: splits"
    assert np.array_equal(ro, rro), f"{what}: receive offsets"
    for d in range(len(lo)):
        if st == 0:
            assert np.array_equal(lo[d], rlo[d]), f"{what}: lengths at {d}"
            assert np.array_equal(ko[d], rko[d]), f"{what}: keys at {d}"
        else:
            assert (lo[d] == LSENT).all() and (ko[d] == KSENT).all(), f"{what}: written at {d}"


@pytest.mark.parametrize("W,NT,batch,pad", [
    (8, 26, 64, 0), (8, 26, 333, 0), (3, 7, 100, 4), (5, 2, 10, 0), (4, 0, 10, 0), (2, 3, 0, 0),
    (1, 5, 33, 0), (16, 300, 7, 0), (64, 100, 3, 0), (3, 4096, 2, 0),
    # keys and lengths in one block copy over 2W ranks up to W = 32, two above
    (32, 40, 5, 4), (33, 50, 4, 0),
    # 63 blocks per receiver (the block copy stages the plan row), 64 and 72
    # (it searches the plan in global memory); more ranks than a DPP row
    (7, 63, 6, 4), (8, 64, 5, 0), (8, 65, 5, 0), (16, 32, 3, 0), (17, 20, 3, 0),
])
def test_keys_exchange_matches_oracle(ref, W, NT, batch, pad):
    _say("keys_exchange", W, NT, batch, pad)
    g = I.rng(W * 7 + NT + batch)
    lengths, keys = _inputs(g, W, NT, batch, lam=3.0, cap=10)
    want = ref.keys_exchange(W, NT, batch, lengths, keys)
    assert want[0] == 0
    got = gpu_keys_exchange(W, NT, batch, lengths, keys, pad=pad, ref=ref)
    _compare_exchange(got, want, f"W={W} NT={NT} batch={batch}")


@pytest.mark.parametrize("case", ["negative", "overrun", "keys_room", "lengths_room", "poisoned"])
@pytest.mark.parametrize("W,NT,batch", [(4, 9, 50), (8, 66, 6)])  # staged plan rows; searched in memory
def test_keys_exchange_errors(ref, case, W, NT, batch):
    g = I.rng(13)
    lengths, keys = _inputs(g, W, NT, batch)
    _, lo, ko, _, _, _ = ref.keys_exchange(W, NT, batch, lengths, keys)
    lcap = [x.size for x in lo]
    kcap = [x.size for x in ko]
    init = 0
    if case == "negative":
        lengths[3][1, 2] = -5
    elif case == "overrun":
        keys[0] = keys[0][:-3]
    elif case == "keys_room":
        kcap[2] -= 1
    elif case == "lengths_room":
        lcap[1] -= 1
    else:
        init = 8
    got = gpu_keys_exchange(W, NT, batch, lengths, keys, lcap, kcap, status_init=init)
    if case == "poisoned":
        st, lo_, ko_, sk, sl, ro, guards = got
        assert guards and st == init and (sk == -7).all() and (ro == -7).all()
        assert all((l == LSENT).all() for l in lo_) and all((k == KSENT).all() for k in ko_)
        return
    want = ref.keys_exchange(W, NT, batch, lengths, keys, np.array(lcap), np.array(kcap))
    assert want[0] != 0
    _compare_exchange(got, want, case)


def test_keys_exchange_full(ref):
    """W=8, 26 tables, batch 8192, lengths min(Poisson(20), 100): the fused
    exchange against the oracle's composition, every byte."""
    W, NT, batch = 8, 26, 8192
    g = I.rng(89)
    ranks = [I.emb_keys_rank(g) for _ in range(W)]
    lengths = [r.lengths for r in ranks]
    keys = [r.keys for r in ranks]
    want = ref.keys_exchange(W, NT, batch, lengths, keys)
    assert want[0] == 0
    got = gpu_keys_exchange(W, NT, batch, lengths, keys, ref=ref)
    _compare_exchange(got, want, "full")
    _say("keys_exchange full: keys received", [k.size for k in got[2]])


def test_keys_exchange_workspace_contents_do_not_matter(ref):
    """The exchange keeps its key counts (and, with a plan launch, the plan) in
    the workspace: whatever the workspace held before (zeros, all ones, random
    bytes, what the last call or a poisoned call left) the result is the
    oracle's, call after call on one workspace, and on a larger one."""
    W, NT, batch = 8, 26, 300
    g = I.rng(77)
    lengths, keys = _inputs(g, W, NT, batch, lam=4.0, cap=20)
    want = ref.keys_exchange(W, NT, batch, lengths, keys)
    lcap = [x.size for x in want[1]]
    kcap = [x.size for x in want[2]]
    need = B.keys_exchange_workspace_bytes(W, NT)
    ws = torch.empty(need + 4096, dtype=torch.uint8, device="cuda")
    lin = [upload_rows(l.reshape(-1).view(np.uint8)) for l in lengths]
    kin = [upload_rows(k.view(np.uint8)) for k in keys]

    def call(status_init=0, wsv=None):
        lout = [GuardedBuffer(c * 4) for c in lcap]
        kout = [GuardedBuffer(c * 8) for c in kcap]
        z = dict(dtype=torch.int64, device="cuda")
        sk, sl, ro = torch.full((W, W), -7, **z), torch.full((W, W), -7, **z), torch.full((W, W + 1), -7, **z)
        status = torch.full((1,), status_init, dtype=torch.int32, device="cuda")
        B.keys_exchange(W, NT, batch, [b.view for b in lin], [b.view for b in kin],
                        [k.size for k in keys], [b.view for b in lout], lcap, [b.view for b in kout],
                        kcap, sk, sl, ro, ws if wsv is None else wsv, status)
        torch.cuda.synchronize()
        return (int(status.item()), [b.host().view(np.int32) for b in lout],
                [b.host().view(np.int64) for b in kout], sk.cpu().numpy(), sl.cpu().numpy(),
                ro.cpu().numpy(), all(b.guards_intact() for b in lin + kin + lout + kout))

    fills = [("zeros", lambda: ws.zero_()), ("ones", lambda: ws.fill_(0xFF)),
             ("random", lambda: ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8,
                                                       device="cuda"))),
             ("as left", lambda: None)]
    for name, fill in fills:
        fill()
        torch.cuda.synchronize()
        for rep in range(2):
            _say("workspace", name, rep)
            _compare_exchange(call(), want, f"{name} {rep}")
    # a poisoned call leaves the counter as it was; the next call is whole
    st = call(status_init=8)
    assert st[0] == 8
    _compare_exchange(call(), want, "after a poisoned call")
    # a larger workspace holding other bytes, twice
    big = torch.empty(B.keys_exchange_workspace_bytes(W, 60), dtype=torch.uint8, device="cuda")
    big.fill_(0x5A)
    _compare_exchange(call(wsv=big), want, "larger workspace")
    _compare_exchange(call(wsv=big), want, "larger workspace again")
