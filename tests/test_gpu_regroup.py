"""GPU parity of the receive-side expert regroup (moe_regroup) against the
CPU oracle: bit-exact bytes, expert offsets and status, at small ragged
shapes, on error paths, and at the full dispatch size."""
import numpy as np
import pytest
import torch

from embeddings_a2av_virtual_amd import _binding as B
from embeddings_a2av_virtual_amd import inputs as I
from gpu_util import SENT, GuardedBuffer, random_rows, upload_rows

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _owned_total(counts, W, E, d):
    P = E // W
    return int(counts[:, d * P:(d + 1) * P].sum())


def gpu_regroup(W, E, R, counts, X, in_rows=None, cap=None, direction=0, pad=0, status_init=0):
    """X: per-rank host uint8 [rows, R]. Returns (status, [out host], eoff [W, P+1], guards)."""
    P = E // W
    in_rows = [x.shape[0] for x in X] if in_rows is None else list(in_rows)
    cap = in_rows if cap is None else list(cap)
    ins = [upload_rows(x, pad=pad) for x in X]
    outs = [GuardedBuffer(int(c) * R, pad=pad) for c in cap]
    cnt = torch.from_numpy(np.ascontiguousarray(counts, dtype=np.int64)).cuda()
    eoff = torch.full((W, P + 1), -7, dtype=torch.int64, device="cuda")
    ws = torch.empty(B.moe_regroup_workspace_bytes(W, E), dtype=torch.uint8, device="cuda")
    status = torch.full((1,), status_init, dtype=torch.int32, device="cuda")
    B.moe_regroup(W, E, R, cnt, [b.view for b in ins], in_rows, [b.view for b in outs], cap, eoff,
                  direction, ws, status)
    torch.cuda.synchronize()
    guards = all(b.guards_intact() for b in outs + ins)
    return int(status.item()), [b.host().reshape(-1, R) for b in outs], eoff.cpu().numpy(), guards


def ref_regroup(ref, W, E, R, counts, X, in_rows=None, cap=None, direction=0):
    """The oracle rank by rank; outputs start as the sentinel, like the GPU's."""
    P = E // W
    in_rows = [x.shape[0] for x in X] if in_rows is None else list(in_rows)
    cap = in_rows if cap is None else list(cap)
    sts, outs, eoffs = 0, [], np.full((W, P + 1), -7, dtype=np.int64)
    per = []
    for d in range(W):
        st, out, eoff = ref.moe_regroup(W, E, d, R, counts, X[d], in_rows[d], cap[d], direction)
        per.append(st)
        sts |= st
        if st == 0:
            eoffs[d] = eoff
        outs.append(out.reshape(-1, R))
    if sts:
        outs = [np.full((int(c), R), SENT, dtype=np.uint8) for c in cap]
    return sts, outs, eoffs, per


def _random_counts(g, W, E, hi, zero_frac=0.3):
    c = g.integers(0, hi + 1, size=(W, E), dtype=np.int64)
    c[g.random((W, E)) < zero_frac] = 0
    return c


@pytest.mark.parametrize("W,E,R,hi,pad,direction", [
    (8, 256, 1024, 3, 0, 0),       # the dispatch layout, small rows
    (8, 256, 1024, 3, 0, 1),
    (4, 16, 7168 * 2, 40, 0, 0),   # full-width rows, pieces span blocks
    (3, 12, 10, 50, 0, 0),         # unaligned row width
    (3, 12, 10, 50, 4, 1),         # misaligned bases
    (2, 4096, 16, 2, 0, 0),        # the most experts: two search levels
    (1, 5, 48, 9, 0, 0),           # one rank
    (5, 5, 64, 300, 0, 1),         # one expert per rank
    (7, 63, 48, 9, 0, 0),          # the most blocks whose plan row a workgroup stages
    (8, 64, 48, 9, 0, 1),          # one block more: the row is searched in global memory
])
def test_regroup_matches_oracle(ref, W, E, R, hi, pad, direction):
    _say("regroup", W, E, R, hi, pad, direction)
    g = I.rng(W * 1000 + E + R + direction)
    counts = _random_counts(g, W, E, hi)
    X = [random_rows(g, _owned_total(counts, W, E, d) + 3, R) for d in range(W)]  # 3 spare rows
    cap = [x.shape[0] + 5 for x in X]
    gst, gout, geoff, guards = gpu_regroup(W, E, R, counts, X, cap=cap, direction=direction, pad=pad)
    rst, rout, reoff, _ = ref_regroup(ref, W, E, R, counts, X, cap=cap, direction=direction)
    assert guards and gst == rst == 0
    assert np.array_equal(geoff, reoff)
    for d in range(W):
        n = _owned_total(counts, W, E, d)
        assert np.array_equal(gout[d][:n], rout[d][:n]), f"rank {d}"
        assert (gout[d][n:] == SENT).all(), f"rank {d} wrote past its rows"


def test_regroup_round_trip_and_expert_blocks(ref):
    """Direction 0 then 1 restores the input; after direction 0, the rows of
    owned expert j are exactly expert_offsets[j] .. expert_offsets[j+1]."""
    W, E, R = 4, 32, 256
    g = I.rng(5)
    counts = _random_counts(g, W, E, 20)
    P = E // W
    X = []
    for d in range(W):
        # tag each row with (expert j, source s) so its block is visible
        rows = []
        for s in range(W):
            for j in range(P):
                n = int(counts[s, d * P + j])
                r = random_rows(g, n, R)
                r[:, 0], r[:, 1] = j, s
                rows.append(r)
        X.append(np.concatenate(rows) if rows else np.zeros((0, R), np.uint8))
    st, mid, eoff, guards = gpu_regroup(W, E, R, counts, X, direction=0)
    assert st == 0 and guards
    st2, back, _, guards2 = gpu_regroup(W, E, R, counts, mid, direction=1)
    assert st2 == 0 and guards2
    for d in range(W):
        assert np.array_equal(back[d], X[d])
        for j in range(P):
            blk = mid[d][eoff[d, j]:eoff[d, j + 1]]
            assert (blk[:, 0] == j).all()
            assert np.array_equal(blk[:, 1], np.repeat(np.arange(W), counts[:, d * P + j]))


@pytest.mark.parametrize("case", ["bad_split", "overrun", "overflow", "mixed", "poisoned"])
def test_regroup_errors_write_nothing(ref, case):
    W, E, R = 4, 16, 32
    g = I.rng(77)
    counts = _random_counts(g, W, E, 6, 0.0) + 1
    X = [random_rows(g, _owned_total(counts, W, E, d), R) for d in range(W)]
    in_rows = [x.shape[0] for x in X]
    cap = list(in_rows)
    init = 0
    if case == "bad_split":
        counts[2, 1 * 4 + 3] = -1              # owned by rank 1
    elif case == "overrun":
        in_rows[2] -= 1
    elif case == "overflow":
        cap[3] -= 1
    elif case == "mixed":
        counts[0, 0] = (1 << 40) + 1           # rank 0: bad split
        in_rows[1] -= 1                        # rank 1: overrun
        cap[2] -= 2                            # rank 2: overflow
    else:
        init = 4
    Xg = [x[:r] for x, r in zip(X, in_rows)]
    gst, gout, geoff, guards = gpu_regroup(W, E, R, counts, Xg, in_rows, cap, status_init=init)
    assert guards
    for d in range(W):
        assert (gout[d] == SENT).all(), f"rank {d} written"
    if case == "poisoned":
        assert gst == init and (geoff == -7).all()
        return
    rst, _, reoff, per = ref_regroup(ref, W, E, R, counts, Xg, in_rows, cap)
    assert gst == rst != 0
    # expert offsets of the ranks that passed are still written
    assert np.array_equal(geoff, reoff)
    if case == "mixed":
        assert per[:3] == [B.ST_BAD_SPLIT, B.ST_SEND_OVERRUN, B.ST_RECV_OVERFLOW] and per[3] == 0


def test_regroup_empty_ranks(ref):
    W, E, R = 4, 8, 64
    counts = np.zeros((W, E), np.int64)
    counts[1, 2:4] = [5, 7]                    # only rank 1 receives anything
    X = [random_rows(I.rng(d), _owned_total(counts, W, E, d), R) for d in range(W)]
    gst, gout, geoff, guards = gpu_regroup(W, E, R, counts, X)
    rst, rout, reoff, _ = ref_regroup(ref, W, E, R, counts, X)
    assert guards and gst == rst == 0
    assert np.array_equal(geoff, reoff)
    for d in range(W):
        assert np.array_equal(gout[d], rout[d])


def test_regroup_full_dispatch(ref):
    """W=8, 8192 tokens x top-8 of 256 Zipf(1.1) experts per rank, rows of
    7168 bf16: every rank's received buffer (about 7 GiB in all) regrouped
    on the GPU and by the oracle, compared byte for byte."""
    W, T, k, E, R = 8, 8192, 8, 256, 7168 * 2
    g = I.rng(4242)
    counts = np.zeros((W, E), np.int64)
    one = np.zeros((T, 1), np.uint8)
    for s in range(W):
        ids = I.topk_ids(g, T, k, E, 1.1)
        st, _, _, _, c = ref.moe_pack(T, k, E, W, 1, one, ids)
        assert st == 0
        counts[s] = c
    tot = [_owned_total(counts, W, E, d) for d in range(W)]
    _say("regroup full: rows per rank", tot)
    ins = [I.payload_bytes(n, R, seed=900 + d, device="cuda") for d, n in enumerate(tot)]
    outs = [torch.empty_like(x) for x in ins]
    cnt = torch.from_numpy(counts).cuda()
    eoff = torch.empty((W, E // W + 1), dtype=torch.int64, device="cuda")
    ws = torch.empty(B.moe_regroup_workspace_bytes(W, E), dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    B.moe_regroup(W, E, R, cnt, ins, tot, outs, tot, eoff, 0, ws, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for d in range(W):
        x = ins[d].cpu().numpy()
        st, want, weoff = ref.moe_regroup(W, E, d, R, counts, x, tot[d], tot[d], 0)
        assert st == 0
        assert np.array_equal(eoff[d].cpu().numpy(), weoff)
        assert np.array_equal(outs[d].cpu().numpy().reshape(-1), want), f"rank {d}"
        del x, want
    _say("regroup full: ok")


# ------------------------------------------------------------------ grouped dispatch
def gpu_grouped(W, E, R, counts, X, in_rows=None, cap=None, direction=0, pad=0, status_init=0):
    in_rows = [x.shape[0] for x in X] if in_rows is None else list(in_rows)
    P = E // W
    if cap is None:
        if direction == 0:
            cap = [_owned_total(counts, W, E, d) for d in range(W)]
        else:
            cap = [int(counts[s].sum()) for s in range(W)]
    ins = [upload_rows(x, pad=pad) for x in X]
    outs = [GuardedBuffer(int(c) * R, pad=pad) for c in cap]
    cnt = torch.from_numpy(np.ascontiguousarray(counts, dtype=np.int64)).cuda()
    eoff = torch.full((W, P + 1), -7, dtype=torch.int64, device="cuda")
    ws = torch.empty(B.moe_dispatch_grouped_workspace_bytes(W, E), dtype=torch.uint8,
                     device="cuda")
    status = torch.full((1,), status_init, dtype=torch.int32, device="cuda")
    B.moe_dispatch_grouped(W, E, R, cnt, [b.view for b in ins], in_rows, [b.view for b in outs],
                           list(cap), eoff, direction, ws, status)
    torch.cuda.synchronize()
    guards = all(b.guards_intact() for b in outs + ins)
    return (int(status.item()), [b.host().reshape(-1, R) for b in outs], eoff.cpu().numpy(),
            guards, cap)


def _check_grouped(ref, W, E, R, counts, X, in_rows, cap, direction, got):
    gst, gout, geoff, guards, cap = got
    rst, rout, reoff = ref.moe_dispatch_grouped(W, E, R, counts, X, in_rows, cap, direction)
    assert guards
    assert gst == rst, f"status {gst} != oracle {rst}"
    assert np.array_equal(geoff, reoff)
    for r in range(W):
        if rst == 0:
            n = (_owned_total(counts, W, E, r) if direction == 0 else int(counts[r].sum())) * R
            assert np.array_equal(gout[r].reshape(-1)[:n], rout[r][:n]), f"rank {r}"
            assert (gout[r].reshape(-1)[n:] == SENT).all(), f"rank {r} past its rows"
        else:
            assert (gout[r] == SENT).all(), f"rank {r} written"


@pytest.mark.parametrize("W,E,R,hi,pad", [
    (8, 256, 1024, 3, 0), (4, 16, 7168 * 2, 40, 0), (3, 12, 10, 50, 0), (3, 12, 10, 50, 4),
    (2, 4096, 16, 2, 0), (1, 5, 48, 9, 0), (5, 5, 64, 300, 0), (64, 128, 32, 3, 0),
    (7, 63, 48, 9, 0), (8, 64, 48, 9, 0),
])
@pytest.mark.parametrize("direction", [0, 1])
def test_grouped_matches_oracle(ref, W, E, R, hi, pad, direction):
    _say("grouped", W, E, R, hi, pad, direction)
    g = I.rng(W * 100 + E + R + direction)
    counts = _random_counts(g, W, E, hi)
    if direction == 0:
        X = [random_rows(g, int(counts[s].sum()) + 2, R) for s in range(W)]
    else:
        X = [random_rows(g, _owned_total(counts, W, E, d) + 2, R) for d in range(W)]
    in_rows = [x.shape[0] for x in X]
    got = gpu_grouped(W, E, R, counts, X, in_rows, direction=direction, pad=pad)
    _check_grouped(ref, W, E, R, counts, X, in_rows, got[4], direction, got)


@pytest.mark.parametrize("case", ["bad_split", "overrun", "overflow", "poisoned"])
@pytest.mark.parametrize("direction", [0, 1])
def test_grouped_errors(ref, case, direction):
    W, E, R = 4, 16, 32
    g = I.rng(78)
    counts = _random_counts(g, W, E, 6, 0.0) + 1
    if direction == 0:
        X = [random_rows(g, int(counts[s].sum()), R) for s in range(W)]
        cap = [_owned_total(counts, W, E, d) for d in range(W)]
    else:
        X = [random_rows(g, _owned_total(counts, W, E, d), R) for d in range(W)]
        cap = [int(counts[s].sum()) for s in range(W)]
    in_rows = [x.shape[0] for x in X]
    init = 0
    if case == "bad_split":
        counts[3, 2] = -1
    elif case == "overrun":
        in_rows[1] -= 1
        X[1] = X[1][:-1]
    elif case == "overflow":
        cap[2] -= 1
    else:
        init = 2
    got = gpu_grouped(W, E, R, counts, X, in_rows, cap, direction, status_init=init)
    if case == "poisoned":
        assert got[0] == init and (got[2] == -7).all() and all((o == SENT).all() for o in got[1])
        return
    _check_grouped(ref, W, E, R, counts, X, in_rows, cap, direction, got)
    assert got[0] != 0


def test_grouped_full_dispatch_round_trip(ref):
    """W=8, 8192 tokens x top-8 of 256 Zipf(1.1) experts per rank, rows of
    7168 bf16: moe_pack, then the grouped dispatch straight to expert-major
    order (checked rank by rank against the oracle's a2av + regroup chain,
    here the one-step oracle), then the grouped return, which must give back
    every packed row."""
    W, T, k, E, hidden = 8, 8192, 8, 256, 7168
    R, Q = hidden * 2, T * k
    g = I.rng(4243)
    ids = [torch.from_numpy(I.topk_ids(g, T, k, E, 1.1).reshape(-1)).cuda() for _ in range(W)]
    tok = [I.payload_bf16(T, hidden, 700 + r, device="cuda") for r in range(W)]
    send = [torch.empty((Q, hidden), dtype=torch.bfloat16, device="cuda") for _ in range(W)]
    perm = [torch.empty(Q, dtype=torch.int64, device="cuda") for _ in range(W)]
    S = torch.empty((W, W), dtype=torch.int64, device="cuda")
    cnt = torch.empty((W, E), dtype=torch.int64, device="cuda")
    ws = torch.empty(B.moe_pack_workspace_bytes(W, T, k, E), dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    B.moe_pack(W, T, k, E, R, tok, ids, send, perm, S, cnt, ws, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    counts = cnt.cpu().numpy()
    P = E // W
    tot = [_owned_total(counts, W, E, d) for d in range(W)]
    exp = [torch.empty((c, hidden), dtype=torch.bfloat16, device="cuda") for c in tot]
    eoff = torch.empty((W, P + 1), dtype=torch.int64, device="cuda")
    gws = torch.empty(B.moe_dispatch_grouped_workspace_bytes(W, E), dtype=torch.uint8,
                      device="cuda")
    B.moe_dispatch_grouped(W, E, R, cnt, send, [Q] * W, exp, tot, eoff, 0, gws, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    sends_h = [x.view(torch.uint8).cpu().numpy().reshape(-1) for x in send]
    st, want, weoff = ref.moe_dispatch_grouped(W, E, R, counts, sends_h, [Q] * W, tot, 0)
    assert st == 0 and np.array_equal(eoff.cpu().numpy(), weoff)
    for d in range(W):
        assert np.array_equal(exp[d].view(torch.uint8).cpu().numpy().reshape(-1), want[d]), d
    del want, sends_h
    back = [torch.empty_like(x) for x in send]
    B.moe_dispatch_grouped(W, E, R, cnt, exp, tot, back, [Q] * W, eoff, 1, gws, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for r in range(W):
        assert torch.equal(back[r].view(torch.int16), send[r].view(torch.int16)), r
    _say("grouped full: ok, rows per owner", tot)
