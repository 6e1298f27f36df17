"""GPU parity of the MoE pack and dispatch in one step (moe_pack_dispatch),
its inverse (moe_unpack_return) and the gate-weighted combine read at the
owners (moe_combine_return) against the CPU oracle: bit-exact receive rows,
perm, splits, counts, block offsets, combined rows and status, in both
receive layouts, at small ragged shapes, on error paths, and at the full
dispatch size."""
import numpy as np
import pytest
import torch

from embeddings_a2av_virtual_amd import _binding as B
from embeddings_a2av_virtual_amd import inputs as I
from gpu_util import SENT, GuardedBuffer, upload_rows

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _dev_array(x, dtype):
    """A device copy of a host array, at least one element long (so that an
    empty one still has an address)."""
    x = np.ascontiguousarray(x, dtype=dtype).reshape(-1)
    t = torch.zeros(max(x.size, 1), dtype=getattr(torch, np.dtype(dtype).name), device="cuda")
    if x.size:
        t[:x.size].copy_(torch.from_numpy(x))
    return t


def gpu_pack_dispatch(W, T, k, E, R, toks, ids, cap, layout, pad=0, status_init=0):
    """toks: per-rank host uint8 [T, R]; ids: per-rank int32 [T*k]. Returns
    (status, [recv host [cap_d, R]], [perm host], S, counts, offsets, guards)."""
    tin = [upload_rows(t, pad=pad) for t in toks]
    idd = [_dev_array(i, np.int32) for i in ids]
    recv = [GuardedBuffer(int(c) * R, pad=pad) for c in cap]
    perm = [torch.full((max(T * k, 1),), -7, dtype=torch.int64, device="cuda") for _ in range(W)]
    S = torch.full((W, W), -7, dtype=torch.int64, device="cuda")
    cnt = torch.full((W, E), -7, dtype=torch.int64, device="cuda")
    G = W if layout == 0 else E // W
    boff = torch.full((W, G + 1), -7, dtype=torch.int64, device="cuda")
    ws = torch.empty(B.moe_pack_dispatch_workspace_bytes(W, T, k, E), dtype=torch.uint8,
                     device="cuda")
    status = torch.full((1,), status_init, dtype=torch.int32, device="cuda")
    B.moe_pack_dispatch(W, T, k, E, R, [b.view for b in tin], idd, [b.view for b in recv], cap,
                        perm, S, cnt, boff, layout, ws, status)
    torch.cuda.synchronize()
    guards = all(b.guards_intact() for b in recv + tin)
    return (int(status.item()), [b.host().reshape(-1, R) for b in recv],
            [p.cpu().numpy()[:T * k] for p in perm], S.cpu().numpy(), cnt.cpu().numpy(),
            boff.cpu().numpy(), guards)


def gpu_unpack_return(W, T, k, E, R, counts, ids, perms, recv, layout, recv_rows=None, pad=0,
                      status_init=0):
    """recv: per-owner host uint8 [rows, R]. Returns (status, [out host [T*k, R]], guards)."""
    rin = [upload_rows(x, pad=pad) for x in recv]
    rows = [x.shape[0] for x in recv] if recv_rows is None else list(recv_rows)
    out = [GuardedBuffer(T * k * R, pad=pad) for _ in range(W)]
    cnt = torch.from_numpy(np.ascontiguousarray(counts, dtype=np.int64)).cuda()
    idd = [_dev_array(i, np.int32) for i in ids]
    pd = [_dev_array(p, np.int64) for p in perms]
    ws = torch.empty(B.moe_unpack_return_workspace_bytes(W, E), dtype=torch.uint8, device="cuda")
    status = torch.full((1,), status_init, dtype=torch.int32, device="cuda")
    B.moe_unpack_return(W, T, k, E, R, cnt, idd, pd, [b.view for b in rin], rows,
                        [b.view for b in out], layout, ws, status)
    torch.cuda.synchronize()
    guards = all(b.guards_intact() for b in out + rin)
    return int(status.item()), [b.host().reshape(-1, R) for b in out], guards


def gpu_combine_return(W, T, k, E, H, counts, ids, perms, recv, weights, layout, recv_rows=None,
                       pad=0, status_init=0):
    """recv: per-owner host uint16 [rows, H]; weights: per-source float32
    [T, k]. Returns (status, [out host uint16 [T, H]], guards)."""
    rin = [upload_rows(np.ascontiguousarray(x).view(np.uint8), pad=pad) for x in recv]
    rows = [x.shape[0] for x in recv] if recv_rows is None else list(recv_rows)
    out = [GuardedBuffer(T * H * 2, pad=pad) for _ in range(W)]
    cnt = torch.from_numpy(np.ascontiguousarray(counts, dtype=np.int64)).cuda()
    idd = [_dev_array(i, np.int32) for i in ids]
    pd = [_dev_array(p, np.int64) for p in perms]
    wd = [_dev_array(w, np.float32) for w in weights]
    ws = torch.empty(B.moe_combine_return_workspace_bytes(W, T, k, E), dtype=torch.uint8,
                     device="cuda")
    status = torch.full((1,), status_init, dtype=torch.int32, device="cuda")
    B.moe_combine_return(W, T, k, E, H, cnt, idd, pd, [b.view for b in rin], rows, wd,
                         [b.view for b in out], layout, ws, status)
    torch.cuda.synchronize()
    guards = all(b.guards_intact() for b in out + rin)
    return (int(status.item()), [b.host().view(np.uint16).reshape(T, H) for b in out], guards)


def _bf16_junk(g, rows, H):
    """Random bf16 bit patterns, specials included (the two sides must agree
    on every bit, NaN included)."""
    x = g.integers(0, 1 << 16, size=(rows, H), dtype=np.uint16)
    sp = np.array([0x7F80, 0xFF80, 0x7FC1, 0x0001, 0x8000, 0x7F7F], dtype=np.uint16)
    m = g.random((rows, H)) < 0.01
    x[m] = sp[g.integers(0, sp.size, size=int(m.sum()))]
    return x


def _case(g, W, T, k, E, R, distinct):
    toks = [g.integers(0, 256, size=(T, R), dtype=np.uint8) for _ in range(W)]
    if distinct:
        ids = [I.topk_ids(g, T, k, E, 1.1).reshape(-1) for _ in range(W)]
    else:
        ids = [g.integers(0, E, size=T * k).astype(np.int32) for _ in range(W)]
    return toks, ids


def _totals(ids, W, E):
    P = E // W
    tot = np.zeros(W, dtype=np.int64)
    for x in ids:
        tot += np.bincount(np.asarray(x, dtype=np.int64) // P, minlength=W)[:W]
    return tot


SHAPES = [
    (8, 64, 8, 256, 1024, True, 0),    # the dispatch layout, small rows
    (4, 100, 3, 12, 48, False, 0),     # repeated experts in a token
    (3, 50, 2, 6, 10, False, 0),       # row width not a multiple of 16
    (3, 50, 2, 6, 32, True, 4),        # misaligned bases
    (1, 33, 4, 5, 64, False, 0),       # one rank
    (5, 40, 1, 5, 16, False, 0),       # one expert per rank, k = 1
    (2, 20, 64, 128, 16, True, 0),     # k = 64, the most a wave holds
    (64, 8, 2, 128, 16, False, 0),     # 64 ranks
    (4, 0, 2, 8, 16, False, 0),        # no tokens
    (2, 40, 8, 4096, 32, False, 0),    # the most experts a plan holds
    (64, 6, 8, 4096, 16, True, 0),     # the most ranks and experts at once
]


@pytest.mark.parametrize("W,T,k,E,R,distinct,pad", SHAPES)
@pytest.mark.parametrize("layout", [0, 1])
def test_pack_dispatch_matches_oracle(ref, W, T, k, E, R, distinct, pad, layout):
    _say("pack_dispatch", W, T, k, E, R, distinct, pad, layout)
    g = I.rng(W * 7919 + T * 31 + k * 7 + E + R + layout)
    toks, ids = _case(g, W, T, k, E, R, distinct)
    tot = _totals(ids, W, E)
    cap = tot + np.arange(W) % 3          # spare rows stay untouched
    st, recv, perm, S, cnt, boff, guards = gpu_pack_dispatch(W, T, k, E, R, toks, ids, cap,
                                                              layout, pad=pad)
    rst, rrecv, rperm, rS, rcnt, rboff = ref.moe_pack_dispatch(W, T, k, E, R, toks, ids, cap,
                                                               layout)
    assert st == rst == 0 and guards
    assert np.array_equal(S, rS) and np.array_equal(cnt, rcnt) and np.array_equal(boff, rboff)
    for s in range(W):
        assert np.array_equal(perm[s], rperm[s]), s
    for d in range(W):
        t = int(tot[d])
        assert np.array_equal(recv[d][:t], rrecv[d].reshape(-1, R)[:t]), d
        assert (recv[d][t:] == SENT).all(), d
    # the inverse on those rows gives every slot its token row
    rows = [recv[d][:int(tot[d])] for d in range(W)]
    st, out, guards = gpu_unpack_return(W, T, k, E, R, cnt, ids, perm, rows, layout, pad=pad)
    assert st == 0 and guards
    for s in range(W):
        assert np.array_equal(out[s], np.repeat(toks[s], k, axis=0)), s
    # and, on arbitrary receive contents, what the oracle gives
    junk = [g.integers(0, 256, size=(int(t), R), dtype=np.uint8) for t in tot]
    st, out, guards = gpu_unpack_return(W, T, k, E, R, cnt, ids, perm, junk, layout, pad=pad)
    rst, rout = ref.moe_unpack_return(W, T, k, E, R, cnt, ids, perm, junk, layout)
    assert st == rst == 0 and guards
    for s in range(W):
        assert np.array_equal(out[s].reshape(-1), rout[s]), s


@pytest.mark.parametrize("case", ["bad_expert", "overflow", "poisoned"])
@pytest.mark.parametrize("layout", [0, 1])
def test_pack_dispatch_errors(ref, case, layout):
    _say("pack_dispatch error", case, layout)
    W, T, k, E, R = 4, 40, 3, 12, 32
    g = I.rng(77 + layout)
    toks, ids = _case(g, W, T, k, E, R, True)
    tot = _totals(ids, W, E)
    cap = tot.copy()
    init = 0
    if case == "bad_expert":
        ids[2] = ids[2].copy()
        ids[2][17] = E
    elif case == "overflow":
        cap[1] -= 1
    else:
        init = B.ST_BAD_OFFSETS
    st, recv, perm, S, cnt, boff, guards = gpu_pack_dispatch(W, T, k, E, R, toks, ids, cap,
                                                              layout, status_init=init)
    assert guards
    assert all((x == SENT).all() for x in recv)
    if case == "poisoned":
        assert st == B.ST_BAD_OFFSETS
    else:
        rst, _, rperm, rS, rcnt, rboff = ref.moe_pack_dispatch(W, T, k, E, R, toks, ids, cap,
                                                               layout)
        assert st == rst
    if case == "overflow":
        assert st == B.ST_RECV_OVERFLOW
        assert np.array_equal(S, rS) and np.array_equal(cnt, rcnt)
        assert np.array_equal(boff, rboff)
        assert all(np.array_equal(a, b) for a, b in zip(perm, rperm))
    else:
        assert st in (B.ST_BAD_EXPERT, B.ST_BAD_OFFSETS)
        assert (S == -7).all() and (cnt == -7).all() and (boff == -7).all()
        assert all((p == -7).all() for p in perm)


@pytest.mark.parametrize("case", ["bad_split", "bad_expert", "bad_perm", "overrun", "two_bits",
                                  "poisoned", "empty_bad_split"])
@pytest.mark.parametrize("layout", [0, 1])
def test_unpack_return_errors(ref, case, layout):
    _say("unpack_return error", case, layout)
    W, T, k, E, R = 3, 30, 2, 6, 16
    g = I.rng(91 + layout)
    toks, ids = _case(g, W, T, k, E, R, True)
    st, recv, perm, S, cnt, boff, _ = gpu_pack_dispatch(W, T, k, E, R, toks, ids,
                                                         _totals(ids, W, E), layout)
    assert st == 0
    rows = None
    init = 0
    ids = [x.copy() for x in ids]
    if case == "bad_split":
        cnt = cnt.copy()
        cnt[1, 4] = -3
    elif case == "bad_expert":
        ids[0][5] = -1
    elif case == "bad_perm":
        q = int(np.nonzero(ids[1] != ids[1][0])[0][0])
        ids[1][0], ids[1][q] = ids[1][q], ids[1][0]
    elif case == "overrun":
        rows = [x.shape[0] for x in recv]
        rows[2] -= 1
    elif case == "two_bits":
        ids[0][5] = E
        q = int(np.nonzero(ids[1] != ids[1][0])[0][0])
        ids[1][0], ids[1][q] = ids[1][q], ids[1][0]
    elif case == "poisoned":
        init = B.ST_BAD_OFFSETS
    if case == "empty_bad_split":
        Tz = 0
        cz = np.zeros((W, E), dtype=np.int64)
        cz[0, 0] = -1
        st, out, guards = gpu_unpack_return(W, Tz, k, E, R, cz, [np.zeros(0, np.int32)] * W,
                                            [np.zeros(0, np.int64)] * W,
                                            [np.zeros((0, R), np.uint8)] * W, layout)
        rst, _ = ref.moe_unpack_return(W, Tz, k, E, R, cz, [np.zeros(0, np.int32)] * W,
                                       [np.zeros(0, np.int64)] * W,
                                       [np.zeros(0, np.uint8)] * W, layout)
        assert st == rst == B.ST_BAD_SPLIT and guards
        return
    st, out, guards = gpu_unpack_return(W, T, k, E, R, cnt, ids, perm, recv, layout,
                                        recv_rows=rows, status_init=init)
    assert guards and all((x == SENT).all() for x in out)
    if case == "poisoned":
        assert st == B.ST_BAD_OFFSETS
        return
    rrecv = recv if rows is None else [x[:n] for x, n in zip(recv, rows)]
    rst, _ = ref.moe_unpack_return(W, T, k, E, R, cnt, ids, perm, rrecv, layout)
    want = {"bad_split": B.ST_BAD_SPLIT, "bad_expert": B.ST_BAD_EXPERT,
            "bad_perm": B.ST_BAD_PERM, "overrun": B.ST_SEND_OVERRUN,
            "two_bits": B.ST_BAD_EXPERT | B.ST_BAD_PERM}[case]
    assert st == rst == want


@pytest.mark.parametrize("layout", [0, 1])
def test_pack_dispatch_full(ref, layout):
    """W=8, 8192 tokens x top-8 of 256 Zipf(1.1) experts per rank, rows of
    7168 bf16, in the launch configuration the benchmark times. The oracle
    runs on the same routing with 8-byte rows that name their (source, token),
    which fixes what every one of the GPU's receive rows must hold; the GPU
    result also equals moe_pack followed by the a2av (layout 0) or the grouped
    dispatch (layout 1), and the inverse brings every slot its token row."""
    W, T, k, E, hidden = 8, 8192, 8, 256, 7168
    R, Q = hidden * 2, T * k
    g = I.rng(5151 + layout)
    ids_h = [I.topk_ids(g, T, k, E, 1.1).reshape(-1) for _ in range(W)]
    ids = [torch.from_numpy(x).cuda() for x in ids_h]
    tok = [I.payload_bf16(T, hidden, 800 + r, device="cuda") for r in range(W)]
    tot = _totals(ids_h, W, E)
    recv = [torch.empty((int(c), hidden), dtype=torch.bfloat16, device="cuda") for c in tot]
    perm = [torch.empty(Q, dtype=torch.int64, device="cuda") for _ in range(W)]
    S = torch.empty((W, W), dtype=torch.int64, device="cuda")
    cnt = torch.empty((W, E), dtype=torch.int64, device="cuda")
    G = W if layout == 0 else E // W
    boff = torch.empty((W, G + 1), dtype=torch.int64, device="cuda")
    ws = torch.empty(B.moe_pack_dispatch_workspace_bytes(W, T, k, E), dtype=torch.uint8,
                     device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    B.moe_pack_dispatch(W, T, k, E, R, tok, ids, recv, tot, perm, S, cnt, boff, layout, ws, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    # the oracle on tag rows: row (s, t) holds s * 2^32 + t
    tags = [(np.int64(s) << 32) + np.arange(T, dtype=np.int64) for s in range(W)]
    rst, rrecv, rperm, rS, rcnt, rboff = ref.moe_pack_dispatch(
        W, T, k, E, 8, [x.view(np.uint8).reshape(T, 8) for x in tags], ids_h, tot, layout)
    assert rst == 0
    assert np.array_equal(S.cpu().numpy(), rS) and np.array_equal(cnt.cpu().numpy(), rcnt)
    assert np.array_equal(boff.cpu().numpy(), rboff)
    for s in range(W):
        assert np.array_equal(perm[s].cpu().numpy(), rperm[s]), s
    tok16 = torch.stack([t.view(torch.int16) for t in tok])        # [W, T, hidden]
    for d in range(W):
        tg = rrecv[d].view(np.int64)
        src = torch.from_numpy(tg >> 32).cuda()
        tt = torch.from_numpy(tg & 0xFFFFFFFF).cuda()
        assert torch.equal(recv[d].view(torch.int16), tok16[src, tt]), d
    del tok16
    # equal to the two-step GPU path
    send = [torch.empty((Q, hidden), dtype=torch.bfloat16, device="cuda") for _ in range(W)]
    pws = torch.empty(B.moe_pack_workspace_bytes(W, T, k, E), dtype=torch.uint8, device="cuda")
    S2 = torch.empty_like(S)
    cnt2 = torch.empty_like(cnt)
    B.moe_pack(W, T, k, E, R, tok, ids, send, perm, S2, cnt2, pws, status)
    two = [torch.empty_like(x) for x in recv]
    if layout == 0:
        from embeddings_a2av_virtual_amd.vranks import A2av
        st = A2av(W)
        st.S.copy_(S2)
        st(R, send, [Q] * W, two, [int(c) for c in tot], fused=True)
        torch.cuda.synchronize()
        assert int(st.status.item()) == 0
    else:
        eoff = torch.empty((W, G + 1), dtype=torch.int64, device="cuda")
        gws = torch.empty(B.moe_dispatch_grouped_workspace_bytes(W, E), dtype=torch.uint8,
                          device="cuda")
        B.moe_dispatch_grouped(W, E, R, cnt2, send, [Q] * W, two, tot, eoff, 0, gws, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for d in range(W):
        assert torch.equal(two[d].view(torch.int16), recv[d].view(torch.int16)), d
    del send, two
    # the inverse: every slot gets its token row back
    out = [torch.empty((Q, hidden), dtype=torch.bfloat16, device="cuda") for _ in range(W)]
    uws = torch.empty(B.moe_unpack_return_workspace_bytes(W, E), dtype=torch.uint8, device="cuda")
    B.moe_unpack_return(W, T, k, E, R, cnt, ids, perm, recv, tot, out, layout, uws, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for s in range(W):
        want = tok[s].view(torch.int16).repeat_interleave(k, dim=0)
        assert torch.equal(out[s].view(torch.int16), want), s
    # the combine at the owners equals the combine over those home rows, and
    # the oracle's on 32 sampled tokens per rank
    w_h = [I.gate_weights(g, T, k) for _ in range(W)]
    wts = [torch.from_numpy(x.reshape(-1)).cuda() for x in w_h]
    cret = [torch.empty((T, hidden), dtype=torch.bfloat16, device="cuda") for _ in range(W)]
    cws = torch.empty(B.moe_combine_return_workspace_bytes(W, T, k, E), dtype=torch.uint8,
                      device="cuda")
    B.moe_combine_return(W, T, k, E, hidden, cnt, ids, perm, recv, tot, wts, cret, layout, cws,
                         status)
    ident = [torch.arange(Q, dtype=torch.int64, device="cuda") for _ in range(W)]
    cref = [torch.empty_like(x) for x in cret]
    cst = torch.zeros(1, dtype=torch.int32, device="cuda")
    B.moe_combine(W, T, k, hidden, out, ident, wts, cref, cst)
    torch.cuda.synchronize()
    assert int(status.item()) == 0 and int(cst.item()) == 0
    for s in range(W):
        assert torch.equal(cret[s].view(torch.int16), cref[s].view(torch.int16)), s
        ts = np.sort(g.choice(T, size=32, replace=False))
        rows = tok[s][torch.from_numpy(ts).cuda()].view(torch.int16).cpu().numpy().view(np.uint16)
        st_, want = ref.moe_combine(32, k, hidden, np.repeat(rows, k, axis=0),
                                    np.arange(32 * k, dtype=np.int64), w_h[s][ts])
        assert st_ == 0
        got = cret[s][torch.from_numpy(ts).cuda()].view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, want), s
    _say("pack_dispatch full: ok, layout", layout, "rows per owner", tot.tolist())


COMBINE_SHAPES = [
    (8, 64, 8, 256, 512, True, 0),     # the dispatch layout, 1 KiB rows
    (4, 50, 3, 12, 24, False, 0),      # repeated experts, three vectors per row
    (3, 40, 2, 6, 13, False, 0),       # odd width: the element path
    (3, 40, 2, 6, 64, True, 4),        # misaligned bases: the element path
    (1, 20, 4, 5, 1000, False, 0),     # a clamped last chunk
    (5, 30, 12, 10, 8, False, 0),      # k = 12: two slot groups
    (2, 0, 2, 8, 16, False, 0),        # no tokens
    (2, 30, 8, 4096, 64, False, 0),    # the most experts a plan holds
    (64, 5, 3, 4096, 8, False, 0),     # the most ranks and experts at once
]


@pytest.mark.parametrize("W,T,k,E,H,distinct,pad", COMBINE_SHAPES)
@pytest.mark.parametrize("layout", [0, 1])
def test_combine_return_matches_oracle(ref, W, T, k, E, H, distinct, pad, layout):
    _say("combine_return", W, T, k, E, H, distinct, pad, layout)
    g = I.rng(W * 131 + T * 7 + k + E + H + layout)
    toks, ids = _case(g, W, T, k, E, 2 * H, distinct)
    tot = _totals(ids, W, E)
    st, recv, perm, S, cnt, boff, _ = gpu_pack_dispatch(W, T, k, E, 2 * H, toks, ids, tot, layout)
    assert st == 0
    wts = [I.gate_weights(g, T, k) for _ in range(W)]
    # on the rows the dispatch left
    rows16 = [x.view(np.uint16).reshape(-1, H) for x in recv]
    gst, out, guards = gpu_combine_return(W, T, k, E, H, cnt, ids, perm, rows16, wts, layout,
                                          pad=pad)
    rst, rout = ref.moe_combine_return(W, T, k, E, H, cnt, ids, perm, rows16, wts, layout)
    assert gst == rst == 0 and guards
    for s in range(W):
        assert np.array_equal(out[s], rout[s]), s
    # on arbitrary bf16 patterns, specials included
    junk = [_bf16_junk(g, int(t), H) for t in tot]
    gst, out, guards = gpu_combine_return(W, T, k, E, H, cnt, ids, perm, junk, wts, layout,
                                          pad=pad)
    rst, rout = ref.moe_combine_return(W, T, k, E, H, cnt, ids, perm, junk, wts, layout)
    assert gst == rst == 0 and guards
    for s in range(W):
        assert np.array_equal(out[s], rout[s]), s


@pytest.mark.parametrize("case", ["bad_split", "bad_expert", "bad_perm", "overrun", "poisoned",
                                  "empty_bad_split"])
@pytest.mark.parametrize("layout", [0, 1])
def test_combine_return_errors(ref, case, layout):
    _say("combine_return error", case, layout)
    W, T, k, E, H = 3, 30, 2, 6, 16
    g = I.rng(191 + layout)
    toks, ids = _case(g, W, T, k, E, 2 * H, True)
    st, recv, perm, S, cnt, boff, _ = gpu_pack_dispatch(W, T, k, E, 2 * H, toks, ids,
                                                         _totals(ids, W, E), layout)
    assert st == 0
    rows16 = [x.view(np.uint16).reshape(-1, H) for x in recv]
    wts = [I.gate_weights(g, T, k) for _ in range(W)]
    ids = [x.copy() for x in ids]
    nrows, init = None, 0
    if case == "bad_split":
        cnt = cnt.copy()
        cnt[2, 1] = -5
    elif case == "bad_expert":
        ids[1][3] = E + 2
    elif case == "bad_perm":
        q = int(np.nonzero(ids[0] != ids[0][0])[0][0])
        ids[0][0], ids[0][q] = ids[0][q], ids[0][0]
    elif case == "overrun":
        nrows = [x.shape[0] for x in rows16]
        nrows[0] -= 1
    elif case == "poisoned":
        init = B.ST_BAD_OFFSETS
    if case == "empty_bad_split":
        cz = np.zeros((W, E), dtype=np.int64)
        cz[1, 0] = -1
        gst, out, guards = gpu_combine_return(W, 0, k, E, H, cz, [np.zeros(0, np.int32)] * W,
                                              [np.zeros(0, np.int64)] * W,
                                              [np.zeros((0, H), np.uint16)] * W,
                                              [np.zeros((0, k), np.float32)] * W, layout)
        assert gst == B.ST_BAD_SPLIT and guards
        return
    gst, out, guards = gpu_combine_return(W, T, k, E, H, cnt, ids, perm, rows16, wts, layout,
                                          recv_rows=nrows, status_init=init)
    assert guards and all((x.view(np.uint8) == SENT).all() for x in out)
    if case == "poisoned":
        assert gst == B.ST_BAD_OFFSETS
        return
    rrows = rows16 if nrows is None else [x[:n] for x, n in zip(rows16, nrows)]
    rst, _ = ref.moe_combine_return(W, T, k, E, H, cnt, ids, perm, rrows, wts, layout)
    want = {"bad_split": B.ST_BAD_SPLIT, "bad_expert": B.ST_BAD_EXPERT,
            "bad_perm": B.ST_BAD_PERM, "overrun": B.ST_SEND_OVERRUN}[case]
    assert gst == rst == want
