"""The entry points under HIP graph capture: a captured one-call a2av, MoE
pack + dispatch, fused key exchange, key bucketing and the one-step MoE trip (pack and
dispatch in one step, the combine at the owners and the one-step inverse),
each replayed several times with eager work and synchronisations between
replays, and every replay compared with the eager result (which is itself
checked against the oracle)."""
import numpy as np
import pytest
import torch

from embeddings_a2av_virtual_amd import _binding as B
from embeddings_a2av_virtual_amd import inputs as I
from embeddings_a2av_virtual_amd.vranks import A2av

pytestmark = pytest.mark.gpu


def _replay_and_check(graph, outputs, want, reset, eager_noise, times=4):
    for i in range(times):
        reset()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, exp in zip(range(len(want)), outputs(), want):
            assert torch.equal(got, exp), f"replay {i}: output {name} differs"
        eager_noise()
        torch.cuda.synchronize()


def _noise():
    # unrelated eager work between replays
    x = torch.randn(1 << 20, device="cuda")
    (x * 2).sum().item()


def test_graph_one_call_a2av(ref):
    W, rows, cols = 4, 2048, 512
    g = I.rng(3)
    S = I.uniform_splits(g, W, rows)
    X = [I.payload_bf16(rows, cols, 40 + r, device="cuda") for r in range(W)]
    cap = [int(c) for c in S.sum(axis=0)]
    Y = [torch.zeros((c, cols), dtype=torch.bfloat16, device="cuda") for c in cap]
    st = A2av(W)
    st.set_splits(S)
    st(cols * 2, X, [rows] * W, Y, cap, fused=True)
    torch.cuda.synchronize()
    assert int(st.status.item()) == 0
    want = [y.clone() for y in Y] + [st.O.clone(), st.send_off.clone(), st.recv_off.clone()]
    rY = [np.empty(c * cols * 2, dtype=np.uint8) for c in cap]
    rst, rO, _, _ = ref.a2av(cols * 2, [x.view(torch.uint8).cpu().numpy().reshape(-1) for x in X],
                             np.full(W, rows), rY, np.array(cap), S)
    assert rst == 0 and np.array_equal(st.O.cpu().numpy(), rO)
    for d in range(W):
        assert np.array_equal(Y[d].view(torch.uint8).cpu().numpy().reshape(-1), rY[d])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        st(cols * 2, X, [rows] * W, Y, cap, fused=True)  # warm-up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            st(cols * 2, X, [rows] * W, Y, cap, fused=True)
    torch.cuda.synchronize()

    def reset():
        for y in Y:
            y.zero_()
        st.O.zero_()
        st.status.zero_()

    _replay_and_check(graph, lambda: Y + [st.O, st.send_off, st.recv_off], want, reset, _noise)
    assert int(st.status.item()) == 0


def test_graph_moe_pack_and_dispatch():
    W, T, k, E, R = 4, 512, 4, 32, 256
    g = I.rng(8)
    tok = [torch.from_numpy(g.integers(0, 256, (T, R), dtype=np.uint8)).cuda() for _ in range(W)]
    ids = [torch.from_numpy(I.topk_ids(g, T, k, E).reshape(-1)).cuda() for _ in range(W)]
    Q = T * k
    send = [torch.zeros(Q * R, dtype=torch.uint8, device="cuda") for _ in range(W)]
    perm = [torch.zeros(Q, dtype=torch.int64, device="cuda") for _ in range(W)]
    fwd = A2av(W)
    cnt = torch.zeros((W, E), dtype=torch.int64, device="cuda")
    ws = torch.empty(B.moe_pack_workspace_bytes(W, T, k, E), dtype=torch.uint8, device="cuda")
    recv = [torch.zeros(Q * W * R, dtype=torch.uint8, device="cuda") for _ in range(W)]
    caps = [Q * W] * W

    def step():
        B.moe_pack(W, T, k, E, R, tok, ids, send, perm, fwd.S, cnt, ws, fwd.status)
        fwd(R, send, [Q] * W, recv, caps, fused=True)

    step()
    torch.cuda.synchronize()
    assert int(fwd.status.item()) == 0
    want = [x.clone() for x in send + perm + recv] + [fwd.S.clone(), cnt.clone()]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        step()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            step()
    torch.cuda.synchronize()

    def reset():
        for x in send + perm + recv:
            x.zero_()
        fwd.S.zero_()
        cnt.zero_()
        fwd.status.zero_()

    _replay_and_check(graph, lambda: send + perm + recv + [fwd.S, cnt], want, reset, _noise)


def test_graph_fused_key_exchange(ref):
    W, NT, batch = 8, 26, 256
    g = I.rng(21)
    ranks = [I.emb_keys_rank(g, tables=NT, batch=batch) for _ in range(W)]
    rst, wlo, wko, wsk, wsl, wro = ref.keys_exchange(W, NT, batch, [r.lengths for r in ranks],
                                                      [r.keys for r in ranks])
    assert rst == 0
    lin = [torch.from_numpy(r.lengths.reshape(-1)).cuda() for r in ranks]
    kin = [torch.from_numpy(r.keys).cuda() for r in ranks]
    lo = [torch.zeros(x.size, dtype=torch.int32, device="cuda") for x in wlo]
    ko = [torch.zeros(x.size, dtype=torch.int64, device="cuda") for x in wko]
    sk = torch.zeros((W, W), dtype=torch.int64, device="cuda")
    sl = torch.zeros((W, W), dtype=torch.int64, device="cuda")
    ro = torch.zeros((W, W + 1), dtype=torch.int64, device="cuda")
    ws = torch.empty(B.keys_exchange_workspace_bytes(W, NT), dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")

    def call():
        B.keys_exchange(W, NT, batch, lin, kin, [r.keys.size for r in ranks], lo,
                        [x.size for x in wlo], ko, [x.size for x in wko], sk, sl, ro, ws, status)

    call()
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for d in range(W):
        assert np.array_equal(lo[d].cpu().numpy(), wlo[d]) and np.array_equal(ko[d].cpu().numpy(), wko[d])
    assert np.array_equal(ro.cpu().numpy(), wro)
    want = [x.clone() for x in lo + ko] + [sk.clone(), sl.clone(), ro.clone()]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        call()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            call()
    torch.cuda.synchronize()

    def reset():
        for x in lo + ko + [sk, sl, ro]:
            x.zero_()
        status.zero_()

    _replay_and_check(graph, lambda: lo + ko + [sk, sl, ro], want, reset, _noise)
    assert int(status.item()) == 0


def test_graph_key_bucketing(ref):
    """keys_bucketize captured (counts, plan, and the one block copy of keys
    and lengths over 2W ranks), replays against the eager result and the
    oracle's per-rank bucketing."""
    W, NT, batch = 8, 26, 200
    g = I.rng(23)
    ranks = [I.emb_keys_rank(g, tables=NT, batch=batch) for _ in range(W)]
    want_o = [ref.keys_bucketize(W, NT, batch, r.lengths, r.keys) for r in ranks]
    assert all(w[0] == 0 for w in want_o)
    lin = [torch.from_numpy(r.lengths.reshape(-1)).cuda() for r in ranks]
    kin = [torch.from_numpy(r.keys).cuda() for r in ranks]
    lo = [torch.zeros(NT * batch, dtype=torch.int32, device="cuda") for _ in range(W)]
    ko = [torch.zeros(r.keys.size, dtype=torch.int64, device="cuda") for r in ranks]
    sk = torch.zeros((W, W), dtype=torch.int64, device="cuda")
    sl = torch.zeros((W, W), dtype=torch.int64, device="cuda")
    ws = torch.empty(B.keys_bucketize_workspace_bytes(W, NT), dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")

    def call():
        B.keys_bucketize(W, NT, batch, lin, kin, [r.keys.size for r in ranks], lo, ko, sk, sl, ws,
                         status)

    call()
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for r in range(W):
        _, rlo, rko, rsk, rsl = want_o[r]
        assert np.array_equal(lo[r].cpu().numpy(), rlo) and np.array_equal(ko[r].cpu().numpy(), rko)
        assert np.array_equal(sk[r].cpu().numpy(), rsk) and np.array_equal(sl[r].cpu().numpy(), rsl)
    want = [x.clone() for x in lo + ko] + [sk.clone(), sl.clone()]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        call()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            call()
    torch.cuda.synchronize()

    def reset():
        for x in lo + ko + [sk, sl]:
            x.zero_()
        status.zero_()

    _replay_and_check(graph, lambda: lo + ko + [sk, sl], want, reset, _noise)
    assert int(status.item()) == 0


def test_graph_one_step_moe_trip(ref):
    W, T, k, E, H = 4, 256, 4, 16, 256
    R, Q = 2 * H, T * k
    g = I.rng(61)
    ids_h = [I.topk_ids(g, T, k, E, 1.1).reshape(-1) for _ in range(W)]
    w_h = [I.gate_weights(g, T, k) for _ in range(W)]
    tok = [I.payload_bf16(T, H, 70 + r, device="cuda") for r in range(W)]
    ids = [torch.from_numpy(x).cuda() for x in ids_h]
    wts = [torch.from_numpy(x.reshape(-1)).cuda() for x in w_h]
    P = E // W
    tot = np.zeros(W, dtype=np.int64)
    for x in ids_h:
        tot += np.bincount(x.astype(np.int64) // P, minlength=W)[:W]
    tot = [int(t) for t in tot]
    recv = [torch.zeros((t, H), dtype=torch.bfloat16, device="cuda") for t in tot]
    perm = [torch.zeros(Q, dtype=torch.int64, device="cuda") for _ in range(W)]
    S = torch.zeros((W, W), dtype=torch.int64, device="cuda")
    cnt = torch.zeros((W, E), dtype=torch.int64, device="cuda")
    boff = torch.zeros((W, P + 1), dtype=torch.int64, device="cuda")
    comb = [torch.zeros((T, H), dtype=torch.bfloat16, device="cuda") for _ in range(W)]
    home = [torch.zeros((Q, H), dtype=torch.bfloat16, device="cuda") for _ in range(W)]
    pws = torch.empty(B.moe_pack_dispatch_workspace_bytes(W, T, k, E), dtype=torch.uint8,
                      device="cuda")
    cws = torch.empty(B.moe_combine_return_workspace_bytes(W, T, k, E), dtype=torch.uint8,
                      device="cuda")
    uws = torch.empty(B.moe_unpack_return_workspace_bytes(W, E), dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")

    def trip():
        B.moe_pack_dispatch(W, T, k, E, R, tok, ids, recv, tot, perm, S, cnt, boff, 1, pws, status)
        B.moe_combine_return(W, T, k, E, H, cnt, ids, perm, recv, tot, wts, comb, 1, cws, status)
        B.moe_unpack_return(W, T, k, E, R, cnt, ids, perm, recv, tot, home, 1, uws, status)

    trip()
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    toks_h = [t.view(torch.uint8).cpu().numpy() for t in tok]
    rst, rrecv, _, _, _, rboff = ref.moe_pack_dispatch(W, T, k, E, R, toks_h, ids_h, tot, 1)
    assert rst == 0 and np.array_equal(boff.cpu().numpy(), rboff)
    for d in range(W):
        assert np.array_equal(recv[d].view(torch.uint8).cpu().numpy().reshape(-1), rrecv[d])
    rst, rcomb = ref.moe_combine_return(W, T, k, E, H, cnt.cpu().numpy(), ids_h,
                                        [p.cpu().numpy() for p in perm],
                                        [x.view(torch.int16).cpu().numpy().view(np.uint16)
                                         for x in recv], w_h, 1)
    assert rst == 0
    for s in range(W):
        assert np.array_equal(comb[s].view(torch.int16).cpu().numpy().view(np.uint16), rcomb[s])
        assert torch.equal(home[s].view(torch.int16),
                           tok[s].view(torch.int16).repeat_interleave(k, dim=0))
    outs = recv + perm + comb + home + [S, cnt, boff]
    want = [x.clone() for x in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        trip()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            trip()
    torch.cuda.synchronize()

    def reset():
        for x in outs:
            x.zero_()
        status.zero_()

    _replay_and_check(graph, lambda: outs, want, reset, _noise)
    assert int(status.item()) == 0
