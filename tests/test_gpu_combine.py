"""GPU parity of the gate-weighted MoE combine (moe_combine) against the CPU
oracle: every output bit, including subnormal, infinite and NaN cases, at
small ragged shapes and on sampled tokens of the full dispatch size."""
import numpy as np
import pytest
import torch

from embeddings_a2av_virtual_amd import _binding as B
from embeddings_a2av_virtual_amd import inputs as I
from gpu_util import GuardedBuffer, upload_rows

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def bf16_bits(g, n, H, special=False):
    """n x H bf16 bit patterns of N(0, 1) values; with special, also +-0,
    subnormals, huge values, infinities and NaNs."""
    x = torch.from_numpy(g.standard_normal((n, H)).astype(np.float32)).to(torch.bfloat16)
    b = x.view(torch.int16).numpy().view(np.uint16).copy()
    if special and b.size:
        pick = g.random(b.shape)
        sub = g.integers(1, 0x80, size=b.shape).astype(np.uint16)          # subnormal
        b[pick < 0.10] = sub[pick < 0.10] | (np.uint16(0x8000) * (pick[pick < 0.10] < 0.05))
        b[(pick >= 0.10) & (pick < 0.12)] = 0x0000
        b[(pick >= 0.12) & (pick < 0.13)] = 0x8000
        b[(pick >= 0.13) & (pick < 0.14)] = 0x7F7F                           # largest finite
        b[(pick >= 0.14) & (pick < 0.145)] = 0x7F80                          # +inf
        b[(pick >= 0.145) & (pick < 0.15)] = 0xFF80                          # -inf
        b[(pick >= 0.15) & (pick < 0.152)] = 0x7FC1                          # quiet NaN
        b[(pick >= 0.152) & (pick < 0.154)] = 0xFF81                         # signalling NaN
    return b


def weights(g, T, k, special=False):
    w = I.gate_weights(g, T, k)
    if special and w.size:
        pick = g.random(w.shape)
        w[pick < 0.1] = 0.0
        w[(pick >= 0.1) & (pick < 0.15)] = -w[(pick >= 0.1) & (pick < 0.15)]
        w[(pick >= 0.15) & (pick < 0.2)] = np.float32(1e-39)                 # fp32 subnormal
        w[(pick >= 0.2) & (pick < 0.22)] = np.float32(3e38)
    return w


def gpu_combine(W, T, k, H, backs, perms, ws, pad=0, status_init=0):
    bufs = [upload_rows(b.view(np.uint8), pad=pad) for b in backs]
    pm = [torch.from_numpy(np.ascontiguousarray(p, dtype=np.int64)).cuda() for p in perms]
    wt = [torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32).reshape(-1)).cuda()
          for w in ws]
    outs = [GuardedBuffer(T * H * 2, pad=pad) for _ in range(W)]
    status = torch.full((1,), status_init, dtype=torch.int32, device="cuda")
    B.moe_combine(W, T, k, H, [b.view for b in bufs], pm, wt, [o.view for o in outs], status)
    torch.cuda.synchronize()
    guards = all(o.guards_intact() for o in outs)
    return (int(status.item()), [o.host().view(np.uint16).reshape(T, H) for o in outs], guards)


def _perm(g, Q):
    return g.permutation(Q).astype(np.int64)


@pytest.mark.parametrize("W,T,k,H,pad,special", [
    (8, 64, 8, 7168, 0, False),     # the dispatch width
    (8, 40, 8, 7168, 0, True),
    (4, 100, 3, 1000, 0, True),     # H % 512 != 0: clamped last step
    (2, 50, 5, 77, 0, True),        # H % 8 != 0: element path
    (2, 30, 4, 64, 2, False),       # misaligned bases: element path
    (3, 9, 70, 512, 0, True),       # k > 64: two slot chunks
    (1, 1, 1, 8, 0, True),
    (3, 17, 1, 24, 0, True),        # k = 1: a rounding of w * x
])
def test_combine_matches_oracle(ref, W, T, k, H, pad, special):
    _say("combine", W, T, k, H, pad, special)
    g = I.rng(T * 31 + k * 7 + H)
    Q = T * k
    backs = [bf16_bits(g, Q, H, special) for _ in range(W)]
    perms = [_perm(g, Q) for _ in range(W)]
    ws = [weights(g, T, k, special) for _ in range(W)]
    st, outs, guards = gpu_combine(W, T, k, H, backs, perms, ws, pad=pad)
    assert st == 0 and guards
    for r in range(W):
        rst, want = ref.moe_combine(T, k, H, backs[r], perms[r], ws[r])
        assert rst == 0
        if not np.array_equal(outs[r], want):
            bad = np.argwhere(outs[r] != want)
            t, h = bad[0]
            raise AssertionError(f"rank {r}: {len(bad)} elements differ, first ({t},{h}): "
                                 f"{outs[r][t, h]:#06x} != {want[t, h]:#06x}")


def test_combine_bad_perm_writes_nothing(ref):
    W, T, k, H = 3, 20, 4, 64
    g = I.rng(3)
    backs = [bf16_bits(g, T * k, H) for _ in range(W)]
    perms = [_perm(g, T * k) for _ in range(W)]
    perms[1][7] = T * k
    ws = [weights(g, T, k) for _ in range(W)]
    st, outs, guards = gpu_combine(W, T, k, H, backs, perms, ws)
    assert st == ref.moe_combine(T, k, H, backs[1], perms[1], ws[1])[0] == B.ST_BAD_PERM
    assert guards and all((o == 0xA5A5).all() for o in outs)
    perms[1][7] = -1
    st, outs, _ = gpu_combine(W, T, k, H, backs, perms, ws)
    assert st == B.ST_BAD_PERM and all((o == 0xA5A5).all() for o in outs)
    # a poisoned word: nothing runs
    perms[1][7] = 0
    st, outs, _ = gpu_combine(W, T, k, H, backs, perms, ws, status_init=2)
    assert st == 2 and all((o == 0xA5A5).all() for o in outs)


def test_combine_no_tokens():
    st, outs, guards = gpu_combine(2, 0, 4, 64, [np.zeros((0, 64), np.uint16)] * 2,
                                   [np.zeros(0, np.int64)] * 2, [np.zeros((0, 4), np.float32)] * 2)
    assert st == 0 and guards


def test_combine_full_dispatch_sampled(ref):
    """W=8, 8192 tokens, top-8, hidden 7168 bf16 (896 MiB of returned rows per
    rank): the whole combine on the GPU, 256 sampled tokens per rank through
    the oracle (a token's result depends only on its own k rows)."""
    W, T, k, H = 8, 8192, 8, 7168
    Q = T * k
    g = I.rng(8080)
    backs = [I.payload_bf16(Q, H, seed=70 + r, device="cuda") for r in range(W)]
    perms = [torch.from_numpy(_perm(g, Q)).cuda() for _ in range(W)]
    wsh = [weights(g, T, k) for _ in range(W)]
    wts = [torch.from_numpy(w.reshape(-1)).cuda() for w in wsh]
    outs = [torch.empty((T, H), dtype=torch.bfloat16, device="cuda") for _ in range(W)]
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    B.moe_combine(W, T, k, H, backs, perms, wts, outs, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for r in range(W):
        ts = np.sort(g.choice(T, size=256, replace=False))
        ts[0], ts[-1] = 0, T - 1
        p = perms[r].cpu().numpy()
        rows = torch.from_numpy(p.reshape(T, k)[ts].reshape(-1)).cuda()
        sub = backs[r][rows].view(torch.int16).cpu().numpy().view(np.uint16)
        st, want = ref.moe_combine(len(ts), k, H, sub, np.arange(len(ts) * k, dtype=np.int64),
                                   wsh[r][ts])
        assert st == 0
        got = outs[r][torch.from_numpy(ts).cuda()].view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, want), f"rank {r}"
    _say("combine full: ok")


# ------------------------------------------------------------------ combine from the expert side
def _grouped_inputs(ref, g, W, T, k, E, H, distinct=True, special=False):
    """Host inputs: ids, the pack's perm and counts (oracle, 1-byte stand-in
    rows), expert-side rows per owner, weights."""
    P = E // W
    ids, perms, counts = [], [], []
    for _ in range(W):
        idr = I.topk_ids(g, T, k, E) if distinct else I.uniform_ids(g, T, k, E)
        st, _, perm, _, cnt = ref.moe_pack(T, k, E, W, 1, np.zeros((T, 1), np.uint8), idr)
        assert st == 0
        ids.append(idr.reshape(-1)); perms.append(perm); counts.append(cnt)
    counts = np.stack(counts)
    rows = [int(counts[:, d * P:(d + 1) * P].sum()) for d in range(W)]
    xs = [bf16_bits(g, rows[d], H, special) for d in range(W)]
    ws = [weights(g, T, k, special) for _ in range(W)]
    return ids, perms, counts, xs, ws


def gpu_combine_grouped(W, T, k, E, H, counts, ids, perms, xs, ws, pad=0, status_init=0,
                        exp_rows=None):
    exp_rows = [x.shape[0] for x in xs] if exp_rows is None else list(exp_rows)
    bufs = [upload_rows(x.view(np.uint8), pad=pad) for x in xs]
    idt = [torch.from_numpy(np.ascontiguousarray(i, dtype=np.int32)).cuda() for i in ids]
    pmt = [torch.from_numpy(np.ascontiguousarray(p, dtype=np.int64)).cuda() for p in perms]
    wt = [torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32).reshape(-1)).cuda() for w in ws]
    outs = [GuardedBuffer(T * H * 2, pad=pad) for _ in range(W)]
    cnt = torch.from_numpy(np.ascontiguousarray(counts, dtype=np.int64)).cuda()
    wsb = torch.empty(B.moe_combine_grouped_workspace_bytes(W, T, k, E), dtype=torch.uint8,
                      device="cuda")
    status = torch.full((1,), status_init, dtype=torch.int32, device="cuda")
    B.moe_combine_grouped(W, T, k, E, H, cnt, idt, pmt, [b.view for b in bufs], exp_rows, wt,
                          [o.view for o in outs], wsb, status)
    torch.cuda.synchronize()
    guards = all(o.guards_intact() for o in outs + bufs)
    return int(status.item()), [o.host().view(np.uint16).reshape(T, H) for o in outs], guards


@pytest.mark.parametrize("W,T,k,E,H,pad,special,distinct", [
    (8, 40, 8, 256, 7168, 0, False, True),    # the dispatch shape, fewer tokens
    (8, 30, 8, 256, 1000, 0, True, True),     # clamped last step, special values
    (4, 50, 3, 12, 77, 0, True, False),       # element path, repeated experts
    (2, 20, 4, 8, 64, 2, False, True),        # misaligned bases: element path
    (3, 9, 12, 24, 512, 0, True, True),       # k > 8: two slot groups
    (1, 7, 1, 5, 8, 0, True, True),           # one rank
    (2, 0, 2, 4, 16, 0, False, True),         # no tokens
])
def test_combine_grouped_matches_oracle(ref, W, T, k, E, H, pad, special, distinct):
    _say("combine grouped", W, T, k, E, H, pad, special, distinct)
    g = I.rng(T * 13 + k + E + H)
    ids, perms, counts, xs, ws = _grouped_inputs(ref, g, W, T, k, E, H, distinct, special)
    st, outs, guards = gpu_combine_grouped(W, T, k, E, H, counts, ids, perms, xs, ws, pad=pad)
    rst, want = ref.moe_combine_grouped(W, T, k, E, H, counts, ids, perms, xs, ws)
    assert guards and st == rst == 0
    for r in range(W):
        assert np.array_equal(outs[r], want[r]), f"rank {r}"


@pytest.mark.parametrize("case", ["bad_split", "bad_expert", "bad_perm", "overrun", "mixed",
                                  "poisoned"])
def test_combine_grouped_errors(ref, case):
    W, T, k, E, H = 2, 20, 4, 8, 64
    g = I.rng(44)
    ids, perms, counts, xs, ws = _grouped_inputs(ref, g, W, T, k, E, H)
    exp_rows = [x.shape[0] for x in xs]
    init = 0
    if case == "bad_split":
        counts[1, 1] = -3
    elif case == "bad_expert":
        ids[0][5] = E
    elif case == "bad_perm":
        q = int(np.nonzero(ids[1] != ids[1][0])[0][0])
        ids[1][0], ids[1][q] = ids[1][q], ids[1][0]
    elif case == "overrun":
        xs[1] = xs[1][:-1]
        exp_rows[1] -= 1
    elif case == "mixed":
        ids[0][5] = -1
        xs[0] = xs[0][:-1]
        exp_rows[0] -= 1
    else:
        init = 8
    st, outs, guards = gpu_combine_grouped(W, T, k, E, H, counts, ids, perms, xs, ws,
                                           status_init=init, exp_rows=exp_rows)
    assert guards and all((o == 0xA5A5).all() for o in outs)
    if case == "poisoned":
        assert st == init
        return
    rst, _ = ref.moe_combine_grouped(W, T, k, E, H, counts, ids, perms, xs, ws)
    assert st == rst != 0
    if case == "mixed":
        assert st == B.ST_BAD_EXPERT | B.ST_SEND_OVERRUN


def test_combine_grouped_full_pipeline(ref):
    """W=8, 8192 tokens x top-8 of 256 Zipf(1.1), hidden 7168: pack, grouped
    dispatch, then the combine read from the expert side, against the combine
    of the grouped return on the GPU (both bit-exact paths), and 128 sampled
    tokens per rank through the oracle's combine of the packed rows."""
    W, T, k, E, H = 8, 8192, 8, 256, 7168
    R, Q = 2 * H, T * k
    g = I.rng(515)
    ids_h = [I.topk_ids(g, T, k, E, 1.1) for _ in range(W)]
    ids = [torch.from_numpy(x.reshape(-1)).cuda() for x in ids_h]
    tok = [I.payload_bf16(T, H, 300 + r, device="cuda") for r in range(W)]
    send = [torch.empty((Q, H), dtype=torch.bfloat16, device="cuda") for _ in range(W)]
    perm = [torch.empty(Q, dtype=torch.int64, device="cuda") for _ in range(W)]
    S = torch.empty((W, W), dtype=torch.int64, device="cuda")
    cnt = torch.empty((W, E), dtype=torch.int64, device="cuda")
    ws = torch.empty(B.moe_pack_workspace_bytes(W, T, k, E), dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    B.moe_pack(W, T, k, E, R, tok, ids, send, perm, S, cnt, ws, status)
    counts = cnt.cpu().numpy()
    P = E // W
    rows = [int(counts[:, d * P:(d + 1) * P].sum()) for d in range(W)]
    exp = [torch.empty((c, H), dtype=torch.bfloat16, device="cuda") for c in rows]
    eoff = torch.empty((W, P + 1), dtype=torch.int64, device="cuda")
    gws = torch.empty(B.moe_dispatch_grouped_workspace_bytes(W, E), dtype=torch.uint8,
                      device="cuda")
    B.moe_dispatch_grouped(W, E, R, cnt, send, [Q] * W, exp, rows, eoff, 0, gws, status)
    wts_h = [weights(g, T, k) for _ in range(W)]
    wts = [torch.from_numpy(w.reshape(-1)).cuda() for w in wts_h]
    out = [torch.empty((T, H), dtype=torch.bfloat16, device="cuda") for _ in range(W)]
    cws = torch.empty(B.moe_combine_grouped_workspace_bytes(W, T, k, E), dtype=torch.uint8,
                      device="cuda")
    B.moe_combine_grouped(W, T, k, E, H, cnt, ids, perm, exp, rows, wts, out, cws, status)
    # the unfused path on the GPU: grouped return, then the combine
    back = [torch.empty_like(x) for x in send]
    B.moe_dispatch_grouped(W, E, R, cnt, exp, rows, back, [Q] * W, eoff, 1, gws, status)
    out2 = [torch.empty_like(x) for x in out]
    B.moe_combine(W, T, k, H, back, perm, wts, out2, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for r in range(W):
        assert torch.equal(out[r].view(torch.int16), out2[r].view(torch.int16)), r
        ts = np.sort(g.choice(T, size=128, replace=False))
        p = perm[r].cpu().numpy().reshape(T, k)[ts].reshape(-1)
        sub = send[r][torch.from_numpy(p).cuda()].view(torch.int16).cpu().numpy().view(np.uint16)
        st, want = ref.moe_combine(len(ts), k, H, sub, np.arange(len(ts) * k, dtype=np.int64),
                                   wts_h[r][ts])
        assert st == 0
        got = out[r][torch.from_numpy(ts).cuda()].view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, want), r
    _say("combine grouped full: ok")
