"""GPU parity of the MoE dispatch pack, the dispatch and return a2av, and the
un-pack, against the CPU oracle (bit-exact)."""
import numpy as np
import pytest
import torch

from embeddings_a2av_virtual_amd import _binding as B
from embeddings_a2av_virtual_amd import inputs as I
from embeddings_a2av_virtual_amd.vranks import A2av
from gpu_util import GuardedBuffer, assert_same, gpu_a2av, random_rows, ref_a2av, upload_rows

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


class MoeRun:
    """Device buffers of one pack -> dispatch a2av -> return a2av -> unpack."""

    def __init__(self, W, T, k, E, R, tokens, ids, pad=0):
        self.W, self.T, self.k, self.E, self.R = W, T, k, E, R
        Q = T * k
        self.tok = [upload_rows(t, pad=pad) for t in tokens]
        self.ids = [torch.from_numpy(np.ascontiguousarray(i).reshape(-1)).cuda() for i in ids]
        self.send = [GuardedBuffer(Q * R, pad=pad) for _ in range(W)]
        self.perm = [torch.full((Q,), -7, dtype=torch.int64, device="cuda") for _ in range(W)]
        self.S = torch.full((W, W), -7, dtype=torch.int64, device="cuda")
        self.counts = torch.full((W, E), -7, dtype=torch.int64, device="cuda")
        wsb = B.moe_pack_workspace_bytes(W, T, k, E)
        assert wsb > 0
        self.ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        self.status = torch.zeros(1, dtype=torch.int32, device="cuda")

    def pack(self):
        B.moe_pack(self.W, self.T, self.k, self.E, self.R, [t.view for t in self.tok], self.ids,
                   [s.view for s in self.send], self.perm, self.S, self.counts, self.ws,
                   self.status)
        torch.cuda.synchronize()
        return int(self.status.item())

    def round_trip(self):
        W, R, Q = self.W, self.R, self.T * self.k
        fwd = A2av(W)
        fwd.S.copy_(self.S)
        fwd.exchange_and_offsets()
        torch.cuda.synchronize()
        cap = fwd.recv_off[:, W].cpu().numpy()
        self.recv = [torch.empty(int(c) * R, dtype=torch.uint8, device="cuda") for c in cap]
        fwd.copy(R, [s.view for s in self.send], [Q] * W, self.recv, [int(c) for c in cap])
        back = A2av(W)
        back.S.copy_(fwd.O)
        back.exchange_and_offsets()
        self.back = [torch.empty(Q * R, dtype=torch.uint8, device="cuda") for _ in range(W)]
        back.copy(R, self.recv, [int(c) for c in cap], self.back, [Q] * W)
        self.out = [GuardedBuffer(Q * R) for _ in range(W)]
        self.ustatus = torch.zeros(1, dtype=torch.int32, device="cuda")
        B.moe_unpack(W, self.T, self.k, R, self.back, self.perm, [o.view for o in self.out],
                     self.ustatus)
        torch.cuda.synchronize()
        return int(fwd.status.item()), int(back.status.item()), int(self.ustatus.item()), fwd


def _moe_inputs(g, W, T, k, E, R, dist="zipf"):
    tokens = [random_rows(g, T, R) for _ in range(W)]
    if dist == "zipf":
        ids = [I.topk_ids(g, T, k, E, 1.1) for _ in range(W)]
    else:
        ids = [I.uniform_ids(g, T, k, E) for _ in range(W)]
    return tokens, ids


@pytest.mark.parametrize("W,T,k,E,R,dist,pad", [
    (8, 512, 8, 256, 7168 * 2, "zipf", 0),     # the dispatch workload, fewer tokens
    (8, 300, 8, 256, 1024, "zipf", 0),         # ragged last segment
    (4, 1500, 3, 12, 10, "uniform", 0),        # unaligned rows, repeated experts
    (2, 700, 2, 2, 16, "uniform", 4),          # one expert per rank, misaligned bases
    (4, 2048, 1, 4096, 64, "uniform", 0),      # k = 1, the most experts
    (4, 4000, 4, 4092, 16, "uniform", 0),      # four passes of the histogram scan, the last ragged
    (1, 100, 4, 7, 32, "uniform", 0),          # one rank
])
def test_moe_pack_round_trip_matches_oracle(ref, W, T, k, E, R, dist, pad):
    _say("moe", W, T, k, E, R, dist, pad)
    g = I.rng(T + E + W)
    tokens, ids = _moe_inputs(g, W, T, k, E, R, dist)
    run = MoeRun(W, T, k, E, R, tokens, ids, pad=pad)
    assert run.pack() == 0
    want = [ref.moe_pack(T, k, E, W, R, tokens[r], ids[r]) for r in range(W)]
    for r in range(W):
        st, send, perm, splits, counts = want[r]
        assert st == 0
        assert np.array_equal(run.perm[r].cpu().numpy(), perm), f"perm rank {r}"
        assert np.array_equal(run.S[r].cpu().numpy(), splits), f"splits rank {r}"
        assert np.array_equal(run.counts[r].cpu().numpy(), counts), f"counts rank {r}"
        assert np.array_equal(run.send[r].host(), send), f"send rank {r}"
        assert run.send[r].guards_intact() and run.tok[r].guards_intact()
    fs, bs, us, fwd = run.round_trip()
    assert (fs, bs, us) == (0, 0, 0)
    # the oracle's own chain on the same bytes
    S = np.stack([w[3] for w in want])
    sends = [w[1].reshape(-1, R) for w in want]
    rst, _, _, _, rY = ref_a2av(ref, R, sends, S)
    assert rst == 0
    for d in range(W):
        assert np.array_equal(run.recv[d].cpu().numpy().reshape(-1, R), rY[d]), f"dispatch rank {d}"
    rst2, _, _, _, rback = ref_a2av(ref, R, rY, np.ascontiguousarray(S.T))
    assert rst2 == 0
    for r in range(W):
        assert np.array_equal(run.back[r].cpu().numpy().reshape(-1, R), rback[r])
        ust, rout = ref.moe_unpack(T, k, R, rback[r], want[r][2])
        assert ust == 0
        got = run.out[r].host()
        assert np.array_equal(got, rout), f"unpack rank {r}"
        # closed form: every slot holds its own token
        assert np.array_equal(got.reshape(T, k, R), np.repeat(tokens[r][:, None, :], k, axis=1))
        assert run.out[r].guards_intact()


def test_moe_bad_expert_writes_nothing(ref):
    g = I.rng(5)
    W, T, k, E, R = 4, 400, 4, 32, 64
    tokens, ids = _moe_inputs(g, W, T, k, E, R, "uniform")
    for bad in (-1, E, 1 << 20):
        ids2 = [i.copy() for i in ids]
        ids2[2][123, 1] = bad
        run = MoeRun(W, T, k, E, R, tokens, ids2)
        assert run.pack() == B.ST_BAD_EXPERT
        assert ref.moe_pack(T, k, E, W, R, tokens[2], ids2[2])[0] == B.ST_BAD_EXPERT
        assert bool((run.S == -7).all()) and bool((run.counts == -7).all())
        assert all(bool((p == -7).all()) for p in run.perm)
        assert all(bool((s.view == 0xA5).all()) and s.guards_intact() for s in run.send)


def test_moe_no_tokens():
    W, T, k, E, R = 4, 0, 2, 8, 16
    run = MoeRun(W, T, k, E, R, [np.zeros((0, R), np.uint8)] * W,
                 [np.zeros((0, k), np.int32)] * W)
    assert run.pack() == 0
    assert not run.S.any() and not run.counts.any()


def test_unpack_bad_perm_writes_nothing(ref):
    g = I.rng(6)
    W, T, k, E, R = 2, 64, 2, 8, 32
    tokens, ids = _moe_inputs(g, W, T, k, E, R, "uniform")
    run = MoeRun(W, T, k, E, R, tokens, ids)
    assert run.pack() == 0
    for bad in (-1, T * k):
        perm = [p.clone() for p in run.perm]
        perm[1][17] = bad
        out = [GuardedBuffer(T * k * R) for _ in range(W)]
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        B.moe_unpack(W, T, k, R, [s.view for s in run.send], perm, [o.view for o in out], status)
        torch.cuda.synchronize()
        assert int(status.item()) == B.ST_BAD_PERM
        assert ref.moe_unpack(T, k, R, run.send[1].host(), perm[1].cpu().numpy())[0] == B.ST_BAD_PERM
        assert all(bool((o.view == 0xA5).all()) for o in out)


def test_moe_dispatch_full_size(ref):
    """W=8, 8192 tokens x 7168 bf16, top-8 of 256 Zipf(1.1) experts. The
    integer outputs are compared whole with the oracle (run on the ids with
    1-byte stand-in rows, which leaves perm, splits and counts unchanged);
    packed rows on a sample; the round trip whole against the closed form."""
    W, T, k, E, hidden = 8, 8192, 8, 256, 7168
    R = hidden * 2
    g = I.rng(77)
    ids = [I.topk_ids(g, T, k, E, 1.1) for _ in range(W)]
    _say("full moe: ids drawn")
    Q = T * k
    tok = [I.payload_bf16(T, hidden, 700 + r, device="cuda").view(torch.uint8).reshape(-1)
           for r in range(W)]
    idd = [torch.from_numpy(i.reshape(-1)).cuda() for i in ids]
    send = [torch.empty(Q * R, dtype=torch.uint8, device="cuda") for _ in range(W)]
    perm = [torch.empty(Q, dtype=torch.int64, device="cuda") for _ in range(W)]
    S = torch.empty((W, W), dtype=torch.int64, device="cuda")
    counts = torch.empty((W, E), dtype=torch.int64, device="cuda")
    ws = torch.empty(B.moe_pack_workspace_bytes(W, T, k, E), dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    B.moe_pack(W, T, k, E, R, tok, idd, send, perm, S, counts, ws, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    gi = np.random.default_rng(1)
    for r in range(W):
        st, _, rperm, rsplits, rcounts = ref.moe_pack(T, k, E, W, 1, np.zeros(T, np.uint8), ids[r])
        assert st == 0
        p = perm[r].cpu().numpy()
        assert np.array_equal(p, rperm) and np.array_equal(S[r].cpu().numpy(), rsplits)
        assert np.array_equal(counts[r].cpu().numpy(), rcounts)
        qs = torch.tensor(gi.integers(0, Q, size=256), dtype=torch.int64, device="cuda")
        rows_send = send[r].view(Q, R)[torch.from_numpy(p).cuda()[qs]]
        rows_tok = tok[r].view(T, R)[qs // k]
        assert torch.equal(rows_send, rows_tok), f"packed rows rank {r}"
    _say("full moe: pack checked; rank 0 sends", S[0].tolist())
    fwd = A2av(W)
    fwd.S.copy_(S)
    fwd.exchange_and_offsets()
    torch.cuda.synchronize()
    cap = fwd.recv_off[:, W].cpu().numpy()
    recv = [torch.empty(int(c) * R, dtype=torch.uint8, device="cuda") for c in cap]
    fwd.copy(R, send, [Q] * W, recv, [int(c) for c in cap])
    del send
    bk = A2av(W)
    bk.S.copy_(fwd.O)
    bk.exchange_and_offsets()
    back = [torch.empty(Q * R, dtype=torch.uint8, device="cuda") for _ in range(W)]
    bk.copy(R, recv, [int(c) for c in cap], back, [Q] * W)
    del recv
    out = [torch.empty(Q * R, dtype=torch.uint8, device="cuda") for _ in range(W)]
    ust = torch.zeros(1, dtype=torch.int32, device="cuda")
    B.moe_unpack(W, T, k, R, back, perm, out, ust)
    torch.cuda.synchronize()
    assert (int(fwd.status.item()), int(bk.status.item()), int(ust.item())) == (0, 0, 0)
    for r in range(W):
        want = tok[r].view(T, 1, R).expand(T, k, R)
        assert torch.equal(out[r].view(T, k, R), want), f"round trip rank {r}"


@pytest.mark.parametrize("env,R", [
    # the scatter's vectors per lane follow the row width: 1, 2, 3, 4, 5 (two
    # chunks), 6, 7 (two chunks), 8
    ({}, 16), ({}, 1040), ({}, 2064), ({}, 3088), ({}, 8208), ({}, 6144), ({}, 14336), ({}, 8192),
    ({"A2AV_MOE_GATHER_UNROLL": "4"}, 1040), ({"A2AV_MOE_GATHER_UNROLL": "8"}, 1040),
])
def test_moe_launch_shapes_give_identical_bytes(ref, monkeypatch, env, R):
    W, T, k, E = 4, 300, 4, 16
    g = I.rng(31)
    tokens, ids = _moe_inputs(g, W, T, k, E, R, "zipf")
    for key, val in env.items():
        monkeypatch.setenv(key, val)
    run = MoeRun(W, T, k, E, R, tokens, ids)
    assert run.pack() == 0
    for r in range(W):
        st, send, perm, splits, counts = ref.moe_pack(T, k, E, W, R, tokens[r], ids[r])
        assert np.array_equal(run.send[r].host(), send)
        assert np.array_equal(run.perm[r].cpu().numpy(), perm)
    assert run.round_trip()[:3] == (0, 0, 0)
    for r in range(W):
        got = run.out[r].host().reshape(T, k, R)
        assert np.array_equal(got, np.repeat(tokens[r][:, None, :], k, axis=1))
