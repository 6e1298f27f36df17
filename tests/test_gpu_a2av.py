"""GPU parity of the a2av (exchange, offsets, payload) against the CPU oracle,
bit-exact, through the C ABI."""
import os

import numpy as np
import pytest
import torch

from embeddings_a2av_virtual_amd import inputs as I
from embeddings_a2av_virtual_amd import _binding as B
from gpu_util import SENT, assert_same, gpu_a2av, random_rows, ref_a2av

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def test_device_is_there():
    assert torch.cuda.is_available()
    _say("device:", torch.cuda.get_device_name(0))
    assert B.a2av_abi_version() == 1


# ------------------------------------------------------------------ the tiny workload
@pytest.mark.parametrize("fused", [False, True], ids=["3call", "fused"])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tiny_workload_and_round_trip(ref, seed, fused):
    """W=4, 256 rows x 64 bf16 per rank, multinomial splits, then back home."""
    _say("tiny seed", seed)
    g = I.rng(seed)
    W, n, cols = 4, 256, 64
    R = cols * 2
    X = [I.payload_bf16(n, cols, seed * 100 + r).view(torch.uint8).numpy().reshape(n, R)
         for r in range(W)]
    S = I.uniform_splits(g, W, n)
    gpu = gpu_a2av(R, X, S, fused=fused)
    want = ref_a2av(ref, R, X, S)
    assert_same(gpu, want, f"tiny seed {seed}")
    # round trip: the received rows go home with the transposed splits
    Y = gpu[4]
    gpu2 = gpu_a2av(R, Y, gpu[1], fused=fused)
    want2 = ref_a2av(ref, R, want[4], want[1])
    assert_same(gpu2, want2, "tiny round trip")
    for r in range(W):
        assert np.array_equal(gpu2[4][r], X[r])


# ------------------------------------------------------------------ several tiles, ragged
@pytest.mark.parametrize("W,R,max_rows,zero_frac,seed", [
    (4, 8192, 700, 0.0, 3),
    (8, 8192, 300, 0.3, 4),
    (5, 4096 + 16, 999, 0.2, 5),
    (3, 128, 20000, 0.0, 6),
    (16, 512, 257, 0.5, 7),
    (64, 48, 40, 0.3, 8),
    (6, 2048, 400, 0.3, 13),   # W > 4: the four waves of a workgroup share the loads
    (7, 1024, 600, 0.5, 14),   # rows k + 4 past W are dropped
    (2, 16, 9000, 0.0, 15),
    (1, 32, 5000, 0.0, 16),
])
@pytest.mark.parametrize("fused", [False, True], ids=["3call", "fused"])
def test_random_splits_many_tiles(ref, W, R, max_rows, zero_frac, seed, fused):
    _say("random", W, R, max_rows, zero_frac, seed)
    g = I.rng(seed)
    S = I.random_splits(g, W, max_rows, zero_frac)
    n = S.sum(axis=1) + g.integers(0, 5, size=W)      # some trailing rows stay home
    X = [random_rows(g, n[s], R) for s in range(W)]
    cap = S.sum(axis=0) + g.integers(0, 3, size=W)     # some room left over
    assert_same(gpu_a2av(R, X, S, cap=cap, fused=fused), ref_a2av(ref, R, X, S, cap=cap), "random")


# ------------------------------------------------------------------ widths and alignment
@pytest.mark.parametrize("R", [1, 2, 3, 4, 5, 7, 8, 12, 16, 24, 100, 8196])
@pytest.mark.parametrize("in_pad,out_pad", [(0, 0), (1, 0), (0, 3), (4, 8), (8, 0), (6, 6)])
@pytest.mark.parametrize("fused", [False, True], ids=["3call", "fused"])
def test_row_widths_and_misaligned_bases(ref, R, in_pad, out_pad, fused):
    g = I.rng(1000 + R * 10 + in_pad)
    W = 4
    max_rows = max(1, 40000 // R)
    S = I.random_splits(g, W, max_rows, 0.2)
    X = [random_rows(g, S[s].sum(), R) for s in range(W)]
    assert_same(gpu_a2av(R, X, S, in_pad=in_pad, out_pad=out_pad, fused=fused), ref_a2av(ref, R, X, S),
                f"R={R} pads={in_pad},{out_pad}")


# ------------------------------------------------------------------ degenerate cases
@pytest.mark.parametrize("fused", [False, True], ids=["3call", "fused"])
def test_degenerate_cases(ref, fused):
    g = I.rng(9)
    R = 64
    cases = {
        "all_zero": (np.zeros((4, 4), np.int64), [3, 0, 5, 1]),
        "w1": (np.array([[77]]), [80]),
        "w1_empty": (np.array([[0]]), [0]),
        "diag": (np.diag([5, 0, 9, 1]).astype(np.int64), [5, 0, 9, 1]),
        "one_rank_sends_nothing": (np.array([[2, 2, 2], [0, 0, 0], [1, 5, 0]]), [6, 0, 6]),
        "one_rank_receives_nothing": (np.array([[2, 0, 2], [4, 0, 0], [1, 0, 9]]), [4, 4, 10]),
        "all_to_one": (np.array([[0, 0, 100]] * 3), [100, 100, 100]),
        "w64_sparse": (np.where(g.random((64, 64)) < 0.05, g.integers(1, 9, (64, 64)), 0), None),
    }
    for name, (S, n) in cases.items():
        S = np.asarray(S, dtype=np.int64)
        if n is None:
            n = S.sum(axis=1)
        X = [random_rows(g, n[s], R) for s in range(S.shape[0])]
        _say("degenerate", name)
        assert_same(gpu_a2av(R, X, S, fused=fused), ref_a2av(ref, R, X, S), name)


# ------------------------------------------------------------------ error paths
# Every payload kernel refuses: the one-call and copy-only wave kernels for
# W <= 8 (aligned rows with the deferred gate, misaligned rows and 16 loads in
# flight with the checks up front), the prep + wave copy for more ranks, and
# the workgroup kernel (LDS metadata up to 16 ranks, global above).
ERROR_ENVS = {"wave": {}, "wave_u16": {"A2AV_WAVE_UNROLL": "16"},
              "block_kernel": {"A2AV_BLOCK_KERNEL": "1"}}


@pytest.mark.parametrize("env", list(ERROR_ENVS), ids=list(ERROR_ENVS))
@pytest.mark.parametrize("R", [16, 24])
@pytest.mark.parametrize("W", [4, 5, 6, 8, 12, 20])
@pytest.mark.parametrize("fused", [False, True], ids=["3call", "fused"])
def test_error_paths_match_oracle(ref, monkeypatch, fused, W, R, env):
    for k, v in ERROR_ENVS[env].items():
        monkeypatch.setenv(k, v)
    g = I.rng(10 + W + R)
    per = 3
    n = W * per
    X = [random_rows(g, n, R) for _ in range(W)]
    good = np.full((W, W), per, dtype=np.int64)
    roomy = np.full(W, 1000)

    neg = good.copy(); neg[2, 1] = -3
    big = good.copy(); big[0, W - 1] = B.MAX_SPLIT + 1
    over = good.copy(); over[1, 0] += 1
    tight = good.sum(axis=0); tight[2] -= 1
    both = good.copy(); both[3, 2] += 2
    both_cap = both.sum(axis=0); both_cap[2] -= 1
    last = good.copy(); last[W - 1, W - 1] += 1  # the last pair overruns and overflows
    last_cap = good.sum(axis=0)
    cases = [("negative", neg, roomy), ("too_large", big, roomy), ("overrun", over, roomy),
             ("overflow", good, tight), ("overrun+overflow", both, both_cap),
             ("last_pair", last, last_cap), ("exact_fit", good, good.sum(axis=0))]
    for name, S, cap in cases:
        _say("error case", name, "W", W, "R", R, env)
        gpu = gpu_a2av(R, X, S, cap=cap, fused=fused)
        want = ref_a2av(ref, R, X, S, cap=cap)
        assert_same(gpu, want, name)
        if want[0]:
            assert all(np.all(y == SENT) for y in gpu[4]), f"{name}: payload written on failure"
        else:
            assert name == "exact_fit"


@pytest.mark.parametrize("env", list(ERROR_ENVS), ids=list(ERROR_ENVS))
@pytest.mark.parametrize("R", [16, 24])
@pytest.mark.parametrize("W", [4, 6, 8, 12, 20])
def test_copy_rejects_foreign_offsets(ref, monkeypatch, W, R, env):
    """Offsets that are not the scans of S: the copy refuses and writes nothing."""
    from embeddings_a2av_virtual_amd.vranks import A2av
    from gpu_util import GuardedBuffer, upload_rows
    g = I.rng(11 + W + R)
    per = 3
    n = W * per
    X = [random_rows(g, n, R) for _ in range(W)]
    S = np.full((W, W), per, dtype=np.int64)
    st = A2av(W)
    st.set_splits(S)
    st.exchange_and_offsets()
    torch.cuda.synchronize()
    for k, v in ERROR_ENVS[env].items():
        monkeypatch.setenv(k, v)
    so0, ro0 = st.send_off.clone(), st.recv_off.clone()
    for which, idx, delta in (("send", (1, 2), 1), ("recv", (0, 1), -1), ("send", (3, 0), 2),
                              ("recv", (2, W), 1), ("send", (W - 1, W - 1), -1),
                              ("recv", (W - 1, W // 2), 1), ("send", (0, W), -1)):
        st.send_off.copy_(so0); st.recv_off.copy_(ro0); st.status.zero_()
        (st.send_off if which == "send" else st.recv_off)[idx] += delta
        ins = [upload_rows(x) for x in X]
        outs = [GuardedBuffer(1000 * R) for _ in range(W)]
        st.copy(R, [b.view for b in ins], [n] * W, [b.view for b in outs], [1000] * W)
        torch.cuda.synchronize()
        caps = np.full(W, 1000, np.int64)
        Y = [np.full(1000 * R, SENT, np.uint8) for _ in range(W)]
        rst = ref.copy(R, [x.reshape(-1) for x in X], np.full(W, n), Y, caps, S,
                       st.send_off.cpu().numpy(), st.recv_off.cpu().numpy())
        gst = int(st.status.item())
        _say("foreign offsets", which, idx, "W", W, "R", R, env, gst, rst)
        assert gst == rst and gst & B.ST_BAD_OFFSETS
        assert all(bool((b.view == SENT).all().item()) and b.guards_intact() for b in outs)
        assert all(b.guards_intact() for b in ins)


@pytest.mark.parametrize("fused", [False, True], ids=["3call", "fused"])
def test_poisoned_status_blocks_every_op(ref, fused):
    g = I.rng(12)
    W, R, n = 4, 16, 20
    X = [random_rows(g, n, R) for _ in range(W)]
    S = np.full((W, W), n // W, dtype=np.int64)
    st, O, so, ro, Y, guards = gpu_a2av(R, X, S, status_init=64, fused=fused)
    assert st == 64 and guards
    assert not O.any() and not so.any() and not ro.any()
    assert all(np.all(y == SENT) for y in Y)


# ------------------------------------------------------------------ launch shapes
@pytest.mark.parametrize("env", [
    {"A2AV_BLOCKS_PER_CU": "1"}, {"A2AV_BLOCKS_PER_CU": "3", "A2AV_UNROLL": "1"},
    {"A2AV_UNROLL": "2", "A2AV_NT": "0"}, {"A2AV_UNROLL": "8", "A2AV_XCD_REMAP": "1"},
    {"A2AV_MIN_PIECE": "4096", "A2AV_BLOCKS_PER_CU": "16"}, {"A2AV_MIN_PIECE": "1048576"},
    {"A2AV_PIECE": "4096"}, {"A2AV_PIECE": "65536", "A2AV_BLOCKS_PER_CU": "2"},
    {"A2AV_PIECE": "1000000"},
    {"A2AV_BLOCK_KERNEL": "1"}, {"A2AV_BLOCK_KERNEL": "1", "A2AV_PIECE": "65536"},
    {"A2AV_WAVE_PIECE": "4096"}, {"A2AV_WAVE_PIECE": "65536", "A2AV_WAVE_UNROLL": "16"},
    {"A2AV_WAVE_PIECE": "1052672", "A2AV_WAVE_UNROLL": "8"},
])
@pytest.mark.parametrize("fused", [False, True], ids=["3call", "fused"])
@pytest.mark.parametrize("W", [3, 8, 12])
def test_launch_shapes_give_identical_bytes(ref, monkeypatch, env, fused, W):
    g = I.rng(13 + W)
    R = 1040
    S = I.random_splits(g, W, 600, 0.25)
    X = [random_rows(g, S[s].sum(), R) for s in range(W)]
    want = ref_a2av(ref, R, X, S)
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    assert_same(gpu_a2av(R, X, S, fused=fused), want, str(env))


# ------------------------------------------------------------------ the 32 MiB workload
@pytest.mark.parametrize("fused", [False, True], ids=["3call", "fused"])
def test_moe32_workload_full(ref, fused):
    """W=4, 4096 rows x 4096 bf16 (32 MiB) per rank, multinomial splits, every
    byte compared."""
    g = I.rng(20)
    W, n, cols = 4, 4096, 4096
    R = cols * 2
    X = [I.payload_bf16(n, cols, 2000 + r).view(torch.uint8).numpy().reshape(n, R)
         for r in range(W)]
    S = I.uniform_splits(g, W, n)
    assert_same(gpu_a2av(R, X, S, fused=fused), ref_a2av(ref, R, X, S), "moe32")


@pytest.mark.parametrize("W", [4, 8])
@pytest.mark.parametrize("mib", [1, 16, 32, 64, 256])
@pytest.mark.parametrize("kind", ["uniform", "half_zero"])
@pytest.mark.parametrize("fused", [False, True], ids=["3call", "fused"])
def test_sweep_sizes_full(ref, W, mib, kind, fused):
    """8 KiB rows, 1..256 MiB per rank, uniform or 50 % zero splits."""
    _say("sweep", W, mib, kind)
    g = I.rng(30 + mib + W)
    R = 8192
    n = I.rows_for_mib(mib, R)
    S = I.uniform_splits(g, W, n) if kind == "uniform" else I.half_zero_splits(g, W, n)
    X = [random_rows(g, n, R) if mib <= 16 else
         I.payload_bytes(n, R, 4000 + s, device="cuda").cpu().numpy() for s in range(W)]
    assert_same(gpu_a2av(R, X, S, fused=fused), ref_a2av(ref, R, X, S), f"sweep {W} {mib} {kind}")
