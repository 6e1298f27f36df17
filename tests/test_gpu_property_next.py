"""Property-based GPU parity of the expert regroup, the weighted combine, the
fused key exchange and the one-step MoE pack + dispatch with its inverse:
random rank counts, expert counts, row widths, base offsets, slot counts,
routings and table layouts, each compared bit-exactly with the CPU oracle.
Derandomized, so every run draws the same examples."""
import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from test_gpu_combine import gpu_combine
from test_gpu_keys import _compare_exchange, gpu_keys_exchange
from test_gpu_pack_dispatch import gpu_pack_dispatch, gpu_unpack_return
from test_gpu_regroup import _owned_total, gpu_regroup, ref_regroup
from gpu_util import SENT

pytestmark = pytest.mark.gpu
SETTINGS = dict(max_examples=40, derandomize=True, deadline=None,
                suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large,
                                       HealthCheck.function_scoped_fixture])


@st.composite
def regroup_cases(draw):
    W = draw(st.integers(1, 12))
    P = draw(st.integers(1, 40))
    R = draw(st.sampled_from([1, 3, 8, 16, 48, 100, 256, 2048]))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    hi = draw(st.sampled_from([0, 1, 4, 30]))
    zero = draw(st.sampled_from([0.0, 0.5, 0.9]))
    pad = draw(st.integers(0, 15))
    direction = draw(st.integers(0, 1))
    return W, W * P, R, seed, hi, zero, pad, direction


@settings(**SETTINGS)
@given(regroup_cases())
def test_random_regroup_matches_oracle(ref, case):
    W, E, R, seed, hi, zero, pad, direction = case
    g = np.random.default_rng(seed)
    counts = g.integers(0, hi + 1, size=(W, E), dtype=np.int64)
    counts[g.random((W, E)) < zero] = 0
    X = [g.integers(0, 256, size=(_owned_total(counts, W, E, d) + int(g.integers(0, 3)), R),
                    dtype=np.uint8) for d in range(W)]
    cap = [x.shape[0] + int(g.integers(0, 3)) for x in X]
    gst, gout, geoff, guards = gpu_regroup(W, E, R, counts, X, cap=cap, direction=direction,
                                           pad=pad)
    rst, rout, reoff, _ = ref_regroup(ref, W, E, R, counts, X, cap=cap, direction=direction)
    assert guards and gst == rst == 0
    assert np.array_equal(geoff, reoff)
    for d in range(W):
        n = _owned_total(counts, W, E, d)
        assert np.array_equal(gout[d][:n], rout[d][:n]), f"rank {d}"
        assert (gout[d][n:] == SENT).all()


@st.composite
def combine_cases(draw):
    W = draw(st.integers(1, 4))
    T = draw(st.integers(0, 40))
    k = draw(st.sampled_from([1, 2, 3, 5, 8, 9, 16, 65]))
    H = draw(st.sampled_from([8, 16, 24, 64, 520, 1000, 7, 13]))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    pad = draw(st.sampled_from([0, 0, 2]))
    return W, T, k, H, seed, pad


@settings(**SETTINGS)
@given(combine_cases())
def test_random_combine_matches_oracle(ref, case):
    W, T, k, H, seed, pad = case
    g = np.random.default_rng(seed)
    Q = T * k
    # any bit pattern: finite values of every size, subnormals, infinities, NaNs
    backs = [g.integers(0, 1 << 16, size=(Q, H), dtype=np.uint16) for _ in range(W)]
    perms = [g.permutation(Q).astype(np.int64) for _ in range(W)]
    ws = [(g.standard_normal((T, k)) * 10.0 ** g.integers(-3, 3, size=(T, k))).astype(np.float32)
          for _ in range(W)]
    st_, outs, guards = gpu_combine(W, T, k, H, backs, perms, ws, pad=pad)
    assert st_ == 0 and guards
    for r in range(W):
        rst, want = ref.moe_combine(T, k, H, backs[r], perms[r], ws[r])
        assert rst == 0
        assert np.array_equal(outs[r], want), f"rank {r}"


@st.composite
def keyx_cases(draw):
    W = draw(st.integers(1, 10))
    NT = draw(st.integers(0, 40))
    batch = draw(st.integers(0, 50))
    lam = draw(st.sampled_from([0.0, 0.5, 3.0, 12.0]))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    pad = draw(st.integers(0, 7))
    return W, NT, batch, lam, seed, pad


@settings(**SETTINGS)
@given(keyx_cases())
def test_random_keys_exchange_matches_oracle(ref, case):
    W, NT, batch, lam, seed, pad = case
    g = np.random.default_rng(seed)
    lengths = [g.poisson(lam, size=(NT, batch)).astype(np.int32) for _ in range(W)]
    keys = [g.integers(0, 1 << 62, size=int(l.sum()), dtype=np.int64) for l in lengths]
    want = ref.keys_exchange(W, NT, batch, lengths, keys)
    assert want[0] == 0
    got = gpu_keys_exchange(W, NT, batch, lengths, keys, pad=pad, ref=ref)
    _compare_exchange(got, want, f"W={W} NT={NT} batch={batch}")


@st.composite
def pack_dispatch_cases(draw):
    W = draw(st.integers(1, 12))
    P = draw(st.integers(1, 24))
    T = draw(st.integers(0, 60))
    k = draw(st.sampled_from([1, 2, 3, 8, 13, 64]))
    R = draw(st.sampled_from([1, 4, 16, 48, 100, 1040, 2064, 8208]))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    skew = draw(st.sampled_from([0.0, 1.1, 3.0]))
    pad = draw(st.integers(0, 15))
    layout = draw(st.integers(0, 1))
    return W, T, k, W * P, R, seed, skew, pad, layout


@settings(**SETTINGS)
@given(pack_dispatch_cases())
def test_random_pack_dispatch_matches_oracle(ref, case):
    W, T, k, E, R, seed, skew, pad, layout = case
    g = np.random.default_rng(seed)
    if skew > 0:   # ids from a Zipf-like law, repeats within a token allowed
        p = 1.0 / np.arange(1, E + 1) ** skew
        ids = [g.choice(E, size=T * k, p=p / p.sum()).astype(np.int32) for _ in range(W)]
    else:
        ids = [g.integers(0, E, size=T * k).astype(np.int32) for _ in range(W)]
    toks = [g.integers(0, 256, size=(T, R), dtype=np.uint8) for _ in range(W)]
    tot = np.zeros(W, dtype=np.int64)
    for x in ids:
        tot += np.bincount(x.astype(np.int64) // (E // W), minlength=W)[:W]
    cap = tot + g.integers(0, 3, size=W)
    gst, recv, perm, S, cnt, boff, guards = gpu_pack_dispatch(W, T, k, E, R, toks, ids, cap,
                                                               layout, pad=pad)
    rst, rrecv, rperm, rS, rcnt, rboff = ref.moe_pack_dispatch(W, T, k, E, R, toks, ids, cap,
                                                               layout)
    assert guards and gst == rst == 0
    assert np.array_equal(S, rS) and np.array_equal(cnt, rcnt) and np.array_equal(boff, rboff)
    for s in range(W):
        assert np.array_equal(perm[s], rperm[s]), s
    for d in range(W):
        t = int(tot[d])
        assert np.array_equal(recv[d][:t], rrecv[d].reshape(-1, R)[:t]), d
        assert (recv[d][t:] == SENT).all()
    rows = [recv[d][:int(tot[d])] for d in range(W)]
    gst, out, guards = gpu_unpack_return(W, T, k, E, R, cnt, ids, perm, rows, layout, pad=pad)
    assert guards and gst == 0
    for s in range(W):
        assert np.array_equal(out[s], np.repeat(toks[s], k, axis=0)), s
