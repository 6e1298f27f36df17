"""Pins of the CPU oracle to facts other than itself.

Each ``pin_*`` function takes an :class:`oracle.ref.Oracle` and raises
``AssertionError`` when the oracle disagrees with what the definition and the
mathematics fix: closed forms (a transpose, exclusive scans), invariants (row
conservation, round trip = identity), special cases that reduce to a textbook
or library routine (W = 1 is a memcpy, equal splits are a block transpose,
stable argsort for the pack), and brute-force enumeration on tiny inputs
against an independent sort-based formulation.

The functions are shared by ``test_oracle_pins.py`` (run on the real oracle)
and ``test_oracle_mutants.py`` (run on copies of the oracle with planted
mistakes, each of which at least one pin must catch).
"""
from __future__ import annotations

import itertools

import numpy as np

import oracle.ref as R

SENT = 0xA5


def _rank_rows(g, W, rows, R_bytes):
    return [g.integers(0, 256, size=(int(n), R_bytes), dtype=np.uint8) for n in rows]


def _out_bufs(W, cap, R_bytes):
    return [np.full((int(c), R_bytes), SENT, dtype=np.uint8) for c in cap]


def _flat(bufs):
    return [b.reshape(-1) for b in bufs]


def run_a2av(o, R_bytes, X, S, cap=None):
    """Run the oracle's whole definition; returns (status, Y list, O, so, ro)."""
    W = len(X)
    S = np.asarray(S, dtype=np.int64)
    if cap is None:
        cap = S.sum(axis=0)
    Y = _out_bufs(W, cap, R_bytes)
    in_rows = np.array([x.shape[0] for x in X], dtype=np.int64)
    st, O, so, ro = o.a2av(R_bytes, _flat(X), in_rows, _flat(Y), np.asarray(cap, np.int64), S)
    return st, Y, O, so, ro


def brute_force_a2av(X, S):
    """Independent formulation: tag every input row, give it the destination
    whose block of the source's row range holds it (found by walking the split
    vector), then gather each destination's rows sorted by (source, row)."""
    W = len(X)
    tagged = []
    for s in range(W):
        i = 0
        for d in range(W):
            for _ in range(int(S[s][d])):
                tagged.append((d, s, i))
                i += 1
    out = []
    for d in range(W):
        mine = sorted((s, i) for (dd, s, i) in tagged if dd == d)
        out.append([X[s][i] for (s, i) in mine])
    return out


# ------------------------------------------------------------------ exchange / offsets
def pin_exchange_is_transpose(o):
    g = np.random.default_rng(11)
    for W in (1, 2, 3, 4, 7, 8, 64):
        S = g.integers(0, 1000, size=(W, W), dtype=np.int64)
        st, O = o.exchange_splits(S)
        assert st == 0
        assert np.array_equal(O, S.T), f"exchange != transpose at W={W}"
        st2, back = o.exchange_splits(O)
        assert st2 == 0 and np.array_equal(back, S)


def pin_offsets_are_exclusive_scans(o):
    g = np.random.default_rng(12)
    for W in (1, 2, 4, 5, 8, 64):
        S = g.integers(0, 1000, size=(W, W), dtype=np.int64)
        O = np.ascontiguousarray(S.T)
        st, so, ro = o.offsets(S, O)
        assert st == 0
        zero = np.zeros((W, 1), dtype=np.int64)
        assert np.array_equal(so, np.hstack([zero, np.cumsum(S, axis=1)])), "send_off"
        assert np.array_equal(ro, np.hstack([zero, np.cumsum(O, axis=1)])), "recv_off"
        # receive totals are column sums of S: rows are conserved
        assert np.array_equal(ro[:, W], S.sum(axis=0))
        assert so[:, W].sum() == ro[:, W].sum()


# ------------------------------------------------------------------ payload
def pin_brute_force_tiny(o):
    """Every split matrix with W <= 3 and at most 3 rows sent per source."""
    g = np.random.default_rng(13)
    R_bytes = 3
    for W in (1, 2, 3):
        rows_choices = [v for v in itertools.product(range(4), repeat=W) if sum(v) <= 3]
        n = [3] * W
        X = _rank_rows(g, W, n, R_bytes)
        for S in itertools.product(rows_choices, repeat=W):
            S = np.array(S, dtype=np.int64)
            st, Y, O, _, _ = run_a2av(o, R_bytes, X, S)
            assert st == 0
            want = brute_force_a2av(X, S)
            for d in range(W):
                got = Y[d]
                exp = np.array(want[d], dtype=np.uint8).reshape(-1, R_bytes)
                assert np.array_equal(got, exp), f"brute force W={W} S={S.tolist()} d={d}"
                for j in range(got.shape[0]):
                    s, i = o.source_of(S, d, j)
                    assert np.array_equal(X[s][i], got[j]), "source_of disagrees"
                assert o.source_of(S, d, got.shape[0]) is None


def pin_round_trip_identity(o):
    """a2av with O as the splits brings every row home when each rank sends
    all of its rows."""
    g = np.random.default_rng(14)
    for W, n, R_bytes in ((4, 256, 128), (8, 300, 12), (3, 17, 1), (5, 64, 8)):
        X = _rank_rows(g, W, [n] * W, R_bytes)
        S = np.stack([g.multinomial(n, [1.0 / W] * W) for _ in range(W)]).astype(np.int64)
        st, Y, O, _, _ = run_a2av(o, R_bytes, X, S)
        assert st == 0
        st, Z, O2, _, _ = run_a2av(o, R_bytes, Y, O)
        assert st == 0
        assert np.array_equal(O2, S)
        for s in range(W):
            assert np.array_equal(Z[s], X[s]), f"round trip W={W} rank {s}"


def pin_equal_splits_block_transpose(o):
    """Equal splits n/W: destination d holds block d of every source, in source
    order, i.e. X.reshape(W, W, n/W, R).transpose(1, 0, 2, 3)."""
    g = np.random.default_rng(15)
    for W, n, R_bytes in ((4, 256, 128), (8, 64, 8), (2, 6, 5)):
        X = _rank_rows(g, W, [n] * W, R_bytes)
        S = np.full((W, W), n // W, dtype=np.int64)
        st, Y, _, _, _ = run_a2av(o, R_bytes, X, S)
        assert st == 0
        blocks = np.stack(X).reshape(W, W, n // W, R_bytes).transpose(1, 0, 2, 3)
        for d in range(W):
            assert np.array_equal(Y[d], blocks[d].reshape(-1, R_bytes)), f"block transpose d={d}"


def pin_w1_is_memcpy(o):
    g = np.random.default_rng(16)
    for n, R_bytes in ((0, 4), (1, 1), (100, 8), (33, 8192)):
        X = _rank_rows(g, 1, [n + 5], R_bytes)
        st, Y, _, _, _ = run_a2av(o, R_bytes, X, np.array([[n]]))
        assert st == 0
        assert np.array_equal(Y[0], X[0][:n])


def pin_diagonal_is_identity(o):
    g = np.random.default_rng(17)
    W, R_bytes = 6, 16
    n = g.integers(0, 50, size=W)
    X = _rank_rows(g, W, n, R_bytes)
    st, Y, _, _, _ = run_a2av(o, R_bytes, X, np.diag(n).astype(np.int64))
    assert st == 0
    for d in range(W):
        assert np.array_equal(Y[d], X[d])


def pin_conservation_and_sentinels(o):
    """Rows are conserved, trailing unsent rows stay home, and output bytes past
    a destination's total are never touched."""
    g = np.random.default_rng(18)
    W, R_bytes = 5, 24
    n = [40, 0, 17, 90, 5]
    X = _rank_rows(g, W, n, R_bytes)
    S = np.zeros((W, W), dtype=np.int64)
    for s in range(W):
        S[s] = g.multinomial(max(n[s] - 3, 0), [1.0 / W] * W) if n[s] >= 3 else 0
    cap = S.sum(axis=0) + np.array([0, 7, 1, 0, 30])
    st, Y, O, so, ro = run_a2av(o, R_bytes, X, S, cap=cap)
    assert st == 0
    assert sum(int(ro[d, W]) for d in range(W)) == int(S.sum())
    for d in range(W):
        tot = int(S[:, d].sum())
        assert np.all(Y[d][tot:] == SENT), "bytes past the total were written"
        got = np.concatenate([Y[d][:tot].reshape(-1)])
        want = np.array(brute_force_a2av(X, S)[d], dtype=np.uint8).reshape(-1)
        assert np.array_equal(got, want)


def pin_error_paths(o):
    """Invalid inputs set the right status bit and write no payload byte."""
    g = np.random.default_rng(19)
    W, R_bytes, n = 4, 8, 20
    X = _rank_rows(g, W, [n] * W, R_bytes)
    good = np.full((W, W), n // W, dtype=np.int64)

    bad = good.copy(); bad[1, 2] = -1
    st, Y, _, _, _ = run_a2av(o, R_bytes, X, bad, cap=np.full(W, 100))
    assert st == R.BAD_SPLIT and all(np.all(y == SENT) for y in Y)

    huge = good.copy(); huge[0, 0] = R.MAX_SPLIT + 1
    st, _, _, _, _ = run_a2av(o, R_bytes, X, huge, cap=np.full(W, 100))
    assert st == R.BAD_SPLIT
    edge = good.copy(); edge[0, 0] = R.MAX_SPLIT
    st_e, _, _ = o.offsets(edge, np.ascontiguousarray(edge.T))
    assert st_e == 0, "a split of exactly the maximum is valid"

    over = good.copy(); over[2, 3] += 1          # rank 2 sends n+1 rows
    st, Y, _, _, _ = run_a2av(o, R_bytes, X, over, cap=np.full(W, 100))
    assert st == R.SEND_OVERRUN and all(np.all(y == SENT) for y in Y)
    exact = good.copy(); exact[2] = [0, 0, 0, n]  # exactly n rows is fine
    st, _, _, _, _ = run_a2av(o, R_bytes, X, exact, cap=np.full(W, 100))
    assert st == 0

    cap = good.sum(axis=0); cap[3] -= 1
    st, Y, _, _, _ = run_a2av(o, R_bytes, X, good, cap=cap)
    assert st == R.RECV_OVERFLOW and all(np.all(y == SENT) for y in Y)
    st, _, _, _, _ = run_a2av(o, R_bytes, X, good, cap=good.sum(axis=0))
    assert st == 0

    # the payload step alone rejects offsets that are not the scans of S
    O = np.ascontiguousarray(good.T)
    _, so, ro = o.offsets(good, O)
    in_rows = np.full(W, n, dtype=np.int64)
    caps = np.full(W, 100, dtype=np.int64)
    for which, idx in (("send", (1, 2)), ("recv", (0, 1)), ("send", (3, 0))):
        so2, ro2 = so.copy(), ro.copy()
        (so2 if which == "send" else ro2)[idx] += 1
        Y = _out_bufs(W, caps, R_bytes)
        st = o.copy(R_bytes, _flat(X), in_rows, _flat(Y), caps, good, so2, ro2)
        assert st & R.BAD_OFFSETS, f"{which} offsets {idx} accepted"
        assert all(np.all(y == SENT) for y in Y)
    Y = _out_bufs(W, caps, R_bytes)
    assert o.copy(R_bytes, _flat(X), in_rows, _flat(Y), caps, good, so, ro) == 0
    # several failures at once report every bit
    both = good.copy(); both[0, 1] += 3
    _, so3, ro3 = o.offsets(both, np.ascontiguousarray(both.T))
    cap3 = both.sum(axis=0); cap3[1] -= 1
    Y = _out_bufs(W, np.full(W, 100), R_bytes)
    st = o.copy(R_bytes, _flat(X), in_rows, _flat(Y), cap3, both, so3, ro3)
    assert st == (R.SEND_OVERRUN | R.RECV_OVERFLOW)
    # host argument errors
    assert o.exchange_splits(np.zeros((0, 0), np.int64))[0] == R.EARG
    assert o.lib.ref_exchange_splits(65, None, None) == R.EARG


# ------------------------------------------------------------------ MoE pack / unpack
def _moe_case(g, T, k, E, R_bytes, distinct=True):
    if distinct:
        ids = np.stack([g.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    else:
        ids = g.integers(0, E, size=(T, k)).astype(np.int32)
    tokens = g.integers(0, 256, size=(T, R_bytes), dtype=np.uint8)
    return tokens, ids


def pin_moe_pack_is_stable_argsort(o):
    g = np.random.default_rng(21)
    for T, k, E, W, R_bytes, distinct in ((64, 8, 256, 8, 16, True), (100, 3, 12, 4, 6, False),
                                          (1, 1, 4, 2, 2, True), (0, 2, 8, 2, 4, False),
                                          (50, 4, 7, 7, 3, False)):
        tokens, ids = _moe_case(g, T, k, E, R_bytes, distinct)
        st, send, perm, splits, counts = o.moe_pack(T, k, E, W, R_bytes, tokens, ids)
        assert st == 0
        flat = ids.reshape(-1)
        order = np.argsort(flat, kind="stable")          # order[p] = slot at row p
        inv = np.empty_like(order); inv[order] = np.arange(order.size)
        assert np.array_equal(perm, inv), "perm != inverse of stable argsort"
        assert np.array_equal(np.sort(perm), np.arange(T * k)), "perm not a bijection"
        rows = send.reshape(-1, R_bytes)
        assert np.array_equal(rows, tokens[order // k]), "send rows"
        assert np.all(np.diff(flat[order]) >= 0)
        assert np.array_equal(counts, np.bincount(flat, minlength=E))
        owner = np.arange(E) // (E // W)
        assert np.array_equal(splits, np.bincount(owner, weights=counts, minlength=W).astype(np.int64))
        assert splits.sum() == T * k


def pin_moe_round_trip(o):
    """pack -> a2av -> a2av with O -> unpack gives every slot its own token."""
    g = np.random.default_rng(22)
    W, T, k, E, R_bytes = 4, 40, 3, 16, 10
    toks, sends, perms, S = [], [], [], np.zeros((W, W), np.int64)
    for r in range(W):
        tokens, ids = _moe_case(g, T, k, E, R_bytes, distinct=True)
        st, send, perm, splits, _ = o.moe_pack(T, k, E, W, R_bytes, tokens, ids)
        assert st == 0
        toks.append(tokens); sends.append(send.reshape(-1, R_bytes)); perms.append(perm)
        S[r] = splits
    st, Y, O, _, _ = run_a2av(o, R_bytes, sends, S)
    assert st == 0
    st, back, _, _, _ = run_a2av(o, R_bytes, Y, O)
    assert st == 0
    for r in range(W):
        st, out = o.moe_unpack(T, k, R_bytes, back[r], perms[r])
        assert st == 0
        out = out.reshape(T, k, R_bytes)
        assert np.array_equal(out, np.repeat(toks[r][:, None, :], k, axis=1))


def pin_moe_errors(o):
    g = np.random.default_rng(23)
    T, k, E, W, R_bytes = 10, 2, 8, 2, 4
    tokens, ids = _moe_case(g, T, k, E, R_bytes, distinct=True)
    for bad in (-1, E, 1 << 30):
        ids2 = ids.copy(); ids2[3, 1] = bad
        st, send, perm, splits, counts = o.moe_pack(T, k, E, W, R_bytes, tokens, ids2)
        assert st == R.BAD_EXPERT
        assert not send.any() and not perm.any() and not splits.any() and not counts.any()
    ids2 = ids.copy(); ids2[0, 0] = E - 1
    assert o.moe_pack(T, k, E, W, R_bytes, tokens, ids2)[0] == 0
    assert o.moe_pack(T, k, 9, 2, R_bytes, tokens, ids)[0] == R.EARG  # E % W != 0
    st, send, perm, _, _ = o.moe_pack(T, k, E, W, R_bytes, tokens, ids)
    for bad in (-1, T * k):
        p2 = perm.copy(); p2[5] = bad
        st, out = o.moe_unpack(T, k, R_bytes, send, p2)
        assert st == R.BAD_PERM and not out.any()


# ------------------------------------------------------------------ embedding keys
def pin_emb_two_call_consistency(o):
    """Keys and lengths exchanged as two calls: for every (d, s) the received
    lengths chunk sums to the keys chunk received from s, and keys received
    from s are exactly the keys that s laid out for d's tables."""
    from embeddings_a2av_virtual_amd.inputs import emb_keys_rank
    g = np.random.default_rng(24)
    W, tables, batch = 4, 7, 16
    ranks = [emb_keys_rank(g, W=W, tables=tables, batch=batch) for _ in range(W)]
    Sk = np.stack([r.split_keys for r in ranks]).astype(np.int64)
    Sl = np.stack([r.split_lengths for r in ranks]).astype(np.int64)
    keys = [r.keys.view(np.uint8).reshape(-1, 8) for r in ranks]
    lens = [r.lengths.view(np.uint8).reshape(-1, 4) for r in ranks]
    st, Yk, Ok, _, rok = run_a2av(o, 8, keys, Sk)
    assert st == 0
    st, Yl, Ol, _, rol = run_a2av(o, 4, lens, Sl)
    assert st == 0
    for d in range(W):
        lv = Yl[d].reshape(-1).view(np.int32)
        kv = Yk[d].reshape(-1).view(np.int64)
        for s in range(W):
            chunk_lens = lv[rol[d, s]:rol[d, s + 1]]
            assert chunk_lens.sum() == Ok[d, s]
            # the keys of s's tables owned by d, in table then sample order
            off = 0
            mine = []
            for p, t in enumerate(ranks[s].table_order):
                n_t = int(ranks[s].lengths[p * batch:(p + 1) * batch].sum())
                if t % W == d:
                    mine.append(ranks[s].keys[off:off + n_t])
                off += n_t
            want = np.concatenate(mine) if mine else np.zeros(0, np.int64)
            assert np.array_equal(kv[rok[d, s]:rok[d, s + 1]], want)
    assert sum(int(r.keys.size) for r in ranks) == int(rok[:, W].sum())


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
