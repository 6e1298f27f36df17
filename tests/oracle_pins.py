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
def _tables_by_owner(W, tables):
    """Table order after bucketing, written as a sort: by (t mod W, t)."""
    return sorted(range(tables), key=lambda t: (t % W, t))


def _bucketize_numpy(W, lengths, keys):
    """Independent formulation of the bucketing: split the keys per table with
    a cumulative sum, reorder tables with a sort, concatenate."""
    tables, batch = lengths.shape
    per_table = lengths.sum(axis=1)
    bounds = np.concatenate([[0], np.cumsum(per_table)])
    order = _tables_by_owner(W, tables)
    lo = np.concatenate([lengths[t] for t in order]) if tables else np.zeros(0, np.int32)
    ko = (np.concatenate([keys[bounds[t]:bounds[t + 1]] for t in order])
          if tables else np.zeros(0, np.int64))
    sk = np.bincount(np.arange(tables) % W, weights=per_table, minlength=W).astype(np.int64)
    sl = np.bincount(np.arange(tables) % W, minlength=W).astype(np.int64) * batch
    return lo, ko, sk, sl


def pin_keys_bucketize_is_sort_by_owner(o):
    from embeddings_a2av_virtual_amd.inputs import emb_keys_rank
    g = np.random.default_rng(25)
    for W, tables, batch in ((8, 26, 64), (4, 7, 16), (3, 1, 5), (5, 3, 0), (1, 4, 9), (6, 0, 4)):
        r = emb_keys_rank(g, tables=tables, batch=batch)
        st, lo, ko, sk, sl = o.keys_bucketize(W, tables, batch, r.lengths, r.keys)
        assert st == 0
        wlo, wko, wsk, wsl = _bucketize_numpy(W, r.lengths, r.keys)
        assert np.array_equal(lo, wlo), "lengths order"
        assert np.array_equal(ko[:wko.size], wko), "keys order"
        assert np.array_equal(sk, wsk) and np.array_equal(sl, wsl), "splits"
        assert sk.sum() == r.keys.size and sl.sum() == tables * batch
    # errors: a negative length, keys shorter than the lengths say
    r = emb_keys_rank(g, tables=4, batch=8)
    bad = r.lengths.copy(); bad[2, 3] = -1
    assert o.keys_bucketize(4, 4, 8, bad, r.keys)[0] == R.BAD_SPLIT
    assert o.keys_bucketize(4, 4, 8, r.lengths, r.keys[:-1])[0] == R.SEND_OVERRUN
    more = np.concatenate([r.keys, [7, 7]])  # spare keys are allowed and not sent
    st, lo, ko, sk, sl = o.keys_bucketize(4, 4, 8, r.lengths, more)
    assert st == 0 and sk.sum() == r.keys.size


def pin_emb_two_call_consistency(o):
    """Keys and lengths bucketed, then exchanged as two calls: for every
    (d, s) the received lengths chunk sums to the keys chunk received from s,
    and the keys received from s are s's keys of the tables d owns."""
    from embeddings_a2av_virtual_amd.inputs import emb_keys_rank
    g = np.random.default_rng(24)
    W, tables, batch = 4, 7, 16
    ranks = [emb_keys_rank(g, tables=tables, batch=batch) for _ in range(W)]
    buck = [o.keys_bucketize(W, tables, batch, r.lengths, r.keys) for r in ranks]
    assert all(b[0] == 0 for b in buck)
    Sk = np.stack([b[3] for b in buck])
    Sl = np.stack([b[4] for b in buck])
    keys = [b[2].view(np.uint8).reshape(-1, 8) for b in buck]
    lens = [b[1].view(np.uint8).reshape(-1, 4) for b in buck]
    st, Yk, Ok, _, rok = run_a2av(o, 8, keys, Sk)
    assert st == 0
    st, Yl, Ol, _, rol = run_a2av(o, 4, lens, Sl)
    assert st == 0
    for d in range(W):
        lv = Yl[d].reshape(-1).view(np.int32)
        kv = Yk[d].reshape(-1).view(np.int64)
        for s in range(W):
            assert lv[rol[d, s]:rol[d, s + 1]].sum() == Ok[d, s]
            bounds = np.concatenate([[0], np.cumsum(ranks[s].lengths.sum(axis=1))])
            mine = [ranks[s].keys[bounds[t]:bounds[t + 1]] for t in range(d, tables, W)]
            want = np.concatenate(mine) if mine else np.zeros(0, np.int64)
            assert np.array_equal(kv[rok[d, s]:rok[d, s + 1]], want)
    assert sum(int(r.keys.size) for r in ranks) == int(rok[:, W].sum())


def pin_keys_exchange_closed_form(o):
    """The fused exchange: receiver d holds, for s = 0..W-1 in order, source
    s's keys and lengths of the tables d owns (ascending), written out from
    the generator's table-order arrays with numpy slicing; the split
    matrices, receive offsets and every failure case as the composition
    defines them."""
    from embeddings_a2av_virtual_amd.inputs import emb_keys_rank
    g = np.random.default_rng(30)
    for W, tables, batch in ((4, 7, 16), (3, 2, 5), (1, 4, 3), (5, 0, 4), (2, 3, 0), (8, 26, 9)):
        ranks = [emb_keys_rank(g, tables=tables, batch=batch) for _ in range(W)]
        L = [r.lengths for r in ranks]
        K = [r.keys for r in ranks]
        st, lo, ko, sk, sl, ro = o.keys_exchange(W, tables, batch, L, K)
        assert st == 0
        for d in range(W):
            own = list(range(d, tables, W))
            wl, wk, col = [], [], []
            for s in range(W):
                bounds = np.concatenate([[0], np.cumsum(L[s].sum(axis=1))]).astype(np.int64)
                mine = [K[s][bounds[t]:bounds[t + 1]] for t in own]
                wk += mine
                wl += [L[s][t] for t in own]
                col.append(sum(m.size for m in mine))
            want_k = np.concatenate(wk) if wk else np.zeros(0, np.int64)
            want_l = np.concatenate(wl) if wl else np.zeros(0, np.int32)
            assert np.array_equal(ko[d], want_k) and np.array_equal(lo[d], want_l)
            assert np.array_equal(sk[:, d], col)
            assert np.array_equal(sl[:, d], [len(own) * batch] * W)
            assert np.array_equal(ro[d], np.concatenate([[0], np.cumsum(col)]))
    # failures: a negative length, keys short of the lengths, a receiver short of room
    W, tables, batch = 3, 5, 6
    ranks = [emb_keys_rank(g, tables=tables, batch=batch) for _ in range(W)]
    L = [r.lengths.copy() for r in ranks]
    K = [r.keys for r in ranks]
    bad = [l.copy() for l in L]; bad[1][2, 3] = -1
    st, lo, ko, sk, sl, ro = o.keys_exchange(W, tables, batch, bad, K)
    assert st == R.BAD_SPLIT and (sk == -7).all() and (ro == -7).all()
    assert not any(x.any() for x in ko) and not any(x.any() for x in lo)
    short = [k.copy() for k in K]; short[2] = short[2][:-1]
    assert o.keys_exchange(W, tables, batch, L, short)[0] == R.SEND_OVERRUN
    st, lo, ko, sk, sl, ro = o.keys_exchange(W, tables, batch, L, K)
    kcap = ro[:, W].copy()
    lcap = np.array([x.size for x in lo], dtype=np.int64)
    kcap[1] -= 1
    st, lo2, ko2, sk2, sl2, ro2 = o.keys_exchange(W, tables, batch, L, K, lcap, kcap)
    assert st == R.RECV_OVERFLOW
    assert not any(x.any() for x in ko2)
    assert (sk2[:, 1] == -7).all() and (ro2[1] == -7).all()
    assert np.array_equal(sk2[:, 0], sk[:, 0]) and np.array_equal(ro2[2], ro[2])


# ------------------------------------------------------------------ expert regroup
def _regroup_by_sort(W, E, d, R, counts, inp):
    """Independent formulation: tag every source-major row with (source,
    owned expert) by walking the counts, then stable-sort the rows by expert."""
    P = E // W
    tags = []
    for s in range(W):
        for j in range(P):
            tags += [(j, s)] * int(counts[s, d * P + j])
    rows = inp.reshape(-1, R)[:len(tags)]
    order = sorted(range(len(tags)), key=lambda i: tags[i][0])  # sorted() is stable
    return rows[order].reshape(-1) if tags else np.zeros(0, np.uint8)


def pin_moe_regroup_is_stable_sort_by_expert(o):
    g = np.random.default_rng(26)
    for W, E, Rb in ((4, 16, 8), (8, 256, 4), (1, 3, 5), (3, 3, 2), (2, 8, 1)):
        counts = g.integers(0, 6, size=(W, E)).astype(np.int64)
        counts[g.random((W, E)) < 0.3] = 0
        P = E // W
        for d in range(W):
            total = int(counts[:, d * P:(d + 1) * P].sum())
            inp = g.integers(0, 256, size=total * Rb + 3 * Rb, dtype=np.uint8)
            st, out, eoff = o.moe_regroup(W, E, d, Rb, counts, inp, total + 3, total + 1, 0)
            assert st == 0
            assert np.array_equal(out[:total * Rb], _regroup_by_sort(W, E, d, Rb, counts, inp))
            assert not out[total * Rb:].any(), "bytes past the total were written"
            col = counts[:, d * P:(d + 1) * P].sum(axis=0)
            assert np.array_equal(eoff, np.concatenate([[0], np.cumsum(col)]))
            st, back, eoff2 = o.moe_regroup(W, E, d, Rb, counts, out, total, total, 1)
            assert st == 0 and np.array_equal(back, inp[:total * Rb]), "inverse"
            assert np.array_equal(eoff2, eoff)
    counts = np.ones((2, 4), np.int64)
    inp = np.zeros(64, np.uint8)
    assert o.moe_regroup(2, 4, 0, 4, counts, inp, 3, 16, 0)[0] == R.SEND_OVERRUN
    assert o.moe_regroup(2, 4, 0, 4, counts, inp, 16, 3, 0)[0] == R.RECV_OVERFLOW
    neg = counts.copy(); neg[1, 1] = -1
    assert o.moe_regroup(2, 4, 0, 4, neg, inp, 16, 16, 0)[0] == R.BAD_SPLIT
    assert o.moe_regroup(2, 4, 1, 4, neg, inp, 16, 16, 0)[0] == 0  # not an owned column


def pin_moe_dispatch_regroup_closed_form(o):
    """pack -> a2av -> regroup: rank d's rows of expert e are the tokens routed
    to e by rank 0, then rank 1, ..., each in (token, slot) order."""
    g = np.random.default_rng(27)
    W, T, k, E, R_bytes = 4, 30, 3, 12, 6
    toks, idss, sends, counts, S = [], [], [], [], np.zeros((W, W), np.int64)
    for r in range(W):
        tokens, ids = _moe_case(g, T, k, E, R_bytes, distinct=True)
        st, send, perm, splits, cnt = o.moe_pack(T, k, E, W, R_bytes, tokens, ids)
        assert st == 0
        toks.append(tokens); idss.append(ids); sends.append(send.reshape(-1, R_bytes))
        counts.append(cnt); S[r] = splits
    counts = np.stack(counts)
    st, Y, O, _, ro = run_a2av(o, R_bytes, sends, S)
    assert st == 0
    P = E // W
    for d in range(W):
        total = int(ro[d, W])
        st, out, eoff = o.moe_regroup(W, E, d, R_bytes, counts, Y[d], total, total, 0)
        assert st == 0
        out = out.reshape(-1, R_bytes)
        for j in range(P):
            e = d * P + j
            want = [toks[s][t] for s in range(W) for t in range(T) for jj in range(k)
                    if idss[s][t, jj] == e]
            got = out[eoff[j]:eoff[j + 1]]
            assert len(want) == got.shape[0]
            assert np.array_equal(got, np.array(want, np.uint8).reshape(-1, R_bytes))


def pin_moe_dispatch_grouped(o):
    """Dispatch with regroup in one step: equals the a2av (splits = counts
    grouped by owner) followed by the per-rank regroup, two functions pinned
    on their own; the inverse direction brings every pack-order row home; and
    after a real pack each expert's rows are its tokens in (source, token)
    order."""
    g = np.random.default_rng(31)
    for W, E, Rb in ((4, 16, 8), (8, 256, 3), (1, 4, 5), (3, 3, 2), (2, 8, 1)):
        P = E // W
        counts = g.integers(0, 5, size=(W, E)).astype(np.int64)
        counts[g.random((W, E)) < 0.3] = 0
        rows = counts.sum(axis=1)
        ins = [g.integers(0, 256, size=(int(rows[s]) + 2) * Rb, dtype=np.uint8) for s in range(W)]
        in_rows = rows + 2
        exp_tot = np.array([int(counts[:, d * P:(d + 1) * P].sum()) for d in range(W)])
        cap = exp_tot + 1
        st, outs, eoff = o.moe_dispatch_grouped(W, E, Rb, counts, ins, in_rows, cap, 0)
        assert st == 0
        # the composition: a2av with owner-grouped splits, then regroup
        S = np.stack([counts[s].reshape(W, P).sum(axis=1) for s in range(W)]).astype(np.int64)
        st2, Y, _, _, _ = run_a2av(o, Rb, [x.reshape(-1, Rb) for x in ins], S)
        assert st2 == 0
        for d in range(W):
            st3, want, weoff = o.moe_regroup(W, E, d, Rb, counts, Y[d], exp_tot[d], cap[d], 0)
            assert st3 == 0
            assert np.array_equal(outs[d][:exp_tot[d] * Rb], want[:exp_tot[d] * Rb])
            assert not outs[d][exp_tot[d] * Rb:].any()
            assert np.array_equal(eoff[d], weoff)
        # inverse
        st4, back, eoff2 = o.moe_dispatch_grouped(W, E, Rb, counts, outs, cap, in_rows, 1)
        assert st4 == 0 and np.array_equal(eoff2, eoff)
        for s in range(W):
            n = int(rows[s]) * Rb
            assert np.array_equal(back[s][:n], ins[s][:n]) and not back[s][n:].any()
    # after a real pack: expert e's rows are the tokens routed to it, source by source
    W, T, k, E, Rb = 4, 30, 3, 12, 6
    P = E // W
    toks, idss, sends, counts = [], [], [], []
    for r in range(W):
        tokens, ids = _moe_case(g, T, k, E, Rb, distinct=True)
        st, send, perm, splits, cnt = o.moe_pack(T, k, E, W, Rb, tokens, ids)
        assert st == 0
        toks.append(tokens); idss.append(ids); sends.append(send); counts.append(cnt)
    counts = np.stack(counts)
    cap = [int(counts[:, d * P:(d + 1) * P].sum()) for d in range(W)]
    st, outs, eoff = o.moe_dispatch_grouped(W, E, Rb, counts, sends, [T * k] * W, cap, 0)
    assert st == 0
    for d in range(W):
        got_rows = outs[d].reshape(-1, Rb)
        for j in range(P):
            e = d * P + j
            want = [toks[s][t] for s in range(W) for t in range(T) for jj in range(k)
                    if idss[s][t, jj] == e]
            got = got_rows[eoff[d, j]:eoff[d, j + 1]]
            assert np.array_equal(got, np.array(want, np.uint8).reshape(-1, Rb))
    # errors
    c2 = counts.copy(); c2[1, 5] = -1
    st, outs2, e2 = o.moe_dispatch_grouped(W, E, Rb, c2, sends, [T * k] * W, cap, 0)
    assert st == R.BAD_SPLIT and (e2 == -7).all() and not any(x.any() for x in outs2)
    st, outs2, e2 = o.moe_dispatch_grouped(W, E, Rb, counts, sends, [T * k - 1] * W, cap, 0)
    assert st == R.SEND_OVERRUN and not any(x.any() for x in outs2)
    assert np.array_equal(e2, eoff)
    cap2 = list(cap); cap2[2] -= 1
    st, outs2, _ = o.moe_dispatch_grouped(W, E, Rb, counts, sends, [T * k] * W, cap2, 0)
    assert st == R.RECV_OVERFLOW and not any(x.any() for x in outs2)


def pin_moe_combine_grouped(o):
    """Combine read from the expert side: after a real pack and grouped
    dispatch, equals the grouped return followed by the combine (pinned on
    their own); bad ids, perm entries outside their expert's block, and short
    expert sides are refused with nothing written."""
    import torch
    g = np.random.default_rng(32)
    for W, T, k, E, H, distinct in ((4, 30, 3, 12, 8, True), (2, 17, 4, 8, 5, False),
                                    (1, 9, 2, 3, 16, True), (3, 0, 2, 6, 4, False)):
        P = E // W
        ids, perms, sends, counts, ws = [], [], [], [], []
        for r in range(W):
            tok = torch.randn(T, H, generator=torch.Generator().manual_seed(100 + r))
            tok = tok.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint8)
            _, idr = _moe_case(g, T, k, E, 1, distinct)
            st, send, perm, splits, cnt = o.moe_pack(T, k, E, W, 2 * H, tok, idr)
            assert st == 0
            ids.append(idr.reshape(-1)); perms.append(perm); sends.append(send)
            counts.append(cnt)
            ws.append((g.random((T, k)) * 2 - 0.5).astype(np.float32))
        counts = np.stack(counts)
        rows = [int(counts[:, d * P:(d + 1) * P].sum()) for d in range(W)]
        st, exp, _ = o.moe_dispatch_grouped(W, E, 2 * H, counts, sends, [T * k] * W, rows, 0)
        assert st == 0
        exp16 = [x.view(np.uint16).reshape(-1, H) for x in exp]
        st, got = o.moe_combine_grouped(W, T, k, E, H, counts, ids, perms, exp16, ws)
        assert st == 0
        st, back, _ = o.moe_dispatch_grouped(W, E, 2 * H, counts, exp, rows, [T * k] * W, 1)
        assert st == 0
        for r in range(W):
            st, want = o.moe_combine(T, k, H, back[r].view(np.uint16).reshape(-1, H), perms[r], ws[r])
            assert st == 0 and np.array_equal(got[r], want), r
    # failures (the last shape above: W=3, T=0 has no slots; rebuild a small one)
    W, T, k, E, H = 2, 6, 2, 4, 8
    P = E // W
    ids, perms, counts, ws = [], [], [], []
    for r in range(W):
        _, idr = _moe_case(g, T, k, E, 1, True)
        st, send, perm, _, cnt = o.moe_pack(T, k, E, W, 1, np.zeros((T, 1), np.uint8), idr)
        ids.append(idr.reshape(-1)); perms.append(perm); counts.append(cnt)
        ws.append(np.ones((T, k), np.float32))
    counts = np.stack(counts)
    exp16 = [np.ones((int(counts[:, d * P:(d + 1) * P].sum()), H), np.uint16) for d in range(W)]
    assert o.moe_combine_grouped(W, T, k, E, H, counts, ids, perms, exp16, ws)[0] == 0
    bad_ids = [x.copy() for x in ids]; bad_ids[1][3] = E
    st, out = o.moe_combine_grouped(W, T, k, E, H, counts, bad_ids, perms, exp16, ws)
    assert st == R.BAD_EXPERT and not any(x.any() for x in out)
    swapped = [x.copy() for x in ids]  # an id of another expert than the row's block
    q = int(np.nonzero(swapped[0] != swapped[0][0])[0][0])
    swapped[0][0], swapped[0][q] = swapped[0][q], swapped[0][0]
    assert o.moe_combine_grouped(W, T, k, E, H, counts, swapped, perms, exp16, ws)[0] == R.BAD_PERM
    short = [x[:-1] for x in exp16]
    assert o.moe_combine_grouped(W, T, k, E, H, counts, ids, perms, short, ws)[0] == R.SEND_OVERRUN
    c2 = counts.copy(); c2[0, 0] = -2
    assert o.moe_combine_grouped(W, T, k, E, H, c2, ids, perms, exp16, ws)[0] == R.BAD_SPLIT


def _return_a2av_unpack(o, W, T, k, R_bytes, S, perms, recv):
    """The unfused return trip of layout 0: the a2av with the transposed
    splits brings every owner's block home, then the un-pack."""
    Ot = np.ascontiguousarray(S.T)
    back = [np.zeros(T * k * R_bytes, np.uint8) for _ in range(W)]
    st, _, _, _ = o.a2av(R_bytes, recv, Ot.sum(axis=1), back, np.full(W, T * k), Ot)
    assert st == 0
    outs = []
    for s in range(W):
        st, out = o.moe_unpack(T, k, R_bytes, back[s], perms[s])
        assert st == 0
        outs.append(out)
    return outs


def pin_moe_pack_dispatch(o):
    """Pack + dispatch in one step: for both layouts equal to the pack
    followed by the a2av (layout 0) or by the grouped dispatch (layout 1),
    both pinned on their own; its inverse brings every slot its token row
    (closed form) and equals the unfused return trip on arbitrary receive
    contents; bad ids, short receivers, bad counts, perm entries outside
    their block are refused with nothing (or only the metadata) written."""
    g = np.random.default_rng(41)
    for W, T, k, E, Rb, distinct in ((4, 40, 3, 12, 6, True), (2, 17, 4, 8, 5, False),
                                     (1, 9, 2, 3, 16, True), (3, 0, 2, 6, 4, False),
                                     (8, 64, 8, 256, 16, True), (5, 23, 2, 5, 3, False)):
        P = E // W
        toks, ids, sends, perms, splits, counts = [], [], [], [], [], []
        for r in range(W):
            tok, idr = _moe_case(g, T, k, E, Rb, distinct)
            st, send, perm, spl, cnt = o.moe_pack(T, k, E, W, Rb, tok, idr)
            assert st == 0
            toks.append(tok); ids.append(idr.reshape(-1)); sends.append(send)
            perms.append(perm); splits.append(spl); counts.append(cnt)
        S = np.stack(splits).reshape(W, W)
        counts = np.stack(counts).reshape(W, E)
        tot = S.sum(axis=0)
        # layout 0 against pack + a2av
        cap = tot + np.arange(W)          # spare rows stay untouched
        st, recv, perm, S0, c0, boff = o.moe_pack_dispatch(W, T, k, E, Rb, toks, ids, cap, 0)
        assert st == 0
        assert np.array_equal(S0, S) and np.array_equal(c0, counts)
        assert all(np.array_equal(a, b) for a, b in zip(perm, perms))
        want = [np.zeros(int(c) * Rb, np.uint8) for c in cap]
        st, _, _, rro = o.a2av(Rb, sends, np.full(W, T * k), want, cap, S)
        assert st == 0 and np.array_equal(boff, rro)
        assert all(np.array_equal(a, b) for a, b in zip(recv, want))
        st, outs = o.moe_unpack_return(W, T, k, E, Rb, counts, ids, perms,
                                       [x[:int(t) * Rb] for x, t in zip(recv, tot)], 0)
        assert st == 0
        for s in range(W):   # every slot gets its token row back
            assert np.array_equal(outs[s].reshape(T * k, Rb), np.repeat(toks[s], k, axis=0))
        # layout 1 against pack + grouped dispatch
        st, recv1, perm1, S1, c1, boff1 = o.moe_pack_dispatch(W, T, k, E, Rb, toks, ids, cap, 1)
        assert st == 0 and np.array_equal(S1, S) and np.array_equal(c1, counts)
        assert all(np.array_equal(a, b) for a, b in zip(perm1, perms))
        st, want1, eoff = o.moe_dispatch_grouped(W, E, Rb, counts, sends, [T * k] * W, cap, 0)
        assert st == 0 and np.array_equal(boff1, eoff)
        assert all(np.array_equal(a, b) for a, b in zip(recv1, want1))
        st, outs1 = o.moe_unpack_return(W, T, k, E, Rb, counts, ids, perms, recv1, 1)
        assert st == 0
        for s in range(W):
            assert np.array_equal(outs1[s].reshape(T * k, Rb), np.repeat(toks[s], k, axis=0))
        # the inverse on arbitrary receive contents equals the unfused return trips
        junk = [g.integers(0, 256, size=int(t) * Rb, dtype=np.uint8) for t in tot]
        st, got0 = o.moe_unpack_return(W, T, k, E, Rb, counts, ids, perms, junk, 0)
        assert st == 0
        w0 = _return_a2av_unpack(o, W, T, k, Rb, S, perms, junk)
        assert all(np.array_equal(a, b) for a, b in zip(got0, w0))
        st, got1 = o.moe_unpack_return(W, T, k, E, Rb, counts, ids, perms, junk, 1)
        assert st == 0
        st, back, _ = o.moe_dispatch_grouped(W, E, Rb, counts, junk, tot, [T * k] * W, 1)
        assert st == 0
        for s in range(W):
            st, w1 = o.moe_unpack(T, k, Rb, back[s], perms[s])
            assert st == 0 and np.array_equal(got1[s], w1), s
    # failures
    W, T, k, E, Rb = 2, 6, 2, 4, 4
    toks, ids = [], []
    for r in range(W):
        tok, idr = _moe_case(g, T, k, E, Rb, True)
        toks.append(tok); ids.append(idr.reshape(-1))
    st, recv, perm, S, counts, boff = o.moe_pack_dispatch(W, T, k, E, Rb, toks, ids, [99] * W, 0)
    assert st == 0
    tot = S.sum(axis=0)
    bad = [x.copy() for x in ids]; bad[1][5] = -1
    for layout in (0, 1):
        st, rv, pm, S2, c2, b2 = o.moe_pack_dispatch(W, T, k, E, Rb, toks, bad, [99] * W, layout)
        assert st == R.BAD_EXPERT and not any(x.any() for x in rv)
        assert all((x == -7).all() for x in pm) and (S2 == -7).all() and (c2 == -7).all()
        short = tot.copy(); short[1] -= 1
        st, rv, pm, S2, c2, b2 = o.moe_pack_dispatch(W, T, k, E, Rb, toks, ids, short, layout)
        assert st == R.RECV_OVERFLOW and not any(x.any() for x in rv)
        assert np.array_equal(S2, S) and np.array_equal(c2, counts)
        assert all(np.array_equal(a, b) for a, b in zip(pm, perm))
        assert b2[1, -1] == tot[1]
        full = [x[:int(t) * Rb] for x, t in zip(recv, tot)]
        st, out = o.moe_unpack_return(W, T, k, E, Rb, counts, bad, perm, full, layout)
        assert st == R.BAD_EXPERT and not any(x.any() for x in out)
        swapped = [x.copy() for x in ids]
        q = int(np.nonzero(swapped[0] != swapped[0][0])[0][0])
        swapped[0][0], swapped[0][q] = swapped[0][q], swapped[0][0]
        st, out = o.moe_unpack_return(W, T, k, E, Rb, counts, swapped, perm, full, layout)
        assert st == R.BAD_PERM and not any(x.any() for x in out)
        st, out = o.moe_unpack_return(W, T, k, E, Rb, counts, ids, perm,
                                      [x[:-Rb] for x in full], layout)
        assert st == R.SEND_OVERRUN and not any(x.any() for x in out)
        c3 = counts.copy(); c3[1, 2] = -1
        st, out = o.moe_unpack_return(W, T, k, E, Rb, c3, ids, perm, full, layout)
        assert st == R.BAD_SPLIT and not any(x.any() for x in out)


def pin_moe_combine_return(o):
    """Combine read at the owners, both layouts: for layout 1 equal to the
    combine from the expert side (written directly, pinned on its own); for
    layout 0 equal to the return a2av with the transposed splits followed by
    the combine over the pack's perm; after the one-step dispatch of real
    tokens, equal to combining the tokens themselves; failures as the
    inverse's."""
    import torch
    g = np.random.default_rng(52)
    for W, T, k, E, H, distinct in ((4, 30, 3, 12, 8, True), (2, 17, 4, 8, 5, False),
                                    (1, 9, 2, 3, 16, True), (3, 0, 2, 6, 4, False)):
        toks, ids = [], []
        for r in range(W):
            tok = torch.randn(T, H, generator=torch.Generator().manual_seed(300 + r))
            toks.append(tok.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
            ids.append(_moe_case(g, T, k, E, 1, distinct)[1].reshape(-1))
        ws = [(g.random((T, k)) * 2 - 0.5).astype(np.float32) for _ in range(W)]
        st, _, perms, S, counts, _ = o.moe_pack_dispatch(W, T, k, E, 2 * H,
                                                         [t.view(np.uint8) for t in toks], ids,
                                                         [10 ** 6] * W, 0)
        assert st == 0
        tot = S.sum(axis=0)
        junk = [g.integers(0, 1 << 16, size=(int(t), H), dtype=np.uint16) for t in tot]
        junk = [np.where((x & 0x7F80) == 0x7F80, x & 0xBFFF, x).astype(np.uint16) for x in junk]
        # layout 1 against the direct combine from the expert side
        st, got = o.moe_combine_return(W, T, k, E, H, counts, ids, perms, junk, ws, 1)
        st2, want = o.moe_combine_grouped(W, T, k, E, H, counts, ids, perms, junk, ws)
        assert st == st2 == 0 and all(np.array_equal(a, b) for a, b in zip(got, want))
        # layout 0 against the return a2av and the combine over perm
        st, got = o.moe_combine_return(W, T, k, E, H, counts, ids, perms, junk, ws, 0)
        assert st == 0
        back = _return_a2av_unpack_back(o, W, T, k, 2 * H, S, junk)
        for s in range(W):
            st, want = o.moe_combine(T, k, H, back[s].view(np.uint16).reshape(-1, H), perms[s],
                                     ws[s])
            assert st == 0 and np.array_equal(got[s], want), s
        # after the one-step dispatch of the tokens: the tokens' own combine
        for layout in (0, 1):
            st, recv, _, _, _, _ = o.moe_pack_dispatch(W, T, k, E, 2 * H,
                                                       [t.view(np.uint8) for t in toks], ids,
                                                       tot, layout)
            assert st == 0
            st, got = o.moe_combine_return(W, T, k, E, H, counts, ids, perms,
                                           [x.view(np.uint16).reshape(-1, H) for x in recv], ws,
                                           layout)
            assert st == 0
            for s in range(W):
                rep = np.ascontiguousarray(np.repeat(toks[s], k, axis=0))
                st, want = o.moe_combine(T, k, H, rep, np.arange(T * k, dtype=np.int64), ws[s])
                assert st == 0 and np.array_equal(got[s], want), (layout, s)
    # failures: the inverse's
    W, T, k, E, H = 2, 6, 2, 4, 8
    ids = [_moe_case(g, T, k, E, 1, True)[1].reshape(-1) for _ in range(W)]
    toks = [np.zeros((T, 2 * H), np.uint8) for _ in range(W)]
    st, _, perms, S, counts, _ = o.moe_pack_dispatch(W, T, k, E, 2 * H, toks, ids, [99] * W, 0)
    ws = [np.ones((T, k), np.float32)] * W
    full = [np.ones((int(t), H), np.uint16) for t in S.sum(axis=0)]
    for layout in (0, 1):
        assert o.moe_combine_return(W, T, k, E, H, counts, ids, perms, full, ws, layout)[0] == 0
        bad = [x.copy() for x in ids]; bad[0][1] = E
        st, out = o.moe_combine_return(W, T, k, E, H, counts, bad, perms, full, ws, layout)
        assert st == R.BAD_EXPERT and not any(x.any() for x in out)
        st, out = o.moe_combine_return(W, T, k, E, H, counts, ids, perms,
                                       [x[:-1] for x in full], ws, layout)
        assert st == R.SEND_OVERRUN and not any(x.any() for x in out)
        c2 = counts.copy(); c2[1, 1] = -4
        assert o.moe_combine_return(W, T, k, E, H, c2, ids, perms, full, ws, layout)[0] == R.BAD_SPLIT


def _return_a2av_unpack_back(o, W, T, k, R_bytes, S, recv):
    """The return a2av of layout 0 alone: every owner's blocks back at their
    sources, in pack order."""
    Ot = np.ascontiguousarray(S.T)
    back = [np.zeros(T * k * R_bytes, np.uint8) for _ in range(W)]
    st, _, _, _ = o.a2av(R_bytes, [np.ascontiguousarray(x).view(np.uint8).reshape(-1) for x in recv],
                         Ot.sum(axis=1), back, np.full(W, T * k), Ot)
    assert st == 0
    return back


# ------------------------------------------------------------------ gate-weighted combine
def _round_f32(x):
    """A Fraction rounded to the nearest binary32, ties to even (finite, in
    range): the rounding step of an IEEE fused multiply-add, from its
    definition."""
    from fractions import Fraction
    import math
    if x == 0:
        return 0.0
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)                      # subnormals share the smallest exponent
    q = a / Fraction(2) ** (e - 23)       # 24 significant bits
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * float(Fraction(n) * Fraction(2) ** (e - 23))


def _bf16_bits_to_f32(b):
    return (np.asarray(b, np.uint32) << 16).view(np.float32)


def pin_moe_combine_is_exact_fma_chain(o):
    """Each output element against the fma chain evaluated in exact rational
    arithmetic with a round-to-nearest-even after every step, then rounded to
    bfloat16 by torch (its own float32 -> bfloat16 conversion)."""
    import torch
    from fractions import Fraction
    g = np.random.default_rng(28)
    for T, k, H in ((5, 3, 7), (3, 8, 4), (2, 1, 9)):
        back = torch.randn(T * k, H).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        perm = g.permutation(T * k).astype(np.int64)
        w = g.random((T, k)).astype(np.float32) * 2 - 0.5
        st, out = o.moe_combine(T, k, H, back, perm, w)
        assert st == 0
        xf = _bf16_bits_to_f32(back)
        want = np.zeros((T, H), np.float32)
        for t in range(T):
            for h in range(H):
                acc = 0.0
                for j in range(k):
                    acc = _round_f32(Fraction(float(w[t, j])) * Fraction(float(xf[perm[t * k + j], h]))
                                     + Fraction(acc))
                want[t, h] = acc
        wb = torch.from_numpy(want).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(out, wb)


def pin_moe_combine_special_cases(o):
    g = np.random.default_rng(29)
    T, k, H = 6, 4, 16
    back = g.integers(0, 0x7F80, size=(T * k, H)).astype(np.uint16)  # finite, >= +0
    perm = g.permutation(T * k).astype(np.int64)
    # one-hot weights copy the chosen row exactly
    w = np.zeros((T, k), np.float32)
    pick = g.integers(0, k, size=T)
    w[np.arange(T), pick] = 1.0
    st, out = o.moe_combine(T, k, H, back, perm, w)
    assert st == 0
    for t in range(T):
        assert np.array_equal(out[t], back[perm[t * k + pick[t]]])
    # infinities and NaN propagate; every NaN comes out as the one quiet NaN
    # 0x7FC0, whatever its sign and payload were
    b2 = back.copy()
    b2[perm[0]] = 0x7F80          # +inf in slot 0 of token 0
    b2[perm[k]] = 0x7FA0          # a signalling NaN in slot 0 of token 1
    w2 = np.full((T, k), 0.25, np.float32)
    st, out = o.moe_combine(T, k, H, b2, perm, w2)
    assert st == 0
    assert np.all(out[0] == 0x7F80)
    assert np.all(out[1] == 0x7FC0)
    b2[perm[k]] = 0xFFC1          # a negative quiet NaN with a payload
    b2[perm[2 * k]] = 0x7F80      # +inf - inf in token 2 makes a new NaN
    b2[perm[2 * k + 1]] = 0xFF80
    st, out = o.moe_combine(T, k, H, b2, perm, w2)
    assert st == 0 and np.all(out[1] == 0x7FC0) and np.all(out[2] == 0x7FC0)
    # zero weights over finite rows give +0 exactly
    st, out = o.moe_combine(T, k, H, back, perm, np.zeros((T, k), np.float32))
    assert st == 0 and not out.any()
    # the order of the chain matters: 2^30 - 2^30 + 1 is 1 in slot order, while
    # 1 - 2^30 rounds to -2^30 in float32, so the reverse order gives 0
    ident = np.arange(3, dtype=np.int64)
    b3 = np.array([[0x4E80], [0xCE80], [0x3F80]], np.uint16)   # 2^30, -2^30, 1
    st, out = o.moe_combine(1, 3, 1, b3, ident, np.ones((1, 3), np.float32))
    assert st == 0 and out[0, 0] == 0x3F80
    # each step is one fused multiply-add: (1 + 2^-23)(1 + 2^-7) carries a 2^-30
    # term that a rounded product would lose before it cancels against slot 0
    b4 = np.array([[0x3F81], [0x3F81]], np.uint16)             # 1 + 2^-7, twice
    w4 = np.array([[-(1 + 2.0 ** -23), 1 + 2.0 ** -23]], np.float32)
    st, out = o.moe_combine(1, 2, 1, b4, ident[:2].copy(), w4)
    assert st == 0 and out[0, 0] == 0x3080                     # 2^-30
    # bad permutation entry
    p2 = perm.copy(); p2[3] = T * k
    assert o.moe_combine(T, k, H, back, p2, w)[0] == R.BAD_PERM


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
