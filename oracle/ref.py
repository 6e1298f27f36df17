"""ctypes wrapper of the CPU oracle (``liba2av_ref.so``), over numpy arrays.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg call this module; the product path never does. It loads only
the oracle's own shared library, built from ``a2av_ref.c`` by :func:`build`.

Payload buffers are numpy ``uint8`` arrays (byte views of whatever dtype the
rows hold); splits, offsets and permutations are ``int64`` arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "a2av_ref.c")
LIB = os.path.join(HERE, "liba2av_ref.so")

BAD_SPLIT = 1
SEND_OVERRUN = 2
RECV_OVERFLOW = 4
BAD_EXPERT = 8
BAD_OFFSETS = 16
BAD_PERM = 32
EARG = -1
MAX_SPLIT = 1 << 40

_lib = None


def build(out: str = LIB, extra_flags: tuple = ()) -> str:
    """Compile the oracle with gcc into a shared library and return its path."""
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-Werror", "-fPIC", "-shared",
           "-ffp-contract=off", *extra_flags, "-o", out, SRC, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def _bind(lib):
    i64p = ctypes.POINTER(ctypes.c_int64)
    i32p = ctypes.POINTER(ctypes.c_int32)
    vpp = ctypes.POINTER(ctypes.c_void_p)
    sz = ctypes.c_size_t
    lib.ref_exchange_splits.argtypes = [ctypes.c_int, i64p, i64p]
    lib.ref_offsets.argtypes = [ctypes.c_int, i64p, i64p, i64p, i64p]
    lib.ref_copy.argtypes = [ctypes.c_int, sz, vpp, i64p, vpp, i64p, i64p, i64p, i64p]
    lib.ref_a2av.argtypes = [ctypes.c_int, sz, vpp, i64p, vpp, i64p, i64p, i64p, i64p, i64p]
    lib.ref_source_of.argtypes = [ctypes.c_int, i64p, ctypes.c_int, ctypes.c_int64,
                                  ctypes.POINTER(ctypes.c_int), i64p]
    lib.ref_moe_pack.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int, sz,
                                 ctypes.c_void_p, i32p, ctypes.c_void_p, i64p, i64p, i64p]
    lib.ref_moe_unpack.argtypes = [ctypes.c_int64, ctypes.c_int, sz, ctypes.c_void_p, i64p,
                                   ctypes.c_void_p]
    lib.ref_moe_regroup.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, sz, i64p,
                                    ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                    ctypes.c_int64, i64p, ctypes.c_int]
    lib.ref_moe_combine.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p,
                                    i64p, ctypes.c_void_p, ctypes.c_void_p]
    lib.ref_keys_bucketize.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int64, i32p,
                                       ctypes.c_void_p, ctypes.c_int64, i32p, ctypes.c_void_p,
                                       i64p, i64p]
    lib.ref_moe_dispatch_grouped.argtypes = [ctypes.c_int, ctypes.c_int, sz, i64p, vpp, i64p, vpp,
                                             i64p, i64p, ctypes.c_int]
    lib.ref_moe_combine_grouped.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_int64, i64p, vpp, vpp, vpp,
                                            i64p, vpp, vpp]
    lib.ref_moe_pack_dispatch.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                          sz, vpp, vpp, vpp, i64p, vpp, i64p, i64p, i64p,
                                          ctypes.c_int]
    lib.ref_moe_unpack_return.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                          sz, i64p, vpp, vpp, vpp, i64p, vpp, ctypes.c_int]
    lib.ref_moe_combine_return.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_int64, i64p, vpp, vpp, vpp, i64p,
                                           vpp, vpp, ctypes.c_int]
    lib.ref_keys_exchange.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int64, vpp, vpp, i64p,
                                      vpp, i64p, vpp, i64p, i64p, i64p, i64p]
    for name in ("ref_exchange_splits", "ref_offsets", "ref_copy", "ref_a2av", "ref_source_of",
                 "ref_moe_pack", "ref_moe_unpack", "ref_moe_regroup", "ref_moe_combine",
                 "ref_keys_bucketize", "ref_keys_exchange", "ref_moe_dispatch_grouped",
                 "ref_moe_combine_grouped", "ref_moe_pack_dispatch", "ref_moe_unpack_return",
                 "ref_moe_combine_return"):
        getattr(lib, name).restype = ctypes.c_int
    return lib


def load(path: str | None = None):
    """Load the oracle library (building it first if it is missing)."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        _lib = _bind(ctypes.CDLL(LIB))
    return _lib


def _i64(a):
    assert a.dtype == np.int64 and a.flags.c_contiguous
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


def _ptrs(bufs):
    arr = (ctypes.c_void_p * len(bufs))()
    for i, b in enumerate(bufs):
        if b is None:
            arr[i] = None
        else:
            assert b.flags.c_contiguous
            arr[i] = b.ctypes.data
    return arr


class Oracle:
    """Thin numpy front end of one loaded oracle library."""

    def __init__(self, lib=None):
        self.lib = lib if lib is not None else load()

    def exchange_splits(self, S):
        S = np.ascontiguousarray(S, dtype=np.int64)
        W = S.shape[0]
        O = np.zeros((W, W), dtype=np.int64)
        st = self.lib.ref_exchange_splits(W, _i64(S), _i64(O))
        return st, O

    def offsets(self, S, O):
        S = np.ascontiguousarray(S, dtype=np.int64)
        O = np.ascontiguousarray(O, dtype=np.int64)
        W = S.shape[0]
        send_off = np.zeros((W, W + 1), dtype=np.int64)
        recv_off = np.zeros((W, W + 1), dtype=np.int64)
        st = self.lib.ref_offsets(W, _i64(S), _i64(O), _i64(send_off), _i64(recv_off))
        return st, send_off, recv_off

    def copy(self, R, ins, in_rows, outs, out_cap, S, send_off, recv_off):
        """Payload step into ``outs`` (modified in place); returns the status."""
        W = len(ins)
        in_rows = np.ascontiguousarray(in_rows, dtype=np.int64)
        out_cap = np.ascontiguousarray(out_cap, dtype=np.int64)
        S = np.ascontiguousarray(S, dtype=np.int64)
        send_off = np.ascontiguousarray(send_off, dtype=np.int64)
        recv_off = np.ascontiguousarray(recv_off, dtype=np.int64)
        return self.lib.ref_copy(W, R, _ptrs(ins), _i64(in_rows), _ptrs(outs), _i64(out_cap),
                                 _i64(S), _i64(send_off), _i64(recv_off))

    def a2av(self, R, ins, in_rows, outs, out_cap, S):
        """Whole definition from S alone; payload lands in ``outs`` in place."""
        W = len(ins)
        in_rows = np.ascontiguousarray(in_rows, dtype=np.int64)
        out_cap = np.ascontiguousarray(out_cap, dtype=np.int64)
        S = np.ascontiguousarray(S, dtype=np.int64)
        O = np.zeros((W, W), dtype=np.int64)
        send_off = np.zeros((W, W + 1), dtype=np.int64)
        recv_off = np.zeros((W, W + 1), dtype=np.int64)
        st = self.lib.ref_a2av(W, R, _ptrs(ins), _i64(in_rows), _ptrs(outs), _i64(out_cap),
                               _i64(S), _i64(O), _i64(send_off), _i64(recv_off))
        return st, O, send_off, recv_off

    def source_of(self, S, d, j):
        S = np.ascontiguousarray(S, dtype=np.int64)
        s = ctypes.c_int(-1)
        i = ctypes.c_int64(-1)
        st = self.lib.ref_source_of(S.shape[0], _i64(S), d, j, ctypes.byref(s), ctypes.byref(i))
        if st == 1:
            return None
        if st != 0:
            raise ValueError(f"ref_source_of failed with {st}")
        return s.value, i.value

    def moe_pack(self, T, k, E, W, R, tokens, ids):
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        tokens = np.ascontiguousarray(tokens).view(np.uint8)
        send = np.zeros(T * k * R, dtype=np.uint8)
        perm = np.zeros(T * k, dtype=np.int64)
        splits = np.zeros(W, dtype=np.int64)
        counts = np.zeros(E, dtype=np.int64)
        st = self.lib.ref_moe_pack(T, k, E, W, R, tokens.ctypes.data,
                                   ids.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                   send.ctypes.data, _i64(perm), _i64(splits), _i64(counts))
        return st, send, perm, splits, counts

    def moe_unpack(self, T, k, R, back, perm):
        back = np.ascontiguousarray(back).view(np.uint8)
        perm = np.ascontiguousarray(perm, dtype=np.int64)
        out = np.zeros(T * k * R, dtype=np.uint8)
        st = self.lib.ref_moe_unpack(T, k, R, back.ctypes.data, _i64(perm), out.ctypes.data)
        return st, out

    def moe_regroup(self, W, E, d, R, counts, inp, in_rows, out_cap, direction=0):
        """Returns (status, out bytes [out_cap * R], expert_offsets [E/W + 1])."""
        counts = np.ascontiguousarray(counts, dtype=np.int64)
        inp = np.ascontiguousarray(inp).view(np.uint8).reshape(-1)
        out = np.zeros(max(int(out_cap), 0) * R, dtype=np.uint8)
        eoff = np.zeros(E // W + 1, dtype=np.int64)
        st = self.lib.ref_moe_regroup(W, E, d, R, _i64(counts), inp.ctypes.data, int(in_rows),
                                      out.ctypes.data, int(out_cap), _i64(eoff), direction)
        return st, out, eoff

    def moe_combine(self, T, k, H, back, perm, w):
        """back: uint16 [T*k, H] (bf16 bits), w: float32 [T, k]; returns uint16 [T, H]."""
        back = np.ascontiguousarray(back, dtype=np.uint16)
        perm = np.ascontiguousarray(perm, dtype=np.int64)
        w = np.ascontiguousarray(w, dtype=np.float32)
        out = np.zeros((T, H), dtype=np.uint16)
        st = self.lib.ref_moe_combine(T, k, H, back.ctypes.data, _i64(perm), w.ctypes.data,
                                      out.ctypes.data)
        return st, out

    def keys_bucketize(self, W, n_tables, batch, lengths, keys):
        """Returns (status, lengths_out, keys_out, split_keys, split_lengths)."""
        lengths = np.ascontiguousarray(lengths, dtype=np.int32).reshape(-1)
        keys = np.ascontiguousarray(keys, dtype=np.int64)
        lo = np.zeros(n_tables * batch, dtype=np.int32)
        ko = np.zeros(keys.size, dtype=np.int64)
        sk = np.zeros(W, dtype=np.int64)
        sl = np.zeros(W, dtype=np.int64)
        st = self.lib.ref_keys_bucketize(W, n_tables, batch,
                                         lengths.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                         keys.ctypes.data, keys.size,
                                         lo.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                         ko.ctypes.data, _i64(sk), _i64(sl))
        return st, lo, ko, sk, sl

    def keys_exchange(self, W, n_tables, batch, lengths, keys, lengths_cap=None, keys_cap=None):
        """All W ranks at once. lengths: per-rank int32 [n_tables, batch]; keys:
        per-rank int64. Capacities default to what each receiver gets. Returns
        (status, [lengths_out], [keys_out], split_keys, split_lengths,
        recv_off_keys); outputs start as zeros (-7 for the matrices)."""
        lengths = [np.ascontiguousarray(l, dtype=np.int32).reshape(-1) for l in lengths]
        keys = [np.ascontiguousarray(k, dtype=np.int64) for k in keys]
        n_keys = np.array([k.size for k in keys], dtype=np.int64)
        if lengths_cap is None or keys_cap is None:
            owned = [len(range(d, n_tables, W)) for d in range(W)]
            lcap = np.array([W * owned[d] * batch for d in range(W)], dtype=np.int64)
            kcap = np.zeros(W, dtype=np.int64)
            for s in range(W):
                tk = lengths[s].reshape(n_tables, batch).sum(axis=1) if n_tables else np.zeros(0)
                for t in range(n_tables):
                    kcap[t % W] += int(tk[t])
            lengths_cap = lcap if lengths_cap is None else lengths_cap
            keys_cap = kcap if keys_cap is None else keys_cap
        lengths_cap = np.ascontiguousarray(lengths_cap, dtype=np.int64)
        keys_cap = np.ascontiguousarray(keys_cap, dtype=np.int64)
        lo = [np.zeros(max(int(c), 0), dtype=np.int32) for c in lengths_cap]
        ko = [np.zeros(max(int(c), 0), dtype=np.int64) for c in keys_cap]
        sk = np.full((W, W), -7, dtype=np.int64)
        sl = np.full((W, W), -7, dtype=np.int64)
        ro = np.full((W, W + 1), -7, dtype=np.int64)
        st = self.lib.ref_keys_exchange(W, n_tables, batch, _ptrs(lengths), _ptrs(keys),
                                        _i64(n_keys), _ptrs(lo), _i64(lengths_cap), _ptrs(ko),
                                        _i64(keys_cap), _i64(sk), _i64(sl), _i64(ro))
        return st, lo, ko, sk, sl, ro

    def moe_dispatch_grouped(self, W, E, R, counts, ins, in_rows, out_cap, direction=0):
        """All W ranks. ins: per-rank uint8 arrays; returns (status, [out bytes,
        out_cap[r] * R each, zero-filled], expert_offsets [W, E/W + 1] (-7 where
        not written))."""
        counts = np.ascontiguousarray(counts, dtype=np.int64)
        ins = [np.ascontiguousarray(x).view(np.uint8).reshape(-1) for x in ins]
        in_rows = np.ascontiguousarray(in_rows, dtype=np.int64)
        out_cap = np.ascontiguousarray(out_cap, dtype=np.int64)
        outs = [np.zeros(max(int(c), 0) * R, dtype=np.uint8) for c in out_cap]
        eoff = np.full((W, E // W + 1), -7, dtype=np.int64)
        st = self.lib.ref_moe_dispatch_grouped(W, E, R, _i64(counts), _ptrs(ins), _i64(in_rows),
                                               _ptrs(outs), _i64(out_cap), _i64(eoff), direction)
        return st, outs, eoff

    def moe_pack_dispatch(self, W, T, k, E, R, tokens, ids, recv_cap, layout=0):
        """All W ranks. tokens: per-rank [T, R] bytes (any dtype); ids: per-rank
        int32 [T*k]. Returns (status, [recv bytes, recv_cap[d] * R each,
        zero-filled where not written], perm [W][T*k], S [W][W], counts [W][E],
        block offsets [W][G+1]); the integer outputs start at -7."""
        toks = [np.ascontiguousarray(x).view(np.uint8).reshape(-1) for x in tokens]
        ids = [np.ascontiguousarray(i, dtype=np.int32).reshape(-1) for i in ids]
        recv_cap = np.ascontiguousarray(recv_cap, dtype=np.int64)
        recv = [np.zeros(max(int(c), 0) * R, dtype=np.uint8) for c in recv_cap]
        perm = [np.full(T * k, -7, dtype=np.int64) for _ in range(W)]
        S = np.full((W, W), -7, dtype=np.int64)
        counts = np.full((W, E), -7, dtype=np.int64)
        G = W if layout == 0 else E // W
        boff = np.full((W, G + 1), -7, dtype=np.int64)
        st = self.lib.ref_moe_pack_dispatch(W, T, k, E, R, _ptrs(toks), _ptrs(ids), _ptrs(recv),
                                            _i64(recv_cap), _ptrs(perm), _i64(S), _i64(counts),
                                            _i64(boff), layout)
        return st, recv, perm, S, counts, boff

    def moe_unpack_return(self, W, T, k, E, R, counts, ids, perms, recv, layout=0):
        """All W ranks. recv: per-owner receive bytes (rows = size // R).
        Returns (status, [out bytes [T*k*R], zero-filled where not written])."""
        counts = np.ascontiguousarray(counts, dtype=np.int64)
        ids = [np.ascontiguousarray(i, dtype=np.int32).reshape(-1) for i in ids]
        perms = [np.ascontiguousarray(p, dtype=np.int64).reshape(-1) for p in perms]
        rv = [np.ascontiguousarray(x).view(np.uint8).reshape(-1) for x in recv]
        rows = np.array([x.size // R for x in rv], dtype=np.int64)
        outs = [np.zeros(T * k * R, dtype=np.uint8) for _ in range(W)]
        st = self.lib.ref_moe_unpack_return(W, T, k, E, R, _i64(counts), _ptrs(ids), _ptrs(perms),
                                            _ptrs(rv), _i64(rows), _ptrs(outs), layout)
        return st, outs

    def moe_combine_return(self, W, T, k, E, H, counts, ids, perms, recv, weights, layout=0):
        """All W ranks. recv: per-owner uint16 [rows, H] in the layout's order;
        weights: float32 [T, k]. Returns (status, [out uint16 [T, H]],
        zero-filled where not written)."""
        counts = np.ascontiguousarray(counts, dtype=np.int64)
        ids = [np.ascontiguousarray(i, dtype=np.int32).reshape(-1) for i in ids]
        perms = [np.ascontiguousarray(p, dtype=np.int64).reshape(-1) for p in perms]
        xs = [np.ascontiguousarray(x, dtype=np.uint16).reshape(-1) for x in recv]
        rows = np.array([x.size // H for x in xs], dtype=np.int64)
        ws = [np.ascontiguousarray(x, dtype=np.float32).reshape(-1) for x in weights]
        outs = [np.zeros((T, H), dtype=np.uint16) for _ in range(W)]
        st = self.lib.ref_moe_combine_return(W, T, k, E, H, _i64(counts), _ptrs(ids), _ptrs(perms),
                                             _ptrs(xs), _i64(rows), _ptrs(ws), _ptrs(outs), layout)
        return st, outs

    def moe_combine_grouped(self, W, T, k, E, H, counts, ids, perms, expert_side, weights):
        """All W ranks. ids: per-rank int32 [T*k]; perms: int64 [T*k]; expert_side:
        per-owner uint16 [rows, H]; weights: float32 [T, k]. Returns (status,
        [out uint16 [T, H]] zero-filled where not written)."""
        counts = np.ascontiguousarray(counts, dtype=np.int64)
        ids = [np.ascontiguousarray(i, dtype=np.int32).reshape(-1) for i in ids]
        perms = [np.ascontiguousarray(p, dtype=np.int64).reshape(-1) for p in perms]
        xs = [np.ascontiguousarray(x, dtype=np.uint16).reshape(-1) for x in expert_side]
        rows = np.array([x.size // H for x in xs], dtype=np.int64)
        ws = [np.ascontiguousarray(x, dtype=np.float32).reshape(-1) for x in weights]
        outs = [np.zeros((T, H), dtype=np.uint16) for _ in range(W)]
        st = self.lib.ref_moe_combine_grouped(W, T, k, E, H, _i64(counts), _ptrs(ids), _ptrs(perms),
                                              _ptrs(xs), _i64(rows), _ptrs(ws), _ptrs(outs))
        return st, outs
