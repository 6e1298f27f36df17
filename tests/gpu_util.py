"""Helpers for the GPU parity tests: run the HIP path through the C ABI on
seeded host inputs and run the oracle on the very same bytes."""
from __future__ import annotations

import numpy as np
import torch

from embeddings_a2av_virtual_amd import _binding as B
from embeddings_a2av_virtual_amd.vranks import A2av

SENT = 0xA5
GUARD = 4096


def dev():
    return torch.device("cuda")


class GuardedBuffer:
    """A device byte range with guard bands on both sides, pre-filled."""

    def __init__(self, nbytes, pad=0, fill=SENT):
        self.nbytes = int(nbytes)
        self.pad = int(pad)
        self.fill = fill
        self.raw = torch.full((GUARD + self.pad + self.nbytes + GUARD,), fill, dtype=torch.uint8,
                              device=dev())
        self.view = self.raw[GUARD + self.pad: GUARD + self.pad + self.nbytes]

    def guards_intact(self):
        lo = self.raw[:GUARD + self.pad]
        hi = self.raw[GUARD + self.pad + self.nbytes:]
        return bool((lo == self.fill).all().item()) and bool((hi == self.fill).all().item())

    def host(self):
        return self.view.cpu().numpy()


def upload_rows(x: np.ndarray, pad=0) -> GuardedBuffer:
    b = GuardedBuffer(x.size, pad=pad, fill=0x5A)
    if x.size:
        b.view.copy_(torch.from_numpy(np.ascontiguousarray(x).reshape(-1)))
    return b


def gpu_a2av(R, X, S, cap=None, in_pad=0, out_pad=0, state=None, status_init=0, fused=False):
    """Run exchange -> offsets -> copy on the GPU (three calls, or the single
    fused call). X: list of host uint8 [n, R] arrays. Returns (status, O,
    send_off, recv_off, [Y_d host uint8 [cap_d, R]], guards_ok)."""
    W = len(X)
    S = np.asarray(S, dtype=np.int64)
    if cap is None:
        cap = np.maximum(S.sum(axis=0), 0)
    ins = [upload_rows(x, pad=in_pad) for x in X]
    outs = [GuardedBuffer(int(c) * R, pad=out_pad) for c in cap]
    st = state if state is not None else A2av(W)
    st.set_splits(S)
    st.status.fill_(status_init)
    st(R, [b.view for b in ins], [x.shape[0] for x in X], [b.view for b in outs],
       [int(c) for c in cap], fused=fused)
    torch.cuda.synchronize()
    Y = [b.host().reshape(-1, R) if R else b.host() for b in outs]
    guards = all(b.guards_intact() for b in outs) and all(b.guards_intact() for b in ins)
    return (int(st.status.item()), st.O.cpu().numpy(), st.send_off.cpu().numpy(),
            st.recv_off.cpu().numpy(), Y, guards)


def ref_a2av(ref, R, X, S, cap=None):
    """The oracle on the same inputs, outputs pre-filled with the sentinel."""
    W = len(X)
    S = np.asarray(S, dtype=np.int64)
    if cap is None:
        cap = np.maximum(S.sum(axis=0), 0)
    Y = [np.full((int(c), R), SENT, dtype=np.uint8) for c in cap]
    in_rows = np.array([x.shape[0] for x in X], dtype=np.int64)
    st, O, so, ro = ref.a2av(R, [x.reshape(-1) for x in X], in_rows, [y.reshape(-1) for y in Y],
                             np.asarray(cap, dtype=np.int64), S)
    return st, O, so, ro, Y


def assert_same(gpu, want, what=""):
    st, O, so, ro, Y, guards = gpu
    rst, rO, rso, rro, rY = want
    assert guards, f"{what}: a guard band was written"
    assert st == rst, f"{what}: status {st} != oracle {rst}"
    # the oracle leaves matrices it does not reach at zero, as a fresh device state
    assert np.array_equal(O, rO), f"{what}: output splits"
    assert np.array_equal(so, rso), f"{what}: send offsets"
    assert np.array_equal(ro, rro), f"{what}: recv offsets"
    for d, (y, ry) in enumerate(zip(Y, rY)):
        if not np.array_equal(y, ry):
            bad = np.argwhere(y != ry)
            raise AssertionError(f"{what}: rank {d} differs at {len(bad)} bytes, first {bad[0]}")


def random_rows(g, n, R):
    return g.integers(0, 256, size=(int(n), R), dtype=np.uint8)
