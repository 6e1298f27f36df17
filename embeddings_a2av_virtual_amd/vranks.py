"""W virtual ranks in one GPU's HBM: the device state of one a2av sequence.

Rank r is row r of the split matrices plus the device buffers (in[r], out[r])
the caller passes. :class:`A2av` owns the small device matrices (splits,
transposed splits, offsets, status word) and enqueues the three library calls
in stream order: splits exchange -> offsets -> payload copy. It allocates
only at construction, so repeated calls allocate nothing.
"""
from __future__ import annotations

import torch

from . import _binding as B


class A2av:
    def __init__(self, W: int, device="cuda"):
        if not 1 <= W <= B.MAX_W:
            raise ValueError(f"W must be in [1, {B.MAX_W}]")
        self.W = W
        self.device = torch.device(device)
        z = dict(dtype=torch.int64, device=self.device)
        self.S = torch.zeros((W, W), **z)
        self.O = torch.zeros((W, W), **z)
        self.send_off = torch.zeros((W, W + 1), **z)
        self.recv_off = torch.zeros((W, W + 1), **z)
        self.status = torch.zeros(1, dtype=torch.int32, device=self.device)

    def set_splits(self, S_host):
        """Upload a W x W split matrix (row s = rank s's split vector)."""
        self.S.copy_(torch.as_tensor(S_host, dtype=torch.int64).reshape(self.W, self.W))

    def reset_status(self):
        self.status.zero_()

    def exchange_and_offsets(self, stream=None):
        B.a2av_exchange_splits(self.S, self.O, self.status, stream)
        B.a2av_offsets(self.S, self.O, self.send_off, self.recv_off, self.status, stream)

    def copy(self, row_bytes, ins, in_rows, outs, out_cap_rows, stream=None):
        B.a2av_copy(row_bytes, ins, in_rows, outs, out_cap_rows, self.S, self.send_off,
                    self.recv_off, self.status, stream)

    def __call__(self, row_bytes, ins, in_rows, outs, out_cap_rows, stream=None, fused=False):
        """Whole a2av on the device-resident splits ``self.S``: three calls, or
        the single a2av_all_to_all_vdev call when ``fused``."""
        if fused:
            B.a2av_all_to_all_vdev(row_bytes, ins, in_rows, outs, out_cap_rows, self.S, self.O,
                                   self.send_off, self.recv_off, self.status, stream)
            return
        self.exchange_and_offsets(stream)
        self.copy(row_bytes, ins, in_rows, outs, out_cap_rows, stream)


def rows_of(t: torch.Tensor, row_bytes: int) -> int:
    """Whole rows of ``row_bytes`` held by a contiguous tensor."""
    return (t.numel() * t.element_size()) // row_bytes
