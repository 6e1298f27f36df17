"""Seeded synthetic inputs for the a2av workloads.

This module only draws inputs: split matrices, payload rows, routing ids and
jagged embedding keys. It holds none of the exchange's own arithmetic (no
transposes, scans, copies or sorts of the payload), so both the HIP path and the
CPU oracle can be fed from it.

Random draws use numpy's PCG64 (``default_rng(seed)``) for everything small and
torch's seeded generator for bulk payload on the device where the payload lives.

Workloads (sizes per virtual rank):

- ``tiny``: W=4, 256 rows x 64 bf16 (128 B rows, 32 KiB), uniform multinomial
  splits summing to 256, with a round trip.
- ``moe32``: W=4, 4096 rows x 4096 bf16 (8 KiB rows, 32 MiB), uniform
  multinomial splits; the message size of the MoE region on the tuning page.
- ``moe_dispatch``: W=8, 8192 tokens x hidden 7168 bf16, top-8 of 256 experts
  (32 per rank), expert ids Zipf(s=1.1).
- ``sweep``: W=4, 8 KiB rows, 1..4096 MiB per rank, uniform or 50 % zero splits.
- ``emb_keys``: W=8, 26 tables, batch 8192, lengths min(Poisson(20), 100), int64
  keys uniform in [0, 1e7), in table order (the exchange buckets them by
  owning rank, t mod 8).
"""
from __future__ import annotations

import numpy as np
import torch

BF16_BYTES = 2


def rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- split matrices
def uniform_splits(g: np.random.Generator, W: int, rows: int) -> np.ndarray:
    """S[s] ~ Multinomial(rows, 1/W) for each source rank s (W x W int64)."""
    return np.stack([g.multinomial(rows, [1.0 / W] * W) for _ in range(W)]).astype(np.int64)


def half_zero_splits(g: np.random.Generator, W: int, rows: int) -> np.ndarray:
    """Per source, W//2 destinations (seeded choice) get zero rows and the rows go
    multinomially over the remaining ones: exactly half of the (src, dst) pairs
    are zero and every rank still sends all its rows."""
    S = np.zeros((W, W), dtype=np.int64)
    for s in range(W):
        live = np.sort(g.choice(W, size=W - W // 2, replace=False))
        S[s, live] = g.multinomial(rows, [1.0 / len(live)] * len(live))
    return S


def random_splits(g: np.random.Generator, W: int, max_rows: int, zero_frac: float = 0.0):
    """Arbitrary splits for property tests: each entry uniform in [0, max_rows],
    a fraction of them forced to zero."""
    S = g.integers(0, max_rows + 1, size=(W, W), dtype=np.int64)
    if zero_frac > 0:
        S[g.random((W, W)) < zero_frac] = 0
    return S


# ---------------------------------------------------------------- payload rows
def payload_bf16(rows: int, cols: int, seed: int, device="cpu") -> torch.Tensor:
    """rows x cols bf16 drawn from N(0, 1) with a seeded torch generator."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    return torch.randn((rows, cols), generator=gen, dtype=torch.float32,
                       device=device).to(torch.bfloat16)


def payload_bytes(rows: int, row_bytes: int, seed: int, device="cpu") -> torch.Tensor:
    """rows x row_bytes uint8 of uniform random bytes (any row width)."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    return torch.randint(0, 256, (rows, row_bytes), generator=gen, dtype=torch.uint8,
                         device=device)


# ---------------------------------------------------------------- MoE routing ids
def zipf_probs(E: int, s: float = 1.1) -> np.ndarray:
    """Truncated Zipf over expert ids 0..E-1: p(e) proportional to (e+1)^-s."""
    w = (np.arange(1, E + 1, dtype=np.float64)) ** (-s)
    return w / w.sum()


def topk_ids(g: np.random.Generator, T: int, k: int, E: int, s: float = 1.1) -> np.ndarray:
    """T x k int32 expert ids: k distinct experts per token drawn without
    replacement from Zipf(s) (Gumbel-top-k), slot j in draw order."""
    logp = np.log(zipf_probs(E, s))
    ids = np.empty((T, k), dtype=np.int32)
    chunk = 4096
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        score = logp[None, :] + g.gumbel(size=(t1 - t0, E))
        top = np.argpartition(-score, k - 1, axis=1)[:, :k]
        order = np.argsort(-np.take_along_axis(score, top, axis=1), axis=1, kind="stable")
        ids[t0:t1] = np.take_along_axis(top, order, axis=1)
    return ids


def uniform_ids(g: np.random.Generator, T: int, k: int, E: int) -> np.ndarray:
    """T x k int32 ids drawn iid uniform over [0, E) (repeats allowed)."""
    return g.integers(0, E, size=(T, k), dtype=np.int64).astype(np.int32)


# ---------------------------------------------------------------- embedding keys
class EmbKeysRank:
    """One rank's sparse features for one batch, in table order.

    ``lengths`` is [tables][batch] int32 (keys per sample); ``keys`` holds the
    keys of table 0 (sample 0, 1, ...), then table 1, ... as int64.
    """

    def __init__(self, lengths, keys):
        self.lengths = lengths
        self.keys = keys


def emb_keys_rank(g: np.random.Generator, tables: int = 26, batch: int = 8192,
                  lam: float = 20.0, cap: int = 100, key_range: int = 10_000_000) -> EmbKeysRank:
    """lengths ~ min(Poisson(lam), cap) per (table, sample); keys uniform int64
    in [0, key_range)."""
    lengths = np.minimum(g.poisson(lam, size=(tables, batch)), cap).astype(np.int32)
    keys = g.integers(0, key_range, size=int(lengths.sum()), dtype=np.int64)
    return EmbKeysRank(lengths, keys)


def gate_weights(g: np.random.Generator, T: int, k: int) -> np.ndarray:
    """T x k float32 gate weights: a softmax over k N(0, 1) logits per token."""
    z = g.standard_normal((T, k))
    e = np.exp(z - z.max(axis=1, keepdims=True))
    return (e / e.sum(axis=1, keepdims=True)).astype(np.float32)


# ---------------------------------------------------------------- workload table
WORKLOADS = {
    "tiny": dict(W=4, rows=256, cols=64, splits="uniform"),
    "moe32": dict(W=4, rows=4096, cols=4096, splits="uniform"),
    "moe_dispatch": dict(W=8, tokens=8192, hidden=7168, k=8, experts=256, zipf=1.1),
    "sweep": dict(W=4, cols=4096, mib=[1 << i for i in range(13)],
                  splits=("uniform", "half_zero")),
    "emb_keys": dict(W=8, tables=26, batch=8192, lam=20.0, cap=100, key_range=10_000_000),
}


def rows_for_mib(mib: float, row_bytes: int) -> int:
    return int(mib * (1 << 20)) // row_bytes
