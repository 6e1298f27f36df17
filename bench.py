#!/usr/bin/env python3
"""Benchmark of the device-split all-to-all-v on one MI355X.

One step = the whole a2av on W virtual ranks held in one GPU's HBM: splits
exchange -> offsets -> payload copy, three C-ABI calls on one stream. The
default workload is W=4 ranks x 32 MiB (4096 rows x 4096 bf16, 8 KiB rows)
with multinomial splits, the message size of the MoE region on the tuning
page. The printed value is effective HBM throughput: payload bytes read plus
bytes written (2 x row bytes x rows moved) per second of GPU time over the
timed steps (HIP events on the launch stream, inside a region synchronized on
both sides), inputs resident in HBM.

Several independent buffer sets are cycled so that no step finds its inputs
in the 256 MB Infinity Cache left behind by the step before.

Also reported on the same JSON line:
  roofline      payload kernel alone, timed with HIP events on its stream,
                against the 8 TB/s HBM peak; `traffic` is the HBM byte count
                from rocprofv3 counters when they were taken on this exact
                kernel source (else null)
  cpu_baseline  the CPU oracle on the same workload on this host
  headline      W in {4, 8} x {32 MiB, 1 GiB} per rank, and W in {16, 64} at
                32 MiB, payload kernel and step
  sweep         W=4 at 1..4096 MiB per rank, uniform and 50%-zero splits
  ceilings      plain device copy of the same bytes (this library's copy loop
                and torch's D2D copy), read-only and write-only streams, and
                the exchange as W*W separate device-to-device copies (the
                library-call baseline)
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "a2av_wave_w4_32mib_traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "embeddings_a2av_virtual_amd", "csrc", f)
                  for f in ("a2av.hip", "common.hpp", "bounds.h")] + [
                      os.path.join(ROOT, "embeddings_a2av_virtual_amd", "build.py")]


def gbps(nbytes: float, seconds: float) -> float:
    """Decimal GB/s (10^9 bytes per second)."""
    return nbytes / seconds / 1e9


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class VSet:
    """One independent set of W virtual ranks: payload, outputs, device
    splits/offsets/status, and pre-marshalled C-ABI argument tuples."""

    def __init__(self, torch, B, I, W, rows, cols, seed, stream_handle, splits="uniform"):
        from embeddings_a2av_virtual_amd.vranks import A2av
        self.W, self.rows, self.R = W, rows, cols * 2
        g = I.rng(seed)
        self.S_host = (I.uniform_splits(g, W, rows) if splits == "uniform"
                       else I.half_zero_splits(g, W, rows))
        self.ins = [I.payload_bf16(rows, cols, seed * 1000 + r, device="cuda") for r in range(W)]
        cap = self.S_host.sum(axis=0)
        self.cap = [int(c) for c in cap]
        self.outs = [torch.empty((c, cols), dtype=torch.bfloat16, device="cuda") for c in self.cap]
        self.st = A2av(W)
        self.st.set_splits(self.S_host)
        self.moved = 2 * self.R * int(self.S_host.sum())
        vp = ctypes.c_void_p
        st = self.st
        hs = vp(stream_handle)
        self.ex_args = (W, vp(st.S.data_ptr()), vp(st.O.data_ptr()), vp(st.status.data_ptr()), hs)
        self.off_args = (W, vp(st.S.data_ptr()), vp(st.O.data_ptr()), vp(st.send_off.data_ptr()),
                         vp(st.recv_off.data_ptr()), vp(st.status.data_ptr()), hs)
        ins = (ctypes.c_void_p * W)(*[t.data_ptr() for t in self.ins])
        outs = (ctypes.c_void_p * W)(*[t.data_ptr() for t in self.outs])
        in_rows = (ctypes.c_int64 * W)(*([rows] * W))
        caps = (ctypes.c_int64 * W)(*self.cap)
        self._keep = (ins, outs, in_rows, caps)
        self.copy_args = (W, self.R, ins, in_rows, outs, caps, vp(st.S.data_ptr()),
                          vp(st.send_off.data_ptr()), vp(st.recv_off.data_ptr()),
                          vp(st.status.data_ptr()), hs)
        self.fused_args = (W, self.R, ins, in_rows, outs, caps, vp(st.S.data_ptr()),
                           vp(st.O.data_ptr()), vp(st.send_off.data_ptr()),
                           vp(st.recv_off.data_ptr()), vp(st.status.data_ptr()), hs)
        # inputs and the zeroed status were written on the current stream; the
        # launch stream may be another one
        torch.cuda.synchronize()


def run_config(torch, B, I, W, mib, steps, warmup, nsets, entry="fused", splits="uniform"):
    """Time `steps` whole a2av steps over `nsets` rotating buffer sets.

    entry="fused": one a2av_all_to_all_vdev call per step (one kernel that
    exchanges, scans and copies); "3call": a2av_exchange_splits, a2av_offsets,
    a2av_copy.

    The timed region holds the steps and nothing else: a barrier-free
    synchronize, host clock, one HIP event on the launch stream, the steps,
    one more event, synchronize. Step throughput is payload bytes over the GPU
    time between the two events (device timing, not the host clock, which
    adds the first launch's latency and the final wake-up to a region of a
    millisecond); the host-clock figure is kept beside it. That time over
    `steps` is also the average launch duration (for the fused entry a step
    is one kernel). For the
    three-call entry a second pass times `steps` a2av_copy launches back to
    back (the offsets the first pass left in every set) to time that kernel
    alone."""
    L = B.lib()
    stream = torch.cuda.current_stream()
    hs = stream.cuda_stream
    cols = 4096
    rows = I.rows_for_mib(mib, cols * 2)
    sets = [VSet(torch, B, I, W, rows, cols, seed=100 + 17 * W + mib + s, stream_handle=hs,
                 splits=splits) for s in range(nsets)]
    torch.cuda.synchronize()

    def step(vs, ev=None):
        if entry == "fused":
            assert L.a2av_all_to_all_vdev(*vs.fused_args) == 0
            return
        assert L.a2av_exchange_splits(*vs.ex_args) == 0
        assert L.a2av_offsets(*vs.off_args) == 0
        if ev is not None:
            ev[0].record(stream)
        assert L.a2av_copy(*vs.copy_args) == 0
        if ev is not None:
            ev[1].record(stream)

    for i in range(warmup):
        step(sets[i % nsets])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        step(sets[i % nsets])
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    gpu_ms = e0.elapsed_time(e1)
    moved = [sets[i % nsets].moved for i in range(steps)]
    wall = t1 - t0
    res = {
        "W": W, "mib_per_rank": mib, "row_bytes": cols * 2, "steps": steps, "entry": entry,
        "bytes_per_step": statistics.mean(moved),
        "step_ms": gpu_ms / steps,
        "step_gbs": gbps(sum(moved), gpu_ms / 1e3),
        "host_step_ms": wall / steps * 1e3,
        "host_step_gbs": gbps(sum(moved), wall),
    }
    if entry == "fused":
        res["kernel_ms_mean"] = gpu_ms / steps
        res["kernel_gbs"] = res["step_gbs"]
        # per-launch distribution from an event pair around each call (the
        # pair adds a little time of its own, so these read slightly high)
        n = min(steps, 100)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        torch.cuda.synchronize()
        for i in range(n):
            evs[i][0].record(stream)
            step(sets[i % nsets])
            evs[i][1].record(stream)
        torch.cuda.synchronize()
        per = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
        res["per_launch_us"] = {"min": round(per[0], 2), "p50": round(per[len(per) // 2], 2),
                                "p90": round(per[min(len(per) - 1, (9 * len(per)) // 10)], 2)}
    else:
        # a2av_copy alone: the passes above left every set's offsets in place,
        # so `steps` copies run back to back between one event pair (an event
        # pair around each launch would add its own time to every launch)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(steps):
            assert L.a2av_copy(*sets[i % nsets].copy_args) == 0
        e1.record(stream)
        torch.cuda.synchronize()
        copy_ms = e0.elapsed_time(e1)
        res["kernel_ms_mean"] = copy_ms / steps
        res["kernel_gbs"] = gbps(sum(moved), copy_ms / 1e3)
        # control: the same copies, each after two launches of a kernel that
        # writes one word (torch's fill of a one-element tensor), in place of
        # the splits exchange and the offsets: what two dependent launches
        # cost between copies, whatever they do
        tiny = torch.zeros(1, dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(steps):
            tiny.fill_(i)
            tiny.fill_(i + 1)
            assert L.a2av_copy(*sets[i % nsets].copy_args) == 0
        e1.record(stream)
        torch.cuda.synchronize()
        res["two_fills_then_copy_ms"] = e0.elapsed_time(e1) / steps
    for vs in sets:
        st = int(vs.st.status.item())
        if st != 0:
            raise RuntimeError(f"status word {st}: {B.a2av_strerror(st)}")
    del sets
    torch.cuda.empty_cache()
    return res


def naive_per_chunk(torch, I, W=4, mib=32, reps=50, nsets=8):
    """The same exchange as W * W separate device-to-device copies (one
    hipMemcpyAsync per (source, destination) chunk, offsets computed on the
    host): the library-call baseline."""
    cols = 4096
    R = cols * 2
    rows = I.rows_for_mib(mib, R)
    sets = []
    for k in range(nsets):
        g = I.rng(100 + 17 * W + mib + k)
        S = I.uniform_splits(g, W, rows)
        ins = [torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda") for _ in range(W)]
        cap = S.sum(axis=0)
        outs = [torch.empty((int(c), cols), dtype=torch.bfloat16, device="cuda") for c in cap]
        so = [[int(S[s, :d].sum()) for d in range(W)] for s in range(W)]
        ro = [[int(S[:s, d].sum()) for s in range(W)] for d in range(W)]
        pairs = [(outs[d][ro[d][s]:ro[d][s] + int(S[s, d])], ins[s][so[s][d]:so[s][d] + int(S[s, d])])
                 for d in range(W) for s in range(W) if S[s, d] > 0]
        sets.append((pairs, 2 * R * int(S.sum())))

    def step(i):
        for dst, src in sets[i % nsets][0]:
            dst.copy_(src)

    for i in range(3):
        step(i)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for i in range(reps):
        step(i)
    b.record()
    torch.cuda.synchronize()
    moved = sum(sets[i % nsets][1] for i in range(reps))
    del sets
    torch.cuda.empty_cache()
    return gbps(moved, a.elapsed_time(b) / 1e3)


def _time_rotating(torch, fn, bufs, reps, nbytes):
    """GB/s of reps calls fn(buf) over rotating buffers, between two events."""
    n = len(bufs)
    for i in range(3):
        fn(bufs[i % n])
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for i in range(reps):
        fn(bufs[i % n])
    b.record()
    torch.cuda.synchronize()
    return gbps(nbytes * reps, a.elapsed_time(b) / 1e3)


def ceilings(torch, B, nbytes, reps=50, nsets=8):
    """Plain contiguous copies of the same byte count (read n/2 + write n/2),
    and one-direction streams of n bytes (read only; written only, with
    non-temporal and with ordinary stores), at that size and at 4 GiB, the
    order of the MoE rows' traffic; and a plain copy of 4 GiB (8 GiB moved,
    the bytes of a W = 4 x 1 GiB exchange). Buffers rotate so the Infinity
    Cache holds none of them."""
    half = nbytes // 2
    srcs = [torch.empty(half, dtype=torch.uint8, device="cuda").fill_(i) for i in range(nsets)]
    dsts = [torch.empty(half, dtype=torch.uint8, device="cuda") for _ in range(nsets)]
    out = {}
    pairs = list(zip(dsts, srcs))
    out["device_copy_gbs"] = _time_rotating(
        torch, lambda p: B.a2av_device_copy(p[0], p[1], half), pairs, reps, 2 * half)
    out["torch_d2d_gbs"] = _time_rotating(torch, lambda p: p[0].copy_(p[1]), pairs, reps, 2 * half)
    del srcs, dsts, pairs
    torch.cuda.empty_cache()
    sink = torch.zeros(B.SINK_WORDS, dtype=torch.int64, device="cuda")
    for tag, size, n, r in (("", nbytes, nsets, reps), ("_4gib", 4 << 30, 2, 6)):
        bufs = [torch.empty(size, dtype=torch.uint8, device="cuda").fill_(i) for i in range(n)]
        out[f"read_only{tag}_gbs"] = _time_rotating(
            torch, lambda t: B.a2av_device_read(t, size, sink), bufs, r, size)
        out[f"write_only_nt{tag}_gbs"] = _time_rotating(
            torch, lambda t: B.a2av_device_fill(t, size, 0x5A5A5A5A, True), bufs, r, size)
        out[f"write_only{tag}_gbs"] = _time_rotating(
            torch, lambda t: B.a2av_device_fill(t, size, 0x5A5A5A5A, False), bufs, r, size)
        if tag:
            # one buffer into the other, then back
            out[f"device_copy{tag}_gbs"] = _time_rotating(
                torch, lambda p: B.a2av_device_copy(p[0], p[1], size),
                [(bufs[1], bufs[0]), (bufs[0], bufs[1])], r, 2 * size)
        del bufs
        torch.cuda.empty_cache()
    return out


def direction_ceiling(ceil, read_bytes, write_bytes):
    """The ceiling a kernel moving read_bytes in and write_bytes out faces if
    HBM serves the two directions one after the other at the one-direction
    rates measured at 4 GiB: total bytes / (reads / read rate + writes /
    write rate), the write rate being the better of the two store kinds."""
    cr = ceil["read_only_4gib_gbs"]
    cw = max(ceil["write_only_nt_4gib_gbs"], ceil["write_only_4gib_gbs"])
    return (read_bytes + write_bytes) / (read_bytes / cr + write_bytes / cw)


def host_cpu():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, os.cpu_count()


def cpu_baseline(torch, I, W=4, mib=32, budget_s=10.0):
    """The CPU oracle on one full set of the workload, repeated for about
    budget_s seconds (at least 3 runs); single-threaded C, pinned to one core
    while it runs."""
    import numpy as np
    sys.path.insert(0, ROOT)
    from oracle.ref import Oracle
    o = Oracle()
    cols = 4096
    R = cols * 2
    rows = I.rows_for_mib(mib, R)
    seed = 100 + 17 * W + mib   # the first buffer set of the GPU run
    g = I.rng(seed)
    S = I.uniform_splits(g, W, rows)
    X = [I.payload_bf16(rows, cols, seed * 1000 + r, device="cuda").view(torch.uint8).cpu().numpy()
         .reshape(-1) for r in range(W)]
    cap = S.sum(axis=0)
    Y = [np.empty(int(c) * R, dtype=np.uint8) for c in cap]
    in_rows = np.full(W, rows, dtype=np.int64)
    times = []
    old_aff = os.sched_getaffinity(0)
    core = min(old_aff)
    os.sched_setaffinity(0, {core})
    try:
        t_start = time.perf_counter()
        while len(times) < 3 or (time.perf_counter() - t_start < budget_s and len(times) < 20000):
            t0 = time.perf_counter()
            st = o.a2av(R, X, in_rows, Y, cap, S)[0]
            times.append(time.perf_counter() - t0)
            assert st == 0
    finally:
        os.sched_setaffinity(0, old_aff)
    moved = 2 * R * int(S.sum())
    med = statistics.median(times)
    model, ncpu = host_cpu()
    return {"value": round(gbps(moved, med), 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"whole W={W} x {mib} MiB/rank a2av (exchange+offsets+copy), "
                      f"{len(times)} runs, median {med * 1e3:.1f} ms, pinned to core {core} of "
                      f"{ncpu} ({model})"}


def time_events(torch, fn, reps, warmup=2):
    """Average GPU ms of fn() over reps launches bracketed by two events."""
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        fn()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(reps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def time_cpu(fn, budget_s=2.0, min_runs=2):
    times = []
    t_start = time.perf_counter()
    while len(times) < min_runs or time.perf_counter() - t_start < budget_s:
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
        if len(times) >= 50:
            break
    return statistics.median(times)


def _vp_array(tensors):
    return (ctypes.c_void_p * len(tensors))(*[t.data_ptr() for t in tensors])


def _i64_array(vals):
    return (ctypes.c_int64 * len(vals))(*[int(x) for x in vals])


def fused_args(st, R, ins, in_rows, outs, caps, stream=None, status=None):
    """Pre-marshalled argument tuple of one a2av_all_to_all_vdev call, so that
    timing a small exchange measures the GPU rather than Python."""
    import torch
    W = len(ins)
    vp = ctypes.c_void_p
    s = stream if stream is not None else torch.cuda.current_stream()
    stat = status if status is not None else st.status
    return (W, R, _vp_array(ins), _i64_array(in_rows), _vp_array(outs), _i64_array(caps),
            vp(st.S.data_ptr()), vp(st.O.data_ptr()), vp(st.send_off.data_ptr()),
            vp(st.recv_off.data_ptr()), vp(stat.data_ptr()), vp(s.cuda_stream))


def row_entry(nbytes, ms, cpu_bytes=None, cpu_s=None, note=""):
    gbs = gbps(nbytes, ms / 1e3)
    e = {"bytes": int(nbytes), "us": round(ms * 1e3, 2), "gbs": round(gbs, 1),
         "frac": round(gbs / HBM_PEAK_GBS, 4)}
    if cpu_bytes is not None:
        e["oracle_gbs"] = round(gbps(cpu_bytes, cpu_s), 3)
        e["oracle_sample"] = note
    return e


def _check_status(B, named):
    for name, st in named:
        v = int(st.item())
        if v != 0:
            raise RuntimeError(f"{name}: status {v} ({B.a2av_strerror(v)})")


class KeyChain:
    """The embedding-key exchange of one batch as pre-marshalled C-ABI calls on
    one stream: keys_bucketize (owner order + the two split matrices on the
    device), then the keys a2av and the lengths a2av reading those splits."""

    NT, BATCH = 26, 8192

    def __init__(self, torch, B, I, W, seed, stream):
        from embeddings_a2av_virtual_amd.vranks import A2av
        self.W = W
        g = I.rng(seed)
        ranks = [I.emb_keys_rank(g) for _ in range(W)]
        self.host = ranks
        self.len_in = [torch.from_numpy(r.lengths.reshape(-1)).cuda() for r in ranks]
        self.key_in = [torch.from_numpy(r.keys).cuda() for r in ranks]
        self.n_keys = [int(r.keys.size) for r in ranks]
        self.len_b = [torch.empty_like(x) for x in self.len_in]
        self.key_b = [torch.empty_like(x) for x in self.key_in]
        self.ka, self.la = A2av(W), A2av(W)
        self.status = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.ws = torch.empty(B.keys_bucketize_workspace_bytes(W, self.NT), dtype=torch.uint8,
                              device="cuda")
        vp = ctypes.c_void_p
        hs = vp(stream.cuda_stream)
        self.b_args = (W, self.NT, self.BATCH, _vp_array(self.len_in), _vp_array(self.key_in),
                       _i64_array(self.n_keys), _vp_array(self.len_b), _vp_array(self.key_b),
                       vp(self.ka.S.data_ptr()), vp(self.la.S.data_ptr()), vp(self.ws.data_ptr()),
                       self.ws.numel(), vp(self.status.data_ptr()), hs)
        self.L = B.lib()
        # the buffers above were filled on the current stream; the calls below
        # run on `stream`, which may be another one
        torch.cuda.synchronize()
        # receive capacity from one bucketing pass (set-up, outside any timing)
        assert self.L.keys_bucketize(*self.b_args) == 0
        torch.cuda.synchronize()
        _check_status(B, [("bucketize", self.status)])
        self.Sk = self.ka.S.cpu().numpy().copy()
        self.Sl = self.la.S.cpu().numpy().copy()
        kc = [int(c) for c in self.Sk.sum(axis=0)]
        lc = [int(c) for c in self.Sl.sum(axis=0)]
        self.key_out = [torch.empty(c, dtype=torch.int64, device="cuda") for c in kc]
        self.len_out = [torch.empty(c, dtype=torch.int32, device="cuda") for c in lc]
        self.k_args = fused_args(self.ka, 8, self.key_b, self.n_keys, self.key_out, kc,
                                 stream=stream, status=self.status)
        self.l_args = fused_args(self.la, 4, self.len_b, [x.numel() for x in self.len_b],
                                 self.len_out, lc, stream=stream, status=self.status)
        self.bucket_bytes = sum(2 * (8 * n + 4 * self.NT * self.BATCH) for n in self.n_keys)
        self.key_bytes = 2 * 8 * int(self.Sk.sum())
        self.len_bytes = 2 * 4 * int(self.Sl.sum())
        # the fused exchange: same inputs, straight into receive buffers of its own
        self.fkey_out = [torch.empty(c, dtype=torch.int64, device="cuda") for c in kc]
        self.flen_out = [torch.empty(c, dtype=torch.int32, device="cuda") for c in lc]
        self.fsk = torch.empty((W, W), dtype=torch.int64, device="cuda")
        self.fsl = torch.empty((W, W), dtype=torch.int64, device="cuda")
        self.fro = torch.empty((W, W + 1), dtype=torch.int64, device="cuda")
        self.fws = torch.empty(B.keys_exchange_workspace_bytes(W, self.NT), dtype=torch.uint8,
                               device="cuda")
        self.fstatus = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.x_args = (W, self.NT, self.BATCH, _vp_array(self.len_in), _vp_array(self.key_in),
                       _i64_array(self.n_keys), _vp_array(self.flen_out), _i64_array(lc),
                       _vp_array(self.fkey_out), _i64_array(kc), vp(self.fsk.data_ptr()),
                       vp(self.fsl.data_ptr()), vp(self.fro.data_ptr()), vp(self.fws.data_ptr()),
                       self.fws.numel(), vp(self.fstatus.data_ptr()), hs)
        # algorithmic bytes of the fused exchange: lengths read once for the
        # counts, then keys and lengths read and written once each
        self.fused_bytes = (sum(4 * self.NT * self.BATCH for _ in range(W)) + self.key_bytes +
                            self.len_bytes)
        torch.cuda.synchronize()   # status words zeroed before any call on `stream`

    def bucketize(self):
        assert self.L.keys_bucketize(*self.b_args) == 0

    def keys(self):
        assert self.L.a2av_all_to_all_vdev(*self.k_args) == 0

    def lengths(self):
        assert self.L.a2av_all_to_all_vdev(*self.l_args) == 0

    def fused(self):
        assert self.L.keys_exchange(*self.x_args) == 0

    def __call__(self):
        self.bucketize()
        self.keys()
        self.lengths()


def time_overlap(torch, fa, fb, sa, sb, reps=20):
    """GPU time (ms) per repetition of a then b on stream sa, and of a on sa
    alongside b on sb (b's stream waits for the repetition's start and sa for
    b's end, so a repetition ends when both have). Also b's latency: from the
    repetition's start to b's end, median over the repetitions, when b is
    queued behind a on one stream and when it runs on its own stream."""
    def ev():
        return torch.cuda.Event(enable_timing=True)

    fb_s = fb["on_a"]
    fb_b = fb["on_b"]
    for _ in range(2):
        fa()
        fb_s()
    torch.cuda.synchronize()
    e0, e1 = ev(), ev()
    starts = [ev() for _ in range(reps)]
    b_done = [ev() for _ in range(reps)]
    e0.record(sa)
    for i in range(reps):
        starts[i].record(sa)
        fa()
        fb_s()
        b_done[i].record(sa)
    e1.record(sa)
    torch.cuda.synchronize()
    t_serial = e0.elapsed_time(e1) / reps
    lat_serial = statistics.median(starts[i].elapsed_time(b_done[i]) for i in range(reps))
    starts = [ev() for _ in range(reps)]
    b_done = [ev() for _ in range(reps)]
    torch.cuda.synchronize()
    e0.record(sa)
    for i in range(reps):
        starts[i].record(sa)
        sb.wait_event(starts[i])
        fa()
        fb_b()
        b_done[i].record(sb)
        sa.wait_event(b_done[i])
    e1.record(sa)
    torch.cuda.synchronize()
    t_over = e0.elapsed_time(e1) / reps
    lat_own = statistics.median(starts[i].elapsed_time(b_done[i]) for i in range(reps))
    return t_serial, t_over, lat_serial, lat_own


def moe_rows(torch, B, I, o, out, ceil=None):
    """MoE dispatch workload: W=8, 8192 tokens x 7168 bf16 per rank, top-8 of
    256 Zipf(1.1) experts. pack -> dispatch a2av -> regroup to expert-major
    and back -> return a2av -> combine (weighted) and un-pack."""
    import numpy as np
    from embeddings_a2av_virtual_amd.vranks import A2av
    W, T, k, E, hidden = 8, 8192, 8, 256, 7168
    R, Q = hidden * 2, T * k
    g = I.rng(900)
    ids_h = [I.topk_ids(g, T, k, E, 1.1) for _ in range(W)]
    w_h = [I.gate_weights(g, T, k) for _ in range(W)]
    tok = [I.payload_bf16(T, hidden, 9000 + r, device="cuda") for r in range(W)]
    ids = [torch.from_numpy(i.reshape(-1)).cuda() for i in ids_h]
    wts = [torch.from_numpy(w.reshape(-1)).cuda() for w in w_h]
    send = [torch.empty((Q, hidden), dtype=torch.bfloat16, device="cuda") for _ in range(W)]
    perm = [torch.empty(Q, dtype=torch.int64, device="cuda") for _ in range(W)]
    S = torch.empty((W, W), dtype=torch.int64, device="cuda")
    counts = torch.empty((W, E), dtype=torch.int64, device="cuda")
    ws = torch.empty(B.moe_pack_workspace_bytes(W, T, k, E), dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    pack = lambda: B.moe_pack(W, T, k, E, R, tok, ids, send, perm, S, counts, ws, status)
    ms = time_events(torch, pack, 5)
    pack_bytes = W * (T * R + Q * R + Q * (4 + 8))
    cpu = {}
    if o is not None:
        Ts = 1024   # one rank, the first 1024 tokens
        th = tok[0][:Ts].view(torch.uint8).cpu().numpy()
        ih = ids_h[0][:Ts]
        cs = time_cpu(lambda: o.moe_pack(Ts, k, E, W, R, th, ih))
        cpu = dict(cpu_bytes=Ts * R + Ts * k * R + Ts * k * 12, cpu_s=cs,
                   note="one rank, 1024 tokens")
    out["moe_pack"] = row_entry(pack_bytes, ms, **cpu)
    # one token row read, k written (plus ids, perm written and read back)
    pack_rw = (W * (T * R + Q * 4 + Q * 8), W * (Q * R + Q * 8))
    # ---- dispatch a2av with the pack's splits (rank 0 receives ~66 % of all rows)
    fwd = A2av(W)
    fwd.S.copy_(S)
    fwd.exchange_and_offsets()
    torch.cuda.synchronize()
    cap = [int(c) for c in fwd.recv_off[:, W].cpu().numpy()]
    recv = [torch.empty((c, hidden), dtype=torch.bfloat16, device="cuda") for c in cap]
    disp = lambda: fwd(R, send, [Q] * W, recv, cap, fused=True)
    ms = time_events(torch, disp, 5)
    moved = 2 * R * sum(cap)
    out["dispatch_a2av"] = row_entry(moved, ms)
    out["dispatch_a2av"]["rows_received_per_rank"] = cap
    # ---- regroup: (source, expert) -> (expert, source) and back
    grp = [torch.empty_like(x) for x in recv]
    eoff = torch.empty((W, E // W + 1), dtype=torch.int64, device="cuda")
    rws = torch.empty(B.moe_regroup_workspace_bytes(W, E), dtype=torch.uint8, device="cuda")
    rst = torch.zeros(1, dtype=torch.int32, device="cuda")
    to_expert = lambda: B.moe_regroup(W, E, R, counts, recv, cap, grp, cap, eoff, 0, rws, rst)
    to_source = lambda: B.moe_regroup(W, E, R, counts, grp, cap, recv, cap, eoff, 1, rws, rst)
    ms0 = time_events(torch, to_expert, 5)
    ms1 = time_events(torch, to_source, 5)
    cpu = {}
    if o is not None:
        cnt_h = counts.cpu().numpy()
        x7 = recv[W - 1].view(torch.uint8).cpu().numpy()
        cs = time_cpu(lambda: o.moe_regroup(W, E, W - 1, R, cnt_h, x7, cap[W - 1], cap[W - 1], 0))
        cpu = dict(cpu_bytes=2 * R * cap[W - 1], cpu_s=cs,
                   note=f"rank {W - 1} whole ({cap[W - 1]} rows)")
    out["moe_regroup_to_expert"] = row_entry(moved, ms0, **cpu)
    out["moe_regroup_to_source"] = row_entry(moved, ms1)
    # ---- the dispatch and the regroup as one copy, and the inverse
    gws = torch.empty(B.moe_dispatch_grouped_workspace_bytes(W, E), dtype=torch.uint8,
                      device="cuda")
    gst = torch.zeros(1, dtype=torch.int32, device="cuda")
    home = [torch.empty((Q, hidden), dtype=torch.bfloat16, device="cuda") for _ in range(W)]
    gdisp = lambda: B.moe_dispatch_grouped(W, E, R, counts, send, [Q] * W, grp, cap, eoff, 0,
                                           gws, gst)
    gret = lambda: B.moe_dispatch_grouped(W, E, R, counts, grp, cap, home, [Q] * W, eoff, 1,
                                          gws, gst)
    ms0 = time_events(torch, gdisp, 5)
    ms1 = time_events(torch, gret, 5)
    cpu = {}
    if o is not None:
        cnt_h = counts.cpu().numpy()
        sh = [x.view(torch.uint8).cpu().numpy().reshape(-1) for x in send]
        cs = time_cpu(lambda: o.moe_dispatch_grouped(W, E, R, cnt_h, sh, [Q] * W, cap, 0),
                      budget_s=3.0, min_runs=1)
        cpu = dict(cpu_bytes=moved, cpu_s=cs, note="all ranks whole (memcpy per block)")
        del sh
    out["moe_dispatch_grouped"] = row_entry(moved, ms0, **cpu)
    out["moe_return_grouped"] = row_entry(moved, ms1)
    torch.cuda.synchronize()
    _check_status(B, [("grouped", gst)])
    for r in range(W):
        if not torch.equal(home[r].view(torch.int16), send[r].view(torch.int16)):
            raise RuntimeError("grouped dispatch + return did not bring the rows home")
    del home
    # ---- the return trip and the weighted combine in one pass, from the expert side
    cgo = [torch.empty((T, hidden), dtype=torch.bfloat16, device="cuda") for _ in range(W)]
    cgws = torch.empty(B.moe_combine_grouped_workspace_bytes(W, T, k, E), dtype=torch.uint8,
                       device="cuda")
    cgst = torch.zeros(1, dtype=torch.int32, device="cuda")
    cgrp = lambda: B.moe_combine_grouped(W, T, k, E, hidden, counts, ids, perm, grp, cap, wts,
                                         cgo, cgws, cgst)
    ms = time_events(torch, cgrp, 5)
    out["moe_combine_grouped"] = row_entry(W * (Q * R + T * R + Q * (8 + 4 + 8)), ms)
    # the whole fused MoE round trip after the pack: grouped dispatch + combine from the expert side
    ms = time_events(torch, lambda: (gdisp(), cgrp()), 5)
    out["moe_fused_round_trip"] = {"us": round(ms * 1e3, 2),
                                   "note": "grouped dispatch + combine from the expert side"}
    torch.cuda.synchronize()
    _check_status(B, [("grouped combine", cgst), ("grouped", gst)])
    # ---- the pack and the dispatch in one step (no send buffer), both receive
    # orders, and the inverse (return trip and un-pack in one step)
    pdws = torch.empty(B.moe_pack_dispatch_workspace_bytes(W, T, k, E), dtype=torch.uint8,
                       device="cuda")
    pdst = torch.zeros(1, dtype=torch.int32, device="cuda")
    S1, cnt1 = torch.empty_like(S), torch.empty_like(counts)
    perm1 = [torch.empty_like(x) for x in perm]
    boff0 = torch.empty((W, W + 1), dtype=torch.int64, device="cuda")
    boff1 = torch.empty((W, E // W + 1), dtype=torch.int64, device="cuda")
    pd0 = lambda: B.moe_pack_dispatch(W, T, k, E, R, tok, ids, recv, cap, perm1, S1, cnt1, boff0,
                                      0, pdws, pdst)
    pd1 = lambda: B.moe_pack_dispatch(W, T, k, E, R, tok, ids, grp, cap, perm1, S1, cnt1, boff1,
                                      1, pdws, pdst)
    out["moe_pack_dispatch"] = row_entry(pack_bytes, time_events(torch, pd0, 5))
    out["moe_pack_dispatch_grouped"] = row_entry(pack_bytes, time_events(torch, pd1, 5))
    if ceil:
        dc = direction_ceiling(ceil, *pack_rw)
        for key in ("moe_pack", "moe_pack_dispatch", "moe_pack_dispatch_grouped"):
            out[key]["direction_ceiling_gbs"] = round(dc, 1)
            out[key]["frac_of_direction_ceiling"] = round(out[key]["gbs"] / dc, 4)
    urws = torch.empty(B.moe_unpack_return_workspace_bytes(W, E), dtype=torch.uint8,
                       device="cuda")
    urst = torch.zeros(1, dtype=torch.int32, device="cuda")
    home = [torch.empty((Q, hidden), dtype=torch.bfloat16, device="cuda") for _ in range(W)]
    ur0 = lambda: B.moe_unpack_return(W, T, k, E, R, cnt1, ids, perm1, recv, cap, home, 0, urws,
                                      urst)
    ur1 = lambda: B.moe_unpack_return(W, T, k, E, R, cnt1, ids, perm1, grp, cap, home, 1, urws,
                                      urst)
    unpack_bytes = W * (2 * Q * R + Q * (8 + 4))
    out["moe_unpack_return"] = row_entry(unpack_bytes, time_events(torch, ur0, 5))
    out["moe_unpack_return_grouped"] = row_entry(unpack_bytes, time_events(torch, ur1, 5))
    # whole round trips from the tokens, each as one-step calls
    cgrp1 = lambda: B.moe_combine_grouped(W, T, k, E, hidden, cnt1, ids, perm1, grp, cap, wts,
                                          cgo, cgws, cgst)
    ms = time_events(torch, lambda: (pd0(), ur0()), 5)
    out["moe_tokens_unpack_round_trip"] = {
        "us": round(ms * 1e3, 2), "note": "moe_pack_dispatch + moe_unpack_return (layout 0)"}
    ms = time_events(torch, lambda: (pd1(), cgrp1()), 5)
    out["moe_tokens_combine_round_trip"] = {
        "us": round(ms * 1e3, 2),
        "note": "moe_pack_dispatch (layout 1) + combine from the expert side"}
    # the weighted combine read at the owners, either receive order
    crws = torch.empty(B.moe_combine_return_workspace_bytes(W, T, k, E), dtype=torch.uint8,
                       device="cuda")
    crst = torch.zeros(1, dtype=torch.int32, device="cuda")
    cr0 = lambda: B.moe_combine_return(W, T, k, E, hidden, cnt1, ids, perm1, recv, cap, wts, cgo,
                                       0, crws, crst)
    cr1 = lambda: B.moe_combine_return(W, T, k, E, hidden, cnt1, ids, perm1, grp, cap, wts, cgo,
                                       1, crws, crst)
    home_comb_bytes = W * (Q * R + T * R + Q * (8 + 4 + 8))
    out["moe_combine_return"] = row_entry(home_comb_bytes, time_events(torch, cr0, 5))
    out["moe_combine_return_grouped"] = row_entry(home_comb_bytes, time_events(torch, cr1, 5))
    ms = time_events(torch, lambda: (pd0(), cr0()), 5)
    out["moe_tokens_combine_round_trip_source_major"] = {
        "us": round(ms * 1e3, 2),
        "note": "moe_pack_dispatch (layout 0) + moe_combine_return (layout 0)"}
    torch.cuda.synchronize()
    _check_status(B, [("pack + dispatch", pdst), ("unpack + return", urst),
                      ("grouped combine", cgst), ("combine at the owners", crst)])
    for r in range(W):
        if not torch.equal(home[r].view(torch.int16),
                           tok[r].view(torch.int16).repeat_interleave(k, dim=0)):
            raise RuntimeError("pack + dispatch and its inverse did not bring every slot home")
    del grp, home
    # ---- return a2av: every row goes home
    bk = A2av(W)
    bk.S.copy_(fwd.O)
    back = [torch.empty((Q, hidden), dtype=torch.bfloat16, device="cuda") for _ in range(W)]
    ret = lambda: bk(R, recv, cap, back, [Q] * W, fused=True)
    ms = time_events(torch, ret, 5)
    out["return_a2av"] = row_entry(moved, ms)
    # ---- weighted combine: read k rows per token, write one
    comb = [torch.empty((T, hidden), dtype=torch.bfloat16, device="cuda") for _ in range(W)]
    cst = torch.zeros(1, dtype=torch.int32, device="cuda")
    combine = lambda: B.moe_combine(W, T, k, hidden, back, perm, wts, comb, cst)
    ms = time_events(torch, combine, 5)
    comb_bytes = W * (Q * R + T * R + Q * (8 + 4))
    cpu = {}
    if o is not None:
        Ts = 128   # one rank, 128 tokens, their own rows
        p0 = perm[0][:Ts * k].cpu().numpy()
        b0 = back[0].view(torch.int16).cpu().numpy().view(np.uint16)
        sub = np.ascontiguousarray(b0[p0])
        ident = np.arange(Ts * k, dtype=np.int64)
        cs = time_cpu(lambda: o.moe_combine(Ts, k, hidden, sub, ident, w_h[0][:Ts]))
        cpu = dict(cpu_bytes=Ts * k * R + Ts * R + Ts * k * 12, cpu_s=cs,
                   note="one rank, 128 tokens (fp32 fma chain, single thread)")
        del b0
    out["moe_combine"] = row_entry(comb_bytes, ms, **cpu)
    del comb
    # ---- un-pack (no weights): every slot gets its row back
    outb = [torch.empty((Q, hidden), dtype=torch.bfloat16, device="cuda") for _ in range(W)]
    ust = torch.zeros(1, dtype=torch.int32, device="cuda")
    unpack = lambda: B.moe_unpack(W, T, k, R, back, perm, outb, ust)
    ms = time_events(torch, unpack, 5)
    out["moe_unpack"] = row_entry(W * (2 * Q * R + 8 * Q), ms)
    torch.cuda.synchronize()
    _check_status(B, [("pack", status), ("dispatch", fwd.status), ("regroup", rst),
                      ("return", bk.status), ("combine", cst), ("unpack", ust)])
    # the same round trip unfused: dispatch a2av, regroup to expert-major and
    # back, return a2av, combine (sum of the rows above)
    out["moe_chain_round_trip"] = {
        "us": round(sum(out[x]["us"] for x in ("dispatch_a2av", "moe_regroup_to_expert",
                                                 "moe_regroup_to_source", "return_a2av",
                                                 "moe_combine")), 2),
        "note": "sum of dispatch a2av, both regroups, return a2av and combine"}
    # from the tokens, unfused: pack, then those steps (weighted), or pack,
    # dispatch a2av, return a2av and un-pack (unweighted)
    out["moe_tokens_combine_round_trip_chain"] = {
        "us": round(out["moe_pack"]["us"] + out["moe_chain_round_trip"]["us"], 2),
        "note": "moe_pack + the chain above"}
    out["moe_tokens_combine_round_trip_source_major_chain"] = {
        "us": round(sum(out[x]["us"] for x in ("moe_pack", "dispatch_a2av", "return_a2av",
                                                 "moe_combine")), 2),
        "note": "sum of pack, dispatch a2av, return a2av and combine"}
    out["moe_tokens_unpack_round_trip_chain"] = {
        "us": round(sum(out[x]["us"] for x in ("moe_pack", "dispatch_a2av", "return_a2av",
                                                 "moe_unpack")), 2),
        "note": "sum of pack, dispatch a2av, return a2av and un-pack"}
    return dict(fwd=fwd, send=send, recv=recv, cap=cap, R=R, Q=Q, W=W)


def key_rows(torch, B, I, o, out):
    """Embedding keys: W=8, 26 tables, batch 8192, lengths min(Poisson(20), 100):
    bucketing by owner, then the keys and lengths a2av."""
    import numpy as np
    stream = torch.cuda.current_stream()
    kc = KeyChain(torch, B, I, 8, 901, stream)
    res = {}
    ms = time_events(torch, kc.bucketize, 50)
    cpu = {}
    if o is not None:
        r0 = kc.host[0]
        cs = time_cpu(lambda: o.keys_bucketize(8, kc.NT, kc.BATCH, r0.lengths, r0.keys))
        cpu = dict(cpu_bytes=2 * (8 * r0.keys.size + 4 * r0.lengths.size), cpu_s=cs,
                   note="one rank whole")
    res["bucketize"] = row_entry(kc.bucket_bytes, ms, **cpu)
    for name, fn, nb, R2 in (("keys", kc.keys, kc.key_bytes, 8),
                             ("lengths", kc.lengths, kc.len_bytes, 4)):
        ms = time_events(torch, fn, 50)
        cpu = {}
        if o is not None:
            Sx = kc.Sk if name == "keys" else kc.Sl
            src = kc.key_b if name == "keys" else kc.len_b
            xh = [x.view(torch.uint8).cpu().numpy() for x in src]
            capx = Sx.sum(axis=0)
            yh = [np.empty(int(c) * R2, dtype=np.uint8) for c in capx]
            rows_in = np.array([x.numel() for x in src], dtype=np.int64)
            cs = time_cpu(lambda: o.a2av(R2, xh, rows_in, yh, capx, Sx))
            cpu = dict(cpu_bytes=nb, cpu_s=cs, note="whole exchange")
        res[name + "_a2av"] = row_entry(nb, ms, **cpu)
    ms = time_events(torch, kc, 50)
    res["chain"] = row_entry(kc.bucket_bytes + kc.key_bytes + kc.len_bytes, ms)
    ms = time_events(torch, kc.fused, 50)
    res["fused_exchange"] = row_entry(kc.fused_bytes, ms)
    # the fused exchange captured once into a HIP graph and replayed
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    kg = KeyChain(torch, B, I, 8, 901, side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        kg.fused()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            kg.fused()
    torch.cuda.synchronize()
    ms = time_events(torch, graph.replay, 50)
    res["fused_exchange_graph"] = row_entry(kg.fused_bytes, ms)
    torch.cuda.synchronize()
    _check_status(B, [("key chain", kc.status), ("fused exchange", kc.fstatus),
                      ("graph replays", kg.fstatus)])
    for a, b in zip(kc.fkey_out + kc.flen_out, kg.fkey_out + kg.flen_out):
        if not torch.equal(a, b):
            raise RuntimeError("graph replay of the key exchange differs from the eager call")
    # the fused exchange delivers the same bytes as the chain
    for a, b in zip(kc.key_out + kc.len_out, kc.fkey_out + kc.flen_out):
        if not torch.equal(a, b):
            raise RuntimeError("fused key exchange differs from the chain")
    out["emb_keys_exchange"] = res
    return kc


def overlap_rows(torch, B, I, moe, out):
    """The next batch's key exchange on a stream of its own, next to the
    current step's traffic on the main stream (both default priority):
    per-repetition GPU time with both on one stream and side by side."""
    sa = torch.cuda.current_stream()
    sb = torch.cuda.Stream()
    kb = KeyChain(torch, B, I, 8, 902, sb)
    ka = KeyChain(torch, B, I, 8, 902, sa)
    res = {}
    t_keys = time_events(torch, ka.fused, 20)
    fwd, W, R, Q = moe["fwd"], moe["W"], moe["R"], moe["Q"]
    disp_args = fused_args(fwd, R, moe["send"], [Q] * W, moe["recv"], moe["cap"], stream=sa)
    L = B.lib()
    disp = lambda: L.a2av_all_to_all_vdev(*disp_args)
    small = VSet(torch, B, I, 4, 4096, 4096, seed=77, stream_handle=sa.cuda_stream)
    a32 = lambda: L.a2av_all_to_all_vdev(*small.fused_args)
    # an expert-sized bf16 GEMM (2048 rows x 7168 -> 4096): compute-bound, so
    # it leaves HBM time for the key exchange to fill
    ga = torch.randn(2048, 7168, device="cuda").to(torch.bfloat16)
    gb = torch.randn(7168, 4096, device="cuda").to(torch.bfloat16).contiguous()
    gc = torch.empty(2048, 4096, dtype=torch.bfloat16, device="cuda")
    gemm = lambda: torch.matmul(ga, gb, out=gc)
    cases = (("dispatch_a2av", disp, None), ("a2av_w4_32mib", a32, None),
             ("gemm_expert", gemm, None),
             # the same a2av neighbours without the occupancy cap (no unused LDS
             # reserved per workgroup): how much of any loss the cap causes
             ("dispatch_a2av_no_cap", disp, "0"), ("a2av_w4_32mib_no_cap", a32, "0"))
    for name, fa, lds in cases:
        old = os.environ.get("A2AV_WAVE_LDS")
        if lds is not None:
            os.environ["A2AV_WAVE_LDS"] = lds
        try:
            t_a = time_events(torch, fa, 10)
            ts, to, ls, lo = time_overlap(torch, fa, {"on_a": ka.fused, "on_b": kb.fused}, sa, sb)
        finally:
            if lds is not None:
                if old is None:
                    del os.environ["A2AV_WAVE_LDS"]
                else:
                    os.environ["A2AV_WAVE_LDS"] = old
        res[name] = {"a_us": round(t_a * 1e3, 2), "keys_us": round(t_keys * 1e3, 2),
                     "serial_us": round(ts * 1e3, 2), "overlapped_us": round(to * 1e3, 2),
                     "hidden_frac_of_keys": round((ts - to) / t_keys, 3),
                     # when the keys are ready: behind the neighbour on its stream,
                     # or on a stream of their own
                     "keys_done_us_same_stream": round(ls * 1e3, 2),
                     "keys_done_us_own_stream": round(lo * 1e3, 2)}
        log("bench: overlap", name, json.dumps(res[name]))
    torch.cuda.synchronize()
    _check_status(B, [("keys a", ka.fstatus), ("keys b", kb.fstatus), ("a2av", small.st.status),
                      ("dispatch", fwd.status)])
    out["key_exchange_overlap"] = res


def row_benchmarks(torch, B, I, with_cpu=True, ceil=None):
    """The other steps of the path, each at its full size. GB/s counts
    algorithmic bytes (payload read + written, plus index and weight bytes
    where a kernel reads them)."""
    sys.path.insert(0, ROOT)
    out = {}
    o = None
    if with_cpu:
        from oracle.ref import Oracle
        o = Oracle()
    moe = moe_rows(torch, B, I, o, out, ceil)
    key_rows(torch, B, I, o, out)
    overlap_rows(torch, B, I, moe, out)
    del moe
    torch.cuda.empty_cache()
    return out


def traffic_entry(bytes_per_launch):
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--sets", type=int, default=8, help="rotating buffer sets (32 MiB case)")
    ap.add_argument("--no-headline", action="store_true", help="skip the W x size matrix")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-rows", action="store_true",
                    help="skip the MoE pack / un-pack and key-exchange measurements")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the size sweep (W=4 at 1..4096 MiB per rank, uniform and "
                         "50%%-zero splits)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} requested, but this benchmark runs on ONE GPU: "
              "the W ranks are virtual (partitions of one GPU's HBM) and there is no "
              "multi-GPU path; run with --gpus 1.", file=sys.stderr)
        return 2
    if int(os.environ.get("RANK", "0")) != 0:
        return 0

    sys.path.insert(0, ROOT)
    import torch
    from embeddings_a2av_virtual_amd import _binding as B
    from embeddings_a2av_virtual_amd import inputs as I
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    B.lib()

    log("bench: W=4 x 32 MiB/rank, steps", args.steps, "warmup", args.warmup, "sets", args.sets)
    main_res = run_config(torch, B, I, 4, 32, args.steps, args.warmup, args.sets, "fused")
    log("bench: main (one-call a2av)", json.dumps(main_res))
    three = run_config(torch, B, I, 4, 32, args.steps, args.warmup, args.sets, "3call")
    log("bench: main (three calls)", json.dumps(three))

    headline = {}
    if not args.no_headline:
        for W, mib, steps, nsets in ((4, 32, 200, 8), (8, 32, 200, 8), (4, 1024, 20, 2),
                                     (8, 1024, 10, 2), (16, 32, 50, 8), (64, 32, 20, 2)):
            for entry in ("fused", "3call"):
                r = run_config(torch, B, I, W, mib, steps, 5, nsets, entry)
                key = f"w{W}_{mib}mib" + ("" if entry == "fused" else "_3call")
                headline[key] = {
                    "kernel_gbs": round(r["kernel_gbs"], 1),
                    "kernel_frac": round(r["kernel_gbs"] / HBM_PEAK_GBS, 4),
                    "step_gbs": round(r["step_gbs"], 1),
                    "step_frac": round(r["step_gbs"] / HBM_PEAK_GBS, 4),
                    "kernel_us": round(r["kernel_ms_mean"] * 1e3, 2),
                    "step_us": round(r["step_ms"] * 1e3, 2)}
                if "per_launch_us" in r:
                    headline[key]["per_launch_us"] = r["per_launch_us"]
                if "two_fills_then_copy_ms" in r:
                    headline[key]["two_fills_then_copy_us"] = round(
                        r["two_fills_then_copy_ms"] * 1e3, 2)
                log("bench: headline", key, json.dumps(headline[key]))
    sweep = {}
    if not args.no_sweep:
        for splits in ("uniform", "half_zero"):
            for mib in [1 << i for i in range(13)]:
                per_step = 2 * 4 * mib << 20
                nsets = max(1, min(8, (2 << 30) // per_step))
                steps = max(5, min(200, (8 << 30) // per_step))
                r = run_config(torch, B, I, 4, mib, steps, 3, nsets, "fused", splits)
                sweep[f"{splits}_{mib}mib"] = {"kernel_gbs": round(r["kernel_gbs"], 1),
                                               "kernel_us": round(r["kernel_ms_mean"] * 1e3, 2),
                                               "frac": round(r["kernel_gbs"] / HBM_PEAK_GBS, 4),
                                               "steps": steps}
                log("bench: sweep", splits, mib, json.dumps(sweep[f"{splits}_{mib}mib"]))
    ceil = ceilings(torch, B, int(main_res["bytes_per_step"]))
    ceil["naive_w2_memcpy_gbs"] = naive_per_chunk(torch, I)
    log("bench: ceilings", json.dumps(ceil))

    rows = {}
    if not args.no_rows:
        rows = row_benchmarks(torch, B, I, with_cpu=not args.no_cpu, ceil=ceil)
        log("bench: rows", json.dumps(rows))

    cpu = None if args.no_cpu else cpu_baseline(torch, I)
    if cpu:
        log("bench: cpu", json.dumps(cpu))

    per_launch = main_res["bytes_per_step"]
    achieved = gbps(per_launch, main_res["kernel_ms_mean"] / 1e3)
    line = {
        "metric": "a2av effective HBM GB/s @32 MiB & 1 GiB per rank, W=4/8; % of HBM peak",
        "value": round(main_res["step_gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_res["step_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # the path copies the payload bit for bit and computes only int64
        # offsets: its arithmetic is on bytes; the payload itself is bf16
        "dtype": "u8",
        "data": "synthetic",
        "config": {"workload": "a2av W=4 virtual ranks x 32 MiB/rank (4096 rows x 4096 bf16), "
                               "uniform multinomial splits; step = splits exchange + offsets + "
                               "copy in one a2av_all_to_all_vdev call",
                   "W": 4, "rows_per_rank": 4096, "row_bytes": 8192, "payload": "bf16",
                   "rotating_sets": args.sets,
                   "frac_of_hbm_peak": round(main_res["step_gbs"] / HBM_PEAK_GBS, 4),
                   "timing": "HIP events on the launch stream around the K steps, inside the "
                             "synchronized region",
                   "host_clock_gbs": round(main_res["host_step_gbs"], 1),
                   "host_clock_ms_per_step": round(main_res["host_step_ms"], 5),
                   "three_call_step_gbs": round(three["step_gbs"], 1),
                   "three_call_copy_kernel_gbs": round(three["kernel_gbs"], 1),
                   "three_call_copy_kernel_frac": round(three["kernel_gbs"] / HBM_PEAK_GBS, 4),
                   "three_call_step_us": round(three["step_ms"] * 1e3, 2),
                   "two_fills_then_copy_us": round(three["two_fills_then_copy_ms"] * 1e3, 2),
                   "per_launch_us": main_res.get("per_launch_us")},
        "roofline": {"bound": "hbm", "kernel": "k_a2av_wave (one launch: exchange+offsets+copy)",
                     "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_entry(per_launch),
                     "algorithmic_bytes_per_launch": int(per_launch),
                     "avg_launch_us": round(main_res["kernel_ms_mean"] * 1e3, 3)},
        "cpu_baseline": cpu,
        "headline": headline,
        "sweep": sweep or None,
        "rows": rows,
        "ceilings": {k: round(v, 1) for k, v in ceil.items()},
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
