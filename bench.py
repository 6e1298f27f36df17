#!/usr/bin/env python3
"""Benchmark of the device-split all-to-all-v on one MI355X.

One step = the whole a2av on W virtual ranks held in one GPU's HBM: splits
exchange -> offsets -> payload copy, three C-ABI calls on one stream. The
default workload is W=4 ranks x 32 MiB (4096 rows x 4096 bf16, 8 KiB rows)
with multinomial splits, the message size of the MoE region on the tuning
page. The printed value is effective HBM throughput: payload bytes read plus
bytes written (2 x row bytes x rows moved) per second of wall clock over the
timed steps, inputs resident in HBM.

Several independent buffer sets are cycled so that no step finds its inputs
in the 256 MB Infinity Cache left behind by the step before.

Also reported on the same JSON line:
  roofline      payload kernel alone, timed with HIP events on its stream,
                against the 8 TB/s HBM peak; `traffic` is the HBM byte count
                from rocprofv3 counters when they were taken on this exact
                kernel source (else null)
  cpu_baseline  the CPU oracle on the same workload on this host
  headline      W in {4, 8} x {32 MiB, 1 GiB} per rank, payload kernel and step
  ceilings      plain device copy of the same bytes (this library's copy loop
                and torch's D2D copy)
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
                  for f in ("a2av.hip", "common.hpp")]


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

    def __init__(self, torch, B, I, W, rows, cols, seed, stream_handle):
        from embeddings_a2av_virtual_amd.vranks import A2av
        self.W, self.rows, self.R = W, rows, cols * 2
        g = I.rng(seed)
        self.S_host = I.uniform_splits(g, W, rows)
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


def run_config(torch, B, I, W, mib, steps, warmup, nsets, entry="fused"):
    """Time `steps` whole a2av steps over `nsets` rotating buffer sets.

    entry="fused": one a2av_all_to_all_vdev call per step (one kernel that
    exchanges, scans and copies); "3call": a2av_exchange_splits, a2av_offsets,
    a2av_copy.

    The timed region holds the steps and nothing else: a barrier-free
    synchronize, host clock, one HIP event on the launch stream, the steps,
    one more event, synchronize. Step throughput is payload bytes over the host
    clock; the GPU time between the two events over `steps` is the average
    launch duration (for the fused entry a step is one kernel). For the
    three-call entry a second pass records an event pair around every
    a2av_copy launch to time that kernel alone."""
    L = B.lib()
    stream = torch.cuda.current_stream()
    hs = stream.cuda_stream
    cols = 4096
    rows = I.rows_for_mib(mib, cols * 2)
    sets = [VSet(torch, B, I, W, rows, cols, seed=100 + 17 * W + mib + s, stream_handle=hs)
            for s in range(nsets)]
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
        "step_ms": wall / steps * 1e3,
        "step_gbs": gbps(sum(moved), wall),
        "gpu_step_ms": gpu_ms / steps,
        "gpu_step_gbs": gbps(sum(moved), gpu_ms / 1e3),
    }
    if entry == "fused":
        res["kernel_ms_mean"] = gpu_ms / steps
        res["kernel_gbs"] = res["gpu_step_gbs"]
    else:
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        torch.cuda.synchronize()
        for i in range(steps):
            step(sets[i % nsets], evs[i])
        torch.cuda.synchronize()
        copy_ms = [evs[i][0].elapsed_time(evs[i][1]) for i in range(steps)]
        res["kernel_ms_mean"] = statistics.mean(copy_ms)
        res["kernel_gbs"] = gbps(sum(moved), sum(copy_ms) / 1e3)
    for vs in sets:
        st = int(vs.st.status.item())
        if st != 0:
            raise RuntimeError(f"status word {st}: {B.a2av_strerror(st)}")
    del sets
    torch.cuda.empty_cache()
    return res


def ceilings(torch, B, nbytes, reps=50, nsets=8):
    """Plain contiguous copies of the same byte count (read n + write n)."""
    half = nbytes // 2
    srcs = [torch.empty(half, dtype=torch.uint8, device="cuda").fill_(i) for i in range(nsets)]
    dsts = [torch.empty(half, dtype=torch.uint8, device="cuda") for _ in range(nsets)]
    out = {}
    for name, fn in (("device_copy", lambda d, s: B.a2av_device_copy(d, s, half)),
                     ("torch_d2d", lambda d, s: d.copy_(s))):
        for i in range(5):
            fn(dsts[i % nsets], srcs[i % nsets])
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for i in range(reps):
            fn(dsts[i % nsets], srcs[i % nsets])
        b.record()
        torch.cuda.synchronize()
        out[name + "_gbs"] = gbps(2 * half * reps, a.elapsed_time(b) / 1e3)
    del srcs, dsts
    torch.cuda.empty_cache()
    return out


def cpu_baseline(torch, I, W=4, mib=32, budget_s=10.0):
    """The CPU oracle on one full set of the workload, repeated for about
    budget_s seconds (at least 3 runs); single-threaded C."""
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
    t_start = time.perf_counter()
    while len(times) < 3 or (time.perf_counter() - t_start < budget_s and len(times) < 500):
        t0 = time.perf_counter()
        st = o.a2av(R, X, in_rows, Y, cap, S)[0]
        times.append(time.perf_counter() - t0)
        assert st == 0
    moved = 2 * R * int(S.sum())
    med = statistics.median(times)
    return {"value": round(gbps(moved, med), 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"whole W={W} x {mib} MiB/rank a2av (exchange+offsets+copy), "
                      f"{len(times)} runs, median {med * 1e3:.1f} ms"}


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


def fused_args(st, R, ins, in_rows, outs, caps):
    """Pre-marshalled argument tuple of one a2av_all_to_all_vdev call, so that
    timing a small exchange measures the GPU rather than Python."""
    import torch
    W = len(ins)
    vp = ctypes.c_void_p
    a_in = (ctypes.c_void_p * W)(*[t.data_ptr() for t in ins])
    a_out = (ctypes.c_void_p * W)(*[t.data_ptr() for t in outs])
    a_rows = (ctypes.c_int64 * W)(*[int(x) for x in in_rows])
    a_caps = (ctypes.c_int64 * W)(*[int(x) for x in caps])
    hs = vp(torch.cuda.current_stream().cuda_stream)
    return (W, R, a_in, a_rows, a_out, a_caps, vp(st.S.data_ptr()), vp(st.O.data_ptr()),
            vp(st.send_off.data_ptr()), vp(st.recv_off.data_ptr()), vp(st.status.data_ptr()), hs)


def row_entry(nbytes, ms, cpu_bytes=None, cpu_s=None, note=""):
    gbs = gbps(nbytes, ms / 1e3)
    e = {"bytes": int(nbytes), "us": round(ms * 1e3, 2), "gbs": round(gbs, 1),
         "frac": round(gbs / HBM_PEAK_GBS, 4)}
    if cpu_bytes is not None:
        e["oracle_gbs"] = round(gbps(cpu_bytes, cpu_s), 3)
        e["oracle_sample"] = note
    return e


def row_benchmarks(torch, B, I, with_cpu=True):
    """The other steps of the path, each at its full size: the MoE dispatch
    pack, the dispatch and return a2av, the un-pack, and the embedding-key
    exchange (keys and lengths). GB/s counts algorithmic bytes (payload read
    + written, index bytes for the pack and un-pack)."""
    import numpy as np
    sys.path.insert(0, ROOT)
    from embeddings_a2av_virtual_amd.vranks import A2av
    out = {}
    o = None
    if with_cpu:
        from oracle.ref import Oracle
        o = Oracle()
    # ---- MoE dispatch: W=8, 8192 tokens x 7168 bf16, top-8 of 256 Zipf(1.1) experts
    W, T, k, E, hidden = 8, 8192, 8, 256, 7168
    R, Q = hidden * 2, T * k
    g = I.rng(900)
    ids_h = [I.topk_ids(g, T, k, E, 1.1) for _ in range(W)]
    tok = [I.payload_bf16(T, hidden, 9000 + r, device="cuda") for r in range(W)]
    ids = [torch.from_numpy(i.reshape(-1)).cuda() for i in ids_h]
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
    del send
    bk = A2av(W)
    bk.S.copy_(fwd.O)
    back = [torch.empty((Q, hidden), dtype=torch.bfloat16, device="cuda") for _ in range(W)]
    ret = lambda: bk(R, recv, cap, back, [Q] * W, fused=True)
    ms = time_events(torch, ret, 5)
    out["return_a2av"] = row_entry(moved, ms)
    del recv
    outb = [torch.empty((Q, hidden), dtype=torch.bfloat16, device="cuda") for _ in range(W)]
    ust = torch.zeros(1, dtype=torch.int32, device="cuda")
    unpack = lambda: B.moe_unpack(W, T, k, R, back, perm, outb, ust)
    ms = time_events(torch, unpack, 5)
    out["moe_unpack"] = row_entry(W * (2 * Q * R + 8 * Q), ms)
    torch.cuda.synchronize()
    for name, st in (("pack", status), ("dispatch", fwd.status), ("return", bk.status),
                     ("unpack", ust)):
        if int(st.item()) != 0:
            raise RuntimeError(f"{name} status {int(st.item())}")
    del back, outb, tok, perm
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
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} requested, but this build runs on ONE GPU: the "
              "W ranks are virtual (partitions of one GPU's HBM) and there is no multi-GPU "
              "path; run with --gpus 1.", file=sys.stderr)
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
                                     (8, 1024, 10, 2)):
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
                log("bench: headline", key, json.dumps(headline[key]))
    ceil = ceilings(torch, B, int(main_res["bytes_per_step"]))
    log("bench: ceilings", json.dumps(ceil))

    rows = {}
    if not args.no_rows:
        rows = row_benchmarks(torch, B, I, with_cpu=not args.no_cpu)
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
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "a2av W=4 virtual ranks x 32 MiB/rank (4096 rows x 4096 bf16), "
                               "uniform multinomial splits; step = splits exchange + offsets + "
                               "copy in one a2av_all_to_all_vdev call",
                   "W": 4, "rows_per_rank": 4096, "row_bytes": 8192,
                   "rotating_sets": args.sets,
                   "frac_of_hbm_peak": round(main_res["step_gbs"] / HBM_PEAK_GBS, 4),
                   "three_call_step_gbs": round(three["step_gbs"], 1),
                   "three_call_copy_kernel_gbs": round(three["kernel_gbs"], 1),
                   "three_call_copy_kernel_frac": round(three["kernel_gbs"] / HBM_PEAK_GBS, 4)},
        "roofline": {"bound": "hbm", "kernel": "k_a2av_wave (one launch: exchange+offsets+copy)",
                     "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_entry(per_launch),
                     "algorithmic_bytes_per_launch": int(per_launch),
                     "avg_launch_us": round(main_res["kernel_ms_mean"] * 1e3, 3)},
        "cpu_baseline": cpu,
        "headline": headline,
        "rows": rows,
        "ceilings": {k: round(v, 1) for k, v in ceil.items()},
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
