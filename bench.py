#!/usr/bin/env python3
"""Throughput of the collective primitives on one MI355X.

The timed step is the ZeRO-style gradient path: ReduceScatter (sum) of
p = 8 logical ranks' 2^26-element bf16 gradients (fp32 accumulation),
then AllGather of the 2^23-element shards back to every rank.  All p
ranks' buffers are resident in the one GPU's HBM, so HBM bandwidth plays
the part of the network.  The JSON line reports

* value: achieved HBM GB/s of the whole step (algorithmic bytes: every
  input element read once, every output element written once, self
  copies included), with busbw/algbw per collective after the bus
  bandwidth conventions of "集合通信：原语、算法、NCCL 实现与拓扑映射"
  (hpc/04, section 2.5), and each kernel's time also cold (after a
  512 MiB overwrite that evicts the Infinity Cache);
* roofline: the dominant kernel's algorithmic bytes per launch over its
  mean duration (HIP events on the launch stream) against 8 TB/s, plus
  the HBM traffic read from rocprofv3 FETCH_SIZE / WRITE_SIZE counters
  when a counter summary for the current kernel sources is on file;
* cpu_baseline: the threaded C++ oracle on the whole step (all host
  threads, and one thread), checked against the GPU output;
* collectives: the other p = 8 collectives (AllReduce in four
  schedules, All-to-All, Alltoallv, the MoE pack -> exchange -> reverse
  exchange -> combine path, Gather, Scatter), the small
  AllReduce at p = 4, the 10,000-call batched AllReduce at p = 16 (also
  as individual calls, with latency percentiles and an alpha-beta fit)
  and the device copy ceiling, each timed with HIP events.  Every row
  carries the attainable ceiling of its read:write stream mix, measured in
  the same run with the library's direction-mix probe (coll_stream_probe:
  the collectives' own tile code), and its fraction of that ceiling.

The JSON line on stdout is a compact summary; the full per-collective
tables go to stderr as "# detail" lines.

Only one GPU is used; --gpus above 1 is refused.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "busbw and achieved HBM GB/s (% of peak) per collective at p=8, 1 GPU"
HBM_PEAK = 8000.0  # GB/s, MI355X HBM3E published peak
PROFILES = os.path.join(ROOT, "profiles")
NO_GRAPHS = False   # set by --no-graphs
CSRC = os.path.join(ROOT, "collective_communication_primitives_coll_amd", "csrc")


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--no-collectives", action="store_true", help="time only the main step")
    ap.add_argument("--only", default=None,
                    help="comma list of extra collectives to time (ar_ring, ar_onepass, ar_hd, "
                         "ar_tree, ar_dbt, ar_literal, ar_avg, ar_premul, a2a, a2av, moe, moe_fp8, moe_direct, moe_fp8_direct, "
                         "gs, ar_small, ar_latency, anyp, batch, copy, ce)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU oracle time budget (all threads)")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the direction-mix ceilings")
    ap.add_argument("--no-graphs", action="store_true", help="skip the HIP-graph replays (for counter runs)")
    return ap.parse_args(argv)


# Sources each timed kernel is built from (its launch code included).
KERNEL_SOURCES = {
    "reduce_scatter": ["coll_api.cpp", "kernel_args.h", "device_common.h", "reduce_tile.h", "reduce_kernels.hip"],
    "allgather": ["coll_api.cpp", "kernel_args.h", "device_common.h", "copy_tile.h", "copy_kernels.hip"],
    "alltoall": ["coll_api.cpp", "kernel_args.h", "device_common.h", "copy_tile.h", "copy_kernels.hip"],
    "alltoall_lds": ["coll_api.cpp", "kernel_args.h", "device_common.h", "copy_tile.h", "a2a_lds_kernels.hip"],
    "alltoallv": ["coll_api.cpp", "kernel_args.h", "device_common.h", "copy_tile.h", "copy_kernels.hip"],
    "allreduce": ["coll_api.cpp", "kernel_args.h", "device_common.h", "reduce_tile.h", "reduce_kernels.hip"],
    "allreduce_small": ["coll_api.cpp", "kernel_args.h", "device_common.h", "reduce_tile.h", "reduce_kernels.hip"],
    "gather_scatter": ["coll_api.cpp", "kernel_args.h", "device_common.h", "copy_tile.h", "copy_kernels.hip"],
    "moe": ["coll_api.cpp", "kernel_args.h", "device_common.h", "copy_tile.h", "moe_direct.h", "moe_kernels.hip"],
    "fp8": ["coll_api.cpp", "kernel_args.h", "device_common.h", "moe_direct.h", "moe_kernels.hip", "fp8_kernels.hip"],
    "batch": ["coll_api.cpp", "kernel_args.h", "device_common.h", "reduce_tile.h", "batch_kernels.hip"],
}


def source_hash(kernel: str | None = None) -> str:
    """SHA-256 over the sources of one timed kernel (all HIP/C++ sources if
    kernel is None): identifies the code a counter summary was taken on."""
    names = KERNEL_SOURCES[kernel] if kernel else sorted(
        n for n in os.listdir(CSRC) if n.endswith((".hip", ".h", ".cpp")))
    h = hashlib.sha256()
    for name in names:
        h.update(name.encode())
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ----------------------------------------------------------------------------
# Device plumbing
# ----------------------------------------------------------------------------

def to_dev(torch, a: np.ndarray, dev):
    if a.dtype == np.uint16:   # bf16 bit patterns
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def to_host_bits(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.cpu().numpy().view(np.uint32)
    return t.cpu().numpy()


def time_launches(torch, fns, iters: int, warmup: int):
    """Run the launch sequence fns warmup + iters times; per fn, the list of
    durations (ms) between HIP events recorded on the launch stream."""
    for _ in range(warmup):
        for f in fns:
            f()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(iters)]
    for i in range(iters):
        ev[i][0].record()
        for k, f in enumerate(fns):
            f()
            ev[i][k + 1].record()
    torch.cuda.synchronize()
    return [[ev[i][k].elapsed_time(ev[i][k + 1]) for i in range(iters)] for k in range(len(fns))]


def stats_us(ms_list):
    a = np.asarray(ms_list, dtype=np.float64) * 1e3
    return float(np.median(a)), float(np.percentile(a, 95)), float(a.mean())


# Probe options swept for each mix: cached or non-temporal loads (1); plain,
# non-temporal (2), device-scope (8) or non-temporal device-scope (2 | 8)
# stores; tiles dealt out or claimed (4).
PROBE_FLAGS = list(range(16))


class Ceilings:
    """Attainable HBM GB/s of a read:write stream mix, measured in this run
    with the library's direction-mix probe (coll_stream_probe: the
    collectives' 16-byte tiles, launch bounds and grid sizing): ns source and
    nd destination streams of stream_bytes each, best over tiles of 1, 2, 4
    and 8 vectors per lane, the cache policies (cached or non-temporal
    loads; plain, non-temporal, device-scope or non-temporal device-scope
    stores), tiles all dealt out
    in turn or three quarters claimed
    (as the large collectives balance their workgroups), and one, two or
    four workgroups per CU.  Results are cached per (ns, nd, stream_bytes)."""

    def __init__(self, torch, coll, dev, enabled=True):
        self.torch, self.coll, self.dev, self.enabled = torch, coll, dev, enabled
        self.cache = {}

    def get(self, ns: int, nd: int, stream_bytes: int):
        if not self.enabled:
            return None
        key = (ns, nd, int(stream_bytes))
        if key in self.cache:
            return self.cache[key]
        torch, coll = self.torch, self.coll
        words = stream_bytes // 4
        src = [torch.empty(words, dtype=torch.int32, device=self.dev) for _ in range(ns)]
        for i, t in enumerate(src):
            t.fill_(i + 1)
        dst = [torch.empty(words, dtype=torch.int32, device=self.dev) for _ in range(nd)]
        sink = torch.zeros(4, dtype=torch.int32, device=self.dev)
        best = None
        try:
            for w in (1, 2, 4):
                coll.coll_set_grid_limit(w)
                for unroll in (1, 2, 4, 8):
                    if ns * unroll > 32:
                        continue
                    for flags in PROBE_FLAGS:
                        f = coll.coll_stream_probe(src, dst, stream_bytes, unroll, flags, sink, defer=True)
                        med = stats_us(time_launches(torch, [f], 4, 1)[0])[0]
                        gbps = (ns + nd) * stream_bytes / (med * 1e-6) / 1e9
                        if best is None or gbps > best[0]:
                            best = (gbps, w, flags, unroll)
        finally:
            coll.coll_set_grid_limit(0)
        del src, dst
        torch.cuda.empty_cache()
        res = {"GBps": round(best[0], 1), "mix": f"{ns}r:{nd}w x {stream_bytes >> 20} MiB",
               "wg_per_cu": best[1], "unroll": best[3], "nt_loads": bool(best[2] & 1),
               "stores": {0: "plain", 2: "non-temporal", 8: "device scope", 10: "non-temporal device scope"}[best[2] & 10],
               "claimed": bool(best[2] & 4)}
        self.cache[key] = res
        return res

    def attach(self, row: dict, ns: int, nd: int, stream_bytes: int, gbps_key: str = "hbm_GBps") -> dict:
        """Add the mix ceiling and the row's fraction of it to row."""
        c = self.get(ns, nd, stream_bytes)
        if c is not None and row.get(gbps_key):
            row["mix"] = c["mix"]
            row["mix_ceiling_GBps"] = c["GBps"]
            row["frac_of_mix_ceiling"] = round(row[gbps_key] / c["GBps"], 4)
        return row


def coll_entry(metrics, name, coll_kind, p, n, d, t_us, algo="ring", extra=None):
    """One row of the per-collective table from a median time."""
    s = t_us * 1e-6
    hbm = metrics.hbm_bytes(coll_kind, p, n, d, algo)
    row = {
        "name": name, "p": p, "n": n, "elem_bytes": d,
        "t_med_us": round(t_us, 2),
        "algbw_GBps": round(metrics.algbw_gbps(coll_kind, p, n, d, s), 1),
        "busbw_GBps": round(metrics.busbw_gbps(coll_kind, p, n, d, s), 1),
        "hbm_bytes": hbm,
        "hbm_GBps": round(hbm / s / 1e9, 1),
        "pct_hbm_peak": round(100.0 * hbm / s / 1e9 / HBM_PEAK, 1),
    }
    if extra:
        row.update(extra)
    return row


# ----------------------------------------------------------------------------
# Counter summary (rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE), if on file
# ----------------------------------------------------------------------------

def read_traffic(kernel_key: str, launches_bytes: int):
    """HBM bytes per launch of kernel_key from profiles/hbm_traffic_*.txt.

    The file holds `source_hash_<key>:`, `copy_fetch_factor:`,
    `copy_write_factor:` and per-kernel `kernel <key> fetch_kib <F>
    write_kib <W>` lines; the factors scale the raw counters by what they
    read for a plain copy of known size.  Returns None when no summary
    matches the kernel's current sources.
    """
    if not os.path.isdir(PROFILES):
        return None
    cur = source_hash(kernel_key)
    for name in sorted(os.listdir(PROFILES)):
        if not (name.startswith("hbm_traffic_") and name.endswith(".txt")):
            continue
        kv, kern = {}, {}
        with open(os.path.join(PROFILES, name), encoding="utf-8") as f:
            for line in f:
                line = line.strip()
                m = re.match(r"^kernel\s+(\S+)\s+fetch_kib\s+([\d.]+)\s+write_kib\s+([\d.]+)", line)
                if m:
                    kern[m.group(1)] = (float(m.group(2)), float(m.group(3)))
                    continue
                m = re.match(r"^([a-z_]+):\s*(\S+)", line)
                if m:
                    kv[m.group(1)] = m.group(2)
        if kv.get("source_hash_" + kernel_key) != cur or kernel_key not in kern:
            continue
        ff = float(kv.get("copy_fetch_factor", "1"))
        wf = float(kv.get("copy_write_factor", "1"))
        fk, wk = kern[kernel_key]
        return int(round(fk * 1024 * ff + wk * 1024 * wf))
    return None


# ----------------------------------------------------------------------------
# Workloads
# ----------------------------------------------------------------------------

def zero_workload(torch, coll, inputs, dev):
    """ReduceScatter then AllGather, p = 8, 2^26 bf16 per rank ~ N(0, 1e-3)."""
    p, total = 8, 1 << 26
    n = total // p
    hx = inputs.rank_buffers(inputs.WL_ZERO_RS_AG, p, total, inputs.BF16, dist="normal", sigma=1e-3)
    send = [to_dev(torch, x, dev) for x in hx]
    shard = [torch.empty(n, dtype=torch.bfloat16, device=dev) for _ in range(p)]
    full = [torch.empty(total, dtype=torch.bfloat16, device=dev) for _ in range(p)]
    rs = coll.coll_reduce_scatter(send, shard, coll.COLL_SUM, defer=True)
    ag = coll.coll_allgather(shard, full, defer=True)
    return dict(p=p, n=n, total=total, hx=hx, send=send, shard=shard, full=full, rs=rs, ag=ag)


def cpu_baseline(torch, wl, cpu_seconds: float):
    """The threaded C++ oracle (oracle/oracle.cpp, as it stands) on the whole
    timed step: ReduceScatter of the full p = 8, 2^26-element bf16 inputs,
    then AllGather of the shards.  Timed with every host thread (repeated
    for about cpu_seconds) and with one thread (once); its result is
    compared with the GPU's whole output."""
    from oracle import native
    from collective_communication_primitives_coll_amd import metrics

    p, n, hx = wl["p"], wl["n"], wl["hx"]
    nt = native.hardware_threads()

    def step(threads):
        shards = native.reduce_scatter(hx, native.SUM, native.BF16, nthreads=threads)
        return shards, native.allgather(shards, nthreads=threads)

    reps, t0 = 0, time.perf_counter()
    while True:
        shards, gathered = step(nt)
        reps += 1
        el = time.perf_counter() - t0
        if el >= cpu_seconds:
            break
    per_all = el / reps
    t1 = time.perf_counter()
    step(1)
    per_one = time.perf_counter() - t1
    alg = metrics.hbm_bytes("reduce_scatter", p, n, 2) + metrics.hbm_bytes("allgather", p, n, 2)

    def same(t, a):
        e = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(t.device)
        return bool(torch.equal(t.view(torch.int16), e))
    agree = all(same(wl["shard"][r], shards[r]) for r in range(p)) and \
        all(same(wl["full"][r], gathered[r]) for r in range(p))
    return {
        "value": round(alg / per_all / 1e9, 3),
        "unit": "GB/s",
        "cores": nt,
        "kind": "oracle",
        "sample": (f"the whole step: oracle/oracle.cpp ReduceScatter + AllGather of the full p=8, 2^26 bf16 "
                   f"per rank inputs, {nt} threads, {reps} repetitions in {el:.1f} s; GB/s of the step's "
                   f"algorithmic HBM bytes"),
        "ms_per_step": round(per_all * 1e3, 1),
        "value_1_thread": round(alg / per_one / 1e9, 3),
        "ms_per_step_1_thread": round(per_one * 1e3, 1),
        "host_cpus": os.cpu_count(),
        "cpu_model": host_cpu_model(),
        "gpu_matches_oracle_whole_step": agree,
    }


def host_cpu_model() -> str | None:
    """The host CPU's model name from /proc/cpuinfo (None if unreadable)."""
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def graph_us_per_call(torch, coll, send, recv, algo, calls=10, replays=20, op=None):
    """Device time per AllReduce call without host overhead: `calls` calls
    captured back to back in one HIP graph, replayed `replays` times."""
    op = coll.COLL_SUM if op is None else op
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm-up off the capture
        coll.coll_allreduce_algo(send, recv, algo, op)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            coll.coll_allreduce_algo(send, recv, algo, op)
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(replays):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / (calls * replays)


def extra_collectives(torch, coll, inputs, metrics, dev, which, ceil, iters=10, warmup=3):
    rows = []
    MiB = 1 << 20
    want = lambda k: which is None or k in which  # noqa: E731

    # --- DP gradient AllReduce, p = 8, 256 MiB fp32 per rank ~ N(0, 1) -------
    if any(want(k) for k in ("ar_ring", "ar_onepass", "ar_hd", "ar_tree", "ar_dbt", "ar_literal", "ar_avg",
                             "ar_premul")):
        p, n = 8, 1 << 26
        send = [to_dev(torch, x, dev) for x in inputs.rank_buffers(inputs.WL_DP_RING_AR, p, n, inputs.F32,
                                                                    dist="normal")]
        recv = [torch.empty(n, dtype=torch.float32, device=dev) for _ in range(p)]
        for key, algo, label, aname in (
                ("ar_ring", coll.COLL_ALGO_RING, "allreduce_ring_fused", "ring"),
                ("ar_onepass", coll.COLL_ALGO_RECURSIVE_DOUBLING, "allreduce_recursive_doubling_order", "ring"),
                ("ar_hd", coll.COLL_ALGO_HALVING_DOUBLING, "allreduce_halving_doubling_order", "ring"),
                ("ar_tree", coll.COLL_ALGO_TREE, "allreduce_tree_order", "ring"),
                ("ar_dbt", coll.COLL_ALGO_DOUBLE_BINARY_TREE, "allreduce_double_binary_tree_order", "ring"),
                ("ar_literal", coll.COLL_ALGO_RING_LITERAL, "allreduce_ring_literal_14_steps",
                 "ring_literal")):
            if not want(key):
                continue
            f = coll.coll_allreduce_algo(send, recv, algo, coll.COLL_SUM, defer=True)
            med, p95, _ = stats_us(time_launches(torch, [f], iters, warmup)[0])
            row = coll_entry(metrics, label, "allreduce", p, n, 4, med, aname,
                             {"dtype": "f32", "op": "sum", "t_p95_us": round(p95, 2),
                              "workload": "DP gradient AllReduce, 256 MiB fp32 per rank"})
            if aname == "ring":
                ceil.attach(row, p, p, n * 4)
            rows.append(row)
        # Scaled variants on the same buffers: AVG (sum then one division by
        # p) and PreMulSum with per-rank weights w_r = 1/p.
        if want("ar_avg"):
            f = coll.coll_allreduce_algo(send, recv, coll.COLL_ALGO_RING, coll.COLL_AVG, defer=True)
            med, p95, _ = stats_us(time_launches(torch, [f], iters, warmup)[0])
            rows.append(ceil.attach(coll_entry(metrics, "allreduce_avg_ring", "allreduce", p, n, 4, med, "ring",
                                               {"dtype": "f32", "op": "avg", "t_p95_us": round(p95, 2),
                                                "workload": "DP gradient AllReduce, 256 MiB fp32 per rank"}),
                                    p, p, n * 4))
        if want("ar_premul"):
            scales = np.full(p, 1.0 / p, dtype=np.float32)
            f = coll.coll_allreduce_premul(send, recv, scales, coll.COLL_ALGO_RING, defer=True)
            med, p95, _ = stats_us(time_launches(torch, [f], iters, warmup)[0])
            rows.append(ceil.attach(coll_entry(metrics, "allreduce_premulsum_ring", "allreduce", p, n, 4, med,
                                               "ring", {"dtype": "f32", "op": "premulsum", "t_p95_us": round(p95, 2),
                                                        "workload": "DP gradient AllReduce, 256 MiB fp32 per rank"}),
                                    p, p, n * 4))
        del send, recv
        torch.cuda.empty_cache()

    # --- MoE dispatch All-to-All, p = 8, 4096 x 7168 bf16 per rank ----------
    if want("a2a") or want("a2av"):
        p, tokens, hidden = 8, 4096, 7168
        per = tokens * hidden
        send = [to_dev(torch, x, dev) for x in inputs.rank_buffers(inputs.WL_MOE_A2A, p, per, inputs.BF16,
                                                                    dist="normal")]
        if want("a2a"):
            recv = [torch.empty(per, dtype=torch.bfloat16, device=dev) for _ in range(p)]
            f = coll.coll_alltoall(send, recv, per // p, defer=True)
            med, p95, _ = stats_us(time_launches(torch, [f], iters, warmup)[0])
            rows.append(ceil.attach(coll_entry(metrics, "alltoall_equal", "alltoall", p, per // p, 2, med, "ring",
                                               {"dtype": "bf16", "t_p95_us": round(p95, 2),
                                                "workload": "MoE dispatch, 512 tokens x 7168 per destination"}),
                                    1, 1, p * per * 2))
            # the same transpose with every vector staged in LDS (gfx950
            # global-to-LDS loads), timed on the same buffers
            f = coll.coll_alltoall_algo(send, recv, coll.COLL_A2A_LDS_STAGED, per // p, defer=True)
            med, p95, _ = stats_us(time_launches(torch, [f], iters, warmup)[0])
            rows.append(ceil.attach(coll_entry(metrics, "alltoall_equal_lds_staged", "alltoall", p, per // p, 2, med,
                                               "ring", {"dtype": "bf16", "t_p95_us": round(p95, 2),
                                                        "workload": "MoE dispatch, 512 tokens x 7168 per destination"}),
                                    1, 1, p * per * 2))
            del recv
        if want("a2av"):
            ctok = inputs.moe_token_counts(p, tokens)
            counts = ctok * hidden
            cols = counts.sum(axis=0)
            recv = [torch.empty(int(c), dtype=torch.bfloat16, device=dev) for c in cols]
            cdev = torch.from_numpy(counts.reshape(-1).copy()).to(dev)
            f = coll.coll_alltoallv(send, recv, cdev, defer=True)
            med, p95, _ = stats_us(time_launches(torch, [f], iters, warmup)[0])
            hbm = int(2 * counts.sum() * 2)
            s = med * 1e-6
            b_local = per * 2
            rows.append({
                "name": "alltoallv_multinomial", "p": p, "elem_bytes": 2, "dtype": "bf16",
                "t_med_us": round(med, 2), "t_p95_us": round(p95, 2),
                "algbw_GBps": round(b_local / s / 1e9, 1),
                "busbw_GBps": round(b_local / s / 1e9 * metrics.busbw_factor("alltoallv", p), 1),
                "hbm_bytes": hbm, "hbm_GBps": round(hbm / s / 1e9, 1),
                "pct_hbm_peak": round(100.0 * hbm / s / 1e9 / HBM_PEAK, 1),
                "max_row_tokens": int(ctok.sum(axis=1).max()), "max_col_tokens": int(ctok.sum(axis=0).max()),
                "zero_ratio": float((ctok == 0).mean()),
                "workload": "MoE dispatch, per-source token counts ~ Multinomial(4096, 1/8)",
            })
            ceil.attach(rows[-1], 1, 1, p * per * 2)
            del recv, cdev
        del send
        torch.cuda.empty_cache()

    # --- MoE dispatch and combine around the ragged exchange -----------------
    if want("moe"):
        rows.append(moe_row(torch, coll, inputs, dev, iters, warmup, ceil))
        torch.cuda.empty_cache()
    if want("moe_fp8"):
        rows.append(moe_fp8_row(torch, coll, inputs, dev, iters, warmup, ceil))
        torch.cuda.empty_cache()
    if want("moe_direct"):
        rows.append(moe_direct_row(torch, coll, inputs, dev, iters, warmup, ceil, fp8=False))
        torch.cuda.empty_cache()
    if want("moe_fp8_direct"):
        rows.append(moe_direct_row(torch, coll, inputs, dev, iters, warmup, ceil, fp8=True))
        torch.cuda.empty_cache()

    # --- Gather / Scatter, p = 8, 2^23 bf16 per rank (root buffer 128 MiB) ----
    if want("gs"):
        p, n = 8, 1 << 23
        ranks = [torch.empty(n, dtype=torch.bfloat16, device=dev).normal_() for _ in range(p)]
        root_buf = torch.empty(p * n, dtype=torch.bfloat16, device=dev)
        fg = coll.coll_gather(ranks, root_buf, 0, defer=True)
        fs = coll.coll_scatter(root_buf, ranks, 0, defer=True)
        tg, ts = time_launches(torch, [fg, fs], iters, warmup)
        for name, kind, ms in (("gather", "gather", tg), ("scatter", "scatter", ts)):
            med, p95, _ = stats_us(ms)
            rows.append(ceil.attach(coll_entry(metrics, name, kind, p, n, 2, med, "ring",
                                               {"dtype": "bf16", "t_p95_us": round(p95, 2), "root": 0,
                                                "workload": "p=8, 2^23 bf16 per rank, 128 MiB root buffer"}),
                                    1, 1, p * n * 2))
        del ranks, root_buf
        torch.cuda.empty_cache()

    # --- small AllReduce, p = 4, 2^20 per rank (Infinity-Cache resident) ------
    if want("ar_small"):
        p, n = 4, 1 << 20
        # 32 MiB of buffers fit in the 256 MB Infinity Cache: back-to-back
        # calls run warm.  A 512 MiB overwrite before each call evicts them
        # (cold); events bracket only the AllReduce.
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        for dt, op, dname, oname in ((inputs.F32, coll.COLL_SUM, "f32", "sum"),
                                     (inputs.I32, coll.COLL_MIN, "i32", "min"),
                                     (inputs.I32, coll.COLL_MAX, "i32", "max")):
            send = [to_dev(torch, x, dev) for x in inputs.rank_buffers(inputs.WL_AR_SMALL, p, n, dt)]
            tdt = torch.float32 if dt == inputs.F32 else torch.int32
            recv = [torch.empty(n, dtype=tdt, device=dev) for _ in range(p)]
            f = coll.coll_allreduce(send, recv, op, defer=True)
            med, p95, _ = stats_us(time_launches(torch, [f], 50, 10)[0])
            cold = []
            for i in range(30):
                scratch.fill_(i & 0xFF)
                ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
                ev[0].record()
                f()
                ev[1].record()
                cold.append(ev)
            torch.cuda.synchronize()
            cmed, cp95, _ = stats_us([a.elapsed_time(b) for a, b in cold])
            g_us = None if NO_GRAPHS else graph_us_per_call(torch, coll, send, recv, coll.COLL_ALGO_RING, calls=20,
                                                            replays=20, op=op)
            rows.append(ceil.attach(coll_entry(
                metrics, f"allreduce_small_{oname}", "allreduce", p, n, 4, med, "ring",
                {"dtype": dname, "op": oname, "t_p95_us": round(p95, 2),
                 "t_cold_med_us": round(cmed, 2), "t_cold_p95_us": round(cp95, 2),
                 "hbm_GBps_cold": round(2 * p * n * 4 / (cmed * 1e-6) / 1e9, 1),
                 "t_graph_us": g_us and round(g_us, 2),
                 "hbm_GBps_graph": g_us and round(2 * p * n * 4 / (g_us * 1e-6) / 1e9, 1),
                 "workload": "AllReduce p=4, 2^20 per rank; t_med back to back (warm, Infinity-Cache resident), "
                             "t_cold after a 512 MiB overwrite, t_graph per call replayed from a HIP graph"}),
                p, p, n * 4))
        del scratch

    # --- latency of every schedule at the batch's small sizes, p = 16 ---------
    # The alpha-beta view of the schedules (hpc/04 page, sections 2.1 and
    # 2.6): on one device every single-pass schedule is one launch whatever
    # its hop count; the literal ring pays 2(p-1) launches.
    if want("ar_latency"):
        p = 16
        table = []
        for nbytes in (4096, 65536, 1 << 20):
            n = nbytes // 4
            send = [to_dev(torch, x, dev) for x in inputs.rank_buffers(inputs.WL_AR_SMALL, p, n, inputs.F32,
                                                                        extra=(nbytes,))]
            recv = [torch.empty(n, dtype=torch.float32, device=dev) for _ in range(p)]
            entry = {"bytes_per_rank": nbytes}
            for key, algo in (("ring", coll.COLL_ALGO_RING), ("recursive_doubling", coll.COLL_ALGO_RECURSIVE_DOUBLING),
                              ("halving_doubling", coll.COLL_ALGO_HALVING_DOUBLING), ("tree", coll.COLL_ALGO_TREE),
                              ("double_binary_tree", coll.COLL_ALGO_DOUBLE_BINARY_TREE),
                              ("ring_literal", coll.COLL_ALGO_RING_LITERAL)):
                f = coll.coll_allreduce_algo(send, recv, algo, coll.COLL_SUM, defer=True)
                med, _, _ = stats_us(time_launches(torch, [f], 50, 10)[0])
                entry[key + "_us"] = round(med, 2)
                if not NO_GRAPHS:
                    entry[key + "_graph_us"] = round(graph_us_per_call(torch, coll, send, recv, algo), 2)
            table.append(entry)
            del send, recv
        rows.append({"name": "allreduce_schedule_latency", "p": p, "dtype": "f32", "op": "sum", "table": table,
                     "workload": "AllReduce p=16, 4 KiB / 64 KiB / 1 MiB per rank, each schedule, back to back"})

    # --- rank counts that are not powers of two: AllReduce 256 MiB fp32 per
    # rank and ReduceScatter of about 2^26 fp32 per rank, p = 3, 5, 6, 7, 12 -
    if want("anyp"):
        table = []
        for p in (3, 5, 6, 7, 12):
            n = 1 << 26
            send = [torch.empty(n, dtype=torch.float32, device=dev).normal_() for _ in range(p)]
            recv = [torch.empty(n, dtype=torch.float32, device=dev) for _ in range(p)]
            f = coll.coll_allreduce(send, recv, coll.COLL_SUM, defer=True)
            ar_us = stats_us(time_launches(torch, [f], iters, warmup)[0])[0]
            del send, recv
            torch.cuda.empty_cache()
            # blocks of a whole number of 16-byte vectors (2^26 / p rounded down to a multiple of 4)
            blk = (1 << 26) // (4 * p) * 4
            send = [torch.empty(p * blk, dtype=torch.float32, device=dev).normal_() for _ in range(p)]
            shard = [torch.empty(blk, dtype=torch.float32, device=dev) for _ in range(p)]
            f = coll.coll_reduce_scatter(send, shard, coll.COLL_SUM, defer=True)
            rs_us = stats_us(time_launches(torch, [f], iters, warmup)[0])[0]
            del send, shard
            torch.cuda.empty_cache()
            ar_b = metrics.hbm_bytes("allreduce", p, n, 4)
            rs_b = metrics.hbm_bytes("reduce_scatter", p, blk, 4)
            e = {"p": p, "allreduce_us": round(ar_us, 1), "allreduce_GBps": round(ar_b / (ar_us * 1e-6) / 1e9, 1),
                 "reduce_scatter_us": round(rs_us, 1), "reduce_scatter_GBps": round(rs_b / (rs_us * 1e-6) / 1e9, 1)}
            c1, c2 = ceil.get(p, p, n * 4), ceil.get(p, 1, p * blk * 4)
            if c1 and c2:
                e["allreduce_frac_of_mix_ceiling"] = round(e["allreduce_GBps"] / c1["GBps"], 4)
                e["reduce_scatter_frac_of_mix_ceiling"] = round(e["reduce_scatter_GBps"] / c2["GBps"], 4)
            table.append(e)
        rows.append({"name": "other_rank_counts", "table": table,
                     "workload": "AllReduce sum 2^26 fp32 per rank and ReduceScatter sum of about 2^26 fp32 per "
                                 "rank (blocks of 2^26/p rounded down to whole vectors), p = 3, 5, 6, 7, 12"})

    # --- 10,000 small AllReduces in one launch, p = 16 -----------------------
    if want("batch"):
        rows.append(batch_row(torch, coll, inputs, dev, ceil))

    # --- copy ceiling ---------------------------------------------------------
    if want("copy"):
        nbytes = 1 << 30
        a = torch.empty(nbytes // 4, dtype=torch.int32, device=dev).fill_(1)
        b = torch.empty_like(a)
        med_t, _, _ = stats_us(time_launches(torch, [lambda: b.copy_(a)], iters, warmup)[0])
        f = coll.coll_broadcast(a, [b], 0, defer=True)
        med_c, _, _ = stats_us(time_launches(torch, [f], iters, warmup)[0])
        rows.append({"name": "copy_ceiling", "bytes_read": nbytes, "bytes_written": nbytes,
                     "torch_copy_GBps": round(2 * nbytes / (med_t * 1e-6) / 1e9, 1),
                     "coll_copy_kernel_GBps": round(2 * nbytes / (med_c * 1e-6) / 1e9, 1),
                     "note": "1 GiB device-to-device: torch copy_ and coll_broadcast with p=1"})
        del a, b
        torch.cuda.empty_cache()

    # --- copy-engine baseline: AllGather and All-to-All as p^2 D2D copies -------
    # The collective built from device-to-device hipMemcpyAsync calls (torch
    # copy_ on slices), one per (source, destination) block, against the
    # library's single launch on the same buffers.
    if want("ce"):
        p = 8
        n = 1 << 23
        shard = [torch.empty(n, dtype=torch.bfloat16, device=dev).normal_() for _ in range(p)]
        full = [torch.empty(p * n, dtype=torch.bfloat16, device=dev) for _ in range(p)]

        def ag_memcpy():
            for r in range(p):
                for s_ in range(p):
                    full[r][s_ * n:(s_ + 1) * n].copy_(shard[s_])
        f = coll.coll_allgather(shard, full, defer=True)
        t_ce, t_k = [stats_us(x)[0] for x in time_launches(torch, [ag_memcpy, f], iters, warmup)]
        b_ag = (p + p * p) * n * 2   # each shard read once, written p times (the copy engine reads it p times)
        rows.append({"name": "allgather_vs_copy_engine", "p": p, "elem_bytes": 2, "hbm_bytes": b_ag,
                     "memcpy_64_calls_us": round(t_ce, 2), "coll_allgather_us": round(t_k, 2),
                     "memcpy_GBps": round(b_ag / (t_ce * 1e-6) / 1e9, 1),
                     "coll_GBps": round(b_ag / (t_k * 1e-6) / 1e9, 1), "speedup": round(t_ce / t_k, 2),
                     "workload": "AllGather p=8, 16 MiB bf16 shards: 64 device-to-device copies vs one launch"})
        del shard, full
        per = 4096 * 7168
        blk = per // p
        send = [torch.empty(per, dtype=torch.bfloat16, device=dev).normal_() for _ in range(p)]
        recv = [torch.empty(per, dtype=torch.bfloat16, device=dev) for _ in range(p)]

        def a2a_memcpy():
            for i in range(p):
                for j in range(p):
                    recv[j][i * blk:(i + 1) * blk].copy_(send[i][j * blk:(j + 1) * blk])
        f = coll.coll_alltoall(send, recv, blk, defer=True)
        t_ce, t_k = [stats_us(x)[0] for x in time_launches(torch, [a2a_memcpy, f], iters, warmup)]
        b_a2a = 2 * p * per * 2
        rows.append({"name": "alltoall_vs_copy_engine", "p": p, "elem_bytes": 2, "hbm_bytes": b_a2a,
                     "memcpy_64_calls_us": round(t_ce, 2), "coll_alltoall_us": round(t_k, 2),
                     "memcpy_GBps": round(b_a2a / (t_ce * 1e-6) / 1e9, 1),
                     "coll_GBps": round(b_a2a / (t_k * 1e-6) / 1e9, 1), "speedup": round(t_ce / t_k, 2),
                     "workload": "All-to-All p=8, 4096x7168 bf16 per rank: 64 device-to-device copies vs one launch"})
        del send, recv
        torch.cuda.empty_cache()
    return rows


def moe_row(torch, coll, inputs, dev, iters, warmup, ceil):
    """Pack -> dispatch Alltoallv -> reverse Alltoallv -> weighted combine
    (in place on a residual), p = 8, 4096 tokens x 7168 bf16 per rank,
    top-2 routing uniform over ranks; each stage timed on its own."""
    p, T, H, k = 8, 4096, 7168, 2
    A = T * k
    d = 2
    toks = [to_dev(torch, x, dev) for x in inputs.rank_buffers(inputs.WL_MOE_A2A, p, T * H, inputs.BF16,
                                                               dist="normal")]
    dest = [torch.from_numpy(r).to(dev) for r in inputs.moe_routes(p, T, k)]
    wts = [torch.from_numpy(w).to(dev) for w in inputs.moe_weights(p, T, k)]
    packed = [torch.empty(A * H, dtype=torch.bfloat16, device=dev) for _ in range(p)]
    pos = [torch.empty(A, dtype=torch.int32, device=dev) for _ in range(p)]
    counts = torch.empty(p * p, dtype=torch.int64, device=dev)
    f_pack = coll.coll_moe_pack(toks, dest, packed, pos, counts, k, H, defer=True)
    f_pack()
    torch.cuda.synchronize()
    cols = counts.cpu().numpy().reshape(p, p).sum(axis=0)
    recv = [torch.empty(int(c), dtype=torch.bfloat16, device=dev) for c in cols]
    back = [torch.empty(A * H, dtype=torch.bfloat16, device=dev) for _ in range(p)]
    out = [torch.empty(T * H, dtype=torch.bfloat16, device=dev).normal_() for _ in range(p)]
    f_disp = coll.coll_alltoallv(packed, recv, counts, defer=True)
    f_rev = coll.coll_alltoallv_transposed(recv, back, counts, defer=True)
    f_comb = coll.coll_moe_combine(back, pos, wts, out, k, H, residual=out, defer=True)
    t = [stats_us(x)[0] for x in time_launches(torch, [f_pack, f_disp, f_rev, f_comb], iters, warmup)]
    # algorithmic HBM bytes per stage (all ranks)
    b_pack = p * (T * H * d + A * H * d + A * 4 * 2)  # tokens once, A rows out, dest, pos
    b_xchg = p * 2 * A * H * d                       # each exchange reads and writes every row once
    b_comb = p * (A * H * d + 2 * T * H * d + A * 8)  # A rows + residual in, T rows out, pos + weights
    stage = {}
    tok_bytes = p * T * H * d
    for name, us, b, mix in (("pack", t[0], b_pack, (1, 2)), ("dispatch_alltoallv", t[1], b_xchg, (1, 1)),
                             ("reverse_alltoallv", t[2], b_xchg, (1, 1)), ("combine", t[3], b_comb, (3, 1))):
        stage[name] = ceil.attach({"t_med_us": round(us, 2), "hbm_bytes": b,
                                   "hbm_GBps": round(b / (us * 1e-6) / 1e9, 1)}, *mix,
                                  tok_bytes * (k if mix == (1, 1) else 1))
    tot_us = sum(t)
    tot_b = b_pack + 2 * b_xchg + b_comb
    return {"name": "moe_dispatch_combine", "p": p, "tokens": T, "hidden": H, "top_k": k, "dtype": "bf16",
            "t_med_us": round(tot_us, 2), "hbm_bytes": tot_b, "hbm_GBps": round(tot_b / (tot_us * 1e-6) / 1e9, 1),
            "pct_hbm_peak": round(100.0 * tot_b / (tot_us * 1e-6) / 1e9 / HBM_PEAK, 1), "stages": stage,
            "workload": "pack -> Alltoallv -> reverse Alltoallv -> weighted combine + residual"}


def moe_fp8_row(torch, coll, inputs, dev, iters, warmup, ceil):
    """The same MoE layer with the dispatch in FP8 e4m3 (one fp32 scale per
    128 elements): quantizing pack -> byte Alltoallv -> dequant (the experts'
    bf16 input) -> bf16 reverse Alltoallv -> weighted combine + residual."""
    p, T, H, k, G = 8, 4096, 7168, 2, 128
    A = T * k
    R = coll.coll_moe_fp8_row_bytes(H, G)
    toks = [to_dev(torch, x, dev) for x in inputs.rank_buffers(inputs.WL_MOE_A2A, p, T * H, inputs.BF16,
                                                               dist="normal")]
    dest = [torch.from_numpy(r).to(dev) for r in inputs.moe_routes(p, T, k)]
    wts = [torch.from_numpy(w).to(dev) for w in inputs.moe_weights(p, T, k)]
    packed = [torch.empty(A * R, dtype=torch.uint8, device=dev) for _ in range(p)]
    pos = [torch.empty(A, dtype=torch.int32, device=dev) for _ in range(p)]
    counts = torch.empty(p * p, dtype=torch.int64, device=dev)
    counts_h = torch.empty(p * p, dtype=torch.int64, device=dev)
    f_pack = coll.coll_moe_pack_fp8(toks, dest, packed, pos, counts, k, H, G, counts_hidden_dev=counts_h,
                                    defer=True)
    f_pack()
    torch.cuda.synchronize()
    rows = counts.cpu().numpy().reshape(p, p).sum(axis=0) // R
    recv = [torch.empty(int(r) * R, dtype=torch.uint8, device=dev) for r in rows]
    ex_in = [torch.empty(int(r) * H, dtype=torch.bfloat16, device=dev) for r in rows]
    back = [torch.empty(A * H, dtype=torch.bfloat16, device=dev) for _ in range(p)]
    out = [torch.empty(T * H, dtype=torch.bfloat16, device=dev).normal_() for _ in range(p)]
    f_disp = coll.coll_alltoallv(packed, recv, counts, defer=True)
    f_deq = coll.coll_moe_dequant_fp8(recv, ex_in, counts, [int(r) for r in rows], H, G, defer=True)
    f_rev = coll.coll_alltoallv_transposed(ex_in, back, counts_h, defer=True)
    f_comb = coll.coll_moe_combine(back, pos, wts, out, k, H, residual=out, defer=True)
    t = [stats_us(x)[0] for x in time_launches(torch, [f_pack, f_disp, f_deq, f_rev, f_comb], iters, warmup)]
    b_pack = p * (T * H * 2 + A * R + A * 4 * 2)      # tokens once, A fp8 rows out, dest, pos
    b_disp = p * 2 * A * R
    b_deq = p * (A * R + A * H * 2)
    b_rev = p * 2 * A * H * 2
    b_comb = p * (A * H * 2 + 2 * T * H * 2 + A * 8)
    stage = {}
    tok_bytes = p * T * H * 2
    for name, us, b, mix, sb in (("pack_fp8", t[0], b_pack, (1, 1), tok_bytes),
                                 ("dispatch_alltoallv_fp8", t[1], b_disp, (1, 1), tok_bytes),
                                 ("dequant_fp8", t[2], b_deq, (1, 2), tok_bytes),
                                 ("reverse_alltoallv_bf16", t[3], b_rev, (1, 1), 2 * tok_bytes),
                                 ("combine", t[4], b_comb, (3, 1), tok_bytes)):
        stage[name] = ceil.attach({"t_med_us": round(us, 2), "hbm_bytes": b,
                                   "hbm_GBps": round(b / (us * 1e-6) / 1e9, 1)}, *mix, sb)
    tot_us = sum(t)
    tot_b = b_pack + b_disp + b_deq + b_rev + b_comb
    return {"name": "moe_fp8_dispatch_bf16_combine", "p": p, "tokens": T, "hidden": H, "top_k": k, "group": G,
            "row_bytes": R, "dtype": "fp8e4m3/bf16", "t_med_us": round(tot_us, 2),
            "dispatch_path_us": round(t[0] + t[1], 2),
            "dispatch_bytes_per_row_vs_bf16": round(R / (H * 2), 4),
            "hbm_bytes": tot_b, "hbm_GBps": round(tot_b / (tot_us * 1e-6) / 1e9, 1),
            "pct_hbm_peak": round(100.0 * tot_b / (tot_us * 1e-6) / 1e9 / HBM_PEAK, 1), "stages": stage,
            "workload": "FP8 pack -> byte Alltoallv -> dequant -> bf16 reverse Alltoallv -> combine + residual"}


def moe_direct_row(torch, coll, inputs, dev, iters, warmup, ceil, fp8: bool):
    """The MoE layer without staging copies: the dispatch writes rows straight
    into the receive buffers (bf16, or FP8 with one scale per 128 elements
    followed by the dequant the experts read), the combine reads the expert
    outputs in place; p = 8, 4096 tokens x 7168 per rank, top-2."""
    p, T, H, k, G = 8, 4096, 7168, 2, 128
    A = T * k
    toks = [to_dev(torch, x, dev) for x in inputs.rank_buffers(inputs.WL_MOE_A2A, p, T * H, inputs.BF16,
                                                               dist="normal")]
    dest = [torch.from_numpy(r).to(dev) for r in inputs.moe_routes(p, T, k)]
    wts = [torch.from_numpy(w).to(dev) for w in inputs.moe_weights(p, T, k)]
    cnt = inputs.moe_routes(p, T, k)
    rows = np.zeros(p, dtype=np.int64)
    for r in cnt:
        rows += np.bincount(r, minlength=p)
    loc = [torch.empty(A, dtype=torch.int64, device=dev) for _ in range(p)]
    counts = torch.empty(p * p, dtype=torch.int64, device=dev)
    out = [torch.empty(T * H, dtype=torch.bfloat16, device=dev).normal_() for _ in range(p)]
    cap = [int(r) for r in rows]
    if fp8:
        R = coll.coll_moe_fp8_row_bytes(H, G)
        recv = [torch.empty(c * R, dtype=torch.uint8, device=dev) for c in cap]
        ex = [torch.empty(c * H, dtype=torch.bfloat16, device=dev) for c in cap]
        f_disp = coll.coll_moe_dispatch_fp8(toks, dest, recv, loc, counts, k, H, G, recv_cap=cap, defer=True)
        f_deq = coll.coll_moe_dequant_fp8(recv, ex, counts, cap, H, G, defer=True)
        fns = [f_disp, f_deq]
        b_disp = p * (T * H * 2 + A * R + A * 20)
        stages = [("dispatch_fp8_direct", b_disp), ("dequant_fp8", p * (A * R + A * H * 2))]
    else:
        R = H * 2
        recv = [torch.empty(c * H, dtype=torch.bfloat16, device=dev) for c in cap]
        ex = recv
        f_disp = coll.coll_moe_dispatch(toks, dest, recv, loc, counts, k, H, recv_cap=cap, defer=True)
        fns = [f_disp]
        stages = [("dispatch_direct", p * (T * H * 2 + A * H * 2 + A * 20))]
    f_comb = coll.coll_moe_combine_direct(ex, loc, wts, out, k, H, y_rows=cap, residual=out, defer=True)
    fns.append(f_comb)
    stages.append(("combine_direct", p * (A * H * 2 + 2 * T * H * 2 + A * 12)))
    t = [stats_us(x)[0] for x in time_launches(torch, fns, iters, warmup)]
    st = {}
    mixes = {"dispatch_fp8_direct": (1, 1), "dequant_fp8": (1, 2), "dispatch_direct": (1, 2), "combine_direct": (3, 1)}
    for (name, b), us in zip(stages, t):
        st[name] = ceil.attach({"t_med_us": round(us, 2), "hbm_bytes": b, "hbm_GBps": round(b / (us * 1e-6) / 1e9, 1)},
                               *mixes[name], p * T * H * 2)
    tot_us = sum(t)
    tot_b = sum(b for _, b in stages)
    return {"name": "moe_fp8_direct" if fp8 else "moe_direct", "p": p, "tokens": T, "hidden": H, "top_k": k,
            "dtype": "fp8e4m3/bf16" if fp8 else "bf16", "t_med_us": round(tot_us, 2), "hbm_bytes": tot_b,
            "hbm_GBps": round(tot_b / (tot_us * 1e-6) / 1e9, 1),
            "pct_hbm_peak": round(100.0 * tot_b / (tot_us * 1e-6) / 1e9 / HBM_PEAK, 1), "stages": st,
            "workload": ("direct FP8 dispatch -> dequant -> combine reading expert outputs in place" if fp8 else
                         "direct dispatch -> combine reading expert outputs in place")}


def batch_row(torch, coll, inputs, dev, ceil, iters=5, warmup=2):
    p = 16
    plan, out_elems = inputs.small_batch_plan(10000)
    pf, pi = inputs.small_batch_pools(p)
    dpf = [to_dev(torch, x, dev) for x in pf]
    dpi = [to_dev(torch, x, dev) for x in pi]
    outs = [torch.empty(out_elems, dtype=torch.int32, device=dev) for _ in range(p)]
    base_f = [t.data_ptr() for t in dpf]
    base_i = [t.data_ptr() for t in dpi]
    base_o = [t.data_ptr() for t in outs]
    calls, total_bytes = [], 0
    for c in plan:
        src = base_f if c.dtype == inputs.F32 else base_i
        calls.append(([b + 4 * c.src_off for b in src], [b + 4 * c.dst_off for b in base_o], c.n, c.dtype, c.op))
        total_bytes += 4 * c.n
    f = coll.coll_allreduce_batch(calls, p, defer=True)
    # wall time of whole calls (host validation + descriptor upload + kernel)
    for _ in range(warmup):
        f()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(iters):
        f()
    torch.cuda.synchronize()
    wall_us = (time.perf_counter() - t0) / iters * 1e6
    med, p95, _ = stats_us(time_launches(torch, [f], iters, 1)[0])
    hbm = 2 * p * total_bytes
    indiv = individual_calls(torch, coll, calls, p)
    del dpf, dpi, outs
    torch.cuda.empty_cache()
    row = {
        "name": "allreduce_batch_10000", "p": p, "calls": len(plan), "dtype": "f32/i32", "op": "sum/min/max",
        "payload_bytes": total_bytes,
        "t_med_us": round(med, 1), "t_p95_us": round(p95, 1), "wall_us_per_batch": round(wall_us, 1),
        "us_per_call": round(med / len(plan), 4),
        "hbm_bytes": hbm, "hbm_GBps": round(hbm / (med * 1e-6) / 1e9, 1),
        "pct_hbm_peak": round(100.0 * hbm / (med * 1e-6) / 1e9 / HBM_PEAK, 1),
        "busbw_GBps": round(total_bytes / (med * 1e-6) / 1e9 * 2 * (p - 1) / p, 1),
        "workload": "10,000 AllReduces, sizes log-uniform 4 KiB-1 MiB, one launch",
        "individual_calls": indiv,
    }
    # ceilings: p reads : p writes at the plan's output footprint (streams of
    # the per-rank output pool), and at a 128 MiB footprint
    ceil.attach(row, p, p, (out_elems * 4 + 255) // 256 * 256)
    small = ceil.get(p, p, 128 << 20)
    if small is not None:
        row["mix_ceiling_128MiB_streams_GBps"] = small["GBps"]
    return row


def individual_calls(torch, coll, calls, p, sample=1000):
    """The same AllReduces as separate coll_allreduce calls.

    back_to_back: all calls enqueued without synchronisation (arguments
    marshalled beforehand), wall time per call; this is the submission
    rate of one host thread.  latency: a seeded sample of calls, each
    followed by a stream synchronisation, end-to-end wall time per call
    (host validation + launch + kernel + completion), with percentiles and
    a least-squares fit t = alpha + bytes / beta (the alpha-beta model of
    "集合通信：原语、算法、NCCL 实现与拓扑映射", section 2.1)."""
    prepared = [coll.coll_allreduce(s, r, op, n=n, dtype=dt, defer=True) for s, r, n, dt, op in calls]
    for f in prepared[:200]:
        f()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for f in prepared:
        f()
    torch.cuda.synchronize()
    b2b_us = (time.perf_counter() - t0) / len(prepared) * 1e6
    rng = np.random.default_rng(11)
    idx = rng.choice(len(prepared), min(sample, len(prepared)), replace=False)
    lat, size = [], []
    for k in idx:
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        prepared[k]()
        torch.cuda.synchronize()
        lat.append((time.perf_counter() - t1) * 1e6)
        size.append(4 * calls[k][2])
    lat, size = np.asarray(lat), np.asarray(size, dtype=np.float64)
    A = np.stack([np.ones_like(size), size], axis=1)
    (alpha, inv_beta), *_ = np.linalg.lstsq(A, lat, rcond=None)
    return {
        "back_to_back_us_per_call": round(b2b_us, 2),
        "latency_sample": int(len(lat)),
        "latency_p50_us": round(float(np.percentile(lat, 50)), 2),
        "latency_p95_us": round(float(np.percentile(lat, 95)), 2),
        "latency_p99_us": round(float(np.percentile(lat, 99)), 2),
        "alpha_us": round(float(alpha), 2),
        "beta_GBps_per_rank_payload": round(float(1e-3 / inv_beta), 1) if inv_beta > 0 else None,
        "note": "alpha-beta fitted on end-to-end latency vs per-rank payload bytes",
    }


# ----------------------------------------------------------------------------

def main(argv=None) -> int:
    global NO_GRAPHS
    args = parse_args(argv)
    NO_GRAPHS = args.no_graphs
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: all p logical ranks live in one device's HBM and "
              "nothing here runs across GPUs; run it with --gpus 1.", file=sys.stderr)
        return 2
    import torch

    import collective_communication_primitives_coll_amd as coll
    from collective_communication_primitives_coll_amd import inputs, metrics

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    coll.lib()

    wl = zero_workload(torch, coll, inputs, dev)
    p, n, total = wl["p"], wl["n"], wl["total"]
    rs, ag = wl["rs"], wl["ag"]
    print(f"# zero_rs_ag: p={p} n_shard={n} bf16, warmup {args.warmup}, steps {args.steps}",
          file=sys.stderr, flush=True)

    for _ in range(args.warmup):
        rs()
        ag()
    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        ev[i][0].record()
        rs()
        ev[i][1].record()
        ag()
        ev[i][2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_rs = [ev[i][0].elapsed_time(ev[i][1]) for i in range(K)]
    t_ag = [ev[i][1].elapsed_time(ev[i][2]) for i in range(K)]
    ms_per_step = wall * 1e3 / K

    hbm_rs = metrics.hbm_bytes("reduce_scatter", p, n, 2)
    hbm_ag = metrics.hbm_bytes("allgather", p, n, 2)
    value = (hbm_rs + hbm_ag) / (ms_per_step * 1e-3) / 1e9
    rs_med, rs_p95, rs_mean = stats_us(t_rs)
    ag_med, ag_p95, ag_mean = stats_us(t_ag)
    per_coll = {
        "reduce_scatter": coll_entry(metrics, "reduce_scatter", "reduce_scatter", p, n, 2, rs_med, "ring",
                                     {"t_p95_us": round(rs_p95, 2), "t_mean_us": round(rs_mean, 2)}),
        "allgather": coll_entry(metrics, "allgather", "allgather", p, n, 2, ag_med, "ring",
                                {"t_p95_us": round(ag_p95, 2), "t_mean_us": round(ag_mean, 2)}),
    }
    # Cold step (outside the timed loop): a 512 MiB overwrite before each
    # step evicts the Infinity Cache; events bracket ReduceScatter and
    # AllGather as above.  ReduceScatter's shards still reach AllGather
    # through the cache within the step.
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cold = []
    for i in range(max(K, 5)):
        scratch.fill_(i & 0xFF)
        ce = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ce[0].record()
        rs()
        ce[1].record()
        ag()
        ce[2].record()
        cold.append(ce)
    torch.cuda.synchronize()
    rs_cold = stats_us([c[0].elapsed_time(c[1]) for c in cold])[0]
    ag_cold = stats_us([c[1].elapsed_time(c[2]) for c in cold])[0]
    del scratch
    per_coll["reduce_scatter"]["t_cold_med_us"] = round(rs_cold, 2)
    per_coll["allgather"]["t_cold_med_us"] = round(ag_cold, 2)
    # dominant kernel: the longer of the two launches
    if rs_mean >= ag_mean:
        dom, dom_bytes, dom_us, kkey = "reduce_kernel<bf16,sum,p=8> (coll_reduce_scatter)", hbm_rs, rs_mean, "reduce_scatter"
    else:
        dom, dom_bytes, dom_us, kkey = "copy_kernel<2B> (coll_allgather)", hbm_ag, ag_mean, "allgather"
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK, 4), "traffic": read_traffic(kkey, dom_bytes),
                "kernel": dom, "algorithmic_bytes_per_launch": dom_bytes, "mean_launch_us": round(dom_us, 2)}
    # Attainable references measured in the same run: the dominant kernel's
    # own read:write stream mix at its stream size (the library's
    # direction-mix probe), and a 1 GiB device copy by the library's copy
    # kernel (Broadcast at p = 1).
    ceil = Ceilings(torch, coll, dev, enabled=not args.no_ceilings)
    mix = ceil.get(p, 1, total * 2) if kkey == "reduce_scatter" else ceil.get(1, p, p * n * 2)
    if mix is not None:
        roofline["attainable_mix_GBps"] = mix["GBps"]
        roofline["mix"] = mix["mix"]
        roofline["frac_of_mix_ceiling"] = round(achieved / mix["GBps"], 4)
        ceil.attach(per_coll["reduce_scatter"], p, 1, total * 2)
        ceil.attach(per_coll["allgather"], 1, p, p * n * 2)
    cbytes = 1 << 30
    ca = torch.empty(cbytes // 4, dtype=torch.int32, device=dev).fill_(1)
    cb = torch.empty_like(ca)
    cmed, _, _ = stats_us(time_launches(torch, [coll.coll_broadcast(ca, [cb], 0, defer=True)], 10, 3)[0])
    copy_gbps = 2 * cbytes / (cmed * 1e-6) / 1e9
    roofline["attainable_copy_GBps"] = round(copy_gbps, 1)
    roofline["frac_of_copy"] = round(achieved / copy_gbps, 4)
    del ca, cb

    cpu = None
    if not args.no_cpu_baseline:
        print("# cpu baseline (threaded C++ oracle, whole step)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(torch, wl, args.cpu_seconds)

    del wl, rs, ag
    torch.cuda.empty_cache()
    rows = []
    if not args.no_collectives:
        which = set(args.only.split(",")) if args.only else None
        print("# per-collective table", file=sys.stderr, flush=True)
        rows = extra_collectives(torch, coll, inputs, metrics, dev, which, ceil)
    for row in rows:
        print("# detail " + json.dumps(row), file=sys.stderr, flush=True)
    print("# ceilings " + json.dumps({f"{k[0]}r:{k[1]}w:{k[2]}": v for k, v in ceil.cache.items()}),
          file=sys.stderr, flush=True)

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 (fp32 accumulation)",
        "data": "synthetic (seeded NumPy PCG64, bf16 ~ N(0, 1e-3))",
        "config": {
            "workload": "zero_rs_ag: ReduceScatter(sum) then AllGather, p=8 logical ranks, "
                        "2^26 bf16 elements per rank, fp32 accumulation, shard 2^23",
            "p": p, "elements_per_rank": total, "storage": "bf16", "accumulate": "f32",
            "hbm_bytes_per_step": hbm_rs + hbm_ag,
            "pct_hbm_peak": round(100.0 * value / HBM_PEAK, 1),
        },
        "per_collective": {k: compact_row(v) for k, v in per_coll.items()},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "collectives": [compact_row(r) for r in rows],
    }
    print("# source_hash " + json.dumps({k: source_hash(k) for k in KERNEL_SOURCES}), file=sys.stderr, flush=True)
    print(json.dumps(line, separators=(",", ":")), flush=True)
    return 0


def _short(v, key: str = ""):
    """A number as the summary line keeps it: GB/s as integers, times to
    0.1 us (0.01 below 10 us), fractions and ratios to three decimals."""
    if not isinstance(v, float):
        return v
    if key.endswith("GBps"):
        return round(v)
    if key.startswith("t_") or key.endswith("_us") or key.endswith("us_per_call"):
        return round(v, 2 if abs(v) < 10 else 1)
    return round(v, 3)


def compact_row(row: dict) -> dict:
    """The figures of a table row that the summary line keeps: time, HBM
    GB/s, busbw, and the fraction of the row's mix ceiling (share of peak
    and the ceiling itself follow from these); nested stages and latency
    tables in the same short form.  The full rows go to stderr."""
    keep = ("name", "t_med_us", "hbm_GBps", "busbw_GBps", "frac_of_mix_ceiling", "t_cold_med_us", "t_graph_us")
    out = {k: _short(row[k], k) for k in keep if k in row}
    if "stages" in row:
        out["stages"] = {k: [_short(v.get(f), f) for f in ("t_med_us", "hbm_GBps", "frac_of_mix_ceiling")]
                         for k, v in row["stages"].items()}
        out["stage_fields"] = ["t_med_us", "hbm_GBps", "frac_of_mix_ceiling"]
    if "table" in row and row["name"] == "other_rank_counts":
        out["table_fields"] = ["p", "allreduce_GBps", "reduce_scatter_GBps", "allreduce_frac_of_mix_ceiling",
                               "reduce_scatter_frac_of_mix_ceiling"]
        out["table"] = [[_short(e.get(k), k) for k in out["table_fields"]] for e in row["table"]]
    elif "table" in row:
        keys = [k for k in row["table"][0] if k.endswith("graph_us")]
        out["bytes_per_rank"] = [e["bytes_per_rank"] for e in row["table"]]
        out["graph_us"] = {k[:-len("_graph_us")]: [_short(e[k], k) for e in row["table"]] for k in keys}
    if "individual_calls" in row:
        ic = row["individual_calls"]
        out["individual_calls"] = {k: _short(ic[k], k) for k in ("back_to_back_us_per_call", "latency_p50_us",
                                                                "latency_p99_us", "alpha_us") if k in ic}
    for k in ("memcpy_GBps", "coll_GBps", "speedup", "torch_copy_GBps", "coll_copy_kernel_GBps"):
        if k in row:
            out[k] = _short(row[k], k)
    return out


if __name__ == "__main__":
    sys.exit(main())
