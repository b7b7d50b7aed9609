#!/usr/bin/env python3
"""Throughput of the row-reduction kernels on one MI355X, as effective HBM GB/s.

A step is one call of the op over one batch of seeded synthetic input (the whole
path: plan, 128-bit loads, register / wave / LDS (/ grid) reductions, epilogue,
stores).  Inputs are resident in HBM before timing starts; several input/output
sets (at least 2 GiB together) rotate so that every step reads cold data rather
than the 256 MB last-level cache.

Printed: one JSON line with
  value      whole-job effective GB/s = algorithmic bytes per step x steps / wall time
  roofline   the kernel's algorithmic bytes / its mean time per launch (two HIP events
             on the launch stream around the timed launches, back to back), against the
             MI355X HBM peak of 8 TB/s, and the HBM bytes the hardware counters measured
             per launch (null if the kernel sources changed since the counters were
             taken)
  cpu_baseline  the double-precision CPU oracle on a bounded sample of the same workload
  copy_ceiling  a 128-bit streaming copy of the same bytes in the same run, and beside it
             a read-only stream of the input bytes and a write-only stream of the output
             bytes (the kernel's reads and writes each at the rate HBM gives them alone)
Algorithmic bytes: softmax M*N*(s_in + s_out); RMSNorm M*N*(s_in + s_out) + N*s;
cross-entropy M*N*s + 12*M (labels in, loss and lse out).

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--sweep] [--ceiling]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective HBM GB/s (1 read+1 write) and % of MI355X peak, per op/N/dtype"
HBM_PEAK_GBPS = 8000.0
# The largest fixed workload, and the shape the pages quote their headline on ([QuACK]
# section NCU 性能分析（Softmax 内核）: fp32 softmax, 16K rows of 131K, 3.01 TB/s on H100).
DEFAULT_WORKLOAD = "softmax_f32_16384x131072_spiky"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = os.path.join(ROOT, "memory_bound_row_softmax_amd", "csrc")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in sorted(os.listdir(KERNEL_SOURCES)):
        if name.endswith((".hip", ".hpp", ".cpp")):  # kernels and the planner that picks them
            with open(os.path.join(KERNEL_SOURCES, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def esize(dtype: str) -> int:
    return 4 if dtype == "f32" else 2


def algorithmic_bytes(w) -> int:
    s = esize(w.dtype)
    if w.op == "softmax":
        return w.M * w.N * 2 * s
    if w.op == "rmsnorm":
        return w.M * w.N * 2 * s + w.N * s
    if w.op == "xent_grad":  # logits in, gradient out; labels, dloss in; loss, lse out
        return w.M * w.N * 2 * s + 16 * w.M
    if w.op == "softmax_bwd":  # y, dy in; dx out
        return w.M * w.N * 3 * s
    if w.op == "rmsnorm_bwd":  # x, dy in; dx out; w, rstd in; dw (fp32) out
        return w.M * w.N * 3 * s + w.N * s + 4 * w.M + 4 * w.N
    return w.M * w.N * s + 12 * w.M


def traffic_for(name: str):
    """Counter-measured HBM bytes per launch, if taken on the current kernel sources."""
    try:
        data = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None, None
    rec = data.get(name)
    if not rec or rec.get("source_hash") != kernel_source_hash():
        return None, rec
    return rec["fetch_bytes"] + rec["write_bytes"], rec


class Runner:
    """Device buffers for one workload and a launcher for step k."""

    def __init__(self, w, min_rotation_bytes: float, device="cuda:0", host_rows=None):
        import numpy as np
        import torch

        import memory_bound_row_softmax_amd as rr
        from synth import workloads as W

        self.w, self.rr, self.torch = w, rr, torch
        self.dev = device
        self.dt = rr.RR_F32 if w.dtype == "f32" else rr.RR_BF16
        s = esize(w.dtype)
        in_bytes = w.M * w.N * s
        out_bytes = in_bytes if w.op != "xent" else 8 * w.M
        if w.op in ("softmax_bwd", "rmsnorm_bwd"):
            in_bytes *= 2  # two input matrices
        has_rows = w.op in ("xent", "xent_grad")  # per-row labels and losses
        self.sets = max(1, min(16, math.ceil(min_rotation_bytes / (in_bytes + out_bytes))))
        tdt = torch.float32 if w.dtype == "f32" else torch.bfloat16

        # host_rows: generate only that many rows and repeat them down the matrix
        # (used by the sweep, whose largest inputs are tens of GiB; throughput does
        # not depend on the values)
        gen_rows = w.M if host_rows is None else min(w.M, host_rows)
        x_np = W.x_rows(w, nrows=gen_rows)
        host = torch.from_numpy(x_np if w.dtype == "f32" else x_np.view(np.int16))
        x0 = torch.empty((w.M, w.N), dtype=host.dtype, device=device)
        block = host.to(device)
        for r0 in range(0, w.M, gen_rows):
            r1 = min(w.M, r0 + gen_rows)
            x0[r0:r1].copy_(block[: r1 - r0])
        del host, x_np, block
        x0 = x0.view(tdt) if w.dtype == "bf16" else x0
        self.x = [x0] + [x0.clone() for _ in range(self.sets - 1)]
        if has_rows:
            lab = torch.from_numpy(W.label_rows(w)).to(device)  # labels are per row: all rows
            self.labels = lab
            self.loss = [torch.empty(w.M, dtype=torch.float32, device=device) for _ in range(self.sets)]
            self.lse = [torch.empty(w.M, dtype=torch.float32, device=device) for _ in range(self.sets)]
        if w.op == "xent_grad":
            self.dloss = torch.from_numpy(W.dloss_rows(w)).to(device)
        if w.op != "xent":
            self.y = [torch.empty_like(x0) for _ in range(self.sets)]
        def tile_rows(gen):
            """A device [M, N] matrix from `gen(nrows)` host rows repeated down it."""
            a = gen(gen_rows)
            h = torch.from_numpy(a if w.dtype == "f32" else a.view(np.int16)).to(device)
            t = torch.empty((w.M, w.N), dtype=h.dtype, device=device)
            for r0 in range(0, w.M, gen_rows):
                r1 = min(w.M, r0 + gen_rows)
                t[r0:r1].copy_(h[: r1 - r0])
            return t.view(tdt) if w.dtype == "bf16" else t

        if w.op in ("rmsnorm", "rmsnorm_bwd"):
            wn = W.weight(w)
            wt = torch.from_numpy(wn if w.dtype == "f32" else wn.view(np.int16)).to(device)
            self.weight = wt.view(tdt) if w.dtype == "bf16" else wt
        if w.op in ("softmax_bwd", "rmsnorm_bwd"):
            # the backward's second input, and the forward outputs it takes (from the
            # library's own forward kernels: these are bench inputs, not references)
            dy0 = tile_rows(lambda n: W.dy_rows(w, nrows=n))
            self.dy = [dy0] + [dy0.clone() for _ in range(self.sets - 1)]
            if w.op == "softmax_bwd":
                for t in self.x:
                    rr.rr_softmax_fwd(t, t)
            else:
                self.rstd = torch.empty(w.M, dtype=torch.float32, device=device)
                rr.rr_rmsnorm_fwd(x0, self.weight, w.eps, y=self.y[0], rstd=self.rstd)
                self.dw = torch.empty(w.N, dtype=torch.float32, device=device)
            torch.cuda.synchronize()
        op = {"softmax": rr.RR_OP_SOFTMAX, "rmsnorm": rr.RR_OP_RMSNORM, "xent": rr.RR_OP_XENT,
              "xent_grad": rr.RR_OP_XENT_GRAD, "softmax_bwd": rr.RR_OP_SOFTMAX_BWD,
              "rmsnorm_bwd": rr.RR_OP_RMSNORM_BWD}[w.op]
        self.op = op
        # The workspace is zero-filled on the launch stream, and everything above is
        # finished before the first launch: a kernel that started before the fill
        # (on another stream) would find stale counters and slots, and have them
        # zeroed under it while its workgroups wait for each other.
        self.stream = torch.cuda.Stream(device=device)
        self.sp = self.stream.cuda_stream
        with torch.cuda.stream(self.stream):
            self.ws = rr.workspace(op, w.M, w.N, self.dt, device)
        torch.cuda.synchronize()
        self.wsp = self.ws.data_ptr() if self.ws is not None else 0
        self.wsb = self.ws.numel() if self.ws is not None else 0
        self.plan = rr.rr_plan_query(op, w.M, w.N, self.dt)
        self.xp = [t.data_ptr() for t in self.x]
        if has_rows:
            self.lp, self.ep = [t.data_ptr() for t in self.loss], [t.data_ptr() for t in self.lse]
            self.labp = self.labels.data_ptr()
        if w.op == "xent_grad":
            self.gp = self.dloss.data_ptr()
        if w.op != "xent":
            self.yp = [t.data_ptr() for t in self.y]
        self.wp = self.weight.data_ptr() if w.op in ("rmsnorm", "rmsnorm_bwd") else 0
        if w.op in ("softmax_bwd", "rmsnorm_bwd"):
            self.dyp = [t.data_ptr() for t in self.dy]
        self.copy_dst = None
        self.sink = None

    def launch(self, k: int) -> int:
        w, rr, i = self.w, self.rr, k % self.sets
        if w.op == "softmax":
            return rr.softmax_fwd_raw(self.xp[i], self.yp[i], w.M, w.N, self.dt, self.wsp, self.wsb,
                                      self.sp)
        if w.op == "rmsnorm":
            return rr.rmsnorm_fwd_raw(self.xp[i], self.wp, self.yp[i], 0, w.M, w.N, self.dt, w.eps,
                                      self.wsp, self.wsb, self.sp)
        if w.op == "softmax_bwd":
            return rr.softmax_bwd_raw(self.xp[i], self.dyp[i], self.yp[i], w.M, w.N, self.dt,
                                      self.wsp, self.wsb, self.sp)
        if w.op == "rmsnorm_bwd":
            return rr.rmsnorm_bwd_raw(self.xp[i], self.wp, self.dyp[i], self.rstd.data_ptr(),
                                      self.yp[i], self.dw.data_ptr(), w.M, w.N, self.dt,
                                      self.wsp, self.wsb, self.sp)
        if w.op == "xent_grad":
            return rr.cross_entropy_fwd_bwd_raw(self.xp[i], self.labp, self.gp, self.lp[i],
                                                self.ep[i], self.yp[i], w.M, w.N, self.dt,
                                                self.wsp, self.wsb, self.sp)
        return rr.cross_entropy_fwd_raw(self.xp[i], self.labp, self.lp[i], self.ep[i], w.M, w.N,
                                        self.dt, self.wsp, self.wsb, self.sp)

    def read_launch(self, k: int) -> int:
        src = self.x[k % self.sets]
        nbytes = src.numel() * src.element_size()
        if self.sink is None:
            self.sink = self.torch.empty(self.rr.stream_read_sink_bytes(nbytes) // 4,
                                         dtype=self.torch.int32, device=self.dev)
        return self.rr.stream_read_raw(src.data_ptr(), nbytes, self.sink.data_ptr(),
                                       self.sink.numel() * 4, self.sp)

    def write_launch(self, k: int) -> int:
        dst = self.y[k % self.sets] if self.w.op != "xent" else self.x[k % self.sets]
        return self.rr.stream_fill_raw(dst.data_ptr(), dst.numel() * dst.element_size(), k,
                                       self.sp)

    def copy_launch(self, k: int) -> int:
        i = k % self.sets
        src = self.x[i]
        nbytes = src.numel() * src.element_size()
        if self.w.op == "xent":
            if self.copy_dst is None:
                self.copy_dst = self.torch.empty_like(self.x[0])
            dst = self.copy_dst
        else:
            dst = self.y[i]
        return self.rr.stream_copy_raw(src.data_ptr(), dst.data_ptr(), nbytes, self.sp)

    def check_workspace(self):
        """Fails if a split row of the timed launches gave up waiting for its peer
        workgroups (its rows would then be NaN, and the launch faster than a real one)."""
        if self.ws is None:
            return
        st = self.rr.rr_workspace_check(self.ws, stream=self.sp)
        if st != 0:
            raise RuntimeError(f"workspace check failed: {self.rr.status_string(st)}")

    def time(self, fn, steps: int, warmup: int, graph: bool = False):
        """Wall time of `steps` back-to-back launches, and the mean time per launch
        from a pair of HIP events on the launch stream around the same region.
        With `graph`, the `steps` launches are captured once in a HIP graph and the
        timed region is one replay of it (no host launch cost between kernels).
        Every launch's status is checked (after the timed region, so that the check
        adds nothing between launches), and so is the workspace's error word."""
        torch = self.torch
        with torch.cuda.stream(self.stream):
            for k in range(warmup):
                st = fn(k)
                if st != 0:
                    raise RuntimeError(f"launch failed: {self.rr.status_string(st)}")
            g = None
            if graph:
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=self.stream):
                    for k in range(steps):
                        st = fn(warmup + k)
                        if st != 0:
                            raise RuntimeError(f"capture failed: {self.rr.status_string(st)}")
                g.replay()  # the first replay uploads the graph
            start = torch.cuda.Event(enable_timing=True)
            end = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            start.record(self.stream)
            bad = 0
            if graph:
                g.replay()
            else:
                for k in range(steps):
                    bad |= fn(warmup + k)
            end.record(self.stream)
            torch.cuda.synchronize()
            t1 = time.perf_counter()
        if bad != 0:
            raise RuntimeError(f"a timed launch failed: {self.rr.status_string(bad)}")
        self.check_workspace()
        return t1 - t0, start.elapsed_time(end) / steps


def cpu_baseline(w, seconds: float, max_threads: int = 16):
    """The oracle, single-threaded, on the first rows of the same workload (for a
    backward pass, only the backward call is timed); then the same oracle function
    row-partitioned over the host's cores (one block of rows per thread; the C
    oracle runs outside the interpreter lock).  Input generation is not timed."""
    import concurrent.futures as cf

    import numpy as np

    import oracle
    import synth
    from synth import workloads as W

    per_row = algorithmic_bytes(w) / w.M

    def prepare(rows, row0=0):
        """Inputs of the timed oracle call for rows row0 .. row0 + rows - 1."""
        x = W.x_rows(w, nrows=rows, row0=row0)
        if w.op == "softmax":
            return (oracle.softmax, x)
        if w.op == "rmsnorm":
            return (oracle.rmsnorm, x, W.weight(w), w.eps)
        if w.op == "xent_grad":
            return (oracle.cross_entropy_grad, x, W.label_rows(w, nrows=rows, row0=row0),
                    W.dloss_rows(w, nrows=rows, row0=row0))
        if w.op == "softmax_bwd":
            y = oracle.softmax(x).astype(np.float32)
            y = y if w.dtype == "f32" else synth.f32_to_bf16(y)
            return (oracle.softmax_backward, y, W.dy_rows(w, nrows=rows, row0=row0))
        if w.op == "rmsnorm_bwd":
            wt = W.weight(w)
            _, r = oracle.rmsnorm(x, wt, w.eps, want_rstd=True)
            return (oracle.rmsnorm_backward, x, wt, W.dy_rows(w, nrows=rows, row0=row0),
                    r.astype(np.float32))
        return (oracle.cross_entropy, x, W.label_rows(w, nrows=rows, row0=row0))

    def run(rows):
        call = prepare(rows)
        t0 = time.perf_counter()
        call[0](*call[1:])
        return time.perf_counter() - t0

    probe = max(1, min(w.M, (1 << 20) // w.N))
    t = run(probe)
    rows = max(1, min(w.M, int(probe * seconds / max(t, 1e-6))))
    passes = 1
    if rows == w.M:  # the whole matrix takes less than `seconds`: repeat it
        t_all = run(rows)
        passes = max(1, int(seconds / max(t_all, 1e-6)))
    total = 0.0
    for _ in range(passes):
        total += run(rows)
    single = {"value": round(per_row * rows * passes / total / 1e9, 4), "unit": "GB/s",
              "cores": 1, "kind": "oracle",
              "sample": f"first {rows} of {w.M} rows x {passes} pass(es), single-threaded "
                        f"double-precision oracle, {total:.1f} s of CPU time"}

    # all cores: one contiguous block of rows per thread (at most 2^27 elements in
    # all), rounds repeated to about half of `seconds`
    threads = max(1, min(max_threads, os.cpu_count() or 1))
    block = max(1, min(rows, w.M // threads, (1 << 27) // (w.N * threads)))
    nblocks = min(threads, max(1, w.M // block))
    calls = [prepare(block, row0=k * block) for k in range(nblocks)]
    with cf.ThreadPoolExecutor(max_workers=nblocks) as ex:
        def one_round():
            t0 = time.perf_counter()
            list(ex.map(lambda c: c[0](*c[1:]), calls))
            return time.perf_counter() - t0

        t_round = one_round()
        rounds = max(1, int(0.5 * seconds / max(t_round, 1e-6)))
        t_mt = sum(one_round() for _ in range(rounds))
    single["all_cores"] = {
        "value": round(per_row * block * nblocks * rounds / t_mt / 1e9, 4), "unit": "GB/s",
        "cores": nblocks, "kind": "oracle",
        "sample": f"{nblocks} blocks of {block} rows, one per thread, x {rounds} round(s), the "
                  f"same oracle function, {t_mt:.1f} s wall"}
    return single


def measure(w, steps: int, warmup: int, min_rotation_bytes: float, with_cpu: bool,
            cpu_seconds: float, host_rows=None, graph=False):
    r = Runner(w, min_rotation_bytes, host_rows=host_rows)
    nbytes = algorithmic_bytes(w)
    wall, mean_ms = r.time(r.launch, steps, warmup, graph)
    copy_wall, copy_mean_ms = r.time(r.copy_launch, steps, warmup, graph)
    _, read_mean_ms = r.time(r.read_launch, steps, warmup, graph)
    in_bytes = r.x[0].numel() * r.x[0].element_size()
    out_bytes = in_bytes if w.op != "xent" else in_bytes  # xent: the fill writes x's size
    if w.op != "xent":
        _, write_mean_ms = r.time(r.write_launch, steps, warmup, graph)
    else:
        write_mean_ms = None  # cross-entropy writes 12 bytes per row
    copy_bytes = 2 * r.x[0].numel() * r.x[0].element_size()
    achieved = nbytes / (mean_ms * 1e-3) / 1e9
    traffic, rec = traffic_for(w.name)
    copy_gbps = copy_bytes / (copy_mean_ms * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": round(nbytes * steps / wall / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(wall / steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "op": w.op, "io_dtype": w.dtype, "M": w.M, "N": w.N,
                   "plan": {k: r.plan[k] for k in ("path", "vals_per_lane", "lanes_per_row",
                                                    "groups_per_row", "block_threads")},
                   "rotating_sets": r.sets, "launch": "graph" if graph else "stream"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "launch_ms_mean": round(mean_ms, 5),
                     "algorithmic_bytes": nbytes},
        "copy_ceiling": {"value": round(copy_gbps, 2), "unit": "GB/s",
                         "frac": round(copy_gbps / HBM_PEAK_GBPS, 4),
                         "kernel_vs_copy": round(achieved / copy_gbps, 4),
                         "read_only": round(in_bytes / (read_mean_ms * 1e-3) / 1e9, 2),
                         "write_only": (round(out_bytes / (write_mean_ms * 1e-3) / 1e9, 2)
                                        if write_mean_ms else None)},
    }
    if rec is not None:
        line["roofline"]["traffic_source"] = rec.get("summary")
    if with_cpu:
        line["cpu_baseline"] = cpu_baseline(w, cpu_seconds)
    del r
    import torch

    torch.cuda.empty_cache()
    return line


def ceiling(steps: int, out=None) -> int:
    """HBM ceilings of this GPU: the library's 128-bit copy (one read and one write per
    byte), read-only and write-only streams, each timed over `steps` launches with HIP
    events, on footprints from 256 MiB to 16 GiB each way (sets rotate up to 4 GiB so
    that launches read cold data)."""
    import torch

    import memory_bound_row_softmax_amd as rr

    dev = "cuda:0"
    stream = torch.cuda.Stream(device=dev)
    sp = stream.cuda_stream
    for size in (256 << 20, 1 << 30, 4 << 30, 16 << 30):
        sets = max(1, (4 << 30) // (2 * size))
        bufs = [(torch.empty(size, dtype=torch.uint8, device=dev),
                 torch.empty(size, dtype=torch.uint8, device=dev)) for _ in range(sets)]
        for a, b in bufs:
            a.fill_(0x5A)
        sink = torch.empty(rr.stream_read_sink_bytes(size) // 4, dtype=torch.int32, device=dev)
        kinds = {
            "copy": (2, lambda k: rr.stream_copy_raw(bufs[k % sets][0].data_ptr(),
                                                     bufs[k % sets][1].data_ptr(), size, sp)),
            "read": (1, lambda k: rr.stream_read_raw(bufs[k % sets][0].data_ptr(), size,
                                                     sink.data_ptr(), sink.numel() * 4, sp)),
            "write": (1, lambda k: rr.stream_fill_raw(bufs[k % sets][1].data_ptr(), size, k, sp)),
        }
        line = {"bytes_each_way": size, "unit": "GB/s"}
        with torch.cuda.stream(stream):
            for name, (ways, fn) in kinds.items():
                for k in range(3):
                    if fn(k) != 0:
                        raise RuntimeError(f"{name} launch failed")
                start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                start.record(stream)
                bad = 0
                for k in range(steps):
                    bad |= fn(k)
                end.record(stream)
                torch.cuda.synchronize()
                if bad:
                    raise RuntimeError(f"{name} launch failed")
                ms = start.elapsed_time(end) / steps
                line[name] = round(ways * size / (ms * 1e-3) / 1e9, 1)
        print(json.dumps(line), flush=True)
        if out:
            with open(out, "a") as f:
                f.write(json.dumps(line) + "\n")
        del bufs, sink
        torch.cuda.empty_cache()
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--sweep", action="store_true",
                    help="run every fixed and sweep workload; one JSON line each to --out")
    ap.add_argument("--out", default="bench_sweep.jsonl")
    ap.add_argument("--rotate-bytes", type=float, default=float(1 << 31))
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep-host-rows", type=int, default=512,
                    help="sweep only: rows generated on the host, repeated down the matrix")
    ap.add_argument("--only", default="",
                    help="sweep only: comma-separated substrings a workload name must contain")
    ap.add_argument("--ceiling", action="store_true",
                    help="time the copy, read-only and write-only streams at 256 MiB, 1 GiB, "
                         "4 GiB and 16 GiB (one JSON line each)")
    ap.add_argument("--graph", action="store_true",
                    help="time one replay of a HIP graph of the steps (kernel and copy) "
                         "instead of launches from the host")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(rows would shard across GPUs with no exchange between them)", file=sys.stderr)
        return 2

    from synth import workloads as W

    if args.ceiling:
        return ceiling(args.steps, args.out if args.out != "bench_sweep.jsonl" else None)
    if args.sweep:
        os.makedirs(os.path.dirname(args.out) or ".", exist_ok=True)
        done = set()
        if os.path.exists(args.out):
            for l in open(args.out):
                try:
                    done.add(json.loads(l)["config"]["workload"])
                except (ValueError, KeyError):
                    pass
        only = [t for t in args.only.split(",") if t]
        for w in W.FIXED + W.sweep() + W.BACKWARD + W.WIDE + W.LONG + W.UNEVEN:
            if w.name in done or (only and not all(t in w.name for t in only)):
                continue
            line = measure(w, args.steps, args.warmup, args.rotate_bytes, False, 0,
                           host_rows=args.sweep_host_rows, graph=args.graph)
            line["config"]["host_rows"] = args.sweep_host_rows
            with open(args.out, "a") as f:
                f.write(json.dumps(line) + "\n")
            print(f"{w.name:34s} {line['roofline']['achieved']:9.1f} GB/s "
                  f"({line['roofline']['frac'] * 100:5.1f}% of peak, copy "
                  f"{line['copy_ceiling']['value']:7.1f})", flush=True)
        return 0

    line = measure(W.by_name(args.workload), args.steps, args.warmup, args.rotate_bytes,
                   not args.no_cpu_baseline, args.cpu_seconds, graph=args.graph)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
