#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X.

A step is one decode step over the whole batch: fd_decode_partial followed by
fd_decode_combine (every query head of every sequence, one new token each),
through the C ABI of libfd.so. Inputs are seeded synthetic tensors already in
HBM when timing starts.

Printed (one JSON line): effective KV bandwidth = counted K+V bytes of the
step (valid keys only) / step time, its fraction of the 8 TB/s HBM peak, the
step time, a roofline object for the partial kernel (its launches timed live
as a region of back-to-back launches with HIP events on the launch stream),
and the fp64 CPU oracle timed on the host over the same workload
("cpu_baseline"), whose outputs also check the GPU result. The default
workload (long-mha) is followed by the other long-context workload, the paged
batch, timed the same way and checked on every output row ("paged_leg").

Workloads (--workload):
  long-mha      batch 4, 32 heads (MHA), head_dim 128, 131072 keys, bf16 (default)
  gqa-32k       batch 1, 32 query / 8 KV heads, 32768 keys, bf16, 64 splits
  paged         batch 16, lengths U[1024, 65536], 32/8 heads, page 16, bf16
  short-batch   batch 128, lengths U[256, 2048], 32/8 heads, bf16
and, beyond those five shapes:
  long-mha-fp8  long-mha with an fp8 (E4M3) cache and per-head scales
  paged-fp8     paged with an fp8 cache
  paged-spec4   paged with 4 query tokens per sequence (multi-token decode,
                causal window), so each KV head's 4 x 4 query rows fill one
                16-row matrix tile
  tiny-fp32     the parity-size case: batch 1, one head, head_dim 64, 1000
                fp32 keys, 4 splits, +30 on three keys' scores (launch-bound;
                for the oracle's single-core figure)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# Element-wise bf16 output tolerance |gpu - ref| <= ATOL + RTOL |ref|; fp32
# outputs: per row max|gpu - ref| / max|ref| <= FP32_ROW_TOL.
BF16_ATOL, BF16_RTOL = 2e-3, 1e-2
FP32_ROW_TOL = 1e-5
METRIC = "decode-attn effective KV HBM GB/s and % of peak; us per decode step"
REGION_REPEATS = 5   # extra timed regions of --steps steps, for the spread of the step time
KERNEL_SRC = os.path.join(ROOT, "decode_attention_12_amd", "csrc", "fd_kernels.hip")


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="long-mha", choices=["long-mha", "gqa-32k", "paged", "short-batch",
                                                                "long-mha-fp8", "paged-fp8", "paged-spec4",
                                                                "tiny-fp32"])
    ap.add_argument("--splits", type=int, default=None, help="force the split count (0 = planner)")
    ap.add_argument("--workers", type=int, default=None, help="override the worker count of a balanced plan")
    ap.add_argument("--lead-pct", type=int, default=None,
                    help="balanced plan: share of the first half of the workers, in percent of the others' (0 = even)")
    ap.add_argument("--path", choices=["auto", "valu", "mfma"], default="auto",
                    help="override the planner's kernel path (auto = keep it)")
    ap.add_argument("--copies", type=int, default=None, help="KV copies rotated across steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-second-leg", action="store_true",
                    help="long-mha only: skip the paged workload that the default run also times")
    ap.add_argument("--fused", action="store_true", help="one fd_decode launch per step instead of partial + combine")
    ap.add_argument("--graph", action="store_true",
                    help="also time the K steps captured in one HIP graph and replayed (kernels_us.graph_*)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB per step (counter calibration)")
    return ap.parse_args()


def kernel_source_hash() -> str:
    """Hash of the kernel source with comments and blank space removed, so
    that a comment edit does not orphan the recorded counters."""
    with open(KERNEL_SRC) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    text = re.sub(r"\s+", " ", text).strip()
    return hashlib.sha256(text.encode()).hexdigest()[:16]


def recorded_traffic(workload: str):
    """HBM bytes per partial launch from the committed counter summary, if it
    was taken on this workload with the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"fd_partial_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    src = re.search(r"kernel_source_sha256[^:]*:\s*([0-9a-f]+)", text)
    if not src or src.group(1) != kernel_source_hash():
        return None
    m = re.search(rf"traffic_bytes_per_launch\[{re.escape(workload)}\]:\s*([0-9.eE+]+)", text)
    return float(m.group(1)) if m else None


def make_workload(name, device):
    import workloads
    if name == "long-mha":
        return workloads.c3_long_mha(device=device), 1
    if name == "gqa-32k":
        return workloads.c2_gqa_32k(device=device), 4
    if name == "paged":
        return workloads.c4_paged(device=device), 1
    if name == "long-mha-fp8":
        return workloads.c3_long_mha(device=device, dtype=workloads.FP8), 1
    if name == "paged-fp8":
        return workloads.c4_paged(device=device, dtype=workloads.FP8), 1
    if name == "paged-spec4":
        return workloads.c4_paged(device=device, q_len=4), 1
    if name == "tiny-fp32":
        return workloads.c1_tiny_fp32("outliers", device=device), 1
    return workloads.c5_short_batch(device=device), 2


def copy_calibration(args):
    """A plain copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = args.copy_calibration << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").random_(0, 255)
    dst = torch.empty_like(src)
    for _ in range(args.warmup + args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": args.warmup + args.steps}))


def host_cpu() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# hipDeviceAttribute_t values (hip_runtime_api.h): peak clocks in kHz, bus width in bits.
_HIP_ATTR_CLOCK_RATE, _HIP_ATTR_MEM_BUS_WIDTH, _HIP_ATTR_MEM_CLOCK_RATE = 5, 59, 60


def device_info(torch) -> dict:
    p = torch.cuda.get_device_properties(0)
    info = {"name": p.name, "gcn_arch": getattr(p, "gcnArchName", ""), "cus": p.multi_processor_count}
    try:
        import ctypes
        hip = ctypes.CDLL("libamdhip64.so")
        for key, attr, scale in (("clock_mhz", _HIP_ATTR_CLOCK_RATE, 1000),
                                 ("mem_clock_mhz", _HIP_ATTR_MEM_CLOCK_RATE, 1000),
                                 ("mem_bus_bits", _HIP_ATTR_MEM_BUS_WIDTH, 1)):
            val = ctypes.c_int(0)
            if hip.hipDeviceGetAttribute(ctypes.byref(val), attr, torch.cuda.current_device()) == 0:
                info[key] = val.value // scale
    except OSError:
        pass
    return info


def cpu_baseline(x, out_gpu):
    """The fp64 oracle over the whole workload on the host cores, timed; its
    outputs also check the GPU outputs element by element."""
    import torch
    import oracle
    t0 = time.time()
    q, k, v, lens = x.q.cpu(), x.k.cpu(), x.v.cpu(), x.seq_lens.cpu()
    bt = x.block_table.cpu() if x.block_table is not None else None
    sc = {} if x.k_scale is None else {"k_scale": x.k_scale.cpu(), "v_scale": x.v_scale.cpu()}
    copy_s = time.time() - t0
    threads = oracle.num_threads()
    oracle.attention(q, k, v, lens, scale=x.scale, block_table=bt, page_size=x.page_size, rows=[(0, 0)],
                     **sc)  # warm pool
    times = []
    ref = None
    for _ in range(3):
        t = time.time()
        ref, ref_lse = oracle.attention(q, k, v, lens, scale=x.scale, block_table=bt, page_size=x.page_size, **sc)
        times.append(time.time() - t)
    t_med = statistics.median(times)
    excess = parity_excess(out_gpu, ref)
    single = None
    if x.kv_bytes <= (256 << 20):
        # Small workloads: the same oracle on one core as well.
        oracle.set_num_threads(1)
        t = time.time()
        oracle.attention(q, k, v, lens, scale=x.scale, block_table=bt, page_size=x.page_size, **sc)
        t_single = time.time() - t
        single = round(x.kv_bytes / t_single / 1e9, 3)
        oracle.set_num_threads(threads)
    return {
        "value": round(x.kv_bytes / t_med / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
        "single_core_value": single, "host_cpu": host_cpu(), "host_nproc": os.cpu_count(),
        "sample": f"whole workload ({x.batch * x.q_len * x.num_q_heads} rows, {x.kv_bytes} KV bytes), fp64, "
                  "median of 3",
        "us_per_step": round(t_med * 1e6, 1), "host_copy_s": round(copy_s, 2),
        "single_core_us_per_step": None if single is None else round(t_single * 1e6, 1),
        "parity_max_err_over_tol": round(excess, 4),
    }


def parity_excess(out_gpu, ref):
    """Largest error over its tolerance (the check passes at <= 1): fp32
    outputs per row, max|gpu - ref| / max|ref| over 1e-5; bf16 outputs per
    element, |gpu - ref| over 2e-3 + 1e-2 |ref|."""
    import torch
    got = out_gpu.double().cpu().reshape(ref.shape)
    if out_gpu.dtype == torch.float32:
        return ((got - ref).abs().amax(dim=-1) / ref.abs().amax(dim=-1)).max().item() / FP32_ROW_TOL
    return ((got - ref).abs() / (BF16_ATOL + BF16_RTOL * ref.abs())).max().item()


class Leg:
    """One workload's timed decode steps on the launch stream: the whole step
    (partial + combine, or the single fd_decode launch), and the partial
    launch and the combine launch each timed as their own region of back to
    back launches (events only at the region ends, so no event sits between
    kernels; a region's average includes the launch gaps, so the partial's
    figure cannot exceed the step's)."""

    def __init__(self, name, args, fd, torch, dev, *, splits=None, copies=None):
        self.name, self.args, self.fd, self.torch = name, args, fd, torch
        x, default_copies = make_workload(name, dev)
        self.x = x
        self.copies = copies or default_copies
        self.kv = [(x.k, x.v)] + [(x.k.clone(), x.v.clone()) for _ in range(self.copies - 1)]
        splits = x.num_splits if splits is None else splits
        self.problem = fd.problem_of(x.q, x.k, x.max_seq_len, out_dtype=x.out_dtype, page_size=x.page_size,
                                     num_pages=x.num_pages)
        self.plan = fd.fd_plan_splits(self.problem, 0, splits)
        # Zeroed once: fd_decode needs its piece counters at zero before first use.
        self.ws = torch.zeros(fd.fd_workspace_size(self.problem, self.plan), dtype=torch.uint8, device=dev)
        self.out = torch.empty(x.q.shape, dtype=x.out_dtype, device=dev)
        self.layout = fd.layout_of(x.k, x.k_scale, x.v_scale)
        self.stream = torch.cuda.current_stream()

    def partial(self, i):
        x, fd = self.x, self.fd
        k, v = self.kv[i % self.copies]
        if self.args.fused:
            fd.fd_decode(self.problem, self.plan, x.q, k, v, self.layout, x.seq_lens, self.ws, self.out, None,
                         scale=x.scale, block_table=x.block_table, stream=self.stream)
        else:
            fd.fd_decode_partial(self.problem, self.plan, x.q, k, v, self.layout, x.seq_lens, self.ws, scale=x.scale,
                                 block_table=x.block_table, stream=self.stream)

    def combine(self):
        if not self.args.fused:
            self.fd.fd_decode_combine(self.problem, self.plan, self.ws, self.out, None, stream=self.stream)

    def region(self, body, steps):
        """Average milliseconds per iteration of `body` over `steps` back-to-back iterations."""
        torch = self.torch
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(self.stream)
        for i in range(steps):
            body(i)
        e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    def step(self, i):
        self.partial(i)
        self.combine()

    def per_step(self, steps):
        """p10 / p50 / p90 of single-step times (ms) over `steps` back-to-back
        steps, an event recorded between every two (the events add a little to
        each figure)."""
        torch = self.torch
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        torch.cuda.synchronize()
        evs[0].record(self.stream)
        for i in range(steps):
            self.step(i)
            evs[i + 1].record(self.stream)
        torch.cuda.synchronize()
        ts = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(steps))
        return {q: ts[min(steps - 1, int(f * steps))] for q, f in (("p10", 0.1), ("p50", 0.5), ("p90", 0.9))}

    def graph_region(self, body, steps):
        """Average milliseconds per iteration of `body` with `steps` iterations
        captured in one HIP graph and the graph replayed (no host launch
        overhead between kernels); the median of 3 replays after one untimed."""
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        eager_stream = self.stream
        with torch.cuda.graph(g):
            self.stream = torch.cuda.current_stream()
            for i in range(steps):
                body(i)
        self.stream = eager_stream
        g.replay()
        torch.cuda.synchronize()
        times = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(self.stream)
            g.replay()
            e1.record(self.stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) / steps)
        del g
        return statistics.median(times)

    def run(self):
        args, torch = self.args, self.torch
        for i in range(args.warmup):
            self.step(i)
        torch.cuda.synchronize()
        t_wall = time.perf_counter()
        step_ms = self.region(self.step, args.steps)
        wall_ms = (time.perf_counter() - t_wall) * 1e3 / args.steps
        repeats = sorted(self.region(self.step, args.steps) for _ in range(REGION_REPEATS))
        singles = self.per_step(args.steps)
        part_ms = [self.region(self.partial, args.steps) for _ in range(3)]
        comb_ms = [self.region(lambda i: self.combine(), args.steps) for _ in range(3)] if not args.fused else [0.0]
        t = {"step_ms": step_ms, "wall_ms": wall_ms, "repeats": repeats, "singles": singles,
             "partial_ms": statistics.median(part_ms), "combine_ms": statistics.median(comb_ms)}
        if args.graph:
            # The same K steps as one captured graph; the replay's last step
            # must leave the outputs an eager step over the same inputs does.
            t["graph_step_ms"] = self.graph_region(self.step, args.steps)
            t["graph_partial_ms"] = self.graph_region(self.partial, args.steps)
            t["graph_combine_ms"] = (self.graph_region(lambda i: self.combine(), args.steps)
                                     if not args.fused else 0.0)
            self.graph_region(self.step, args.steps)
            torch.cuda.synchronize()
            replayed = self.out.clone()
            self.step(args.steps - 1)
            torch.cuda.synchronize()
            t["graph_matches_eager"] = bool(torch.equal(replayed, self.out))
        self.step(0)   # leave the outputs of a whole step in self.out
        torch.cuda.synchronize()
        return t

    def config(self):
        fd, plan, x = self.fd, self.plan, self.x
        return {**x.describe(), "num_splits": plan.num_splits, "chunk_len": plan.chunk_len, "path": plan.path_name,
                "mode": "balanced" if plan.mode == fd.FD_MODE_BALANCED else "splits", "workers": plan.workers,
                "lead_workers": plan.lead_workers, "lead_pct": plan.lead_pct,
                "launches_per_step": 1 if self.args.fused else 2, "kv_copies_rotated": self.copies,
                "counted_kv_bytes": x.kv_bytes, "workspace_bytes": self.ws.numel()}

    def overhead(self):
        """Bytes a step moves besides the counted K/V (reported, not in the
        metric): query rows, outputs and LSEs, the block-table entries in use,
        the lengths, and the records, which the partial writes once and the
        combine reads once (at most the workspace each way)."""
        x, torch = self.x, self.torch
        rows = x.q.numel() // x.head_dim
        out_esz = torch.tensor([], dtype=x.out_dtype).element_size()
        pages = sum(-(-L // x.page_size) for L in x.seq_lens_host) if x.page_size else 0
        return {"q": x.q.numel() * x.q.element_size(), "out": rows * x.head_dim * out_esz, "lse_out": 4 * rows,
                "block_table": 4 * pages, "seq_lens": 4 * x.batch,
                "records_written_and_read_at_most": 2 * self.ws.numel()}

    def free(self):
        self.kv = self.x = self.ws = self.out = None
        self.torch.cuda.empty_cache()


def oracle_parity(x, out_gpu):
    """Every output row against the fp64 oracle over the whole workload:
    the largest |gpu - ref| / (ATOL + RTOL |ref|) (the check passes at <= 1)."""
    import oracle
    q, k, v, lens = x.q.cpu(), x.k.cpu(), x.v.cpu(), x.seq_lens.cpu()
    bt = x.block_table.cpu() if x.block_table is not None else None
    sc = {} if x.k_scale is None else {"k_scale": x.k_scale.cpu(), "v_scale": x.v_scale.cpu()}
    ref, _ = oracle.attention(q, k, v, lens, scale=x.scale, block_table=bt, page_size=x.page_size, **sc)
    return parity_excess(out_gpu, ref)


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the library runs on one GPU "
              "(a multi-GPU step would shard by KV head or sequence and exchange only the small merge records)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_calibration:
        copy_calibration(args)
        return
    import decode_attention_12_amd as fd

    dev = torch.device("cuda:0")
    leg = Leg(args.workload, args, fd, torch, dev, splits=args.splits, copies=args.copies)
    # The second leg's inputs are made now, before anything is freed: made
    # after the 8.6 GB of the first workload had been freed, the paged pool
    # streamed ~4 % slower than in a process of its own (its random page
    # order meets a fragmented address space).
    second = None
    if args.workload == "long-mha" and not args.no_second_leg:
        second = Leg("paged", args, fd, torch, dev)
    plan = leg.plan
    if args.workers and plan.mode == fd.FD_MODE_BALANCED:
        plan.workers = args.workers
    if args.lead_pct is not None and plan.mode == fd.FD_MODE_BALANCED:
        plan.lead_pct = args.lead_pct
        plan.lead_workers = plan.workers // 2 if args.lead_pct else 0
    if args.path != "auto":
        plan.path = {"valu": fd.FD_PATH_VALU, "mfma": fd.FD_PATH_MFMA}[args.path]
    if fd.fd_workspace_size(leg.problem, plan) > leg.ws.numel():
        leg.ws = torch.zeros(fd.fd_workspace_size(leg.problem, plan), dtype=torch.uint8, device=dev)
    t = leg.run()
    x = leg.x
    step_ms, part_ms = t["step_ms"], t["partial_ms"]
    gbs = x.kv_bytes / (step_ms * 1e-3) / 1e9
    achieved = x.kv_bytes / (part_ms * 1e-3) / 1e9
    rep = t["repeats"]
    line = {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(step_ms, 5), "us_per_step": round(step_ms * 1e3, 2),
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": str(x.k.dtype).replace("torch.", ""), "data": "synthetic",
        "config": leg.config(),
        "overhead_bytes": leg.overhead(),
        "kernels_us": {"partial_region_avg": round(part_ms * 1e3, 2),
                       "combine_region_avg": round(t["combine_ms"] * 1e3, 2),
                       "step_median_of_repeats": round(rep[len(rep) // 2] * 1e3, 2),
                       "step_min_of_repeats": round(rep[0] * 1e3, 2),
                       "step_max_of_repeats": round(rep[-1] * 1e3, 2),
                       **{f"single_step_{q}": round(v * 1e3, 2) for q, v in t["singles"].items()},
                       "host_wall_per_step": round(t["wall_ms"] * 1e3, 2),
                       **({"graph_step_avg": round(t["graph_step_ms"] * 1e3, 2),
                           "graph_partial_avg": round(t["graph_partial_ms"] * 1e3, 2),
                           "graph_combine_avg": round(t["graph_combine_ms"] * 1e3, 2),
                           "graph_matches_eager": t["graph_matches_eager"]} if args.graph else {})},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if args.fused else recorded_traffic(args.workload),
                     "kernel": "decode (partial + merge)" if args.fused else "partial",
                     "kernel_time": "average over back-to-back launches, events at the region ends",
                     "algorithmic_bytes_per_launch": x.kv_bytes},
        "cpu_baseline": None,
        "device": device_info(torch),
    }
    tp = None
    if second is not None:
        # The other long-context workload: the paged GQA batch, timed the same
        # way right after the first (before the host-side oracle work below,
        # while the device is still busy), every output row checked against
        # the oracle afterwards.
        tp = second.run()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(x, leg.out)
    if second is not None:
        leg.free()
        pg = second
        pgbs = pg.x.kv_bytes / (tp["step_ms"] * 1e-3) / 1e9
        line["paged_leg"] = {
            "config": pg.config(), "overhead_bytes": pg.overhead(),
            "us_per_step": round(tp["step_ms"] * 1e3, 2), "value": round(pgbs, 2),
            "unit": "GB/s", "pct_of_hbm_peak": round(100 * pgbs / HBM_PEAK_GBS, 2),
            "us_per_step_median_of_repeats": round(tp["repeats"][len(tp["repeats"]) // 2] * 1e3, 2),
            "partial_region_avg_us": round(tp["partial_ms"] * 1e3, 2),
            "combine_region_avg_us": round(tp["combine_ms"] * 1e3, 2),
            "partial_frac_of_peak": round(pg.x.kv_bytes / (tp["partial_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "parity_max_err_over_tol": round(oracle_parity(pg.x, pg.out), 4),
            "parity": "every output row against the fp64 oracle, |gpu - ref| <= 2e-3 + 1e-2 |ref|",
        }
        pg.free()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
