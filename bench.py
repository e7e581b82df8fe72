#!/usr/bin/env python3
"""Throughput of the unified paged attention forward pass on one MI355X.

A step is one ``ua_run`` over one batch of synthetic inputs already resident in
HBM: the host plan, then the attention kernel (and, on the split-KV path, the
log-sum-exp reduce).  The default workload is the decode batch (64 sequences,
S_k ~ U{512..8192}, H_q/H_k = 32/8, d = 128, b = 16, bf16, causal), which is
HBM-bound: its value is algorithmic GB/s.  MFMA-bound workloads report
TFLOP/s.  One JSON line is printed.

Algorithmic work (counted from the realised lengths):
  bytes = K+V of every key visible to at least one row, once per (sequence,
          KV head) + Q + O + the block-table entries of visited blocks +
          sequence metadata (+ slopes / sinks);
  flops = 4 d per visible (query row, key, query head) triple.
The roofline object prices the dominant (attention) kernel alone: its bytes
(the above without O when a reduce kernel writes O) or flops per launch over
its mean duration, from HIP events recorded around it on its own stream.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 / fp16 MFMA
METRIC = "paged-attn TFLOPS (prefill) & HBM GB/s (decode) on 1 MI355X, % of roofline"
CSRC = os.path.join(ROOT, "varlen_attention_serving_amd", "csrc")


def algorithmic_work(w):
    """Visible (row, key) pairs and visited keys per sequence, from lengths."""
    pairs = 0
    visited = np.zeros(w.num_seqs, dtype=np.int64)
    blocks = 0
    for s in range(w.num_seqs):
        ql, sk = int(w.q_lens[s]), int(w.seq_lens[s])
        if ql == 0:
            continue
        ctx = sk - ql
        q_abs = ctx + np.arange(ql, dtype=np.int64)
        kmax = np.minimum(q_abs, sk - 1) if w.causal else np.full(ql, sk - 1)
        kmin = np.maximum(q_abs - w.window + 1, 0) if w.window > 0 else np.zeros(ql, np.int64)
        pairs += int((kmax - kmin + 1).sum())
        lo, hi = int(kmin[0]), int(kmax[-1])
        visited[s] = hi - lo + 1
        blocks += hi // w.block_size - lo // w.block_size + 1
    esz_kv = 1 if w.kv_dtype == 2 else 2
    kv_bytes = int(visited.sum()) * w.num_kv_heads * w.head_dim * esz_kv * 2
    q_bytes = w.total_q * w.num_q_heads * w.head_dim * 2
    # paged: one table entry per visited block, S_k and cu_seqlens_q; dense:
    # cu_seqlens_q and cu_seqlens_k only
    meta = (2 * (w.num_seqs + 1) * 4 if getattr(w, "dense", False)
            else blocks * 4 + w.num_seqs * 4 + (w.num_seqs + 1) * 4)
    meta += (w.num_q_heads * 4 if w.use_alibi else 0) + (w.num_q_heads * 4 if w.use_sinks else 0)
    flops = 4 * w.head_dim * w.num_q_heads * pairs
    dense_flops = 4 * w.head_dim * w.num_q_heads * int(
        (w.q_lens.astype(np.int64) * w.seq_lens.astype(np.int64)).sum())
    return dict(kv_bytes=kv_bytes, q_bytes=q_bytes, o_bytes=q_bytes, meta_bytes=meta,
                bytes=kv_bytes + 2 * q_bytes + meta, flops=flops, dense_flops=dense_flops,
                pairs=pairs, visited_keys=int(visited.sum()))


class ClockSampler:
    """GFX (SCLK) and memory (MCLK) clocks of the benchmarked GPU, sampled by
    amdsmi on a host thread while the timed steps run (the pages note a
    25-30% automatic clock swing, so a figure without its clock is hard to
    compare).  Any failure leaves a reason instead of samples."""

    def __init__(self, period_s=0.001):
        import threading
        self.period = period_s
        self.samples = []
        self.error = None
        self.handle = None
        self._stop = threading.Event()
        self._thread = None
        try:
            import amdsmi
            import torch
            self.smi = amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            props = torch.cuda.get_device_properties(torch.cuda.current_device())
            want = (getattr(props, "pci_domain_id", 0), getattr(props, "pci_bus_id", -1),
                    getattr(props, "pci_device_id", -1))
            for h in handles:
                bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)  # "dddd:bb:dd.f"
                dom, bus, rest = bdf.split(":")
                if (int(dom, 16), int(bus, 16), int(rest.split(".")[0], 16)) == want:
                    self.handle = h
            if self.handle is None and len(handles) == 1:
                self.handle = handles[0]
            if self.handle is None:
                self.error = f"no amdsmi device matches PCI {want}"
        except Exception as e:  # no amdsmi, no permission, ...
            self.error = f"{type(e).__name__}: {e}"

    def _read(self):
        # the firmware's metrics table: one current gfx clock per XCD, and the
        # memory (UMC) clock
        mt = self.smi.amdsmi_get_gpu_metrics_info(self.handle)
        xcd = [float(v) for v in (mt.get("current_gfxclks") or [])
               if isinstance(v, (int, float)) and v > 0]
        g = float(np.mean(xcd)) if xcd else float(mt["current_gfxclk"])
        return g, float(mt["current_uclk"])

    def _loop(self):
        while not self._stop.is_set():
            try:
                self.samples.append(self._read() + (time.perf_counter(),))
            except Exception as e:
                self.error = f"{type(e).__name__}: {e}"
                return
            self._stop.wait(self.period)

    def start(self):
        import threading
        if self.handle is not None:
            self._thread = threading.Thread(target=self._loop, daemon=True)
            self._thread.start()

    def stop(self):
        if self._thread is not None:
            self._stop.set()
            self._thread.join()
        if self.handle is not None:
            try:
                self.smi.amdsmi_shut_down()
            except Exception:
                pass
        if not self.samples:
            return {"samples": 0, "error": self.error or "no samples"}
        s = np.array(self.samples)
        window = float(s[-1, 2] - s[0, 2])
        # The metrics table refreshes slowly: values read before its first
        # change after the start describe the idle GPU, so they are dropped.
        moved = np.nonzero(s[:, 0] != s[0, 0])[0]
        if len(moved) == 0:
            return {"samples": len(s), "window_s": round(window, 3),
                    "note": "the firmware clock table did not refresh during the timed steps "
                            "(it lags by tens of ms); run more --steps to read clocks"}
        live = s[moved[0]:]
        return {"samples": len(live), "window_s": round(window, 3),
                "gfx_mhz_median": round(float(np.median(live[:, 0])), 1),
                "gfx_mhz_min": round(float(live[:, 0].min()), 1),
                "gfx_mhz_max": round(float(live[:, 0].max()), 1),
                "mem_mhz_median": round(float(np.median(live[:, 1])), 1)}


def kernel_source_hash():
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def load_traffic(workload, path_id):
    """HBM bytes per launch of the attention kernel from the committed counter
    summary, if it was taken on the current kernel sources; else None."""
    f = os.path.join(ROOT, "profiles", f"{workload}_hbm_traffic.json")
    if not os.path.exists(f):
        return None
    with open(f) as fh:
        t = json.load(fh)
    if t.get("kernel_source_hash") != kernel_source_hash() or t.get("path") != path_id:
        return None
    return t.get("bytes_per_launch")


def _counter_per_launch(csv_path, kernel_substr, counter):
    import csv
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(csv_path))
            if kernel_substr in r["Kernel_Name"] and r["Counter_Name"] == counter]
    if not vals:
        raise SystemExit(f"no {counter} rows for {kernel_substr} in {csv_path}")
    return float(np.mean(vals)), len(vals)


ATTENTION_KERNELS = ("ua_decode_sk_kernel", "ua_decode16_kernel", "ua_attn_lds_kernel",
                     "ua_attn_kernel")


def _plan(args):
    """The bench's plan for the workload (host-side query, no GPU)."""
    from varlen_attention_serving_amd import binding as B
    from varlen_attention_serving_amd import device as D
    from varlen_attention_serving_amd import workloads as W
    w = W.named(args.workload)
    extra = {"auto": 0, "2d": B.UA_FLAG_FORCE_2D, "3d": B.UA_FLAG_FORCE_3D}[args.force]
    h = B.ua_create_problem(D.problem_desc(w, extra, split_segment_tiles=args.segment_tiles))
    try:
        return B.ua_query_plan(h, w.num_seqs, w.total_q, w.max_seqlen_q, w.max_seqlen_k)
    finally:
        B.ua_destroy_problem(h)


def summarize_traffic(args):
    """HBM bytes per launch of the attention kernel from rocprofv3 --pmc CSVs
    (FETCH_SIZE and WRITE_SIZE runs of this bench, and of --copy-calibration),
    each scaled by what the counter reads for the plain copy of known size."""
    fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, copy_bytes = args.summarize_traffic
    copy_bytes = int(copy_bytes)
    cf, _ = _counter_per_launch(copy_fetch_csv, "copyBuffer", "FETCH_SIZE")
    cw, _ = _counter_per_launch(copy_write_csv, "copyBuffer", "WRITE_SIZE")
    f_scale = copy_bytes / (cf * 1024.0)
    w_scale = copy_bytes / (cw * 1024.0)
    out = {"workload": args.workload, "kernel_source_hash": kernel_source_hash(),
           "copy_calibration_bytes": copy_bytes,
           "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4), "kernels": {}}
    for sub in ATTENTION_KERNELS + ("ua_reduce_kernel",):
        try:
            f, n = _counter_per_launch(fetch_csv, sub, "FETCH_SIZE")
            wv, _ = _counter_per_launch(write_csv, sub, "WRITE_SIZE")
        except SystemExit:
            continue
        out["kernels"][sub] = {"fetch_kib_raw": round(f, 1), "write_kib_raw": round(wv, 1),
                               "bytes_read": round(f * 1024 * f_scale),
                               "bytes_written": round(wv * 1024 * w_scale), "launches": n}
    # the dominant kernel: the attention launch that reads the most (a class
    # split's other launch may find no rows of its class)
    att = max((k for k in out["kernels"] if k in ATTENTION_KERNELS),
              key=lambda k: out["kernels"][k]["bytes_read"])
    plan = _plan(args)
    out["path"] = plan.path
    if plan.class_split:
        # the timed span of a class split holds both attention launches and
        # the stream-K reduce: price their traffic together
        out["attention_kernel"] = "+".join(sorted(out["kernels"]))
        out["bytes_per_launch"] = sum(k["bytes_read"] + k["bytes_written"]
                                      for k in out["kernels"].values())
    else:
        out["attention_kernel"] = att
        a = out["kernels"][att]
        out["bytes_per_launch"] = a["bytes_read"] + a["bytes_written"]
    path = os.path.join(ROOT, "profiles", f"{args.workload}_hbm_traffic.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    print(json.dumps(out, indent=1))


def cpu_baseline(w, budget_s):
    """The oracle, untuned, on whole sequences drawn in a seeded order until
    about `budget_s` of wall time; reported in the metric's unit."""
    import oracle
    threads = oracle.default_threads()
    order = np.random.default_rng(123).permutation(w.num_seqs)
    done_bytes = done_flops = 0
    seqs = 0
    t_total = 0.0
    passes = 0
    while t_total < budget_s:
        for s in order:
            lo, hi = int(w.cu_seqlens_q[s]), int(w.cu_seqlens_q[s + 1])
            if hi == lo:
                continue
            rows = np.arange(lo * w.num_q_heads, hi * w.num_q_heads, dtype=np.int64)
            t0 = time.perf_counter()
            oracle.rows(w, rows, nthreads=threads)
            t_total += time.perf_counter() - t0
            a = algorithmic_work(_subset(w, s))
            done_bytes += a["bytes"]
            done_flops += a["flops"]
            seqs += 1
            if t_total >= budget_s:
                break
        passes += 1
    return dict(seconds=t_total, bytes=done_bytes, flops=done_flops, seqs=seqs, cores=threads,
                passes=passes)


def _subset(w, s):
    import copy
    sub = copy.copy(w)
    sub.q_lens = w.q_lens[s:s + 1]
    sub.seq_lens = w.seq_lens[s:s + 1]
    sub.cu_seqlens_q = np.array([0, int(w.q_lens[s])], dtype=np.int32)
    return sub


def cpu_baseline_rows(w, budget_s, chunk=256):
    """The oracle, untuned, on seeded random (token, head) rows of the batch,
    chunk by chunk until about `budget_s` of wall time (for batches whose
    sequences are too long to run whole); reported work is counted per row."""
    import oracle
    threads = oracle.default_threads()
    rng = np.random.default_rng(321)
    vis = np.concatenate([_visible(w, s) for s in range(w.num_seqs)]) if w.num_seqs else []
    row_bytes = 2 * w.head_dim * (1 if w.kv_dtype == 2 else 2)
    done_flops = done_bytes = rows_done = 0
    t_total = 0.0
    while t_total < budget_s:
        rows = rng.integers(0, w.total_q * w.num_q_heads, size=chunk)
        t0 = time.perf_counter()
        oracle.rows(w, rows, nthreads=threads)
        t_total += time.perf_counter() - t0
        keys = vis[rows // w.num_q_heads]
        done_flops += int(keys.sum()) * 4 * w.head_dim
        done_bytes += int(keys.sum()) * row_bytes + 4 * w.head_dim * len(rows)
        rows_done += len(rows)
    return dict(seconds=t_total, bytes=done_bytes, flops=done_flops, rows=rows_done,
                cores=threads)


def _visible(w, s):
    """Keys visible to each local query row of sequence s."""
    ql, sk = int(w.q_lens[s]), int(w.seq_lens[s])
    q_abs = sk - ql + np.arange(ql, dtype=np.int64)
    kmax = np.minimum(q_abs, sk - 1) if w.causal else np.full(ql, sk - 1)
    kmin = np.maximum(q_abs - w.window + 1, 0) if w.window > 0 else np.zeros(ql, np.int64)
    return np.maximum(kmax - kmin + 1, 0)


class Runner:
    """One workload on the device: its batch, problem handle and plan."""

    def __init__(self, name, force="auto", segment_tiles=0, extra_flags=0, w=None):
        from varlen_attention_serving_amd import binding as B
        from varlen_attention_serving_amd import device as D
        from varlen_attention_serving_amd import workloads as W
        import torch
        self.B, self.torch = B, torch
        self.name = name
        if w is None:
            print(f"[bench] generating {name}", file=sys.stderr, flush=True)
            w = W.named(name)
        self.w = w
        extra = {"auto": 0, "2d": B.UA_FLAG_FORCE_2D, "3d": B.UA_FLAG_FORCE_3D}[force] | extra_flags
        self.batch = D.DeviceBatch(w)
        self.ua = D.UnifiedAttention(D.problem_desc(w, extra, split_segment_tiles=segment_tiles))
        self.plan = self.ua.plan(w)
        self.work = algorithmic_work(w)
        self.t_hbm = self.work["bytes"] / (HBM_PEAK_GBS * 1e9)
        self.t_mfma = self.work["flops"] / (BF16_PEAK_TFLOPS * 1e12)
        self.bound = "hbm" if self.t_hbm >= self.t_mfma else "mfma"
        self.stream = torch.cuda.current_stream()
        self.args = self.batch.run_args(self.ua.workspace)

    def step(self):
        self.B.ua_run(self.ua.handle, self.args, self.stream.cuda_stream)

    def time(self, steps, warmup, every=4, flush=None):
        """Warm-up, then `steps` timed steps.  HIP events around the kernels
        of every `every`-th step (every step with a flush); with `flush` (a
        callable that evicts the caches) it runs before each step, outside
        the events, and the step time is the events' sum."""
        torch = self.torch
        print(f"[bench] {self.name}: plan path={self.plan.path} split={self.plan.class_split} "
              f"stream_k={self.plan.stream_k} waves={self.plan.waves} "
              f"segments={self.plan.num_segments}; warmup {warmup}, "
              f"{steps} steps{' (cold)' if flush else ''}", file=sys.stderr, flush=True)
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        # Recording events costs GPU time (about 10 us per step on the decode
        # batch), so warm runs time the kernels on every `every`-th step only
        # and leave the other steps as the workload runs in service.
        every = 1 if flush else max(1, every)
        sampled = list(range(0, steps, every))
        evs = {i: [torch.cuda.Event(enable_timing=True) for _ in range(3)] for i in sampled}
        for trio in evs.values():
            for e in trio:
                e.record(self.stream)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            if flush is not None:
                flush()
            for j in range(3):
                self.args.timing_events[j] = evs[i][j].cuda_event if i in evs else None
            self.step()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        for j in range(3):
            self.args.timing_events[j] = None
        attn = np.array([evs[i][0].elapsed_time(evs[i][1]) for i in sampled])
        whole = np.array([evs[i][0].elapsed_time(evs[i][2]) for i in sampled])
        return dict(wall_ms=wall * 1e3 / steps, attn=attn, whole=whole, sampled=len(sampled))

    def figures(self, t):
        """Throughput and roofline from one timing: `value` over the wall
        clock (warm) or the summed events (cold); the roofline prices the
        attention kernel alone over its own events."""
        work, plan = self.work, self.plan
        attn_ms = float(np.mean(t["attn"]))
        whole_ms = float(np.mean(t["whole"]))
        if self.bound == "hbm":
            per = lambda units, ms: units / (ms * 1e-3) / 1e9
            units = work["bytes"]
            # a split run's reduce writes O: the attention kernel does not
            kernel_units = units - (work["o_bytes"] if plan.path == 3 else 0)
            peak, unit = HBM_PEAK_GBS, "GB/s"
        else:
            per = lambda units, ms: units / (ms * 1e-3) / 1e12
            units = kernel_units = work["flops"]
            peak, unit = BF16_PEAK_TFLOPS, "TFLOP/s"
        achieved = per(kernel_units, attn_ms)
        return dict(attn_ms=attn_ms, whole_ms=whole_ms, unit=unit, peak=peak,
                    achieved=achieved, frac=achieved / peak,
                    value_wall=per(units, t["wall_ms"]), value_events=per(units, whole_ms),
                    frac_whole_forward=max(self.t_hbm, self.t_mfma) / (whole_ms * 1e-3))

    def roofline(self, f, traffic_workload=None):
        name = traffic_workload or self.name
        traffic = load_traffic(name, self.plan.path)
        return {"bound": self.bound, "achieved": round(f["achieved"], 3), "peak": f["peak"],
                "unit": f["unit"], "frac": round(f["frac"], 4), "traffic": traffic,
                "scope": ("the attention kernel alone, over HIP events on its stream"
                          + ("; the split-KV reduce (which writes O) and O's bytes excluded"
                             if self.plan.path == 3 and self.bound == "hbm" else "")),
                "traffic_source": (f"profiles/{name}_hbm_traffic.json: rocprofv3 --pmc "
                                   "FETCH_SIZE + WRITE_SIZE per launch on these kernel sources"
                                   if traffic is not None else
                                   "no counter summary on the current kernel sources")}

    def config(self):
        w, plan, work = self.w, self.plan, self.work
        return {"workload": self.name,
                "num_seqs": w.num_seqs, "total_q": w.total_q, "max_seqlen_k": w.max_seqlen_k,
                "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
                "head_dim": w.head_dim, "block_size": w.block_size,
                "kv_layout": "dense (cu_seqlens_k)" if w.dense else "paged (block table)",
                "path": {2: "2d", 3: "3d-split-kv"}[plan.path], "segments": plan.num_segments,
                "class_split": bool(plan.class_split), "stream_k": bool(plan.stream_k),
                "algorithmic_bytes": work["bytes"], "algorithmic_flops": work["flops"],
                "dense_equivalent_flops": work["dense_flops"]}

    def dtype(self):
        return {0: "bf16", 1: "f16"}[self.w.q_dtype] + ("+fp8kv" if self.w.kv_dtype == 2 else "")

    def close(self):
        self.ua.close()
        del self.batch
        self.torch.cuda.empty_cache()


def clocks_under(runner, seconds, ms_per_step, flush=None):
    """GPU clocks during an untimed replay of the step: the firmware's table
    refreshes too slowly to be read inside a short timed region."""
    if seconds <= 0:
        return None
    clocks = ClockSampler()
    if clocks.handle is not None:
        reps = int(min(50000, max(1, seconds * 1e3 / max(ms_per_step, 1e-3))))
        clocks.start()
        for _ in range(reps):
            if flush is not None:
                flush()
            runner.step()
        runner.torch.cuda.synchronize()
    info = clocks.stop()
    info["replay"] = f"untimed replay of the step for about {seconds:g} s"
    return info


def single_thread_oracle(names=("tiny_varlen", "decode_batch"), budget_s=3.0):
    """The oracle on one host thread: the whole tiny batch, and whole
    sequences of the decode batch for about `budget_s`, in the metric's units."""
    import oracle
    out = {}
    for name in names:
        from varlen_attention_serving_amd import workloads as W
        w = W.named(name)
        if name == "tiny_varlen":
            t0 = time.perf_counter()
            reps = 0
            while time.perf_counter() - t0 < 0.5:
                oracle.attention(w, nthreads=1)
                reps += 1
            sec = (time.perf_counter() - t0) / reps
            a = algorithmic_work(w)
            out[name] = {"seconds_per_batch": round(sec, 6), "GB/s": round(a["bytes"] / sec / 1e9, 6),
                         "threads": 1, "sample": f"the whole batch, {reps} runs"}
        else:
            order = np.random.default_rng(7).permutation(w.num_seqs)
            done = 0
            t = 0.0
            seqs = 0
            for s in order:
                lo, hi = int(w.cu_seqlens_q[s]), int(w.cu_seqlens_q[s + 1])
                rows = np.arange(lo * w.num_q_heads, hi * w.num_q_heads, dtype=np.int64)
                t0 = time.perf_counter()
                oracle.rows(w, rows, nthreads=1)
                t += time.perf_counter() - t0
                done += algorithmic_work(_subset(w, s))["bytes"]
                seqs += 1
                if t >= budget_s:
                    break
            out[name] = {"GB/s": round(done / t / 1e9, 6), "threads": 1, "seconds": round(t, 2),
                         "sample": f"{seqs} whole sequences of the batch (all rows and heads)"}
    return out


def cpu_object(w, bound, unit, budget_s, by_rows):
    print(f"[bench] oracle CPU baseline on {w.name} (~{budget_s:.0f} s)", file=sys.stderr,
          flush=True)
    if by_rows:
        c = cpu_baseline_rows(w, budget_s)
        sample = (f"{c['rows']} seeded random (token, head) rows of the batch, "
                  f"{c['seconds']:.1f} s of fp64 oracle time on {c['cores']} threads")
    else:
        c = cpu_baseline(w, budget_s)
        sample = (f"{c['seqs']} sequence runs over {c['passes']} pass(es) of the "
                  f"{w.num_seqs}-sequence batch (all rows and heads of each), "
                  f"{c['seconds']:.1f} s of fp64 oracle time on {c['cores']} threads")
    value = (c["bytes"] / c["seconds"] / 1e9) if bound == "hbm" else \
        (c["flops"] / c["seconds"] / 1e12)
    return {"value": round(value, 6), "unit": unit, "cores": c["cores"], "kind": "oracle",
            "sample": sample}


def part_batches(w):
    """The parts of a batch that `--parts` times: the decode-shaped sequences
    alone (q_len * g <= 32: rows of one single-wave q-block), the others
    alone, and the whole batch with each optional feature switched off."""
    import dataclasses
    parts = [("all", w)]
    dec = [s for s in range(w.num_seqs) if int(w.q_lens[s]) * w.group <= 32]
    wide = [s for s in range(w.num_seqs) if int(w.q_lens[s]) * w.group > 32]
    if dec and wide and not w.dense:
        parts += [("decode_seqs", w.select(dec, f"{w.name}:decode_seqs")),
                  ("wide_seqs", w.select(wide, f"{w.name}:wide_seqs"))]
    off = {"softcap": dict(softcap=0.0), "alibi": dict(use_alibi=False, alibi_slopes=None),
           "sinks": dict(use_sinks=False, sinks=None), "window": dict(window=0)}
    on = {"softcap": w.softcap > 0, "alibi": w.use_alibi, "sinks": w.use_sinks,
          "window": w.window > 0}
    for feat, kw in off.items():
        if on[feat]:
            parts.append((f"no_{feat}", dataclasses.replace(w, name=f"{w.name}:no_{feat}", **kw)))
    return parts


def time_parts(args, extra_flags):
    """One JSON line with the time of each part of the workload (see
    part_batches); every part is its own batch, planned on its own."""
    from varlen_attention_serving_amd import workloads as W
    print(f"[bench] generating {args.workload}", file=sys.stderr, flush=True)
    w = W.named(args.workload)
    rows = []
    for label, pw in part_batches(w):
        r = Runner(pw.name, args.force, args.segment_tiles, extra_flags, w=pw)
        t = r.time(args.steps, args.warmup, 1)
        f = r.figures(t)
        rows.append({"part": label, "num_seqs": pw.num_seqs, "total_q": pw.total_q,
                     "plan": {"path": r.plan.path, "class_split": bool(r.plan.class_split),
                              "stream_k": bool(r.plan.stream_k), "waves": r.plan.waves,
                              "segments": r.plan.num_segments},
                     "attention_kernel_ms_median": round(float(np.median(t["attn"])), 5),
                     "gpu_ms_per_step_events_median": round(float(np.median(t["whole"])), 5),
                     "algorithmic_bytes": r.work["bytes"], "algorithmic_flops": r.work["flops"],
                     "bound": r.bound, "achieved": round(f["achieved"], 3), "unit": f["unit"],
                     "frac": round(f["frac"], 4)})
        r.close()
        print(f"[bench]   {label:12s} attn {rows[-1]['attention_kernel_ms_median']:.4f} ms  "
              f"step {rows[-1]['gpu_ms_per_step_events_median']:.4f} ms", file=sys.stderr,
              flush=True)
    print(json.dumps({"workload": args.workload, "steps": args.steps, "warmup": args.warmup,
                      "timing": "HIP events around every step, medians", "parts": rows}),
          flush=True)


def make_read_flush(torch, nbytes=1 << 30):
    """A cache flush that only reads: the sum of a `nbytes` buffer (larger
    than L2 plus the 256 MiB MALL) into one value, so no dirty lines are left
    to write back during the next timed step."""
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    sink = torch.empty((), dtype=torch.float32, device="cuda")

    def flush():
        torch.sum(buf, dim=0, out=sink)
    return flush


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode_batch",
                    choices=["decode_batch", "chunked_prefill_mix", "long_prefill",
                             "variant_mix", "tiny_varlen", "dense_prefill", "mha_prefill",
                             "d256_prefill", "decode_large"])
    ap.add_argument("--force", choices=["auto", "2d", "3d"], default="auto")
    ap.add_argument("--cold", action="store_true",
                    help="time the main workload cold: a read-only 1 GiB flush before every "
                         "step (outside the events) so no step finds K/V in L2 or the MALL; "
                         "value then comes from the summed step events")
    ap.add_argument("--extras", default="auto",
                    help="comma list of extra figures added to the line: 'cold' (the main "
                         "workload again, cold) and 'prefill' (long_prefill, the MFMA-bound "
                         "half of the metric); 'auto' = both for the decode batch, 'none'")
    ap.add_argument("--event-every", type=int, default=4,
                    help="record the kernel-timing events on every N-th timed step (warm runs)")
    ap.add_argument("--segment-tiles", type=int, default=0,
                    help="split-KV segment length in KV tiles (0 = the plan's choice)")
    ap.add_argument("--bf16-partials", action="store_true",
                    help="keep the split-KV partial o in bf16 (UA_FLAG_BF16_PARTIALS)")
    ap.add_argument("--persistent", action="store_true",
                    help="run a 2D LDS-ring launch on the persistent schedule (UA_FLAG_PERSISTENT)")
    ap.add_argument("--clock-seconds", type=float, default=1.0,
                    help="seconds of untimed replay after timing during which amdsmi "
                         "samples the GPU clocks (0 = skip)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="wall-time budget of the oracle CPU baseline (0 = skip)")
    ap.add_argument("--prefill-cpu-seconds", type=float, default=10.0,
                    help="wall-time budget of the prefill figure's oracle baseline (0 = skip)")
    ap.add_argument("--parts", action="store_true",
                    help="instead of the bench line, time the parts of the workload: the "
                         "whole batch, its decode-shaped and its wide sequences alone, and the "
                         "batch with each optional feature (softcap, ALiBi, sinks, window) off")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes (5 launches): the "
                         "reference dispatch for scaling HBM traffic counters")
    ap.add_argument("--summarize-traffic", nargs=5, default=None,
                    metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV",
                             "COPY_BYTES"),
                    help="write profiles/<workload>_hbm_traffic.json from rocprofv3 --pmc "
                         "counter CSVs (no GPU needed)")
    args = ap.parse_args()

    if args.summarize_traffic:
        summarize_traffic(args)
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(this build has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if args.copy_calibration:
        n = args.copy_calibration // 16
        src = torch.empty(n, 4, dtype=torch.int32, device="cuda").random_()
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n * 16, "copy_bytes_written": n * 16,
                          "launches": 5}))
        return

    extras = set()
    if args.extras == "auto":
        if args.workload == "decode_batch" and args.force == "auto" and not args.cold:
            extras = {"cold", "prefill"}
    elif args.extras != "none":
        extras = {e.strip() for e in args.extras.split(",") if e.strip()}
        unknown = extras - {"cold", "prefill"}
        if unknown:
            ap.error(f"unknown extras {sorted(unknown)}")

    from varlen_attention_serving_amd import binding as B
    extra_flags = ((B.UA_FLAG_BF16_PARTIALS if args.bf16_partials else 0) |
                   (B.UA_FLAG_PERSISTENT if args.persistent else 0))
    if args.parts:
        time_parts(args, extra_flags)
        return
    r = Runner(args.workload, args.force, args.segment_tiles, extra_flags)
    flush = make_read_flush(torch) if (args.cold or "cold" in extras) else None
    t = r.time(args.steps, args.warmup, args.event_every, flush if args.cold else None)
    f = r.figures(t)
    # warm: whole-job wall clock over the K steps; cold: the steps' own GPU time
    ms_per_step = f["whole_ms"] if args.cold else t["wall_ms"]
    value = f["value_events"] if args.cold else f["value_wall"]
    clock_info = clocks_under(r, args.clock_seconds, ms_per_step, flush if args.cold else None)

    config = r.config()
    config.update({
        "gpu_ms_per_step_events": round(f["whole_ms"], 5),
        "attention_kernel_ms": round(f["attn_ms"], 5),
        "timed_steps_with_events": t["sampled"],
        "attention_kernel_ms_median": round(float(np.median(t["attn"])), 5),
        "attention_kernel_ms_min": round(float(np.min(t["attn"])), 5),
        "cache": "cold (read-only 1 GiB flush before each step)" if args.cold else "warm",
        "split_partials": "bf16" if args.bf16_partials else "f32",
        "schedule": "persistent" if args.persistent else "grid",
        "roofline_frac_whole_step": round(max(r.t_hbm, r.t_mfma) / (ms_per_step * 1e-3), 4),
        "roofline_frac_whole_forward_events": round(f["frac_whole_forward"], 4),
        "clocks": clock_info,
    })
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": f["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": r.dtype(),
        "data": "synthetic (seeded N(0,1) values, seeded lengths and block tables)",
        "config": config,
        "roofline": r.roofline(f),
        "cpu_baseline": None,
    }

    if "cold" in extras:
        tc = r.time(args.steps, 2, 1, flush)
        fc = r.figures(tc)
        out["cold"] = {
            "workload": r.name, "value": round(fc["value_events"], 3), "unit": fc["unit"],
            "ms_per_step_events": round(fc["whole_ms"], 5),
            "attention_kernel_ms": round(fc["attn_ms"], 5),
            "attention_kernel_ms_median": round(float(np.median(tc["attn"])), 5),
            "roofline": {"bound": r.bound, "achieved": round(fc["achieved"], 3),
                         "peak": fc["peak"], "unit": fc["unit"], "frac": round(fc["frac"], 4),
                         "scope": "the attention kernel alone"},
            "roofline_frac_whole_forward_events": round(fc["frac_whole_forward"], 4),
            "flush": "torch.sum over a 1 GiB buffer before each step, outside the events "
                     "(reads only: nothing dirty is left to write back in the timed step)",
        }
    if args.cpu_seconds > 0:
        out["cpu_baseline"] = cpu_object(r.w, r.bound, f["unit"], args.cpu_seconds,
                                         by_rows=False)
        if args.workload == "decode_batch":
            out["cpu_baseline"]["single_thread"] = single_thread_oracle()
    r.close()
    del flush

    if "prefill" in extras:
        rp = Runner("long_prefill")
        tp = rp.time(args.steps, args.warmup, args.event_every)
        fp = rp.figures(tp)
        pre = {
            "workload": rp.name, "value": round(fp["value_wall"], 3), "unit": fp["unit"],
            "ms_per_step": round(tp["wall_ms"], 5), "dtype": rp.dtype(),
            "config": rp.config(),
            "attention_kernel_ms": round(fp["attn_ms"], 5),
            "attention_kernel_ms_median": round(float(np.median(tp["attn"])), 5),
            "roofline_frac_whole_step": round(max(rp.t_hbm, rp.t_mfma) / (tp["wall_ms"] * 1e-3), 4),
            "roofline": rp.roofline(fp),
            "cpu_baseline": None,
        }
        if args.prefill_cpu_seconds > 0:
            pre["cpu_baseline"] = cpu_object(rp.w, rp.bound, fp["unit"],
                                             args.prefill_cpu_seconds, by_rows=True)
        rp.close()
        out["prefill"] = pre

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
