"""Benchmark: paged GQA decode attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--path split|direct]

One step is one decode step of one attention layer of the Llama-3-8B-shaped workload
(batch 64, 32 query / 8 KV heads, head_dim 128, bf16 KV, contexts U[512, 4096], seed
1001): kv_append of the 64 new tokens followed by paged decode attention -- by default
the balanced kernel (the batch's blocks dealt evenly over the workgroups) and its merge;
--path split / direct time the fixed-partition split + merge or the single-pass kernel.
Inputs are resident in HBM before the timed region; two copies of the KV pool are used in
turn so that consecutive steps do not find the previous step's KV in the 256 MB Infinity
Cache.

Printed: ONE JSON line.  value = algorithmic KV bytes per step / step time (GB/s);
roofline.achieved = the same bytes / the attention kernel's mean duration, timed with
HIP events on the stream the kernels run on.  The other workloads (Llama-2-70B shared
prefix, 128K context, int8 verify) are timed the same way and reported under "others".
cpu_baseline times the fp64 oracle on a bounded sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "paged decode attention: KV-read GB/s (% of HBM peak) and µs/step per layer"

# partition sizes (tokens) used by the split path, per workload
PARTITION = {"llama3_8b": 512, "llama2_70b_prefix": 1024, "long_128k": 2048,
             "verify_int8": None, "tiny_fp32": None}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--path", choices=["balanced", "split", "direct"], default="balanced")
    ap.add_argument("--workgroups", type=int, default=0, help="balanced path; 0 = library default")
    ap.add_argument("--partition", type=int, default=None)
    ap.add_argument("--no-others", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--calibrate", action="store_true",
                    help="first run a 1 GiB device copy (reference for HBM counters)")
    return ap.parse_args()


class Runner:
    """Device-resident inputs of one workload and one decode step through the C ABI."""

    def __init__(self, P, wl, path, partition, copies=2, workgroups=0):
        import torch
        self.P, self.wl, self.torch = P, wl, torch
        c = wl.cfg
        dev = torch.device("cuda:0")
        self.q = wl.q.to(dev)
        self.tables = wl.block_tables.to(dev)
        self.lens = wl.seq_lens.to(dev)
        self.pools = []
        for _ in range(copies):
            self.pools.append((wl.k_cache.to(dev), wl.v_cache.to(dev),
                               None if wl.k_scale is None else wl.k_scale.to(dev),
                               None if wl.v_scale is None else wl.v_scale.to(dev)))
        self.append = wl.slot_mapping is not None
        if self.append:
            self.k_new, self.v_new = wl.k_new.to(dev), wl.v_new.to(dev)
            self.slots = wl.slot_mapping.to(dev)
        self.dims = P.make_dims(c.batch, c.num_q_heads, c.num_kv_heads, c.head_dim,
                                wl.block_tables.shape[1], wl.k_cache.shape[0], c.q_dtype,
                                c.kv_dtype)
        self.sm = float(np.float32(c.sm_scale))
        self.out = torch.empty((c.batch, c.num_q_pos, c.num_q_heads, c.head_dim),
                               dtype=torch.float32, device=dev)
        self.path = path
        self.split = path == "split" and c.num_q_pos == 1 and partition
        if path == "split" and not self.split:
            self.path = "direct"
        if self.split:
            self.pt = partition
            self.maxp = -(-int(wl.seq_lens.max()) // partition)
            self.part_out = torch.empty((c.batch, c.num_q_heads, self.maxp, c.head_dim),
                                        dtype=torch.float32, device=dev)
            self.part_lse = torch.empty((c.batch, c.num_q_heads, self.maxp),
                                        dtype=torch.float32, device=dev)
        if path == "balanced":
            self.G = workgroups or P.paged_attn_balanced_workgroups(self.dims, c.num_q_pos)
            nbytes = P.paged_attn_balanced_workspace_bytes(self.dims, c.num_q_pos, self.G)
            self.ws = torch.empty((nbytes,), dtype=torch.uint8, device=dev)

    def step(self, i, ev=None):
        P, c = self.P, self.wl.cfg
        kc, vc, ks, vs = self.pools[i % len(self.pools)]
        if ev is not None:
            ev[0].record()
        if self.append:
            P.kv_append(self.dims, self.k_new, self.v_new, self.slots, c.batch, kc, vc)
        if ev is not None:
            ev[1].record()
        if self.path == "balanced":
            P.paged_attn_balanced(self.dims, c.num_q_pos, self.q, kc, vc, ks, vs, self.tables,
                                  self.lens, self.sm, self.G, self.ws, self.out)
            if ev is not None:
                ev[2].record()
            P.paged_attn_balanced_merge(self.dims, c.num_q_pos, self.G, self.ws, self.out)
        elif self.split:
            P.paged_decode_attn_split(self.dims, self.q, kc, vc, ks, vs, self.tables, self.lens,
                                      self.sm, self.pt, self.maxp, self.part_out, self.part_lse)
            if ev is not None:
                ev[2].record()
            P.lse_merge(self.dims, self.part_out, self.part_lse, self.lens, self.pt, self.maxp,
                        self.out)
        else:
            P.paged_verify_attn(self.dims, c.num_q_pos, self.q, kc, vc, ks, vs, self.tables,
                                self.lens, self.sm, self.out)
            if ev is not None:
                ev[2].record()
        if ev is not None:
            ev[3].record()

    def measure(self, steps, warmup):
        torch = self.torch
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.step(i, evs[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        app = [e[0].elapsed_time(e[1]) * 1e3 for e in evs]     # us
        attn = [e[1].elapsed_time(e[2]) * 1e3 for e in evs]
        merge = [e[2].elapsed_time(e[3]) * 1e3 for e in evs]
        return wall, np.array(app), np.array(attn), np.array(merge)


def summarize(wl, wall, steps, app, attn, merge):
    kv = wl.kv_bytes()
    us_step = wall / steps * 1e6
    srt = np.sort(attn)
    return {
        "kv_bytes": kv,
        "us_per_step": us_step,
        "kv_GBps": kv / (us_step * 1e-6) / 1e9,
        "attn_kernel_us_mean": float(attn.mean()),
        "attn_kernel_us_median": float(np.median(attn)),
        "attn_kernel_us_p95": float(srt[int((len(srt) - 1) * 0.95)]),
        "attn_kernel_GBps": kv / (attn.mean() * 1e-6) / 1e9,
        "append_us_mean": float(app.mean()),
        "merge_us_mean": float(merge.mean()),
    }


def cpu_baseline(wl, seconds):
    """The fp64 oracle, as it stands, run on the host over the same workload: whole
    passes over all (sequence, KV head) pairs, repeated until about `seconds` of host time
    is spent (a pass cut short when one pass alone is longer); rate in the same unit."""
    import torch
    from oracle import attention, paging
    c = wl.cfg

    def raw(x):
        if x is None:
            return None
        return x.view(torch.int16).numpy() if x.dtype == torch.bfloat16 else x.numpy()
    kc, vc = raw(wl.k_cache), raw(wl.v_cache)
    if wl.slot_mapping is not None:
        kc, vc = paging.append(kc, vc, raw(wl.k_new), raw(wl.v_new), wl.slot_mapping.numpy())
    elem = {"f32": 4, "bf16": 2, "i8": 1}[c.kv_dtype]
    pairs_done, nbytes = 0, 0
    t0 = time.perf_counter()
    done = False
    while not done:
        for b in range(c.batch):
            for g in range(c.num_kv_heads):
                attention.paged_attention(raw(wl.q), c.q_dtype, kc, vc, c.kv_dtype,
                                          wl.block_tables.numpy(), wl.seq_lens.numpy(),
                                          float(np.float32(c.sm_scale)), c.num_q_pos,
                                          raw(wl.k_scale), raw(wl.v_scale), pairs=[(b, g)])
                pairs_done += 1
                nbytes += int(wl.seq_lens[b]) * 2 * c.head_dim * elem
                done = time.perf_counter() - t0 > seconds
                if done:
                    break
            if done:
                break
    dt = time.perf_counter() - t0
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas = int(os.environ.get("OMP_NUM_THREADS", "1"))
    npairs = c.batch * c.num_kv_heads
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": blas,
            "kind": "oracle",
            "sample": f"{pairs_done} (sequence, KV head) pairs ({pairs_done / npairs:.2f} passes "
                      f"over the {npairs} of {c.name}, seed {wl.meta['seed']}), fp64 numpy, "
                      f"{dt:.1f} s",
            "host_cpus": len(os.sched_getaffinity(0))}


KERNEL_SOURCES = ["paged_gqa_decode_kv_amd/csrc/attn.hip", "paged_gqa_decode_kv_amd/csrc/pa_common.hpp"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "llama3_8b_balanced_traffic.json")


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch of the attention kernel from the committed counter summary,
    or None if there is none or the kernel source changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha") != kernel_source_hash():
        return None
    return t.get("traffic_bytes_per_launch")


def calibration_copy(torch, nbytes=1 << 30):
    """A plain device-to-device copy of known size, for scaling the HBM counters."""
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    del a, b


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this path is single-GPU); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import paged_gqa_decode_kv_amd as P
    import workloads as W
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.calibrate:
        calibration_copy(torch)

    main_name = "llama3_8b"
    wl = W.generate(main_name, poison=False)
    part = args.partition or PARTITION[main_name]
    r = Runner(P, wl, args.path, part, workgroups=args.workgroups)
    res = summarize(wl, *_m(r, args))
    G = getattr(r, "G", None)
    del r
    torch.cuda.empty_cache()

    others = {}
    if not args.no_others:
        for name in ("llama2_70b_prefix", "long_128k", "verify_int8"):
            w2 = W.generate(name, poison=False)
            copies = 1 if name == "long_128k" else 2
            r2 = Runner(P, w2, "balanced", None, copies=copies)
            s = summarize(w2, *_m(r2, args, steps=min(args.steps, 20), warmup=3))
            s["path"] = "balanced"
            s["workgroups"] = r2.G
            s["pct_hbm_peak"] = s["kv_GBps"] / HBM_PEAK_GBS * 100
            s["attn_kernel_frac_of_peak"] = s["attn_kernel_GBps"] / HBM_PEAK_GBS
            others[name] = {k: (round(v, 3) if isinstance(v, float) else v) for k, v in s.items()}
            del r2, w2
            torch.cuda.empty_cache()

    achieved = res["attn_kernel_GBps"]
    kernel = {"balanced": "paged_attn_balanced_kernel", "split": "paged_attn_kernel (split)",
              "direct": "paged_attn_kernel (direct)"}[args.path]
    line = {
        "metric": METRIC,
        "value": round(res["kv_GBps"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["us_per_step"] / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama3_8b_layer_decode", "batch": 64, "q_heads": 32,
                   "kv_heads": 8, "head_dim": 128, "block_size": 16, "kv_dtype": "bf16",
                   "context": "uniform [512, 4096] (+ the appended token)", "seed": 1001,
                   "path": args.path, "workgroups": G,
                   "partition_tokens": part if args.path == "split" else None,
                   "kv_bytes_per_step": res["kv_bytes"]},
        "us_per_step": round(res["us_per_step"], 2),
        "pct_hbm_peak": round(res["kv_GBps"] / HBM_PEAK_GBS * 100, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic() if args.path == "balanced" else None,
                     "kernel": kernel, "kernel_us_mean": round(res["attn_kernel_us_mean"], 2),
                     "bytes_per_launch": res["kv_bytes"]},
        "timing": {k: round(v, 3) for k, v in res.items() if k.endswith("_us_mean") or
                   k.endswith("_us_median") or k.endswith("_us_p95")},
        "others": others,
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(line), flush=True)


def _m(r, args, steps=None, warmup=None):
    steps = args.steps if steps is None else steps
    warmup = args.warmup if warmup is None else warmup
    wall, app, attn, merge = r.measure(steps, warmup)
    return (wall, steps, app, attn, merge)


if __name__ == "__main__":
    main()
