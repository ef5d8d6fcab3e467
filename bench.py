"""Benchmark: paged GQA decode attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--event-steps E]
                    [--path step|balanced|split|direct] [--layout interleaved|separate]

One step is one decode step of one attention layer of the Llama-3-8B-shaped workload
(batch 64, 32 query / 8 KV heads, head_dim 128, bf16 KV, contexts U[512, 4096], seed
1001): the append of the 64 new tokens and paged decode attention over the cache that
includes them.  Paths for that workload:
  step      (default) paged_decode_step + paged_attn_balanced_merge: the append folded
            into the balanced attention kernel, then the merge of cut segments
  balanced  kv_append, paged_attn_balanced, paged_attn_balanced_merge
  split     kv_append, fixed-partition split attention, lse_merge
  direct    kv_append, the single-pass kernel
--layout: K and V tiles of one (block, head) side by side in one pool (interleaved,
default) or two separate pools.  Inputs are resident in HBM before the timed region;
two copies of the KV pool are used in turn so that consecutive steps do not find the
previous step's KV in the 256 MB Infinity Cache.

Timing: W untimed warm-up steps, then EXACTLY K steps between two synchronisations with
no events in between (value, ms_per_step), then a separate pass of E steps in which HIP
events (no system fence, on the stream the kernels run on) bracket the attention kernel
and the merge of every step (kernel means and percentiles, roofline.achieved).

Printed: ONE JSON line.  value = algorithmic KV bytes per step / wall-clock step time
(GB/s).  "configs" holds the same columns for the five configurations of the task -- c1
tiny fp32 (with a standalone kv_append), c2 Llama-3-8B (the headline), c3 Llama-2-70B
shared prefix, c4 128K context (decode step, and split + LSE merge at the partition size
the bench picks), c5 int8 speculative verify -- each with its max abs error against the
fp64 oracle over every output element and the oracle's own time on the same inputs.
"others" holds the further workloads (sliding window, fp8, block copy, quantising
append, chunked prefill, tree verify); cpu_baseline times the oracle on a bounded sample
of the headline workload.

Profiler summaries (profiles/) from rocprofv3 runs of this script with the same flags:
    --trace-summary DIR            kernel trace (per workload and kernel)
    --counter-summary DIR [NAME]   one --pmc pass of counters
    --pmc-summary FETCH_DIR WRITE_DIR   HBM bytes per launch of every workload's kernels
                                   (FETCH_SIZE and WRITE_SIZE passes, with --calibrate)
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
MFMA_BF16_PEAK_TFLOPS = 2500.0
METRIC = "paged decode attention: KV-read GB/s (% of HBM peak) and µs/step per layer"

# partition sizes (tokens) tried by the split path, per workload; the 128K configuration
# picks the fastest of its candidates
PARTITION = {"llama3_8b": 512, "llama2_70b_prefix": 1024, "long_128k": 2048,
             "verify_int8": None, "tiny_fp32": None}
SPLIT_CANDIDATES = (1024, 2048, 4096, 8192)

# the task's configurations: label, workload, attention path
CONFIGS = [("c1", "tiny_fp32", "step"), ("c2", "llama3_8b", "step"),
           ("c3", "llama2_70b_prefix", "step"), ("c4", "long_128k", "step"),
           ("c5", "verify_int8", "step")]
TOL = {"f32": 1e-5, "bf16": 2e-3, "i8": 4e-3, "fp8": 4e-3}

# Workloads in the order the bench runs them; each starts with a separator kernel (mark),
# which is how the profiler summaries tell them apart.  (name, warm-up launches of its
# kernels before the timed ones)
ORDER = ["llama3_8b", "tiny_fp32", "llama2_70b_prefix", "long_128k",
         "long_128k_split_candidates", "long_128k_split", "verify_int8", "mistral_7b_window",
         "llama3_8b_fp8", "kv_copy_blocks_2048", "kv_copy_blocks_64", "kv_append_quant",
         "prefill_chunk", "tree_verify"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--event-steps", type=int, default=50,
                    help="steps of the separate pass whose kernels are bracketed by events")
    ap.add_argument("--path", choices=["step", "balanced", "split", "direct"], default="step")
    ap.add_argument("--layout", choices=["interleaved", "separate"], default="interleaved")
    ap.add_argument("--workgroups", type=int, default=0, help="balanced path; 0 = library default")
    ap.add_argument("--partition", type=int, default=None)
    ap.add_argument("--no-others", action="store_true",
                    help="the headline workload only (no other configurations or workloads)")
    ap.add_argument("--no-cpu", action="store_true", help="no oracle timing or parity")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--calibrate", action="store_true",
                    help="first run a 1 GiB device copy (reference for HBM counters)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 --pmc runs into profiles/hbm_traffic.json")
    ap.add_argument("--counter-summary", nargs="+", metavar=("PMC_DIR", "NAME"),
                    help="summarise one rocprofv3 --pmc run of this script into "
                         "profiles/NAME.md (default kernel_counters) and exit")
    ap.add_argument("--trace-summary", metavar="TRACE_DIR",
                    help="summarise a rocprofv3 --kernel-trace run of this script (profiles/) "
                         "and exit")
    return ap.parse_args()


def log(msg):
    """Progress on stderr (stdout carries only the JSON line)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)

class HipEvent:
    """A HIP timing event recorded on the current torch stream (the stream the binding
    launches on), created with hipEventDisableSystemFence: the record writes a timestamp
    and no system-scope cache writeback / invalidate, which would otherwise sit between
    the bracketed kernel and its neighbours (about 2 us per bracket here).  The HIP runtime
    is the one torch has already loaded (same soname)."""

    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        cls = type(self)
        if cls._hip is None:
            hip = ctypes.CDLL("libamdhip64.so.7")
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p),
                                                    ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = hip
        self._c = ctypes
        self.h = ctypes.c_void_p()
        rc = cls._hip.hipEventCreateWithFlags(ctypes.byref(self.h), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self):
        import torch
        stream = self._c.c_void_p(torch.cuda.current_stream().cuda_stream)
        rc = self._hip.hipEventRecord(self.h, stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_time(self, end):
        """Milliseconds from this event to `end` (both complete)."""
        f = self._c.c_float()
        rc = self._hip.hipEventElapsedTime(self._c.byref(f), self.h, end.h)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return f.value

    def __del__(self):
        try:
            if self.h:
                self._hip.hipEventDestroy(self.h)
        except Exception:       # interpreter shutdown
            pass

class Runner:
    """Device-resident inputs of one workload and one step through the C ABI."""

    def __init__(self, P, wl, path, partition, copies=2, workgroups=0, layout="interleaved"):
        import torch
        self.P, self.wl, self.torch = P, wl, torch
        c = wl.cfg
        dev = torch.device("cuda:0")
        self.q = wl.q.to(dev)
        self.tables = wl.block_tables.to(dev)
        self.lens = wl.seq_lens.to(dev)
        self.pools = []
        self.keep = []
        tile = wl.k_cache[0, 0].numel()
        for _ in range(copies):
            ks = None if wl.k_scale is None else wl.k_scale.to(dev)
            vs = None if wl.v_scale is None else wl.v_scale.to(dev)
            if layout == "interleaved":
                # [NB][Hkv][2][tile]: K then V tile of each (block, head), tile stride 2 tiles
                nb, h = wl.k_cache.shape[:2]
                comb = torch.empty((nb, h, 2, tile), dtype=wl.k_cache.dtype, device=dev)
                comb[:, :, 0] = wl.k_cache.reshape(nb, h, tile).to(dev)
                comb[:, :, 1] = wl.v_cache.reshape(nb, h, tile).to(dev)
                self.keep.append(comb)
                self.pools.append((comb, comb.data_ptr() + tile * comb.element_size(), ks, vs))
            else:
                self.pools.append((wl.k_cache.to(dev), wl.v_cache.to(dev), ks, vs))
        self.append = wl.slot_mapping is not None
        if self.append:
            self.k_new, self.v_new = wl.k_new.to(dev), wl.v_new.to(dev)
            self.slots = wl.slot_mapping.to(dev)
        self.dims = P.make_dims(c.batch, c.num_q_heads, c.num_kv_heads, c.head_dim,
                                wl.block_tables.shape[1], wl.k_cache.shape[0], c.q_dtype,
                                c.kv_dtype,
                                kv_tile_stride=2 * tile if layout == "interleaved" else 0,
                                sliding_window=c.sliding_window)
        self.sm = float(np.float32(c.sm_scale))
        self.out = torch.empty((c.batch, c.num_q_pos, c.num_q_heads, c.head_dim),
                               dtype=torch.float32, device=dev)
        if path == "step" and not (self.append and c.num_q_pos == 1):
            path = "balanced"        # the fused step is the decode step with an append
        self.path = path
        self.split = path == "split" and c.num_q_pos == 1 and partition
        if path == "split" and not self.split:
            self.path = "direct"
        self.pt = self.maxp = None
        if self.split:
            self.pt = partition
            self.maxp = -(-int(wl.seq_lens.max()) // partition)
            self.part_out = torch.empty((c.batch, c.num_q_heads, self.maxp, c.head_dim),
                                        dtype=torch.float32, device=dev)
            self.part_lse = torch.empty((c.batch, c.num_q_heads, self.maxp),
                                        dtype=torch.float32, device=dev)
        self.G = None
        if self.path in ("balanced", "step"):
            self.G = workgroups or P.paged_attn_balanced_workgroups(self.dims, c.num_q_pos)
            nbytes = P.paged_attn_balanced_workspace_bytes(self.dims, c.num_q_pos, self.G)
            self.ws = torch.empty((nbytes,), dtype=torch.uint8, device=dev)

    def append_part(self, i):
        """The separate kv_append of the non-fused paths (nothing for the decode step)."""
        c = self.wl.cfg
        kc, vc, _, _ = self.pools[i % len(self.pools)]
        if self.append and self.path != "step":
            self.P.kv_append(self.dims, self.k_new, self.v_new, self.slots, c.batch, kc, vc)

    def attention(self, i):
        """The attention kernel of step i (for the decode step, with the append folded in)."""
        P, c = self.P, self.wl.cfg
        kc, vc, ks, vs = self.pools[i % len(self.pools)]
        if self.path == "step":
            P.paged_decode_step(self.dims, self.q, self.k_new, self.v_new, kc, vc, self.tables,
                                self.lens, self.sm, self.G, self.ws, self.out)
        elif self.path == "balanced":
            P.paged_attn_balanced(self.dims, c.num_q_pos, self.q, kc, vc, ks, vs, self.tables,
                                  self.lens, self.sm, self.G, self.ws, self.out)
        elif self.split:
            P.paged_decode_attn_split(self.dims, self.q, kc, vc, ks, vs, self.tables, self.lens,
                                      self.sm, self.pt, self.maxp, self.part_out, self.part_lse)
        else:
            P.paged_verify_attn(self.dims, c.num_q_pos, self.q, kc, vc, ks, vs, self.tables,
                                self.lens, self.sm, self.out)

    def merge(self, i=0):
        """The merge that completes the step (nothing for the single-pass kernel)."""
        P, c = self.P, self.wl.cfg
        if self.path in ("step", "balanced"):
            P.paged_attn_balanced_merge(self.dims, c.num_q_pos, self.G, self.ws, self.out)
        elif self.split:
            P.lse_merge(self.dims, self.part_out, self.part_lse, self.lens, self.pt, self.maxp,
                        self.out)

    def step(self, i, ev=None):
        """One step; with ev = (e0, e1, e2), HIP events bracket its attention kernel
        (e0 .. e1) and its merge (e1 .. e2); the separate append stays outside them."""
        self.append_part(i)
        if ev is not None:
            ev[0].record()
        self.attention(i)
        if ev is not None:
            ev[1].record()
        self.merge()
        if ev is not None:
            ev[2].record()

    def measure(self, steps, warmup, event_steps):
        """Wall time of exactly `steps` steps with nothing else in between, then a separate
        pass of `event_steps` steps with the attention kernel and the merge of every step
        bracketed by events (a bracket adds ~1 us to what it measures; kernels launched
        back to back instead would run into dispatch gaps of the short merge and measure
        those).  Returns (wall seconds, attention us array, merge us array)."""
        torch = self.torch
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.step(i)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        evs = [[HipEvent() for _ in range(3)] for _ in range(event_steps)]
        torch.cuda.synchronize()
        for i in range(event_steps):
            self.step(i, evs[i])
        torch.cuda.synchronize()
        attn = np.array([e[0].elapsed_time(e[1]) * 1e3 for e in evs])
        merge = np.array([e[1].elapsed_time(e[2]) * 1e3 for e in evs])
        return wall, attn, merge


def pct(a, p):
    """Percentile by the rule int((n - 1) * p) of the sorted samples."""
    s = np.sort(np.asarray(a))
    return float(s[int((len(s) - 1) * p)])


def summarize(wl, wall, steps, attn, merge):
    kv = wl.kv_bytes()
    us_step = wall / steps * 1e6
    kern = attn + merge
    return {
        "kv_bytes": kv,
        "us_per_step": us_step,
        "kv_GBps": kv / (us_step * 1e-6) / 1e9,
        "pct_hbm_peak": kv / (us_step * 1e-6) / 1e9 / HBM_PEAK_GBS * 100,
        "attn_kernel_us_mean": float(attn.mean()),
        "attn_kernel_us_median": float(np.median(attn)),
        "attn_kernel_us_p95": pct(attn, 0.95),
        "merge_us_mean": float(merge.mean()),
        "merge_us_p95": pct(merge, 0.95),
        "kernels_us_mean": float(kern.mean()),
        "kernels_us_p95": pct(kern, 0.95),
        "attn_kernel_GBps": kv / (attn.mean() * 1e-6) / 1e9,
        "kernels_GBps": kv / (kern.mean() * 1e-6) / 1e9,
        "event_samples": len(attn),
    }


def total_bytes(wl):
    """Bytes a step moves beyond the KV stream, added to it: queries read, outputs written,
    the used block-table entries and lengths read once, the appended tokens (K and V rows
    read, then written into their slots)."""
    c = wl.cfg
    qe = {"f32": 4, "bf16": 2}[c.q_dtype]
    ke = {"f32": 4, "bf16": 2, "i8": 1, "fp8": 1}[c.kv_dtype]
    rows = c.batch * c.num_q_pos * c.num_q_heads * c.head_dim
    ents = sum(-(-int(L) // 16) for L in wl.seq_lens.tolist())
    app = 2 * 2 * c.batch * c.num_kv_heads * c.head_dim * ke if wl.slot_mapping is not None else 0
    return wl.kv_bytes() + rows * qe + rows * 4 + ents * 4 + c.batch * 4 + app


def unique_kv_bytes(wl):
    """KV bytes of the distinct physical blocks the batch reads (shared blocks once)."""
    c = wl.cfg
    elem = {"f32": 4, "bf16": 2, "i8": 1, "fp8": 1}[c.kv_dtype]
    return int(wl.occupancy.sum()) * 2 * c.num_kv_heads * c.head_dim * elem


_ORACLE = {}   # workload name -> (reference output, seconds, threads): one pass each


def oracle_parity(wl, out):
    """The fp64 oracle over every (sequence, KV head) pair of the workload, on the caches
    after the step's append; returns (max |out - oracle| over every element, oracle
    seconds, threads it kept busy).  A workload measured twice (the 128K decode step and
    its split path) reuses the first pass."""
    key = (wl.cfg.name, wl.meta["seed"])
    if key in _ORACLE:
        ref, dt, cores = _ORACLE[key]
        g = out.detach().cpu().numpy().astype(np.float64).reshape(ref.shape)
        err = float(np.abs(g - ref).max()) if np.isfinite(g).all() else float("inf")
        return err, dt, cores
    import torch
    from oracle import attention, paging

    def raw(x):
        if x is None:
            return None
        return x.view(torch.int16).numpy() if x.dtype == torch.bfloat16 else x.numpy()
    c = wl.cfg
    kc, vc = raw(wl.k_cache), raw(wl.v_cache)
    t0, c0 = time.perf_counter(), time.process_time()
    if wl.slot_mapping is not None:
        kc, vc = paging.append(kc, vc, raw(wl.k_new), raw(wl.v_new), wl.slot_mapping.numpy())
    ref, _ = attention.paged_attention(raw(wl.q), c.q_dtype, kc, vc, c.kv_dtype,
                                       wl.block_tables.numpy(), wl.seq_lens.numpy(),
                                       float(np.float32(c.sm_scale)), c.num_q_pos,
                                       raw(wl.k_scale), raw(wl.v_scale),
                                       window=c.sliding_window)
    dt = time.perf_counter() - t0
    busy = (time.process_time() - c0) / max(dt, 1e-9)
    _ORACLE.clear()
    _ORACLE[key] = (ref, dt, max(1, int(round(busy))))
    g = out.detach().cpu().numpy().astype(np.float64).reshape(ref.shape)
    err = float(np.abs(g - ref).max()) if np.isfinite(g).all() else float("inf")
    return err, dt, max(1, int(round(busy)))


def config_entry(P, torch, W, label, name, path, args, partition=None, main=None):
    """One configuration's columns: wall-clock step, kernel times and percentiles, bytes,
    rates, HBM fraction, counter-measured HBM bytes (when the committed summary matches
    the kernel sources), and parity with the oracle over every output element."""
    wl = W.generate(name, poison=False)
    copies = 1 if name == "long_128k" else 2
    if main is None:
        r = Runner(P, wl, path, partition, copies=copies)
        meas = r.measure(args.steps, 3, args.event_steps)
    else:
        r, meas = main
    s = summarize(wl, meas[0], args.steps, *meas[1:])
    c = wl.cfg
    e = {"workload": name, "path": r.path, "workgroups": r.G,
         "partition_tokens": r.pt, "kv_dtype": c.kv_dtype, "batch": c.batch,
         "q_heads": c.num_q_heads, "kv_heads": c.num_kv_heads, "head_dim": c.head_dim,
         "num_q_pos": c.num_q_pos, "seed": wl.meta["seed"]}
    e.update({k: (round(v, 3) if isinstance(v, float) else v) for k, v in s.items()})
    e["total_bytes"] = total_bytes(wl)
    e["attn_kernel_frac_of_peak"] = round(s["attn_kernel_GBps"] / HBM_PEAK_GBS, 4)
    e["kernels_frac_of_peak"] = round(s["kernels_GBps"] / HBM_PEAK_GBS, 4)
    if c.shared_groups:
        # shared prefix: the HBM fractions are taken over the distinct blocks' bytes (each
        # read at most once from HBM); the logical rate is reported beside them
        ub = unique_kv_bytes(wl)
        e["unique_kv_bytes"] = ub
        e["logical_kv_GBps"] = e["kv_GBps"]
        e["unique_kv_GBps"] = round(ub / (s["us_per_step"] * 1e-6) / 1e9, 1)
        e["pct_hbm_peak"] = round(e["unique_kv_GBps"] / HBM_PEAK_GBS * 100, 2)
        e["attn_kernel_frac_of_peak"] = round(ub / (s["attn_kernel_us_mean"] * 1e-6) / 1e9 /
                                              HBM_PEAK_GBS, 4)
        e["kernels_frac_of_peak"] = round(ub / (s["kernels_us_mean"] * 1e-6) / 1e9 /
                                          HBM_PEAK_GBS, 4)
    tr = measured_traffic(name if r.path != "split" else name + "_split")
    e["fetched_bytes"] = None if tr is None else tr.get("attn_fetch_bytes")
    e["hbm_traffic_step_bytes"] = None if tr is None else tr.get("step_traffic_bytes")
    if not args.no_cpu:
        err, dt, cores = oracle_parity(wl, r.out)
        e["max_abs_err"] = err
        e["tol"] = TOL[c.kv_dtype]
        e["oracle"] = {"seconds": round(dt, 3), "kv_GBps": round(wl.kv_bytes() / dt / 1e9, 4),
                       "cores": cores, "kind": "oracle", "sample": "every (sequence, KV head) "
                       "pair of the workload, one pass, fp64 numpy"}
    return e, r, wl


def split_entry(P, torch, W, name, args):
    """Split + LSE merge on a workload: every candidate partition size timed over a short
    run, the fastest measured in full (its kv_append is outside the events)."""
    wl = W.generate(name, poison=False)
    cand = {}
    for p in SPLIT_CANDIDATES:
        r = Runner(P, wl, "split", p, copies=1)
        _, attn, merge = r.measure(5, 2, 10)
        cand[p] = round(float((attn + merge).mean()), 2)
        del r
        torch.cuda.empty_cache()
    best = min(cand, key=cand.get)
    mark(torch)   # the chosen size, measured in full, is a workload of its own in the traces
    e, r, _ = config_entry(P, torch, W, "split", name, "split", args, partition=best)
    e["candidates_us"] = {str(k): v for k, v in cand.items()}
    del r
    torch.cuda.empty_cache()
    return e


def append_entry(P, torch, W, steps):
    """kv_append alone on the tiny configuration: its 4 new tokens (fp32, 2 KV heads, d 64)
    written into their slots, launches back to back between two events."""
    wl = W.generate("tiny_fp32", poison=False)
    c = wl.cfg
    dev = torch.device("cuda:0")
    kc, vc = wl.k_cache.to(dev), wl.v_cache.to(dev)
    kn, vn, sm = wl.k_new.to(dev), wl.v_new.to(dev), wl.slot_mapping.to(dev)
    d = P.make_dims(c.batch, c.num_q_heads, c.num_kv_heads, c.head_dim, wl.block_tables.shape[1],
                    kc.shape[0], c.q_dtype, c.kv_dtype)
    for _ in range(3):
        P.kv_append(d, kn, vn, sm, c.batch, kc, vc)
    torch.cuda.synchronize()
    e0, e1 = HipEvent(), HipEvent()
    e0.record()
    for _ in range(steps):
        P.kv_append(d, kn, vn, sm, c.batch, kc, vc)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    nbytes = 2 * 2 * c.batch * c.num_kv_heads * c.head_dim * 4
    return {"tokens": c.batch, "kv_heads": c.num_kv_heads, "bytes": nbytes,
            "us_per_launch": round(us, 2), "launches": steps}

def copy_blocks_bench(P, torch, W, steps):
    """kv_copy_blocks on the Llama-3-8B pool (interleaved layout): a bulk copy of 2048
    blocks and the copy-on-write of one block per sequence (64 pairs).  Two disjoint pair
    sets alternate so a launch does not find the previous one's blocks in the Infinity
    Cache.  Bytes = pairs * Hkv * (K + V tile) * 2 (read and write).  The launches run
    back to back between two HIP events on the stream they run on (one event pair per
    launch would add its own idle gap to a launch this short)."""
    wl = W.generate(W.scaled("llama3_8b", append=False), poison=False, spare_blocks=4096)
    c = wl.cfg
    dev = torch.device("cuda:0")
    nb, h = wl.k_cache.shape[:2]
    tile = wl.k_cache[0, 0].numel()
    comb = torch.empty((nb, h, 2, tile), dtype=wl.k_cache.dtype, device=dev)
    comb[:, :, 0] = wl.k_cache.reshape(nb, h, tile).to(dev)
    comb[:, :, 1] = wl.v_cache.reshape(nb, h, tile).to(dev)
    vptr = comb.data_ptr() + tile * comb.element_size()
    dims = P.make_dims(c.batch, c.num_q_heads, c.num_kv_heads, c.head_dim,
                       wl.block_tables.shape[1], nb, c.q_dtype, c.kv_dtype,
                       kv_tile_stride=2 * tile)
    pairs = W.copy_pairs(wl, 4096, seed=3).to(dev)
    res = {}
    for label, n in (("bulk", 2048), ("cow_step", c.batch)):
        mark(torch)    # each copy size is a workload of its own in the traces
        sets = [pairs[:n].contiguous(), pairs[2048:2048 + n].contiguous()]
        for i in range(4):
            P.kv_copy_blocks(dims, sets[i % 2], n, comb, vptr)
        torch.cuda.synchronize()
        e0, e1 = (HipEvent() for _ in range(2))
        e0.record()
        for i in range(steps):
            P.kv_copy_blocks(dims, sets[i % 2], n, comb, vptr)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        nbytes = n * h * 2 * tile * comb.element_size() * 2
        res[label] = {"pairs": n, "bytes": nbytes, "us_mean": round(us, 2),
                      "GBps": round(nbytes / us / 1e3, 1),
                      "frac_of_peak": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)}
    del comb
    torch.cuda.empty_cache()
    return res

def append_quant_bench(P, torch, W, steps):
    """kv_append_quant for one decode step of a Llama-3-8B-shaped int8 cache: 64 new tokens
    (one per sequence, at the end of each sequence of the seeded Llama-3-8B lengths) into
    8 KV heads, each re-encoding its open block from a bf16 staging row.  Bytes per (token,
    head) = staged tokens read + new token read + staged token written + the block's live
    codes written (K and V) + the two scales; launches back to back between two events."""
    wl = W.generate(W.scaled("llama3_8b", kv_dtype="i8", append=False), poison=False,
                    spare_blocks=64)
    c = wl.cfg
    dev = torch.device("cuda:0")
    nb, h = wl.k_cache.shape[:2]
    d = c.head_dim
    kc, vc = wl.k_cache.to(dev), wl.v_cache.to(dev)
    ks, vs = wl.k_scale.to(dev), wl.v_scale.to(dev)
    alloc = wl.meta["allocator"]
    slots = torch.tensor([alloc.append_token(b)[0] for b in range(c.batch)], dtype=torch.int64)
    gen = torch.Generator().manual_seed(7)
    kn = torch.randn((c.batch, h, d), generator=gen).to(torch.bfloat16).to(dev)
    vn = torch.randn((c.batch, h, d), generator=gen).to(torch.bfloat16).to(dev)
    kst = torch.randn((c.batch, h, 16, d), generator=gen).to(torch.bfloat16).to(dev)
    vst = torch.randn((c.batch, h, 16, d), generator=gen).to(torch.bfloat16).to(dev)
    rows = torch.arange(c.batch, dtype=torch.int32, device=dev)
    sl = slots.to(dev)
    dims = P.make_dims(c.batch, c.num_q_heads, h, d, wl.block_tables.shape[1], nb, "bf16", "i8")
    for _ in range(3):
        P.kv_append_quant(dims, kn, vn, sl, rows, c.batch, kst, vst, kc, vc, ks, vs)
    torch.cuda.synchronize()
    e0, e1 = (HipEvent() for _ in range(2))
    e0.record()
    for _ in range(steps):
        P.kv_append_quant(dims, kn, vn, sl, rows, c.batch, kst, vst, kc, vc, ks, vs)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    offs = (slots % 16).tolist()
    nbytes = sum(h * (2 * (o * d * 2) + 2 * d * 2 + 2 * d * 2 + 2 * (o + 1) * d + 8)
                 for o in offs)
    del kc, vc
    torch.cuda.empty_cache()
    return {"tokens": c.batch, "kv_heads": h, "bytes": nbytes, "us_per_launch": round(us, 2),
            "GBps": round(nbytes / us / 1e3, 1)}

def multi_query_bench(P, torch, W, name, steps):
    """paged_multi_query_attn on a multi-query workload (chunked prefill: 256 causal
    positions per sequence; speculative tree verify: 64 candidates per sequence), interleaved
    pool, two pool copies used in turn, launches back to back between two events.  FLOPs =
    for every query row, 4 * head_dim per visible token (q.K and P.V, multiply-add = 2)."""
    wl = W.generate(name, poison=False)
    c = wl.cfg
    dev = torch.device("cuda:0")
    nb, h = wl.k_cache.shape[:2]
    tile = wl.k_cache[0, 0].numel()
    pools = []
    for _ in range(2):
        comb = torch.empty((nb, h, 2, tile), dtype=wl.k_cache.dtype, device=dev)
        comb[:, :, 0] = wl.k_cache.reshape(nb, h, tile).to(dev)
        comb[:, :, 1] = wl.v_cache.reshape(nb, h, tile).to(dev)
        pools.append((comb, comb.data_ptr() + tile * comb.element_size()))
    dims = P.make_dims(c.batch, c.num_q_heads, c.num_kv_heads, c.head_dim,
                       wl.block_tables.shape[1], nb, c.q_dtype, c.kv_dtype,
                       kv_tile_stride=2 * tile)
    q, tables, lens = wl.q.to(dev), wl.block_tables.to(dev), wl.seq_lens.to(dev)
    words = None if wl.tree_mask is None else W.tree_mask_words(wl.tree_mask).to(dev)
    out = torch.empty((c.batch, c.num_q_pos, c.num_q_heads, c.head_dim), device=dev)
    sm = float(np.float32(c.sm_scale))

    def launch(i):
        kc, vc = pools[i % 2]
        P.paged_multi_query_attn(dims, c.num_q_pos, q, kc, vc, None, None, tables, lens, sm, out,
                                 None, words)
    for i in range(3):
        launch(i)
    torch.cuda.synchronize()
    e0, e1 = (HipEvent() for _ in range(2))
    e0.record()
    for i in range(steps):
        launch(i)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    nq = c.num_q_pos
    vis = 0
    for b, L in enumerate(wl.seq_lens.tolist()):
        for i in range(nq):
            if wl.tree_mask is None:
                vis += max(0, L - nq + 1 + i)
            else:
                vis += max(0, L - nq) + int(wl.tree_mask[b, i].sum())
    flops = vis * c.num_q_heads * 4 * c.head_dim
    tflops = flops / us / 1e6
    del pools
    torch.cuda.empty_cache()
    return {"batch": c.batch, "num_q_pos": nq, "tree": wl.tree_mask is not None,
            "flops": flops, "kv_bytes": wl.kv_bytes(), "us_per_launch": round(us, 2),
            "TFLOPs": round(tflops, 1),
            "frac_of_bf16_mfma_peak": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "kv_GBps": round(wl.kv_bytes() / us / 1e3, 1)}

def _blas_threads():
    """Threads numpy's BLAS may use (the oracle's matrix-vector products)."""
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        return int(os.environ.get("OMP_NUM_THREADS", "1"))

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
    pairs_done, nbytes, t_depage = 0, 0, 0.0
    t0 = time.perf_counter()
    c0 = time.process_time()           # CPU time of all the process's threads
    done = False
    while not done:
        for b in range(c.batch):
            for g in range(c.num_kv_heads):
                attention.paged_attention(raw(wl.q), c.q_dtype, kc, vc, c.kv_dtype,
                                          wl.block_tables.numpy(), wl.seq_lens.numpy(),
                                          float(np.float32(c.sm_scale)), c.num_q_pos,
                                          raw(wl.k_scale), raw(wl.v_scale), pairs=[(b, g)])
                if pairs_done % 16 == 0:    # the de-page step alone, on every 16th pair
                    td = time.perf_counter()
                    paging.depage_fast(kc, vc, c.kv_dtype, wl.block_tables[b].numpy(),
                                       int(wl.seq_lens[b]), g, raw(wl.k_scale), raw(wl.v_scale))
                    t_depage += 16 * (time.perf_counter() - td)
                pairs_done += 1
                nbytes += int(wl.seq_lens[b]) * 2 * c.head_dim * elem
                done = time.perf_counter() - t0 > seconds
                if done:
                    break
            if done:
                break
    # t_depage estimates the de-page time of all pairs from every 16th one; the sampled
    # calls themselves (t_depage / 16) were extra work and leave the oracle's time
    wall = time.perf_counter() - t0
    busy = (time.process_time() - c0) / max(wall, 1e-9)   # threads busy on average
    dt = max(wall - t_depage / 16, 1e-9)
    npairs = c.batch * c.num_kv_heads
    # cores: the threads the oracle kept busy on average (CPU time / wall time), at least
    # one; blas_threads: the pool numpy's BLAS could use
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s",
            "cores": max(1, int(round(busy))), "cpu_time_per_wall": round(busy, 2),
            "blas_threads": _blas_threads(),
            "oracle_ms_per_pass": round(dt / (pairs_done / npairs) * 1e3, 1),
            "depage_share": round(min(1.0, t_depage / dt), 3),
            "kind": "oracle",
            "sample": f"{pairs_done} (sequence, KV head) pairs ({pairs_done / npairs:.2f} passes "
                      f"over the {npairs} of {c.name}, seed {wl.meta['seed']}), fp64 numpy, "
                      f"{dt:.1f} s",
            "host_cpus": len(os.sched_getaffinity(0))}

def cpu_oracle_others(W, seconds=3.0):
    """The oracle beside the measured paths that have no full oracle pass in "configs" /
    "others", each on a bounded sample for about `seconds` of host time, in the unit the GPU
    line reports: the multi-query rows in TFLOP/s over whole (sequence, KV head) pairs; the
    block copy in GB/s moved; the quantising append in tokens x heads / s."""
    import torch
    from oracle import attention, paging, quant

    def raw(x):
        if x is None:
            return None
        return x.view(torch.int16).numpy() if x.dtype == torch.bfloat16 else x.numpy()

    busy = []   # threads kept busy on average (CPU time / wall time), per timed sample

    def timed(fn):
        n, t0, c0 = 0, time.perf_counter(), time.process_time()
        while True:
            fn(n)
            n += 1
            if time.perf_counter() - t0 > seconds:
                wall = time.perf_counter() - t0
                busy.append((time.process_time() - c0) / wall)
                return n, wall

    res = {}
    for name in ("prefill_chunk", "tree_verify"):
        wl = W.generate(W.scaled(name, append=False), poison=False)
        c = wl.cfg
        pairs = [(b, g) for b in range(c.batch) for g in range(c.num_kv_heads)]
        tm = None if wl.tree_mask is None else wl.tree_mask.numpy()
        kc, vc = raw(wl.k_cache), raw(wl.v_cache)
        args = (raw(wl.q), c.q_dtype, kc, vc, c.kv_dtype, wl.block_tables.numpy(),
                wl.seq_lens.numpy(), float(np.float32(c.sm_scale)), c.num_q_pos,
                raw(wl.k_scale), raw(wl.v_scale))
        n, dt = timed(lambda i: attention.paged_attention(*args, pairs=[pairs[i % len(pairs)]],
                                                          window=c.sliding_window, tree_mask=tm))
        done = [pairs[i % len(pairs)] for i in range(n)]
        if c.num_q_pos == 1:
            per = wl.kv_bytes() / len(pairs)
            res[name] = {"value": round(n * per / dt / 1e9, 4), "unit": "GB/s"}
        else:
            vis = 0
            for b, _ in done:
                L = int(wl.seq_lens[b])
                for i in range(c.num_q_pos):
                    vis += (max(0, L - c.num_q_pos + 1 + i) if tm is None
                            else max(0, L - c.num_q_pos) + int(tm[b, i].sum()))
            flops = vis * c.group_size * 4 * c.head_dim
            res[name] = {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s"}
        res[name]["sample"] = f"{n} (sequence, KV head) pairs of {name}, {dt:.1f} s"
    wl = W.generate(W.scaled("llama3_8b", append=False), poison=False, spare_blocks=4096)
    pairs = W.copy_pairs(wl, 2048, seed=3).numpy()
    kc, vc = raw(wl.k_cache), raw(wl.v_cache)
    n, dt = timed(lambda i: paging.copy_blocks(kc, vc, pairs))
    moved = 2048 * wl.cfg.num_kv_heads * 2 * wl.k_cache[0, 0].numel() * 2 * 2
    res["kv_copy_blocks"] = {"value": round(n * moved / dt / 1e9, 4), "unit": "GB/s",
                             "sample": f"{n} copies of 2048 blocks, {dt:.1f} s"}
    h, d, T = 8, 128, 64
    gen = torch.Generator().manual_seed(7)
    kn = torch.randn((T, h, d), generator=gen).to(torch.bfloat16)
    st = torch.randn((T, h, 16, d), generator=gen).to(torch.bfloat16)
    nb = 128
    cache = (np.zeros((nb, h, d // 16, 16, 16), np.int8), np.zeros((nb, h, d, 16), np.int8),
             np.zeros((nb, h), np.float32), np.zeros((nb, h), np.float32), raw(st), raw(st))
    slots = np.arange(T) * 16 + (np.arange(T) * 7) % 16
    n, dt = timed(lambda i: quant.append_quant(*cache, raw(kn), raw(kn), slots, np.arange(T)))
    res["kv_append_quant"] = {"value": round(n * T * h / dt, 1), "unit": "token-heads/s",
                              "sample": f"{n} calls of {T} tokens x {h} heads, {dt:.1f} s"}
    assert len(busy) == len(res)
    for v, bz in zip(res.values(), busy):
        v.update(kind="oracle", cores=max(1, int(round(bz))), cpu_time_per_wall=round(bz, 2),
                 blas_threads=_blas_threads())
    return res

def calibration_copy(torch, nbytes=1 << 30):
    """A plain device-to-device copy of known size, for scaling the HBM counters."""
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    del a, b

KERNEL_SOURCES = ["paged_gqa_decode_kv_amd/csrc/attn.hip", "paged_gqa_decode_kv_amd/csrc/merge.hip",
                  "paged_gqa_decode_kv_amd/csrc/append.hip", "paged_gqa_decode_kv_amd/csrc/pa_common.hpp",
                  "paged_gqa_decode_kv_amd/csrc/launch.hpp"]
TRAFFIC_FILE = "hbm_traffic.json"
MARKER = "FillFunctor<short>"


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per launch of a workload's kernels from the committed counter summary,
    or None if there is none or the kernel sources changed since it was taken."""
    try:
        with open(os.path.join(ROOT, "profiles", TRAFFIC_FILE)) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha") != kernel_source_hash():
        return None
    return t.get("workloads", {}).get(workload)


def mark(torch):
    """A small fill kernel (int16, used nowhere else) that opens a workload in a profiler
    trace; the summaries split the dispatch list at it."""
    torch.empty(64, dtype=torch.int16, device="cuda:0").fill_(1)
    torch.cuda.synchronize()


def _short(n):
    import re
    if "pa::" not in n:
        return None
    n = n.replace("(anonymous namespace)::", "")
    m = re.match(r"void pa::(\w+)<(.*)>\(", n)
    if m:
        return f"{m.group(1)}<{m.group(2)}>"
    m = re.match(r"void pa::(\w+)\(", n)
    return m.group(1) if m else n.split("(")[0][:60]


def _grouped(rows):
    """(kernel name, value) pairs in dispatch order -> [(workload, {kernel: [values]})],
    one group per marker, named by ORDER."""
    groups, cur = [], None
    for name, val in rows:
        if MARKER in name:
            cur = {}
            groups.append(cur)
            continue
        k = _short(name)
        if cur is None or k is None:
            continue
        cur.setdefault(k, []).append(val)
    return list(zip(ORDER, groups))


def _warm(name, args):
    """Warm-up launches of each kernel of a workload, left out of the summaries."""
    if name == ORDER[0]:
        return args.warmup
    return 4 if name.startswith("kv_copy_blocks") else 3


def _flags(args):
    return (f"--steps {args.steps} --warmup {args.warmup} --event-steps {args.event_steps}" +
            (" --no-cpu" if args.no_cpu else "") + (" --calibrate" if args.calibrate else "") +
            f" --path {args.path} --layout {args.layout}")


def trace_summary(args, trace_dir):
    """Markdown summary of a rocprofv3 --kernel-trace run of this script (same flags):
    per workload and kernel, launches and mean / median duration, warm-up launches left
    out (the split workload's figures pool all its candidate partition sizes)."""
    import sqlite3
    db = sqlite3.connect(os.path.join(trace_dir, "run_results.db"))
    rows = db.execute("select name, start, end from kernels order by start").fetchall()
    groups = _grouped([(n, (e - s0) / 1000) for n, s0, e in rows])
    lines = [f"# rocprofv3 kernel trace: bench.py {_flags(args)}", "",
             "Command (MI355X, one GPU):", "",
             f"    rocprofv3 --kernel-trace --stats -d {trace_dir} -o run -- python bench.py {_flags(args)}",
             f"    python bench.py {_flags(args)} --trace-summary {trace_dir}", "",
             f"Kernel sources sha: {kernel_source_hash()}", "",
             "| workload | kernel | launches | mean us | median us |", "|---|---|---|---|---|"]
    for name, g in groups:
        for k, v in g.items():
            w = _warm(name, args)
            v = v[w:] if len(v) > w else v
            lines.append(f"| {name} | `{k}` | {len(v)} | {np.mean(v):.2f} | {np.median(v):.2f} |")
    out = os.path.join(ROOT, "profiles", f"{args.path}_{args.layout}_kernel_trace.md")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _pmc_rows(pmc_dir):
    import sqlite3
    db = sqlite3.connect(os.path.join(pmc_dir, "run_results.db"))
    rows = db.execute("select dispatch_id, kernel_name, counter_name, value from "
                      "counters_collection order by dispatch_id").fetchall()
    disp = {}
    for did, name, cname, val in rows:
        d = disp.setdefault(did, {"name": name, "c": {}})
        d["c"][cname] = d["c"].get(cname, 0.0) + float(val)
    return [(disp[d]["name"], disp[d]["c"]) for d in sorted(disp)]


def counter_summary(args, pmc_dir, out_name="kernel_counters"):
    """Markdown summary of one rocprofv3 --pmc run of this script (same flags): per
    workload and kernel, the mean per-dispatch value of every counter collected (warm-up
    dispatches left out), and per-wave ratios where the counters allow them."""
    disp = _pmc_rows(pmc_dir)
    groups = _grouped(disp)
    counters = sorted({cn for _, c in disp for cn in c})
    lines = [f"# rocprofv3 counters: bench.py {_flags(args)}", "",
             "Command (MI355X, one GPU):", "",
             f"    rocprofv3 --pmc {' '.join(counters)} -d {pmc_dir} -o run -- python "
             f"bench.py {_flags(args)}",
             f"    python bench.py {_flags(args)} --counter-summary {pmc_dir}"
             f"{'' if out_name == 'kernel_counters' else ' ' + out_name}", "",
             f"Kernel sources sha: {kernel_source_hash()}", "",
             "Mean per dispatch (counters summed over the device). Derived, where collected: "
             "VALU/wave = SQ_INSTS_VALU / SQ_WAVES, MFMA/wave = SQ_INSTS_MFMA / SQ_WAVES, "
             "VALU issue = SQ_ACTIVE_INST_VALU / SQ_WAVE_CYCLES.", "",
             "| workload | kernel | dispatches | " + " | ".join(counters) +
             " | VALU/wave | MFMA/wave | VALU issue |",
             "|---|---|---|" + "---|" * (len(counters) + 3)]
    for name, g in groups:
        for k, cs in g.items():
            w = _warm(name, args)
            cs = cs[w:] if len(cs) > w else cs
            mean = {cn: float(np.mean([c.get(cn, 0.0) for c in cs])) for cn in counters}
            wv = mean.get("SQ_WAVES", 0.0)
            der = [f"{mean['SQ_INSTS_VALU'] / wv:.0f}" if wv and "SQ_INSTS_VALU" in mean else "",
                   f"{mean['SQ_INSTS_MFMA'] / wv:.0f}" if wv and "SQ_INSTS_MFMA" in mean else "",
                   f"{mean['SQ_ACTIVE_INST_VALU'] / mean['SQ_WAVE_CYCLES']:.3f}"
                   if mean.get("SQ_WAVE_CYCLES") and "SQ_ACTIVE_INST_VALU" in mean else ""]
            lines.append(f"| {name} | `{k}` | {len(cs)} | " +
                         " | ".join(f"{mean[cn]:.4g}" for cn in counters) + " | " +
                         " | ".join(der) + " |")
    out = os.path.join(ROOT, "profiles", f"{out_name}.md")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def pmc_summary(args, fetch_dir, write_dir):
    """profiles/hbm_traffic.json from two rocprofv3 --pmc runs of this script with
    --calibrate (FETCH_SIZE, then WRITE_SIZE): per workload, the attention kernel's and the
    merge's HBM bytes per launch, each counter scaled by what it reads for the 1 GiB
    calibration copy (copy bytes / counter bytes)."""
    copy_bytes = 1 << 30

    def load(d, counter):
        disp = _pmc_rows(d)
        cal = [c[counter] for n, c in disp if "copyBuffer" in n and counter in c][:3]
        scale = copy_bytes / (float(np.mean(cal)) * 1024)
        res = {}
        for name, g in _grouped(disp):
            for k, cs in g.items():
                w = _warm(name, args)
                cs = cs[w:] if len(cs) > w else cs
                role = ("attn" if k.startswith("paged_attn") else
                        "merge" if "merge" in k else "append" if "append" in k else None)
                if role is None or counter not in cs[0]:
                    continue
                res.setdefault(name, {})[role] = (k, float(np.mean([c[counter] for c in cs])) *
                                                  1024 * scale, len(cs))
        return float(np.mean(cal)), scale, res
    cf, fs, fetch = load(fetch_dir, "FETCH_SIZE")
    cw, wsc, write = load(write_dir, "WRITE_SIZE")
    import workloads as W
    out = {"kernel_source_sha": kernel_source_hash(), "kernel_sources": KERNEL_SOURCES,
           "calibration": {"copy_bytes": copy_bytes, "FETCH_SIZE_KiB": round(cf, 1),
                           "WRITE_SIZE_KiB": round(cw, 1), "fetch_scale": round(fs, 5),
                           "write_scale": round(wsc, 5)},
           "commands": [
               f"rocprofv3 --pmc FETCH_SIZE -d {fetch_dir} -o run -- python bench.py {_flags(args)}",
               f"rocprofv3 --pmc WRITE_SIZE -d {write_dir} -o run -- python bench.py {_flags(args)}",
               f"python bench.py {_flags(args)} --pmc-summary {fetch_dir} {write_dir}"],
           "workloads": {}}
    for name in fetch:
        f, w = fetch[name], write.get(name, {})
        e = {}
        for role in ("attn", "merge", "append"):
            if role in f:
                e[f"{role}_kernel"] = f[role][0]
                e[f"{role}_fetch_bytes"] = round(f[role][1])
                e[f"{role}_write_bytes"] = round(w[role][1]) if role in w else None
                e[f"{role}_dispatches"] = f[role][2]
        e["step_traffic_bytes"] = sum(v for k, v in e.items()
                                      if k.endswith(("_fetch_bytes", "_write_bytes")) and v)
        base = name[:-len("_split")] if name.endswith("_split") else name
        if base in W.CONFIGS:
            e["algorithmic_kv_bytes"] = W.generate(base, poison=False).kv_bytes()
        out["workloads"][name] = e
    with open(os.path.join(ROOT, "profiles", TRAFFIC_FILE), "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out))


KERNEL_NAME = {"step": "paged_attn_balanced_kernel (decode step: append folded in)",
               "balanced": "paged_attn_balanced_kernel",
               "split": "paged_attn_kernel (split)", "direct": "paged_attn_kernel (direct)"}


def main():
    args = parse()
    if args.pmc_summary:
        pmc_summary(args, *args.pmc_summary)
        return
    if args.trace_summary:
        trace_summary(args, args.trace_summary)
        return
    if args.counter_summary:
        counter_summary(args, *args.counter_summary[:2])
        return
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

    # ---- headline: the Llama-3-8B decode step (c2) --------------------------------------
    mark(torch)
    main_name = "llama3_8b"
    wl = W.generate(main_name, poison=False)
    part = args.partition or PARTITION[main_name]
    r = Runner(P, wl, args.path, part, workgroups=args.workgroups, layout=args.layout)
    meas = r.measure(args.steps, args.warmup, args.event_steps)
    log(f"{main_name} {args.path}: {meas[0] / args.steps * 1e6:.2f} us/step, attention "
        f"{meas[1].mean():.2f} us, merge {meas[2].mean():.2f} us")
    configs = {}
    configs["c2"], _, _ = config_entry(P, torch, W, "c2", main_name, args.path, args,
                                       main=(r, meas))
    res = summarize(wl, meas[0], args.steps, *meas[1:])
    del r
    torch.cuda.empty_cache()

    others = {}
    if not args.no_others:
        mark(torch)
        kv_app = append_entry(P, torch, W, max(args.steps, 20))
        configs["c1"], r1, _ = config_entry(P, torch, W, "c1", "tiny_fp32", "step", args)
        configs["c1"]["kv_append"] = kv_app
        del r1
        log(f"c1 done: {configs['c1']['us_per_step']:.2f} us/step, kv_append "
            f"{kv_app['us_per_launch']} us")
        for label, name in (("c3", "llama2_70b_prefix"), ("c4", "long_128k")):
            mark(torch)
            configs[label], rr, _ = config_entry(P, torch, W, label, name, "step", args)
            del rr
            torch.cuda.empty_cache()
            log(f"{label} done: {configs[label]['us_per_step']:.2f} us/step")
        mark(torch)
        configs["c4"]["split"] = split_entry(P, torch, W, "long_128k", args)
        log(f"c4 split done: partition {configs['c4']['split']['partition_tokens']}, "
            f"{configs['c4']['split']['us_per_step']:.2f} us/step")
        mark(torch)
        configs["c5"], rr, _ = config_entry(P, torch, W, "c5", "verify_int8", "step", args)
        del rr
        torch.cuda.empty_cache()
        log(f"c5 done: {configs['c5']['us_per_step']:.2f} us/step")
        for name in ("mistral_7b_window", "llama3_8b_fp8"):
            mark(torch)
            others[name], rr, _ = config_entry(P, torch, W, name, name, "step", args)
            del rr
            torch.cuda.empty_cache()
            log(f"{name} done")
        others["kv_copy_blocks"] = copy_blocks_bench(P, torch, W, min(args.steps, 40))
        mark(torch)
        others["kv_append_quant"] = append_quant_bench(P, torch, W, min(args.steps, 40))
        for name in ("prefill_chunk", "tree_verify"):
            mark(torch)
            others[name] = multi_query_bench(P, torch, W, name, min(args.steps, 20))
        log("others done")

    c2 = configs["c2"]
    tr = measured_traffic(main_name if args.path != "split" else main_name + "_split")
    traffic = None
    if tr is not None and tr.get("attn_fetch_bytes") is not None:
        traffic = tr["attn_fetch_bytes"] + (tr.get("attn_write_bytes") or 0)
    achieved = res["attn_kernel_GBps"]
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
                   "path": args.path, "layout": args.layout, "workgroups": c2["workgroups"],
                   "partition_tokens": part if args.path == "split" else None,
                   "kv_bytes_per_step": res["kv_bytes"]},
        "us_per_step": round(res["us_per_step"], 2),
        "pct_hbm_peak": round(res["pct_hbm_peak"], 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": KERNEL_NAME[args.path],
                     "kernel_us_mean": round(res["attn_kernel_us_mean"], 2),
                     "bytes_per_launch": res["kv_bytes"]},
        # the step as the task defines it: the attention call and its merge together
        "step_roofline": {"achieved": round(res["kernels_GBps"], 1), "peak": HBM_PEAK_GBS,
                          "unit": "GB/s", "frac": round(res["kernels_GBps"] / HBM_PEAK_GBS, 4),
                          "kernels_us_mean": round(res["kernels_us_mean"], 2),
                          "traffic": None if tr is None else tr.get("step_traffic_bytes")},
        "timing": {k: round(res[k], 3) for k in ("attn_kernel_us_mean", "attn_kernel_us_median",
                                                 "attn_kernel_us_p95", "merge_us_mean",
                                                 "merge_us_p95", "kernels_us_mean",
                                                 "kernels_us_p95")}
                  | {"event_samples": res["event_samples"]},
        "configs": configs,
        "others": others,
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
        if not args.no_others:
            line["cpu_oracle_others"] = cpu_oracle_others(W)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
