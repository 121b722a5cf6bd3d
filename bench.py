"""Benchmark of the paged KV-cache attention hot path on one MI355X.

A step is one batch through the whole path: validate + plan (host, once per
batch) and then, for each of the model's layers, append the new K/V rows,
run attention and merge split tiles ("Deep Dive - FlashInfer", "Plan then
run": one plan serves every layer of a batch; "GPU attention backends",
"FlashInfer: plan and run": 28 layers share one plan).  Every layer has its
own KV pool, so the working set is far larger than the 256 MB MALL and the
KV stream comes from HBM.

Headline workload: batch paged decode, 64 requests, kv_len U[512, 4096],
page 16, 20k-page pool, 32 query / 8 kv heads, head_dim 128, bf16, NHD.
value = algorithmic bytes of all layers / step time (GB/s).  The same JSON
line carries the roofline of the attention kernel (HIP events around each
launch), the chunked-prefill TFLOP/s secondary, the skewed and MLA decode
secondaries, and the CPU oracle baseline.

    python bench.py [--steps K] [--warmup W] [--layers L] [--gpus 1]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0                  # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2516.6              # MI355X dense bf16 MFMA, published (256 CU x 2.4 GHz x 4096)
METRIC = "paged decode KV-read GB/s + prefill TFLOP/s, each as fraction of MI355X peak"
KERNEL_SOURCES = ["attn_rows.hip", "attn_rows_one_wave.hip", "prefill_mfma.hip", "mla_decode.hip", "merge_append.hip",
                  "device.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "paged_kv_cache_plan_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ------------------------------------------------------------ work counts --

def decode_bytes(b) -> dict:
    """Algorithmic HBM bytes of one decode layer: every K and V row read once
    per kv head, Q read, O and LSE written, page ids read; append reads and
    writes the new rows."""
    es = 2 if b.dtype == "bf16" else 4
    es_kv = {"bf16": 2, "fp8": 1}.get(b.kv_dtype, 4)
    kv = sum(b.kv_lens) * b.num_kv_heads * b.head_dim * 2 * es_kv
    q = b.nnz * b.num_qo_heads * b.head_dim * es
    o = q
    lse = b.nnz * b.num_qo_heads * 4
    idx = int(b.kv_indptr[-1]) * 4
    append = 0 if b.k_new is None else 2 * 2 * b.k_new.size * es_kv
    attn = kv + q + o + lse + idx
    # With the append fused into the attention launch the new rows are read
    # once (as keys, already in kv) and written once into the cache.
    return {"kv": kv, "attn": attn, "append": append, "layer": attn + append,
            "attn_fused": attn + append // 2, "layer_fused": attn + append // 2}


def prefill_flops(b) -> int:
    """2 * Hq * (d_qk + d_vo) per visible (row, key) pair; masked pairs are not counted."""
    pairs = sum(q * (k - q) + q * (q + 1) // 2 for q, k in zip(b.qo_lens, b.kv_lens))
    return 2 * b.num_qo_heads * (2 * b.head_dim) * pairs


def mla_bytes(b) -> dict:
    kv = sum(b.kv_lens) * 576 * 2
    q = b.batch_size * 128 * 576 * 2
    o = b.batch_size * 128 * 512 * 2
    lse = b.batch_size * 128 * 4
    idx = int(b.kv_indptr[-1]) * 4
    flops = sum(b.kv_lens) * 128 * (576 + 512) * 2
    return {"kv": kv, "attn": kv + q + o + lse + idx, "flops": flops}


def cascade_bytes(b) -> dict:
    """Algorithmic bytes of one cascade run: every node's K and V rows once per
    kv head (shared nodes once, not once per request), Q read, O and LSE
    written, page ids read.  ``flat_kv`` is what the same batch reads through
    a flat page table (every request reading its whole path)."""
    es = 2 if b.dtype == "bf16" else 4
    row = b.num_kv_heads * b.head_dim * 2 * es
    levels = b.extra["levels"]
    kv = sum(sum(lv["kv_lens"]) for lv in levels) * row
    q = b.nnz * b.num_qo_heads * b.head_dim * es
    lse = b.nnz * b.num_qo_heads * 4
    idx = sum(int(lv["kv_indptr"][-1]) for lv in levels) * 4
    flat_tokens = 0
    for r in range(b.batch_size):
        row0 = int(b.qo_indptr[r])
        for lv in levels:
            n = int(np.searchsorted(lv["qo_indptr"], row0, side="right")) - 1
            flat_tokens += lv["kv_lens"][n]
    return {"kv": kv, "attn": kv + 2 * q + lse + idx, "flat_kv": flat_tokens * row}


# ---------------------------------------------------------------- runners --

class Runner:
    """Device copies of one batch with ``layers`` independent KV pools."""

    def __init__(self, b, layers: int, time_merge: bool = False):
        import torch
        import paged_kv_cache_plan_amd as pkv
        self.b, self.torch, self.pkv = b, torch, pkv
        self.time_merge = time_merge
        # Decode attention is timed with events that the kernel's own dispatch
        # records (pkv_time_next_attention): no event packets in the stream.
        # Other runs record events on the stream around the timed launches.
        self.kernel_events = not time_merge and b.mode == "decode"
        # Decode batches with new rows append them inside the attention launch
        # (pkv_run_append) unless a separate append kernel is asked for.
        self.fused_append = b.mode == "decode" and b.k_new is not None
        # Decode plans may fold the split merge into the attention launch
        # (plan_params merge_in_launch); set before make_plan.
        self.separate_merge = True
        dev = lambda x, bf: (torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
                             if bf else torch.from_numpy(np.ascontiguousarray(x)).cuda())
        bf = b.dtype == "bf16"
        kv_bf = b.kv_dtype == "bf16"   # fp8 caches stay uint8 codes
        self.q = dev(b.q, bf)
        self.kv_indices = dev(b.kv_indices, False)
        if b.mode == "mla":
            self.q_kpe = dev(b.q_kpe, True)
            base = dev(b.k_cache, True)
            self.pools = [base] + [base.clone() for _ in range(layers - 1)]
            self.out = torch.empty((b.batch_size, 128, 512), dtype=torch.bfloat16, device="cuda")
            self.lse = torch.empty((b.batch_size, 128), dtype=torch.float32, device="cuda")
        else:
            k0, v0 = dev(b.k_cache, kv_bf), dev(b.v_cache, kv_bf)
            self.pools = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(layers - 1)]
            self.out = torch.empty_like(self.q)
            self.lse = torch.empty((b.nnz, b.num_qo_heads), dtype=torch.float32, device="cuda")
            if b.k_new is not None:
                self.k_new, self.v_new = dev(b.k_new, kv_bf), dev(b.v_new, kv_bf)
                self.append_indptr = dev(b.append_indptr, False)
                self.kv_indptr_d = dev(b.kv_indptr, False)
                self.last_d = dev(b.kv_last_page_len, False)
        self.params = pkv.plan_params(
            mode=b.mode, batch_size=b.batch_size, num_qo_heads=b.num_qo_heads, num_kv_heads=b.num_kv_heads,
            head_dim_qk=576 if b.mode == "mla" else b.head_dim, head_dim_vo=512 if b.mode == "mla" else b.head_dim,
            page_size=b.page_size, causal=b.causal, dtype=b.dtype, max_num_pages=b.max_num_pages,
            kv_dtype=b.kv_dtype)
        info, _, _ = pkv.plan_compute(self.params, qo_indptr=b.qo_indptr if b.mode == "prefill" else None,
                                      kv_indptr=b.kv_indptr, kv_indices=b.kv_indices,
                                      kv_last_page_len=b.kv_last_page_len)
        self.workspace = torch.empty(max(info["workspace_bytes"], 256), dtype=torch.uint8, device="cuda")
        self.staging = torch.empty(max(info["staging_bytes"], 256), dtype=torch.uint8, pin_memory=True)
        self.plan = None

    def make_plan(self):
        b = self.b
        self.plan = self.pkv.Plan(self.params, qo_indptr=b.qo_indptr if b.mode == "prefill" else None,
                                  kv_indptr=b.kv_indptr, kv_indices=b.kv_indices, kv_last_page_len=b.kv_last_page_len,
                                  workspace=self.workspace, staging=self.staging)
        # o is final after the attention call (the split merge inside it)
        self.merged = (b.mode == "decode" and not self.separate_merge
                       and bool(self.plan.info["merge_in_launch"]))
        return self.plan

    def append(self, i: int):
        """append_paged_kv of the batch's new rows into layer i's pool."""
        b = self.b
        k, v = self.pools[i % len(self.pools)]
        self.pkv.append_paged_kv(self.k_new, self.v_new, self.append_indptr, self.kv_indptr_d, self.kv_indices,
                                 self.last_d, k, v, layout=b.layout, page_size=b.page_size)

    def layer(self, i: int, ev=None):
        """append + attention + merge for layer i; ev = (start, end) events around
        attention (and the merge too when time_merge is set; run_mla always merges)."""
        b, plan = self.b, self.plan
        if b.mode == "mla":
            pool = self.pools[i % len(self.pools)]
            if ev:
                ev[0].record()
            plan.run_mla(self.q, self.q_kpe, pool[..., :512], pool[..., 512:], self.kv_indices, self.out, self.lse,
                         sm_scale=b.sm_scale)
            if ev:
                ev[1].record()
            return
        k, v = self.pools[i % len(self.pools)]
        if b.k_new is not None and not self.fused_append:
            self.append(i)
        if ev:
            if self.kernel_events:
                self.pkv.time_next_attention(ev[0], ev[1])
            else:
                ev[0].record()
        merged = self.merged
        if self.fused_append:
            plan.run_append(self.q, k, v, self.kv_indices, self.out, self.lse, k_new=self.k_new, v_new=self.v_new,
                            append_indptr=self.append_indptr, kv_indptr=self.kv_indptr_d,
                            kv_last_page_len=self.last_d, layout=b.layout, sm_scale=b.sm_scale, with_merge=merged)
        elif merged:
            plan.run(self.q, k, v, self.kv_indices, self.out, self.lse, layout=b.layout, sm_scale=b.sm_scale)
        else:
            plan.run_attention(self.q, k, v, self.kv_indices, self.out, self.lse, layout=b.layout,
                               sm_scale=b.sm_scale)
        if self.time_merge and not merged:
            plan.run_merge(self.out, self.lse)
        if ev and not self.kernel_events:
            ev[1].record()
        if not self.time_merge and not merged:
            plan.run_merge(self.out, self.lse)


class CascadeRunner(Runner):
    """A cascade batch: per layer, append the new rows into the leaves, then
    pkv_cascade_run (one attention launch per level + the row merge)."""

    def __init__(self, b, layers: int, target_per_cu: int = 0):
        import torch
        import paged_kv_cache_plan_amd as pkv
        self.b, self.torch, self.pkv = b, torch, pkv
        self.time_merge = True
        self.kernel_events = False
        dev = lambda x, bf: (torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
                             if bf else torch.from_numpy(np.ascontiguousarray(x)).cuda())
        bf = b.dtype == "bf16"
        self.levels = b.extra["levels"]
        self.q = dev(b.q, bf)
        self.all_indices = dev(np.concatenate([lv["kv_indices"][:lv["kv_indptr"][-1]] for lv in self.levels]), False)
        self.kv_indices = dev(b.kv_indices, False)
        k0, v0 = dev(b.k_cache, bf), dev(b.v_cache, bf)
        self.pools = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(layers - 1)]
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty((b.nnz, b.num_qo_heads), dtype=torch.float32, device="cuda")
        self.k_new, self.v_new = dev(b.k_new, bf), dev(b.v_new, bf)
        self.append_indptr = dev(b.append_indptr, False)
        self.kv_indptr_d = dev(b.kv_indptr, False)
        self.last_d = dev(b.kv_last_page_len, False)
        self.params = pkv.plan_params(mode="prefill", batch_size=0, num_qo_heads=b.num_qo_heads,
                                      num_kv_heads=b.num_kv_heads, head_dim_qk=b.head_dim, page_size=b.page_size,
                                      causal=b.causal, dtype=b.dtype, max_num_pages=b.max_num_pages,
                                      target_per_cu=target_per_cu)
        info = pkv.cascade_plan_compute(self.params, self.levels)[0]
        self.workspace = torch.empty(max(info["workspace_bytes"], 256), dtype=torch.uint8, device="cuda")
        self.staging = torch.empty(max(info["staging_bytes"], 256), dtype=torch.uint8, pin_memory=True)
        self.plan = None

    def make_plan(self):
        self.plan = self.pkv.CascadePlan(self.params, self.levels, workspace=self.workspace, staging=self.staging)
        return self.plan

    def layer(self, i: int, ev=None):
        b = self.b
        k, v = self.pools[i % len(self.pools)]
        self.pkv.append_paged_kv(self.k_new, self.v_new, self.append_indptr, self.kv_indptr_d, self.kv_indices,
                                 self.last_d, k, v, layout=b.layout, page_size=b.page_size)
        if ev:
            ev[0].record()
        self.plan.run(self.q, k, v, self.all_indices, self.out, self.lse, layout=b.layout, sm_scale=b.sm_scale)
        if ev:
            ev[1].record()


def measure_append(runner: Runner, layers: int, reps: int = 24) -> dict:
    """Append on its own: ``reps`` launches into the layers' pools back to
    back between two stream events, three times; the per-launch time is the
    median of the three group means (it includes the small gap between
    consecutive launches)."""
    torch = runner.torch
    for i in range(layers):
        runner.append(i)
    torch.cuda.synchronize()
    per = []
    for _ in range(3):
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record()
        for i in range(reps):
            runner.append(i)
        s1.record()
        torch.cuda.synchronize()
        per.append(s0.elapsed_time(s1) / reps)
    return {"ms_mean": float(np.mean(per)), "ms_median": float(np.median(per)), "launches": 3 * reps}


def measure(runner: Runner, layers: int, steps: int, warmup: int, ev_every: int = 1) -> dict:
    """Time `steps` steps (plan + `layers` layers each).  The attention launch
    of every `ev_every`-th layer is also timed with a pair of HIP events inside
    the same timed region: recorded by the kernel's own dispatch when the
    runner times attention alone, else recorded on the stream around the
    timed launches (a stream event pair costs a few microseconds)."""
    torch = runner.torch
    for _ in range(warmup):
        runner.make_plan()
        for i in range(layers):
            runner.layer(i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           if i % ev_every == 0 else None for _ in range(steps) for i in range(layers)]
    for e in evs:                       # create the events outside the timed region
        if e is not None:
            e[0].record()
            e[1].record()
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    for s in range(steps):
        runner.make_plan()
        for i in range(layers):
            runner.layer(i, evs[s * layers + i])
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    step_ms = t_start.elapsed_time(t_end) / steps
    attn_ms = [e[0].elapsed_time(e[1]) for e in evs if e is not None]
    # Host planning time on its own: inside the timed steps make_plan also
    # waits until the GPU has consumed the previous plan's pinned staging, so
    # it is timed again here with the GPU idle.
    plan_host = []
    for _ in range(10):
        torch.cuda.synchronize()
        p0 = time.perf_counter()
        runner.make_plan()
        plan_host.append(time.perf_counter() - p0)
    torch.cuda.synchronize()
    return {"ms_per_step": step_ms, "wall_ms_per_step": wall * 1e3 / steps,
            "attn_ms_mean": float(np.mean(attn_ms)), "attn_ms_median": float(np.median(attn_ms)),
            "attn_ms_p10": float(np.percentile(attn_ms, 10)), "attn_ms_p90": float(np.percentile(attn_ms, 90)),
            "plan_host_ms": float(np.median(plan_host)) * 1e3, "plan_info": runner.plan.info,
            "launches_timed": len(attn_ms)}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


_ORACLE_BATCHES = {}   # host batches the forked oracle workers read (copy-on-write)


_WORKER_LIMITS = []


def _oracle_worker_init():
    """Each worker process runs BLAS on one thread (set once per process)."""
    from threadpoolctl import threadpool_limits
    _WORKER_LIMITS.append(threadpool_limits(limits=1))


def _oracle_task(task):
    """One oracle call in a worker process: (workload, heads, requests)."""
    from oracle import attention as oat
    name, heads, reqs = task
    b = _ORACLE_BATCHES[name]
    if name == "mla":
        oat.mla_decode(b.q, b.q_kpe, b.k_cache[..., :512], b.k_cache[..., 512:], kv_indptr=list(b.kv_indptr),
                       kv_indices=list(b.kv_indices), kv_last_page_len=list(b.kv_last_page_len),
                       page_size=b.page_size, sm_scale=b.sm_scale, requests=reqs)
    else:
        oat.paged_attention(b.q, b.k_cache, b.v_cache, qo_indptr=list(b.qo_indptr), kv_indptr=list(b.kv_indptr),
                            kv_indices=b.kv_indices, kv_last_page_len=list(b.kv_last_page_len),
                            page_size=b.page_size, layout=b.layout, num_kv_heads=b.num_kv_heads, causal=b.causal,
                            sm_scale=b.sm_scale, q_dtype=b.dtype, kv_dtype=b.kv_dtype, heads=heads, requests=reqs)
    return None


def _oracle_tasks(name, b, workers):
    """A task is one request with all its heads (an oracle call gathers a
    request's keys once for the heads it computes), unless the request holds
    more than a quarter of a worker's share of the work: then its kv-head
    groups are split over several tasks.  Largest tasks first."""
    if name == "mla":
        return [("mla", None, [r]) for r in sorted(range(b.batch_size), key=lambda r: -b.kv_lens[r])]
    g = b.num_qo_heads // b.num_kv_heads
    cost = [q * k for q, k in zip(b.qo_lens, b.kv_lens)]
    share = max(1, sum(cost) / (4 * workers))
    tasks = []
    for r in range(b.batch_size):
        parts = min(b.num_kv_heads, max(1, int(-(-cost[r] // share))))
        while b.num_kv_heads % parts:
            parts -= 1
        per = b.num_kv_heads // parts
        for i in range(parts):
            tasks.append((cost[r] / parts, (name, list(range(i * per * g, (i + 1) * per * g)), [r])))
    return [t for _, t in sorted(tasks, key=lambda t: -t[0])]


def cpu_baseline(batches: dict) -> dict:
    """The float64 oracle, as it stands, on every host core, for each of the
    five workloads: the worked example, the decode, skewed-decode, prefill and
    MLA batches (the same host arrays the GPU runs use).  Oracle calls run in
    a pool of worker processes, one per core and one BLAS thread each, forked
    before anything in this process touches the GPU; a task is a request (or
    a kv-head group of a long one).  The worked example and the two decode
    batches are timed three times (median), prefill and MLA once.  Throughput
    counts the GPU's algorithmic bytes or FLOPs (the oracle scores every pair
    and masks afterwards, so prefill does more work than it is credited
    with)."""
    import multiprocessing
    import workloads as wl
    workers = os.cpu_count() or 1
    plan = [("C1 worked example", "worked", 3), ("C2 decode", "decode", 3), ("C3 skewed decode", "skewed", 3),
            ("C4 prefill", "prefill", 1), ("C5 MLA decode", "mla", 1)]
    for _, name, _ in plan:
        if name not in batches:
            batches[name] = wl.make(name, literal_pages=True) if name == "worked" else wl.make(name)
        _ORACLE_BATCHES[name] = batches[name]
    configs = {}
    with multiprocessing.get_context("fork").Pool(workers, initializer=_oracle_worker_init) as pool:
        pool.map(_oracle_task, _oracle_tasks("worked", batches["worked"], workers))   # start the workers
        for label, name, runs in plan:
            b = batches[name]
            tasks = _oracle_tasks(name, b, workers)
            times = []
            for _ in range(runs):
                t0 = time.perf_counter()
                pool.map(_oracle_task, tasks, chunksize=1)
                times.append(time.perf_counter() - t0)
            sec = float(np.median(times))
            ent = {"seconds": round(sec, 4), "runs": runs, "tasks": len(tasks)}
            if name in ("decode", "skewed"):
                ent["GB/s"] = round(decode_bytes(b)["attn"] / sec / 1e9, 4)
            elif name == "prefill":
                ent["GFLOP/s"] = round(prefill_flops(b) / sec / 1e9, 3)
            elif name == "mla":
                mb = mla_bytes(b)
                ent["GB/s"] = round(mb["attn"] / sec / 1e9, 4)
                ent["GFLOP/s"] = round(mb["flops"] / sec / 1e9, 3)
            configs[label] = ent
            log(f"cpu oracle {label}: {sec:.3f} s ({runs} run(s), {len(tasks)} tasks on {workers} processes)")
    _ORACLE_BATCHES.clear()
    c2 = configs["C2 decode"]
    return {"value": c2["GB/s"], "unit": "GB/s", "cores": workers, "kind": "oracle",
            "sample": f"the float64 numpy oracle over every request and head of each workload, in {workers} "
                      "worker processes with one BLAS thread each (tasks: a request, or a kv-head group of a "
                      "long one); value = the decode batch (median of 3 runs), its algorithmic "
                      "KV+Q+O+LSE+index bytes / oracle seconds",
            "cpu_model": _cpu_model(), "host_cpus": os.cpu_count(), "blas_threads_per_worker": 1,
            "configs": configs}


def device_facts(torch) -> dict:
    """CU count and peak engine clock of the GPU (rocminfo), next to the
    published peaks the fractions use."""
    import subprocess
    props = torch.cuda.get_device_properties(0)
    out = {"name": props.name, "cus": props.multi_processor_count, "max_clock_mhz": None,
           "arch": getattr(props, "gcnArchName", None), "hbm_peak_gbs": HBM_PEAK_GBS,
           "bf16_peak_tflops": BF16_PEAK_TFLOPS,
           "peaks": "published MI355X figures: 8 TB/s HBM3E; 256 CU x 2.4 GHz x 4096 bf16 flop/clk"}
    try:
        txt = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=30).stdout
        agent = None
        for line in txt.splitlines():
            line = line.strip()
            if line.startswith("Name:") and "gfx" in line:
                agent = line.split(":", 1)[1].strip()
            if agent and agent.startswith("gfx950") and line.startswith("Max Clock Freq. (MHz):"):
                out["max_clock_mhz"] = int(line.split(":", 1)[1].strip())
                break
    except (OSError, ValueError, subprocess.SubprocessError):
        pass
    return out


COUNTER_KERNELS = {"decode": "attn_rows_kernel", "skewed": "attn_rows_kernel", "prefill": "prefill_mfma_kernel",
                   "mla": "mla_decode_kernel", "cascade": "prefill_mfma_kernel", "fp8": "attn_rows_kernel",
                   "fp8_prefill": "prefill_mfma_kernel"}


def ingest_counters(workload: str, fetch_csv: str, write_csv: str, command: str) -> dict:
    """HBM bytes per launch of the workload's attention kernel from two rocprofv3
    --pmc runs (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch) of
    ``bench.py --only W --calibrate-copy-mib M``.  Each counter is scaled by
    what it reads for the calibration pass: the fill of the M MiB source (its
    WRITE_SIZE) and the plain device copy right after it (its FETCH_SIZE)."""
    import csv

    def rows(path):
        with open(path) as f:
            out = {}
            for r in csv.DictReader(f):
                out[int(r["Dispatch_Id"])] = (r["Kernel_Name"], float(r["Counter_Value"]))
            return [out[k] for k in sorted(out)]

    def calib(rs, counter):
        for i, (name, val) in enumerate(rs):
            if "FillFunctor" in name:
                copy = next(v for n, v in rs[i + 1:] if "copyBuffer" in n)
                return val if counter == "WRITE_SIZE" else copy
        raise ValueError("no calibration fill/copy dispatch in the counter file")

    f_rows, w_rows = rows(fetch_csv), rows(write_csv)
    known_kib = None
    for name, val in w_rows:
        if "FillFunctor" in name:
            known_kib = val        # fill of the calibration source: written once, exactly
            break
    if known_kib is None:
        raise ValueError("no calibration fill dispatch")
    f_scale = known_kib / calib(f_rows, "FETCH_SIZE")
    w_scale = known_kib / calib(w_rows, "WRITE_SIZE")
    sub = COUNTER_KERNELS[workload]
    fetch = [v for n, v in f_rows if sub in n]
    write = [v for n, v in w_rows if sub in n]
    fb = float(np.mean(fetch)) * 1024 * f_scale
    wb = float(np.mean(write)) * 1024 * w_scale
    return {"source_hash": source_hash(), "kernel": sub, "dispatches": len(fetch),
            "fetch_kib_raw": float(np.mean(fetch)), "write_kib_raw": float(np.mean(write)),
            "fetch_scale": round(f_scale, 5), "write_scale": round(w_scale, 5),
            "fetch_bytes": round(fb), "write_bytes": round(wb), "bytes_per_launch": round(fb + wb),
            "command": command}


def read_traffic(kernel: str):
    """Counter-measured HBM traffic per launch from profiles/, if taken on this kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    ent = data.get(kernel)
    if not ent or ent.get("source_hash") != source_hash():
        return None
    return ent.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=28)
    ap.add_argument("--secondary-layers", type=int, default=4)
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["decode", "prefill", "fp8_prefill", "skewed", "mla", "cascade", "fp8"],
                    default=None,
                    help="time one workload (profiling runs)")
    ap.add_argument("--cascade-target", type=int, default=0,
                    help="planner target items per CU for every cascade level (0: the per-mode default)")
    ap.add_argument("--no-flat", action="store_true", help="skip the flat-page-table comparison run")
    ap.add_argument("--event-every", type=int, default=4,
                    help="time the attention launch of every N-th layer of the decode workloads")
    ap.add_argument("--stream-events", action="store_true",
                    help="record timing events on the stream around launches instead of by the dispatch")
    ap.add_argument("--separate-append", action="store_true",
                    help="decode workloads: launch append_paged_kv on its own before each attention launch "
                         "instead of fusing it into the attention launch (pkv_run_append)")
    ap.add_argument("--merge-in-launch", action="store_true",
                    help="decode workloads: plans with merge_in_launch = 1, which fold the split merge into the "
                         "attention launch where they can (default: a merge launch of its own)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--ingest-counters", nargs=3, metavar=("WORKLOAD", "FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter files into profiles/traffic.json (no GPU)")
    args = ap.parse_args()
    if args.ingest_counters:
        w, fcsv, wcsv = args.ingest_counters
        path = os.path.join(ROOT, "profiles", "traffic.json")
        data = json.load(open(path)) if os.path.exists(path) else {}
        cmd = (f"rocprofv3 --pmc {{FETCH_SIZE|WRITE_SIZE}} -f csv -d <dir> -o p -- python3 bench.py --only {w} "
               "--steps 2 --warmup 1 --layers 4 --secondary-layers 4 --no-cpu-baseline --no-flat --calibrate-copy-mib 512")
        data[w] = ingest_counters(w, fcsv, wcsv, cmd)
        with open(path, "w") as f:
            json.dump(data, f, indent=1, sort_keys=True)
        print(json.dumps(data[w]))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path; run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import workloads as wl
    which = [args.only] if args.only else ["decode"] + ([] if args.no_secondary else
                                                        ["prefill", "fp8_prefill", "skewed", "mla",
                                                         "cascade", "fp8"])
    # Host batches of the five workloads the CPU baseline times (the GPU runs
    # reuse them).  The baseline forks its worker processes before anything
    # in this process touches the GPU.
    host = {}
    with_cpu = not args.no_cpu_baseline and not args.only
    for name in ("decode", "prefill", "skewed", "mla"):
        if name in which or with_cpu:
            host[name] = wl.make(name, with_append=True) if name == "decode" else wl.make(name)
    cpu = cpu_baseline(host) if with_cpu else None

    import torch
    import paged_kv_cache_plan_amd as pkv
    assert torch.cuda.is_available(), "bench.py needs a ROCm GPU"
    pkv.lib()
    dev = device_facts(torch)
    log(f"device: {dev['name']} {dev['arch']}, CUs {dev['cus']}, max clock {dev['max_clock_mhz']} MHz")

    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy: {n} bytes read, {n} bytes written")

    result = {}

    if "decode" in which:
        b = host["decode"]
        r = Runner(b, args.layers)
        r.kernel_events = r.kernel_events and not args.stream_events
        r.fused_append = r.fused_append and not args.separate_append
        r.separate_merge = not args.merge_in_launch
        r.params.merge_in_launch = int(args.merge_in_launch)
        m = measure(r, args.layers, args.steps, args.warmup, ev_every=args.event_every)
        m["append"] = measure_append(r, args.layers)
        nb = decode_bytes(b)
        fused = r.fused_append
        merge_in = bool(r.plan.info["merge_in_launch"]) and not r.separate_merge
        value = nb["layer_fused" if fused else "layer"] * args.layers / (m["ms_per_step"] * 1e-3) / 1e9
        launch_bytes = nb["attn_fused" if fused else "attn"]
        achieved = launch_bytes / (m["attn_ms_mean"] * 1e-3) / 1e9
        result["decode"] = dict(m, value=value, bytes=nb, achieved=achieved, fused=fused, merge_in=merge_in,
                                launch_bytes=launch_bytes)
        log(f"decode: {value:.1f} GB/s per step, attention kernel {achieved:.1f} GB/s "
            f"({m['attn_ms_mean'] * 1e3:.1f} us), plan {m['plan_host_ms']:.3f} ms host")
        del r
    if "prefill" in which:
        b = host["prefill"]
        layers = args.secondary_layers
        r = Runner(b, layers)
        m = measure(r, layers, max(1, min(args.steps, 5)), 1)
        m["append"] = measure_append(r, layers)
        fl = prefill_flops(b)
        tf = fl / (m["attn_ms_mean"] * 1e-3) / 1e12
        step_tf = fl * layers / (m["ms_per_step"] * 1e-3) / 1e12
        ab = decode_bytes(b)["append"]
        result["prefill"] = dict(m, tflops=tf, step_tflops=step_tf, flops=fl, append_bytes=ab,
                                 append_gbs=ab / (m["append"]["ms_median"] * 1e-3) / 1e9)
        log(f"prefill: attention {tf:.1f} TFLOP/s ({m['attn_ms_mean']:.3f} ms), step {step_tf:.1f} TFLOP/s, "
            f"append {result['prefill']['append_gbs']:.1f} GB/s ({m['append']['ms_median'] * 1e3:.1f} us)")
        del r
    if "fp8_prefill" in which:
        # The prefill batch over an E4M3 cache (bf16 queries and outputs).
        b = wl.make("prefill", kv_dtype="fp8")
        layers = args.secondary_layers
        r = Runner(b, layers)
        m = measure(r, layers, max(1, min(args.steps, 5)), 1)
        fl = prefill_flops(b)
        tf = fl / (m["attn_ms_mean"] * 1e-3) / 1e12
        result["fp8_prefill"] = dict(m, tflops=tf, flops=fl)
        log(f"fp8 prefill: attention {tf:.1f} TFLOP/s ({m['attn_ms_mean']:.3f} ms)")
        del r
    if "skewed" in which:
        b = host["skewed"]
        layers = args.secondary_layers
        r = Runner(b, layers, time_merge=True)
        r.separate_merge = not args.merge_in_launch
        r.params.merge_in_launch = int(args.merge_in_launch)
        m = measure(r, layers, args.steps, args.warmup)
        nb = decode_bytes(b)
        result["skewed"] = dict(m, gbs=nb["attn"] / (m["attn_ms_mean"] * 1e-3) / 1e9, bytes=nb)
        log(f"skewed: attention + merge {result['skewed']['gbs']:.1f} GB/s ({m['attn_ms_mean'] * 1e3:.1f} us)")
        del r
    if "mla" in which:
        b = host["mla"]
        layers = args.secondary_layers
        r = Runner(b, layers)
        m = measure(r, layers, args.steps, args.warmup)
        nb = mla_bytes(b)
        result["mla"] = dict(m, gbs=nb["attn"] / (m["attn_ms_mean"] * 1e-3) / 1e9,
                             tflops=nb["flops"] / (m["attn_ms_mean"] * 1e-3) / 1e12, bytes=nb)
        log(f"mla: run {result['mla']['gbs']:.1f} GB/s, {result['mla']['tflops']:.1f} TFLOP/s "
            f"({m['attn_ms_mean'] * 1e3:.1f} us)")
        del r

    if "fp8" in which:
        # The headline decode batch over an E4M3 cache (one byte per element).
        b = wl.make("decode", with_append=True, kv_dtype="fp8")
        layers = args.layers
        r = Runner(b, layers)
        r.kernel_events = r.kernel_events and not args.stream_events
        r.fused_append = r.fused_append and not args.separate_append
        r.separate_merge = not args.merge_in_launch
        r.params.merge_in_launch = int(args.merge_in_launch)
        m = measure(r, layers, args.steps, args.warmup, ev_every=args.event_every)
        nb = decode_bytes(b)
        fz = "_fused" if r.fused_append else ""
        result["fp8"] = dict(m, bytes=nb, gbs=nb["attn" + fz] / (m["attn_ms_mean"] * 1e-3) / 1e9,
                             step_gbs=nb["layer" + fz] * layers / (m["ms_per_step"] * 1e-3) / 1e9,
                             launch_bytes=nb["attn" + fz])
        log(f"fp8: attention {result['fp8']['gbs']:.1f} GB/s ({m['attn_ms_mean'] * 1e3:.1f} us), "
            f"step {result['fp8']['step_gbs']:.1f} GB/s")
        del r
    if "cascade" in which:
        b = wl.make("cascade")
        layers = args.secondary_layers
        r = CascadeRunner(b, layers, args.cascade_target)
        m = measure(r, layers, args.steps, args.warmup)
        nb = cascade_bytes(b)
        del r
        flat_us = float("nan")
        if not args.no_flat:
            # The same batch through a flat page table (each request reads its whole path).
            fl = wl.flat_levels(b)
            bf = wl.Batch(**{**b.__dict__, "mode": "decode", "kv_indptr": fl["kv_indptr"],
                             "kv_indices": fl["kv_indices"], "kv_last_page_len": fl["kv_last_page_len"],
                             "kv_lens": fl["kv_lens"], "extra": {}})
            rf = Runner(bf, layers, time_merge=True)
            flat_us = measure(rf, layers, max(2, args.steps // 4), 1)["attn_ms_mean"] * 1e3
            del rf
        result["cascade"] = dict(m, bytes=nb, gbs=nb["attn"] / (m["attn_ms_mean"] * 1e-3) / 1e9, flat_us=flat_us)
        log(f"cascade: run {m['attn_ms_mean'] * 1e3:.1f} us ({result['cascade']['gbs']:.1f} GB/s unique), "
            f"flat decode {flat_us:.1f} us")

    if args.only and args.only != "decode":
        print(json.dumps({k: {kk: vv for kk, vv in v.items() if kk != "plan_info"} for k, v in result.items()}))
        return

    d = result["decode"]
    line = {
        "metric": METRIC,
        "value": round(d["value"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(d["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "batch paged decode: 64 requests, qo_len 1, kv_len U[512,4096], page_size 16, "
                               "20000-page shuffled pool, 32 qo / 8 kv heads, head_dim 128, bf16, NHD; "
                               f"step = plan + {args.layers} layers x ("
                               + ("one attention launch with the append fused in" if d["fused"]
                                  else "append + attention")
                               + (" and the split merge folded in)" if d["merge_in"] else " + merge)"),
                   "layers": args.layers, "batch": 64, "page_size": 16, "heads": [32, 8], "head_dim": 128},
        "roofline": {"bound": "hbm", "achieved": round(d["achieved"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(d["achieved"] / HBM_PEAK_GBS, 4), "traffic": read_traffic("decode"),
                     "kernel": "attention (decode)" + (", append fused in" if d["fused"] else "")
                               + (", split merge folded in" if d["merge_in"] else ""),
                     "bytes_per_launch": d["launch_bytes"],
                     "launch_us_mean": round(d["attn_ms_mean"] * 1e3, 2),
                     "launch_us_median": round(d["attn_ms_median"] * 1e3, 2),
                     "launch_us_p10_p90": [round(d["attn_ms_p10"] * 1e3, 2), round(d["attn_ms_p90"] * 1e3, 2)],
                     "launches_timed": d["launches_timed"]},
        "device": dev,
        "decode_append": {"launch_us_median": round(d["append"]["ms_median"] * 1e3, 2),
                          "bytes_per_launch": d["bytes"]["append"],
                          "gbs": round(d["bytes"]["append"] / (d["append"]["ms_median"] * 1e-3) / 1e9, 1),
                          "timed": "back-to-back launches between two stream events"},
        "plan_host_ms": round(d["plan_host_ms"], 4),
        "plan": {k: d["plan_info"][k] for k in ("num_items", "num_merges", "chunk_pages", "split")},
        "kernel_source": source_hash(),
    }
    if "prefill" in result:
        p = result["prefill"]
        line["prefill"] = {"value": round(p["tflops"], 2), "unit": "TFLOP/s", "peak": BF16_PEAK_TFLOPS,
                           "frac": round(p["tflops"] / BF16_PEAK_TFLOPS, 4),
                           "launch_ms_mean": round(p["attn_ms_mean"], 4),
                           "launch_ms_median": round(p["attn_ms_median"], 4), "flops_per_launch": p["flops"],
                           "step_tflops_incl_append": round(p["step_tflops"], 2),
                           "append": {"value": round(p["append_gbs"], 1), "unit": "GB/s",
                                      "frac": round(p["append_gbs"] / HBM_PEAK_GBS, 4),
                                      "launch_us_median": round(p["append"]["ms_median"] * 1e3, 2),
                                      "bytes_per_launch": p["append_bytes"],
                                      "timed": "back-to-back launches between two stream events"},
                           "workload": "chunked prefill/append: 8 requests, qo U[512,2048], prefix U[0,8192], "
                                       "page 16, HND, 32/8 heads, d128, bf16, causal"}
    if "fp8_prefill" in result:
        p = result["fp8_prefill"]
        line["fp8_prefill"] = {"value": round(p["tflops"], 2), "unit": "TFLOP/s", "peak": BF16_PEAK_TFLOPS,
                               "frac": round(p["tflops"] / BF16_PEAK_TFLOPS, 4),
                               "launch_ms_mean": round(p["attn_ms_mean"], 4),
                               "launch_ms_median": round(p["attn_ms_median"], 4),
                               "workload": "the chunked prefill batch with an E4M3 K/V cache (bf16 queries and "
                                           "outputs; the products run in bf16)"}
    if "skewed" in result:
        s = result["skewed"]
        line["skewed_decode"] = {"value": round(s["gbs"], 1), "unit": "GB/s", "frac": round(s["gbs"] / HBM_PEAK_GBS, 4),
                                 "run_us_mean": round(s["attn_ms_mean"] * 1e3, 2),
                                 "run_us_median": round(s["attn_ms_median"] * 1e3, 2), "timed": "attention + merge",
                                 "merge_items": s["plan_info"]["num_merges"]}
    if "mla" in result:
        mm = result["mla"]
        line["mla_decode"] = {"value": round(mm["gbs"], 1), "unit": "GB/s", "frac": round(mm["gbs"] / HBM_PEAK_GBS, 4),
                              "tflops": round(mm["tflops"], 2), "run_us_mean": round(mm["attn_ms_mean"] * 1e3, 2),
                              "run_us_median": round(mm["attn_ms_median"] * 1e3, 2),
                              "timed": "attention + merge"}
    if "fp8" in result:
        f = result["fp8"]
        line["fp8_decode"] = {"value": round(f["gbs"], 1), "unit": "GB/s", "frac": round(f["gbs"] / HBM_PEAK_GBS, 4),
                              "launch_us_mean": round(f["attn_ms_mean"] * 1e3, 2),
                              "launch_us_median": round(f["attn_ms_median"] * 1e3, 2),
                              "bytes_per_launch": f["launch_bytes"],
                              "step_gbs": round(f["step_gbs"], 1),
                              "workload": "the decode batch with an E4M3 K/V cache (bf16 queries and outputs), "
                                          "the append fused into the attention launch as in the decode step"}
    if "cascade" in result:
        c = result["cascade"]
        run_s = c["attn_ms_mean"] * 1e-3
        line["cascade"] = {"value": round(c["gbs"], 1), "unit": "GB/s", "frac": round(c["gbs"] / HBM_PEAK_GBS, 4),
                           "run_us_mean": round(c["attn_ms_mean"] * 1e3, 2),
                           "run_us_median": round(c["attn_ms_median"] * 1e3, 2),
                           "timed": "all level launches + row merge",
                           "flat_equivalent_gbs": round(c["bytes"]["flat_kv"] / run_s / 1e9, 1),
                           "flat_decode_us_mean": round(c["flat_us"], 2),
                           "speedup_vs_flat_decode": round(c["flat_us"] / (c["attn_ms_mean"] * 1e3), 2),
                           "workload": "shared-prefix decode: 64 requests, 3-level tree (16384-token root, "
                                       "8 branches U[1024,4096], leaves U[128,1024]), page 16, 32/8 heads, "
                                       "d128, bf16"}
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
