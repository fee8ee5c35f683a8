#!/usr/bin/env python3
"""Benchmark of ragged (varlen) batched prefill attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one call of the library's one-shot C entry point
``ragged_prefill_bf16`` on a synthetic ragged batch already resident in HBM:
argument validation, the plan lookup (the plan is built on the first call and
cached per offsets/shape, i.e. planned once per batch as in the plan/run
design), the tile kernel and, when the plan splits KV, the merge kernel.
Prints ONE JSON line.

Default workload: 8 requests, qo_len = kv_len ~ U[128, 2048] (recorded lengths),
32 qo / 8 kv heads, head_dim 128, causal, bf16 N(0,1) inputs.  Without --warmup,
the untimed warmup runs for at least 0.3 s (the GPU needs tens of ms of sustained
load to reach its steady clock; 20 steps of this workload are 2 ms).

roofline.bound is "mfma" when the workload's algorithmic flop/byte ratio is at
or above the MI355X ridge (2.5 PF/s / 8 TB/s = 312.5 flop/B), else "hbm" (decode-
like batches), with achieved algorithmic GB/s against 8 TB/s.

Other modes:
  --kv-fp8             K/V stored as FP8 E4M3 codes (per-tensor scales); the
                       algorithmic bytes count K/V at one byte per element.
  --paged P            the same batch with K/V scattered into a page pool of
                       P-key pages in random order; a step is one rp_run_paged
                       call on a plan built once before the timed region.
  --shared-prefix P    the workload with its first P keys shared by all requests
                       (SharedPrefixPlan: all queries against the prefix once,
                       each request against its own keys, state merge), and
                       the flat run over the same keys for comparison.
  --merge-states K     the state-merge kernel alone (K states per row-head),
                       reported in GB/s against the HBM peak.
  --copy-probe-mib M   run a plain device copy of M MiB (read M, write M) a few
                       times; used to scale rocprofv3 FETCH_SIZE/WRITE_SIZE.
  --record-traffic KDIR CDIR
                       (no GPU) turn the rocprofv3 counter CSVs of the
                       workload's run (KDIR: fetch_/write_counter_collection.csv)
                       and of the copy probe (CDIR, same names) into
                       profiles/traffic_<kernel>_<workload>.json, which later
                       runs report as roofline.traffic while the kernel source
                       is unchanged.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ragged causal prefill TFLOP/s & tok/s (bf16 GQA hd128) + % of MFMA peak"
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (published)
WARMUP_SECONDS = 0.3             # default warmup: at least this much wall time of steps
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E (published)
RIDGE_FLOP_PER_BYTE = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)   # 312.5
KERNEL_SRC = os.path.join(ROOT, "varlen_prefill_amd", "csrc", "rp_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_{kernel}_{workload}.json")


def kernel_source_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def parse_args():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=None,
                   help="untimed warmup steps (default: as many as take >= %.1f s, at least 20; "
                        "the GPU needs tens of ms of sustained load to reach its steady clock)"
                        % WARMUP_SECONDS)
    p.add_argument("--workload", default="hd128_gqa_causal")
    p.add_argument("--noncausal", action="store_true", help="run the workload without the causal mask")
    p.add_argument("--shared-prefix", type=int, default=0, metavar="P",
                   help="the workload's first P keys are one prefix shared by every request: "
                        "shared-prefix attention (two levels + state merge), timed beside the "
                        "flat run over the same keys")
    p.add_argument("--merge-states", type=int, default=0, metavar="K",
                   help="time rp_merge_states over K states per (token, qo head) of the workload")
    p.add_argument("--kv-fp8", action="store_true",
                   help="K/V as FP8 E4M3 codes with per-tensor scales max|x| / 448 "
                        "(rp_run_fp8kv / rp_run_paged_fp8kv on a prebuilt plan)")
    p.add_argument("--paged", type=int, default=0, metavar="PAGE_SIZE",
                   help="keep K/V in a paged cache of this page size (rp_run_paged on a prebuilt plan)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--sample-steps", type=int, default=100,
                   help="steps timed one by one (HIP events per step) after the timed region, "
                        "for the per-step median and std, warm and cold (0: skip)")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target CPU time of the oracle baseline sample")
    p.add_argument("--copy-probe-mib", type=int, default=0)
    p.add_argument("--record-traffic", nargs=2, metavar=("KDIR", "CDIR"))
    return p.parse_args()


def copy_probe(mib: int) -> None:
    import torch
    n = mib * (1 << 20)
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n, "launches": 5}))


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(batch, cfg, causal: bool, sm_scale: float, target_s: float) -> dict:
    """Time the fp64 oracle (as it stands) on the host cores: the whole batch
    once on all threads when that fits in about 2.5x target_s, else the
    batch's leading requests up to about target_s of work; plus a
    single-thread run of one request of the batch for a per-core rate."""
    import oracle
    qo = np.diff(batch.q_indptr).astype(np.int64)
    kv = np.diff(batch.kv_indptr).astype(np.int64)

    def req_pairs(r):
        i = np.arange(qo[r])
        lim = np.clip(i + kv[r] - qo[r] + 1, 0, kv[r]) if causal else np.full(qo[r], kv[r])
        return float(lim.sum())

    pairs = np.array([req_pairs(r) for r in range(batch.batch)])
    flops_req = 4.0 * cfg.head_dim * cfg.num_qo_heads * pairs

    def run(n_req):
        qi, ki = batch.q_indptr[: n_req + 1], batch.kv_indptr[: n_req + 1]
        t0 = time.perf_counter()
        oracle.ragged_attention(batch.q, batch.k, batch.v, qi, ki, cfg.num_qo_heads,
                                cfg.num_kv_heads, causal, sm_scale)
        return time.perf_counter() - t0

    threads = oracle.num_threads()
    # rate estimate from the smallest non-empty leading prefix worth timing
    nz = [r for r in range(batch.batch) if flops_req[r] > 0]
    if not nz:
        return None
    cum = np.cumsum(flops_req)
    n_cal = int(np.searchsorted(cum, min(cum[-1], 2e9))) + 1
    rate = cum[n_cal - 1] / max(run(n_cal), 1e-6)
    if cum[-1] / rate <= 2.5 * target_s:
        n_req = batch.batch
    else:
        n_req = max(1, int(np.searchsorted(cum, rate * target_s)) + 1)
    dt = run(n_req)
    flops = float(cum[n_req - 1])
    toks = int(batch.q_indptr[n_req] - batch.q_indptr[0])
    sample = (f"the whole batch ({batch.batch} requests)" if n_req == batch.batch else
              f"requests 0..{n_req - 1} of {batch.batch} (in batch order)")
    # per-core rate: one request (the one with the least work above 0.1 GFLOP, else the largest) on one thread
    cand = [r for r in nz if flops_req[r] >= 1e8]
    r1 = min(cand, key=lambda r: flops_req[r]) if cand else max(nz, key=lambda r: flops_req[r])
    sub_q = np.array([0, qo[r1]], dtype=np.int32) + batch.q_indptr[r1]
    sub_kv = np.array([0, kv[r1]], dtype=np.int32) + batch.kv_indptr[r1]
    oracle.set_num_threads(1)
    try:
        t0 = time.perf_counter()
        oracle.ragged_attention(batch.q, batch.k, batch.v, sub_q, sub_kv, cfg.num_qo_heads,
                                cfg.num_kv_heads, causal, sm_scale)
        dt1 = time.perf_counter() - t0
    finally:
        oracle.set_num_threads(threads)
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{sample}: {toks} query tokens, {flops / 1e9:.1f} GFLOP, {dt:.1f} s",
        "tokens_per_s": toks / dt,
        "seconds": dt,
        "cpu_model": _cpu_model(),
        "per_core": {"value": float(flops_req[r1] / dt1 / 1e12), "unit": "TFLOP/s", "threads": 1,
                     "sample": f"request {r1} ({qo[r1]} query x {kv[r1]} key tokens, "
                               f"{flops_req[r1] / 1e9:.2f} GFLOP), {dt1:.2f} s"},
    }


def record_traffic(kdir: str, cdir: str, workload: str, head_dim: int, alg_bytes: float,
                   copy_mib: int = 1024) -> str:
    """HBM bytes per tile-kernel launch from FETCH_SIZE / WRITE_SIZE (KiB per
    dispatch), each scaled by what the same counter reads for the copy probe
    of known size."""
    import csv

    def values(path, pick):
        with open(path) as f:
            return [float(r["Counter_Value"]) for r in csv.DictReader(f) if pick(r["Kernel_Name"])]

    tile = lambda name: f"tile_kernel<{head_dim}" in name
    copy = lambda name: "copyBuffer" in name
    fetch = values(os.path.join(kdir, "fetch_counter_collection.csv"), tile)
    write = values(os.path.join(kdir, "write_counter_collection.csv"), tile)
    cfetch = values(os.path.join(cdir, "fetch_counter_collection.csv"), copy)
    cwrite = values(os.path.join(cdir, "write_counter_collection.csv"), copy)
    if not (fetch and write and cfetch and cwrite):
        raise SystemExit("record-traffic: a counter file holds no matching dispatch")
    nbytes = copy_mib * (1 << 20)
    fetch_scale = nbytes / (float(np.mean(cfetch)) * 1024.0)
    write_scale = nbytes / (float(np.mean(cwrite)) * 1024.0)
    hbm = float(np.mean(fetch)) * 1024.0 * fetch_scale + float(np.mean(write)) * 1024.0 * write_scale
    kernel = f"tile_kernel_hd{head_dim}"
    rec = {
        "kernel": kernel,
        "workload": workload,
        "kernel_source_sha256_16": kernel_source_hash(),
        "dispatches": len(fetch),
        "fetch_size_kib_per_dispatch": float(np.mean(fetch)),
        "write_size_kib_per_dispatch": float(np.mean(write)),
        "copy_probe": {"bytes_read": nbytes, "bytes_written": nbytes,
                       "fetch_size_kib": float(np.mean(cfetch)),
                       "write_size_kib": float(np.mean(cwrite))},
        "fetch_scale": fetch_scale,
        "write_scale": write_scale,
        "hbm_bytes_per_launch": hbm,
        "algorithmic_bytes_per_launch": alg_bytes,
    }
    path = TRAFFIC_FILE.format(kernel=kernel, workload=workload)
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    return path


def load_traffic(kernel: str, workload: str):
    path = TRAFFIC_FILE.format(kernel=kernel, workload=workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None  # counters were taken on another version of the kernel
    return rec.get("hbm_bytes_per_launch")


def warm_up(step, warmup) -> int:
    """Run `warmup` untimed steps, or (None) steps until WARMUP_SECONDS of wall
    time have passed and at least 20 ran.  Returns the number run."""
    import torch
    if warmup is not None:
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        return warmup
    n = 0
    t0 = time.perf_counter()
    while n < 20 or time.perf_counter() - t0 < WARMUP_SECONDS:
        for _ in range(10):
            step()
        n += 10
        torch.cuda.synchronize()
    return n


FLUSH_BYTES = 512 << 20   # larger than L2 (4 MB per XCD) and MALL (256 MB) together


def per_step_times(step, stream, n: int, flops: float):
    """Per-step GPU times (HIP events around each step on `stream`), after the
    timed region: warm (back to back) and cold (a 512 MiB device write between
    steps evicts L2 and MALL).  Median and standard deviation in ms, and the
    median as TFLOP/s."""
    import torch
    if n <= 0:
        return None
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=torch.device("cuda:0"))

    def run(cold: bool):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        for i, (a, b) in enumerate(evs):
            if cold:
                flush.fill_(i & 0xff)
            a.record(stream)
            step()
            b.record(stream)
        torch.cuda.synchronize()
        t = np.array([a.elapsed_time(b) for a, b in evs])
        med = float(np.median(t))
        return {"median_ms": med, "std_ms": float(np.std(t)), "median_tflops": flops / (med * 1e-3) / 1e12}

    with torch.cuda.stream(stream):
        res = {"n": n, "warm": run(False), "cold": run(True), "flush_bytes": FLUSH_BYTES}
    del flush
    return res


def _time_steps(step, warmup, steps: int, stream):
    """Wall time and HIP-event time (on `stream`) of `steps` calls, ms/step,
    and the number of warmup steps run."""
    import torch
    warmup = warm_up(step, warmup)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    return wall, ev0.elapsed_time(ev1) / steps, warmup


def bench_shared_prefix(args, cfg, causal: bool) -> dict:
    import torch
    import varlen_prefill_amd as vp
    from varlen_prefill_amd import _lib
    from workloads import make_batch, request_tensors
    p_len = args.shared_prefix
    own = [kv - p_len for kv in cfg.kv_lens]
    if min(own) < 0 or (causal and any(q > k for q, k in zip(cfg.qo_lens, own))):
        raise SystemExit(f"--shared-prefix {p_len}: every request needs kv_len - P >= qo_len")
    d, hq, hkv = cfg.head_dim, cfg.num_qo_heads, cfg.num_kv_heads
    b = make_batch(cfg.qo_lens, own, hq, hkv, d, cfg.seed)
    _, ks, vs = request_tensors(cfg.seed, 10**6, 0, p_len, hq, hkv, d)
    sm = float(np.float32(1.0 / math.sqrt(d)))
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    lib = _lib.load()
    q = b.q.to(dev)
    ks_d, vs_d, ku, vu = ks.to(dev), vs.to(dev), b.k.to(dev), b.v.to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((q.shape[0], hq), dtype=torch.float32, device=dev)
    sp = vp.SharedPrefixPlan(b.q_indptr, b.kv_indptr, p_len, hq, hkv, d, causal)
    ws = torch.empty(max(sp.workspace_bytes, 256), dtype=torch.uint8, device=dev)
    info = sp.info
    P = ctypes.c_void_p
    sp_args = (sp.handle, P(q.data_ptr()), P(ks_d.data_ptr()), P(vs_d.data_ptr()), P(ku.data_ptr()),
               P(vu.data_ptr()), P(o.data_ptr()), P(lse.data_ptr()), ctypes.c_float(sm),
               P(ws.data_ptr()), ws.numel(), P(stream.cuda_stream))

    def step_sp():
        _lib.check(lib.rp_run_shared_prefix(*sp_args), "rp_run_shared_prefix")
    wall, gpu, n_warm = _time_steps(step_sp, args.warmup, args.steps, stream)
    # the flat run over the same keys: every request holds its own copy of the prefix
    kf, vf = [], []
    for r in range(b.batch):
        sl = slice(int(b.kv_indptr[r]), int(b.kv_indptr[r + 1]))
        kf += [ks, b.k[sl]]
        vf += [vs, b.v[sl]]
    kf, vf = torch.cat(kf).to(dev), torch.cat(vf).to(dev)
    flat_kv = np.concatenate([[0], np.cumsum(cfg.kv_lens)]).astype(np.int32)
    flat = vp.Plan(b.q_indptr, flat_kv, hq, hkv, d, causal)
    fws = torch.empty(max(flat.workspace_bytes, 256), dtype=torch.uint8, device=dev)
    of = torch.empty_like(q)
    f_args = (flat.handle, P(q.data_ptr()), P(kf.data_ptr()), P(vf.data_ptr()), P(of.data_ptr()),
              P(lse.data_ptr()), ctypes.c_float(sm), P(fws.data_ptr()), fws.numel(),
              P(stream.cuda_stream))

    def step_flat():
        _lib.check(lib.rp_run(*f_args), "rp_run")
    fwall, fgpu, _ = _time_steps(step_flat, args.warmup, args.steps, stream)
    flops = info["flops"]
    assert abs(flops - flat.info["flops"]) < 1e-6 * flops
    value = flops / (wall * 1e-3) / 1e12
    achieved = flops / (gpu * 1e-3) / 1e12
    return {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": n_warm, "ms_per_step": wall, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{cfg.name}_shared{p_len}" + ("" if causal else "_noncausal"),
                   "requests": cfg.batch, "num_qo_heads": hq, "num_kv_heads": hkv,
                   "head_dim": d, "causal": causal, "shared_kv_len": p_len,
                   "total_q": cfg.total_q, "own_kv": int(sum(own)), "seed": cfg.seed},
        "tokens_per_s": cfg.total_q / (wall * 1e-3),
        "mfma_peak_frac": value / MFMA_BF16_PEAK_TFLOPS,
        "alg_gflop_per_step": flops / 1e9, "alg_mb_per_step": info["bytes"] / 1e6,
        "gpu_ms_per_step": gpu,
        "flat_gpu_ms_per_step": fgpu, "flat_ms_per_step": fwall,
        "flat_alg_mb_per_step": flat.info["bytes"] / 1e6,
        "speedup_vs_flat": fgpu / gpu,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / MFMA_BF16_PEAK_TFLOPS, "traffic": None,
                     "kernel": "tile_kernel_hd%d (both levels) + merge_kernel + state_merge_kernel" % d},
        "cpu_baseline": None,
    }


def bench_merge_states(args, cfg) -> dict:
    import torch
    import varlen_prefill_amd as vp
    from varlen_prefill_amd import _lib
    k, rows, h, d = args.merge_states, cfg.total_q, cfg.num_qo_heads, cfg.head_dim
    gen = torch.Generator().manual_seed(cfg.seed)
    dev = torch.device("cuda:0")
    v = torch.randn((rows, k, h, d), generator=gen).to(torch.bfloat16).to(dev)
    s = (torch.rand((rows, k, h), generator=gen) * 20 - 10).to(dev)
    vo = torch.empty((rows, h, d), dtype=torch.bfloat16, device=dev)
    so = torch.empty((rows, h), dtype=torch.float32, device=dev)
    lib = _lib.load()
    stream = torch.cuda.current_stream()
    P = ctypes.c_void_p
    a = (P(v.data_ptr()), P(s.data_ptr()), P(vo.data_ptr()), P(so.data_ptr()), rows, k, h, d,
         P(stream.cuda_stream))

    def step():
        _lib.check(lib.rp_merge_states(*a), "rp_merge_states")
    wall, gpu, n_warm = _time_steps(step, args.warmup, args.steps, stream)
    nbytes = rows * h * ((k + 1) * (2 * d + 4))       # read k states, write one
    gbs = nbytes / (gpu * 1e-3) / 1e9
    return {
        "metric": "state merge GB/s", "value": nbytes / (wall * 1e-3) / 1e9, "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": n_warm, "ms_per_step": wall,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"merge_states_k{k}_{cfg.name}", "rows": rows, "num_states": k,
                   "num_heads": h, "head_dim": d},
        "gpu_ms_per_step": gpu,
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": None, "kernel": "state_merge_kernel"},
        "cpu_baseline": None,
    }


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(this path runs on a single GPU; see DESIGN.md for how it would shard)",
              file=sys.stderr)
        sys.exit(2)
    if args.record_traffic:
        from workloads import get_config
        from workloads.gen import indptr_from_lens
        import varlen_prefill_amd as vp
        cfg = get_config(args.workload)
        causal = cfg.causal and not args.noncausal
        plan = vp.Plan(indptr_from_lens(cfg.qo_lens), indptr_from_lens(cfg.kv_lens),
                       cfg.num_qo_heads, cfg.num_kv_heads, cfg.head_dim, causal, host_only=True)
        alg = plan.info["bytes"]
        if args.kv_fp8:
            alg -= 2.0 * cfg.num_kv_heads * cfg.head_dim * cfg.total_kv   # K/V at one byte
        path = record_traffic(args.record_traffic[0], args.record_traffic[1],
                              cfg.name + ("" if causal else "_noncausal")
                              + ("_fp8kv" if args.kv_fp8 else "")
                              + (f"_paged{args.paged}" if args.paged else ""), cfg.head_dim, alg)
        print(path)
        return
    import torch
    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib)
        return
    import varlen_prefill_amd as vp
    from varlen_prefill_amd import _lib
    from workloads import get_config, make_config_batch

    cfg = get_config(args.workload)
    causal = cfg.causal and not args.noncausal
    if args.shared_prefix or args.merge_states:
        if not vp.available():
            raise SystemExit("the gfx950 library is not usable on this device")
        res = (bench_shared_prefix(args, cfg, causal) if args.shared_prefix
               else bench_merge_states(args, cfg))
        print(json.dumps(res))
        return
    workload = (cfg.name + ("" if causal else "_noncausal") + ("_fp8kv" if args.kv_fp8 else "")
                + (f"_paged{args.paged}" if args.paged else ""))
    batch = make_config_batch(cfg)
    sm_scale = float(np.float32(1.0 / math.sqrt(cfg.head_dim)))
    dev = torch.device("cuda:0")
    q, k, v = batch.q.to(dev), batch.k.to(dev), batch.v.to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((q.shape[0], cfg.num_qo_heads), dtype=torch.float32, device=dev)
    if not vp.available():
        raise SystemExit("the gfx950 library is not usable on this device")

    # plan statistics and host plan time (a fresh plan + worklist upload)
    plan_times = []
    for _ in range(5):
        t0 = time.perf_counter()
        plan = vp.Plan(batch.q_indptr, batch.kv_indptr, cfg.num_qo_heads, cfg.num_kv_heads,
                       cfg.head_dim, causal)
        plan_times.append(time.perf_counter() - t0)
        info = plan.info
        plan.close()
    flops = info["flops"]
    alg_bytes = info["bytes"]
    launches = 1 + (1 if info["num_merge_items"] > 0 else 0)

    lib = _lib.load()
    stream = torch.cuda.current_stream()
    qi = np.ascontiguousarray(batch.q_indptr, dtype=np.int32)
    ki = np.ascontiguousarray(batch.kv_indptr, dtype=np.int32)
    call_args = (ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                 ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(o.data_ptr()),
                 ctypes.c_void_p(lse.data_ptr()), qi.ctypes.data_as(ctypes.c_void_p),
                 ki.ctypes.data_as(ctypes.c_void_p), cfg.batch, cfg.num_qo_heads,
                 cfg.num_kv_heads, cfg.head_dim, 1 if causal else 0, ctypes.c_float(sm_scale),
                 ctypes.c_void_p(stream.cuda_stream))
    step = lib.ragged_prefill_bf16
    step_name = "ragged_prefill_bf16"
    if args.kv_fp8:
        from workloads import make_fp8_kv, make_paged
        ks = float(batch.k.float().abs().max()) / 448.0
        vs = float(batch.v.float().abs().max()) / 448.0
        k8, v8 = make_fp8_kv(batch, ks, vs)
        fplan = vp.Plan(batch.q_indptr, batch.kv_indptr, cfg.num_qo_heads, cfg.num_kv_heads,
                        cfg.head_dim, causal)
        ws = torch.empty(max(fplan.workspace_bytes, 1), dtype=torch.uint8, device=dev)
        if args.paged:
            pk = make_paged(batch, args.paged, seed=cfg.seed, k=k8, v=v8)
            kp, vpg = pk.k_pages.to(dev), pk.v_pages.to(dev)
            table = torch.from_numpy(pk.block_table).to(dev)
            call_args = (fplan.handle, ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(kp.data_ptr()),
                         ctypes.c_void_p(vpg.data_ptr()), ctypes.c_void_p(table.data_ptr()),
                         int(table.shape[1]), args.paged, ctypes.c_float(ks), ctypes.c_float(vs),
                         ctypes.c_void_p(o.data_ptr()), ctypes.c_void_p(lse.data_ptr()),
                         ctypes.c_float(sm_scale), ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                         ctypes.c_void_p(stream.cuda_stream))
            step, step_name = lib.rp_run_paged_fp8kv, "rp_run_paged_fp8kv"
        else:
            k8d, v8d = k8.to(dev), v8.to(dev)
            call_args = (fplan.handle, ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k8d.data_ptr()),
                         ctypes.c_void_p(v8d.data_ptr()), ctypes.c_float(ks), ctypes.c_float(vs),
                         ctypes.c_void_p(o.data_ptr()), ctypes.c_void_p(lse.data_ptr()),
                         ctypes.c_float(sm_scale), ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                         ctypes.c_void_p(stream.cuda_stream))
            step, step_name = lib.rp_run_fp8kv, "rp_run_fp8kv"
        # K and V at one byte per element
        alg_bytes -= 2.0 * cfg.num_kv_heads * cfg.head_dim * cfg.total_kv
    elif args.paged:
        from workloads import make_paged
        pk = make_paged(batch, args.paged, seed=cfg.seed)
        kp, vpg = pk.k_pages.to(dev), pk.v_pages.to(dev)
        table = torch.from_numpy(pk.block_table).to(dev)
        paged_plan = vp.Plan(batch.q_indptr, batch.kv_indptr, cfg.num_qo_heads, cfg.num_kv_heads,
                             cfg.head_dim, causal)
        ws = torch.empty(max(paged_plan.workspace_bytes, 1), dtype=torch.uint8, device=dev)
        call_args = (paged_plan.handle, ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(kp.data_ptr()),
                     ctypes.c_void_p(vpg.data_ptr()), ctypes.c_void_p(table.data_ptr()),
                     int(table.shape[1]), args.paged, ctypes.c_void_p(o.data_ptr()),
                     ctypes.c_void_p(lse.data_ptr()), ctypes.c_float(sm_scale),
                     ctypes.c_void_p(ws.data_ptr()), ws.numel(), ctypes.c_void_p(stream.cuda_stream))
        step = lib.rp_run_paged
        step_name = "rp_run_paged"

    n_warm = warm_up(lambda: _lib.check(step(*call_args), step_name), args.warmup)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        st = step(*call_args)
        if st != 0:
            _lib.check(st, step_name)
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall_s = t1 - t0
    event_ms = ev0.elapsed_time(ev1)
    ms_per_step = wall_s * 1e3 / args.steps
    gpu_ms_per_step = event_ms / args.steps

    per_step = per_step_times(lambda: _lib.check(step(*call_args), step_name), stream,
                              args.sample_steps, flops)

    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (gpu_ms_per_step * 1e-3) / 1e12
    kernel = f"tile_kernel_hd{cfg.head_dim}"
    traffic = load_traffic(kernel, workload)
    alg_gbs = alg_bytes / (gpu_ms_per_step * 1e-3) / 1e9
    kernels = kernel if launches == 1 else f"{kernel} + merge_kernel"
    if flops / alg_bytes >= RIDGE_FLOP_PER_BYTE:
        roofline = {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                    "traffic": traffic, "kernel": kernels, "alg_hbm_gbs": alg_gbs}
    else:
        # below the ridge (decode-like batches): the HBM bound applies
        roofline = {"bound": "hbm", "achieved": alg_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": alg_gbs / HBM_PEAK_GBS, "traffic": traffic, "kernel": kernels,
                    "alg_tflops": achieved}
    result = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": n_warm,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": workload,
            "requests": cfg.batch,
            "num_qo_heads": cfg.num_qo_heads,
            "num_kv_heads": cfg.num_kv_heads,
            "head_dim": cfg.head_dim,
            "causal": causal,
            "total_q": cfg.total_q,
            "total_kv": cfg.total_kv,
            "seed": cfg.seed,
            "kv_layout": f"paged, page_size {args.paged}" if args.paged else "ragged",
            "kv_dtype": "fp8_e4m3 (per-tensor scales)" if args.kv_fp8 else "bf16",
        },
        "tokens_per_s": cfg.total_q / (ms_per_step * 1e-3),
        "mfma_peak_frac": value / MFMA_BF16_PEAK_TFLOPS,
        "alg_gflop_per_step": flops / 1e9,
        "alg_mb_per_step": alg_bytes / 1e6,
        "gpu_ms_per_step": gpu_ms_per_step,
        "launches_per_step": launches,
        "plan_ms_median": float(np.median(plan_times) * 1e3),
        "per_step": per_step,
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(batch, cfg, causal, sm_scale, args.cpu_seconds)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
