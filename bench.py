"""Benchmark: paged decode attention on one MI355X.

One step = one decode-attention call over the whole batch (every sequence,
every query head): the context-partition kernel, then the combine kernel when
the plan splits contexts.  Inputs are synthetic and resident in HBM before
timing starts.

Prints one JSON line: KV-read throughput (GB/s of K+V bytes of every logical
token, once per (sequence, kv head)) of the median cold-cache step, plus the
dominant kernel's roofline figures (HIP events on the launch stream), the
warm back-to-back rate, the other decode configurations measured the same
way in the same process, and the CPU oracle timed on the host as a baseline.

Timing.  Each of the K timed steps runs on a cold cache: a 1 GiB scratch
write before it (outside its events) evicts the L2s and the 256 MB
last-level cache, so every K / V byte comes from HBM.  One HIP event pair on
the launch stream brackets each step; ms_per_step is their median and
`value` the KV bytes over it.  The kernel durations come the same way, each
kernel launched alone between one event pair after an eviction.  The warm
figure runs K steps back to back between one event pair (an event recorded
between two launches costs about 4 us of GPU time, so none is recorded
inside that loop).

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload mha_7b]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0}   # dense matrix-core peaks
METRIC = "Paged decode attention: achieved KV-read GB/s and % of HBM peak; seqs/s"
KERNEL_NAMES = {0: "auto", 1: "generic", 2: "valu", 3: "mfma"}


def time_loop(fn, n, stream):
    """Run fn() n times back to back; returns (wall ms per call, GPU ms per
    call from one event pair around the loop).  Synchronises before and
    after."""
    import torch
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(n):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall * 1e3 / n, e0.elapsed_time(e1) / n


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mha_7b",
                    help="mha_small | mha_7b | gqa_70b | gqa_long | mqa (default: mha_7b, the batch-64 case)")
    ap.add_argument("--block-size", type=int, default=None, help="override B (gqa_long sweeps 1/8/16/32)")
    ap.add_argument("--q-heads", type=int, default=None, help="override Hq (e.g. mqa with 32 query heads)")
    ap.add_argument("--seqs", type=int, default=None, help="override the number of sequences S")
    ap.add_argument("--fixed-len", type=int, default=None,
                    help="every sequence this many tokens (a uniform batch; the table fits it)")
    ap.add_argument("--kernel", default="auto", choices=["auto", "generic", "valu", "mfma"])
    ap.add_argument("--partition-tokens", type=int, default=0)
    ap.add_argument("--token-waves", type=int, default=0, choices=[0, 1, 2, 4],
                    help="waves per decode item (0: the planner's choice)")
    ap.add_argument("--kv-reuse", choices=["on", "off"], default="off",
                    help="cached (on) or streamed (off, default) K/V loads")
    ap.add_argument("--graph", action="store_true",
                    help="decode: also time the step captured in one HIP graph and replayed")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-read-peak", action="store_true",
                    help="decode: skip the plain device reads (the 4 GiB measured HBM peak and "
                         "each configuration's same-size read floor)")
    ap.add_argument("--no-extra-configs", action="store_true",
                    help="decode: skip the other decode configurations (C2 mha_small, C4 "
                         "gqa_70b, C5 gqa_long at B = 16) measured after the headline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--print-source-sha", action="store_true",
                    help="print each kernel's source hash (used to match counter records), then exit")
    ap.add_argument("--op", choices=["decode", "write_kv", "append_kv", "copy_blocks", "prefill"],
                    default="decode",
                    help="decode (default): the attention step; write_kv: store a prompt chunk's "
                         "K/V through a slot mapping; append_kv: store one new token per sequence; "
                         "copy_blocks: copy-on-write copies of --pairs whole blocks; "
                         "prefill: causal attention of --new-tokens per sequence (workload 'prefill')")
    ap.add_argument("--new-tokens", type=int, default=0,
                    help="prefill: new tokens per sequence (default: the workload's chunk)")
    ap.add_argument("--pairs", type=int, default=1024, help="copy_blocks: blocks copied per step")
    ap.add_argument("--tokens", type=int, default=16384,
                    help="write_kv: tokens in the chunk")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="before timing, run one plain device-to-device copy of this many MiB "
                         "(a known-size reference for hardware byte counters)")
    return ap.parse_args()


# Sources each kernel is built from: a traffic record stays valid while these
# files are unchanged.
_COMMON = ["pa_device.h", "pa_args.h"]
KERNEL_SOURCES = {
    "pa_valu_partitions": ["pa_valu.hip", "pa_tile.h", "pa_table.h", "pa_sched.h"] + _COMMON,
    "pa_mfma_partitions": ["pa_mfma.hip", "pa_mfma_core.h", "pa_tile.h", "pa_table.h",
                           "pa_sched.h"] + _COMMON,
    "pa_generic_partitions": ["pa_generic.hip", "pa_rows.h"] + _COMMON,
    "pa_prefill_mfma": ["pa_prefill.hip", "pa_mfma_core.h", "pa_tile.h", "pa_table.h",
                        "pa_rows.h"] + _COMMON,
    "pa_prefill_generic": ["pa_generic.hip", "pa_rows.h"] + _COMMON,
    "pa_kv_write": ["pa_kvwrite.hip"] + _COMMON,
    "pa_copy_blocks": ["pa_kvwrite.hip"] + _COMMON,
}


def _code_only(text: str) -> str:
    """C / C++ source without comments and with whitespace collapsed (a record
    stays valid across comment edits; the sources hold no comment markers
    inside string literals)."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_sha256(kernel: str) -> str:
    """Hash of one kernel's source code (ties hardware-counter records to a build)."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_cache_301_amd", "csrc")
    for name in sorted(KERNEL_SOURCES[kernel]):
        with open(os.path.join(csrc, name)) as f:
            h.update(name.encode() + b"\0" + _code_only(f.read()).encode())
    return h.hexdigest()


def prefill_roofline(kv_bytes: int, flops: int, dtype: str, kernel_s: float):
    """The roofline that binds a multi-token call: HBM when reading the unique
    K+V once at the HBM peak takes longer than its flops at the type's dense
    matrix-core peak (a few new tokens per sequence), else the matrix cores.
    Returns (bound, achieved, peak, unit) for a kernel time of kernel_s."""
    flop_peak = MFMA_PEAK_TFLOPS.get(dtype, 157.3)
    if kv_bytes / (HBM_PEAK_GBS * 1e9) > flops / (flop_peak * 1e12):
        return "hbm", kv_bytes / kernel_s / 1e9, HBM_PEAK_GBS, "GB/s"
    return "mfma", flops / kernel_s / 1e12, flop_peak, "TFLOP/s"


def record_key(workload: str, args) -> str:
    """Workload name of a traffic record: the named workload plus the
    overrides that change its shape (query heads, new tokens per sequence)."""
    key = workload
    if args.q_heads:
        key += f"_hq{args.q_heads}"
    if getattr(args, "seqs", None):
        key += f"_s{args.seqs}"
    if getattr(args, "fixed_len", None):
        key += f"_len{args.fixed_len}"
    if args.op == "prefill" and args.new_tokens:
        key += f"_new{args.new_tokens}"
    return key


def recorded_traffic(kernel: str, workload: str, block_size: int, partition: int = 0,
                     token_waves: int = 1):
    """HBM bytes per launch from a rocprofv3 --pmc summary under profiles/,
    if one was recorded for these exact kernel sources, the same partition
    size (0: the kernel has none) and the same waves per decode item; else
    None."""
    import glob
    import re
    if kernel not in KERNEL_SOURCES:
        return None
    sha = source_sha256(kernel)
    pat = re.compile(r"traffic-record: kernel=(\S+) workload=(\S+) B=(\d+) P=(\d+) TW=(\d+) "
                     r"source_sha256=([0-9a-f]+) read_bytes=(\d+) write_bytes=(\d+)")
    want = (kernel, workload, block_size, partition, token_waves, sha)
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        for m in pat.finditer(open(path).read()):
            if (m.group(1), m.group(2), int(m.group(3)), int(m.group(4)), int(m.group(5)),
                    m.group(6)) == want:
                return int(m.group(7)) + int(m.group(8))
    return None


def measured_read_peak(dev, calls=5):
    """Achievable HBM read rate: the library's plain streaming read (16-byte
    non-temporal loads, as the paged kernels use) over a 4 GiB buffer, far
    larger than every cache level; median of a few calls after one warm-up."""
    import numpy as np
    import torch
    from paged_kv_cache_301_amd import binding
    nbytes = 4 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    binding.read_bytes(buf, sink, stream=stream)
    ms = []
    for _ in range(calls):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        binding.read_bytes(buf, sink, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    del buf
    med = float(np.median(ms))
    return {"gbs": round(nbytes / (med * 1e-3) / 1e9, 2), "bytes": nbytes,
            "kernel": "pa_read_bytes over a 4 GiB buffer", "calls": calls}


def evict_and_time(fn, n, stream, scratch):
    """n calls of fn(), each after a write of `scratch` (outside the events)
    and bracketed by one HIP event pair on `stream`; returns the per-call
    durations in ms."""
    import torch
    torch.cuda.synchronize()
    pairs = []
    for i in range(n):
        scratch.fill_(i & 0xFF)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        pairs.append((e0, e1))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in pairs]


def stats_us(ms):
    import numpy as np
    a = np.asarray(ms) * 1e3
    return {"median_us": round(float(np.median(a)), 2), "mean_us": round(float(a.mean()), 2),
            "p10_us": round(float(np.percentile(a, 10)), 2),
            "p90_us": round(float(np.percentile(a, 90)), 2)}


def measure_decode(w, args, dev, scratch, kernel="auto", partition_tokens=0, kv_reuse=False,
                   token_waves=0):
    """Cold-cache and warm timings of one decode workload (see the module
    docstring).  Returns (plan, timing dict, prepared step callables)."""
    import torch
    from paged_kv_cache_301_amd import binding
    plan = binding.plan(w.S, w.Hq, w.Hkv, w.D, w.B, w.NB, w.max_blocks, w.dtype,
                        kernel=kernel, partition_tokens=partition_tokens, token_waves=token_waves)
    ws = None
    if plan["workspace_bytes"]:
        ws = torch.empty(plan["workspace_bytes"], dtype=torch.uint8, device=dev)
    out = torch.empty_like(w.query)
    stream = torch.cuda.current_stream(dev)
    kw = dict(kernel=kernel, partition_tokens=partition_tokens, workspace=ws, stream=stream,
              kv_reuse=kv_reuse, token_waves=token_waves)
    args_ = (w.query, w.key_cache, w.value_cache, w.block_tables, w.seq_lens, w.scale, out)
    run_parts = binding.prepare(*args_, stages=binding.STAGE_PARTITIONS, **kw)
    run_combine = binding.prepare(*args_, stages=binding.STAGE_COMBINE, **kw)

    def step():
        run_parts()
        if plan["split"]:
            run_combine()

    for _ in range(args.warmup):
        step()
    t = {}
    # the timed region: K cold steps
    cold = evict_and_time(step, args.steps, stream, scratch)
    t["cold"] = stats_us(cold)
    # each kernel alone, cold
    t["partitions"] = stats_us(evict_and_time(run_parts, args.steps, stream, scratch))
    t["combine"] = (stats_us(evict_and_time(run_combine, args.steps, stream, scratch))
                    if plan["split"] else None)
    # warm: K steps back to back, and the partition kernel alone back to back
    warm_ms, warm_gpu_ms = time_loop(step, args.steps, stream)
    t["warm"] = {"ms_per_step": round(warm_ms, 5), "gpu_us": round(warm_gpu_ms * 1e3, 2),
                 "partitions_us": round(time_loop(run_parts, args.steps, stream)[1] * 1e3, 2)}
    return plan, t, (step, args_, kw)


def plain_read_floor(nbytes, args, dev, scratch):
    """Cold median of the library's plain streaming read (pa_read_bytes) over
    a contiguous buffer of the same size as a workload's unique K/V: what one
    launch moving that many bytes takes on this GPU, the floor for a step."""
    import numpy as np
    import torch
    from paged_kv_cache_301_amd import binding
    nbytes = (nbytes + 15) // 16 * 16
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    binding.read_bytes(buf, sink, stream=stream)
    ms = evict_and_time(lambda: binding.read_bytes(buf, sink, stream=stream), args.steps, stream,
                        scratch)
    del buf
    med = float(np.median(ms))
    return {"median_us": round(med * 1e3, 2), "gbs": round(nbytes / (med * 1e-3) / 1e9, 2),
            "bytes": nbytes}


def decode_summary(w, plan, t, kname, floor=None):
    """Rates of one measured decode workload: logical and unique bytes."""
    kv = w.kv_bytes()
    unique = w.unique_kv_bytes() if w.spec.prefix_tokens else kv
    step_s = t["cold"]["median_us"] * 1e-6
    k_s = t["partitions"]["mean_us"] * 1e-6
    extra = {}
    if floor:
        extra = {"plain_read_floor": floor,
                 "step_vs_floor": round(floor["median_us"] / t["cold"]["median_us"], 4)}
    return {**extra,
        "S": w.S, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D, "B": w.B,
        "tokens": int(w.lens.sum()), "kv_bytes": kv, "unique_kv_bytes": unique,
        "kernel": kname, "partition_tokens": plan["partition_tokens"], "split": bool(plan["split"]),
        "token_waves": plan["token_waves"], "step_cold_us": t["cold"], "kernel_cold_us": t["partitions"],
        "combine_cold_us": t["combine"], "warm": t["warm"],
        "gbs": round(kv / step_s / 1e9, 2), "hbm_frac": round(kv / step_s / 1e9 / HBM_PEAK_GBS, 4),
        "unique_gbs": round(unique / step_s / 1e9, 2),
        "unique_hbm_frac": round(unique / step_s / 1e9 / HBM_PEAK_GBS, 4),
        "kernel_gbs": round(kv / k_s / 1e9, 2),
        "kernel_unique_hbm_frac": round(unique / k_s / 1e9 / HBM_PEAK_GBS, 4),
        "seqs_per_s": round(w.S / step_s, 1),
    }


def cpu_model() -> str:
    """The host CPU's model name (Linux), for the CPU baseline's record."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, target_s):
    """Time the oracle on the host: whole batch, repeated until target_s."""
    import oracle
    q, kc, vc = w.query.cpu(), w.key_cache.cpu(), w.value_cache.cpu()
    bt, sl = w.block_tables.cpu(), w.seq_lens.cpu()
    # one sequence (after one untimed call that touches the host copies) to
    # size the sample
    oracle.decode(q, kc, vc, bt, sl, w.scale, rows=range(w.Hq))
    t0 = time.perf_counter()
    oracle.decode(q, kc, vc, bt, sl, w.scale, rows=range(w.Hq))
    t_one = max(time.perf_counter() - t0, 1e-6)
    per_seq_bytes = int(w.lens[0]) * w.Hkv * w.D * 2 * w.esz
    est_full = t_one * w.kv_bytes() / max(per_seq_bytes, 1)
    if est_full > 3 * target_s:
        # bounded sample: the first n sequences
        n = max(1, int(w.S * target_s / est_full))
        rows = range(n * w.Hq)
        sample_bytes = int(w.lens[:n].sum()) * w.Hkv * w.D * 2 * w.esz
        reps, desc = 1, f"first {n} of {w.S} sequences, all heads, once"
    else:
        rows = None
        sample_bytes = w.kv_bytes()
        reps = max(1, int(target_s / max(est_full, 1e-3)))
        desc = f"whole batch ({w.S} sequences, all heads), {reps} pass(es)"
    t0 = time.perf_counter()
    for _ in range(reps):
        oracle.decode(q, kc, vc, bt, sl, w.scale, rows=rows)
    dt = time.perf_counter() - t0
    return {"value": round(sample_bytes * reps / dt / 1e9, 4), "unit": "GB/s",
            "cores": oracle.num_threads(), "cpu": cpu_model(), "kind": "oracle",
            "sample": desc, "seconds": round(dt, 2)}


def write_slots(w, T, seed=11):
    """Slot mapping of a T-token prompt chunk: the tokens fill whole blocks in
    order, the blocks drawn at random (without repeats) from the pool."""
    import numpy as np
    rng = np.random.default_rng(seed)
    nblk = (T + w.B - 1) // w.B
    if nblk > w.NB:
        raise SystemExit(f"bench.py: {T} tokens need {nblk} blocks, the pool has {w.NB}")
    blocks = rng.choice(w.NB, size=nblk, replace=False)
    t = np.arange(T)
    return (blocks[t // w.B] * w.B + t % w.B).astype(np.int32)


def bench_write(args, w, dev):
    """K/V write step: read the new rows, write them into their slots."""
    import numpy as np
    import torch

    from paged_kv_cache_301_amd import binding
    g = torch.Generator(device=dev).manual_seed(12)
    stream = torch.cuda.current_stream(dev)
    if args.op == "copy_blocks":
        rng = np.random.default_rng(13)
        ids = rng.choice(w.NB, size=2 * args.pairs, replace=False)
        pairs_h = torch.from_numpy(ids.reshape(2, -1).T.copy().astype(np.int32))
        pairs = pairs_h.to(dev)
        T = args.pairs

        def step():
            binding.copy_blocks(w.key_cache, w.value_cache, pairs, stream=stream)
        block_bytes = w.Hkv * w.B * w.D * w.esz
        row_bytes = T * block_bytes * 2                  # K and V blocks
        meta_bytes = 8 * T
    elif args.op == "write_kv":
        T = args.tokens
        slots = torch.from_numpy(write_slots(w, T)).to(dev)
        key = torch.randn((T, w.Hkv, w.D), generator=g, device=dev).to(w.dtype)
        value = torch.randn((T, w.Hkv, w.D), generator=g, device=dev).to(w.dtype)

        def step():
            binding.write_kv(key, value, slots, w.key_cache, w.value_cache, stream=stream)
        meta_bytes = 4 * T
    else:
        T = w.S
        key = torch.randn((T, w.Hkv, w.D), generator=g, device=dev).to(w.dtype)
        value = torch.randn((T, w.Hkv, w.D), generator=g, device=dev).to(w.dtype)

        def step():
            binding.append_kv(key, value, w.block_tables, w.seq_lens, w.key_cache,
                              w.value_cache, stream=stream)
        meta_bytes = 8 * T       # length + one table entry per sequence
    if args.op != "copy_blocks":
        row_bytes = T * w.Hkv * w.D * w.esz * 2      # K and V rows
    alg_bytes = 2 * row_bytes + meta_bytes           # read once, write once
    for _ in range(args.warmup):
        step()
    # one launch per step: the loop's event pair gives the kernel's average
    step_ms, k_ms = time_loop(step, args.steps, stream)
    gbs = alg_bytes / (step_ms * 1e-3) / 1e9
    achieved = alg_bytes / (k_ms * 1e-3) / 1e9
    kernel = "pa_copy_blocks" if args.op == "copy_blocks" else "pa_kv_write"
    print(f"[bench] {args.op}: T={T} rows {row_bytes / 1e6:.2f} MB, kernel {k_ms * 1e3:.2f} us, "
          f"step {step_ms * 1e3:.2f} us", file=sys.stderr, flush=True)
    res = {
        "metric": f"Paged KV {args.op.replace('_kv', '')}: K/V bytes moved per second (read + write)",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(step_ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": {torch.bfloat16: "bf16", torch.float16: "f16", torch.float32: "f32"}[w.dtype],
        "data": "synthetic",
        "config": {"workload": f"{args.op}_{args.workload}",
                   ("pairs" if args.op == "copy_blocks" else "tokens"): T, "Hkv": w.Hkv,
                   "D": w.D, "B": w.B, "NB": w.NB, "bytes": alg_bytes},
        "kernel_us": round(k_ms * 1e3, 2),
        "roofline": {"bound": "hbm", "kernel": kernel, "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic(kernel, record_key(f"{args.op}_{args.workload}", args), w.B)},
    }
    if not args.no_cpu_baseline and args.op == "copy_blocks":
        from oracle.block_manager import copy_blocks as oracle_copy
        # host pool of just the blocks the copies touch (renumbered)
        ids_h = pairs_h.flatten().numpy()
        small = torch.arange(len(ids_h), dtype=torch.int32).reshape(-1, 2)
        hk = w.key_cache[torch.from_numpy(ids_h.astype(np.int64)).to(dev)].cpu()
        hv = w.value_cache[torch.from_numpy(ids_h.astype(np.int64)).to(dev)].cpu()
        reps, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < min(args.cpu_seconds, 5.0):
            oracle_copy(hk, hv, small.tolist())
            reps += 1
        dt = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": round(alg_bytes * reps / dt / 1e9, 4), "unit": "GB/s",
                               "cores": 1, "cpu": cpu_model(), "kind": "oracle",
                               "sample": f"{T} block copies in a host pool of the {2 * T} blocks "
                                         f"they touch (the oracle also clones that pool), {reps} pass(es)",
                               "seconds": round(dt, 2)}
    elif not args.no_cpu_baseline:
        import oracle
        # host copy of the same rows; the pool holds just the blocks the
        # write touches (renumbered in first-touch order), so the sample
        # measures the row copies, not a copy of the whole pool
        sm = (write_slots(w, T) if args.op == "write_kv" else
              np.array([int(w.tables_host[s, (L - 1) // w.B]) * w.B + (L - 1) % w.B
                        for s, L in enumerate(w.lens)], dtype=np.int64))
        blk, off = sm // w.B, sm % w.B
        _, ren = np.unique(blk, return_inverse=True)
        sm_h = torch.from_numpy((ren * w.B + off).astype(np.int32))
        nb = int(ren.max()) + 1
        hk, hv = key.cpu(), value.cpu()
        hkc = torch.zeros((nb, w.Hkv, w.B, w.D), dtype=w.dtype)
        hvc = torch.zeros_like(hkc)
        reps, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < min(args.cpu_seconds, 5.0):
            oracle.write_kv(hk, hv, sm_h, hkc, hvc, inplace=True)
            reps += 1
        dt = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": round(alg_bytes * reps / dt / 1e9, 4), "unit": "GB/s",
                               "cores": 1, "cpu": cpu_model(), "kind": "oracle",
                               "sample": f"whole write ({T} tokens) into a host pool of the "
                                         f"{nb} blocks it touches, {reps} pass(es)",
                               "seconds": round(dt, 2)}
    print(json.dumps(res), flush=True)


def bench_prefill(args, dev):
    """Causal multi-token step: every sequence's chunk of new tokens against its
    cache (all rows, all heads); matrix-core bound."""
    import numpy as np
    import torch

    from paged_kv_cache_301_amd import binding, workloads
    over = {}
    if args.block_size:
        over["B"] = args.block_size
    if args.q_heads:
        over["Hq"] = args.q_heads
    if args.seqs:
        over["S"] = args.seqs
    if args.fixed_len:
        S = args.seqs or workloads.SPECS["prefill"].S
        over["lens"] = ("fixed", (args.fixed_len,) * S)
        over["max_len"] = args.fixed_len
    name = args.workload if args.workload in workloads.PREFILL_NEW else "prefill"
    pw = workloads.make_prefill_workload(name, args.new_tokens or None, device=dev, **over)
    w = pw.base
    torch.cuda.synchronize()
    plan = binding.plan_prefill(w.S, pw.T, w.Hq, w.Hkv, w.D, w.B, w.NB, w.max_blocks,
                                pw.max_query_len, w.dtype, kernel=args.kernel,
                                partition_tokens=args.partition_tokens)
    ws = (torch.empty(plan["workspace_bytes"], dtype=torch.uint8, device=dev)
          if plan["workspace_bytes"] else None)
    out = torch.empty_like(pw.query)
    stream = torch.cuda.current_stream(dev)
    kw = dict(max_query_len=pw.max_query_len, kernel=args.kernel,
              partition_tokens=args.partition_tokens, workspace=ws, stream=stream)
    a = (pw.query, w.key_cache, w.value_cache, w.block_tables, w.seq_lens, pw.query_start, w.scale, out)

    def parts():
        binding.prefill(*a, stages=binding.STAGE_PARTITIONS, **kw)

    def combine():
        binding.prefill(*a, stages=binding.STAGE_COMBINE, **kw)

    def step():
        parts()
        if plan["split"]:
            combine()

    for _ in range(args.warmup):
        step()
    step_ms, _ = time_loop(step, args.steps, stream)
    _, k_ms = time_loop(parts, args.steps, stream)
    c_ms = time_loop(combine, args.steps, stream)[1] if plan["split"] else 0.0
    flops = pw.flops()
    tf = flops / (step_ms * 1e-3) / 1e12
    kname = {1: "generic", 3: "mfma"}[plan["kernel"]]
    dts = {torch.bfloat16: "bf16", torch.float16: "f16", torch.float32: "f32"}[w.dtype]
    # the unique K+V the chunks attend, read once
    kv = w.unique_kv_bytes() if w.spec.prefix_tokens else w.kv_bytes()
    bound, achieved, peak, unit = prefill_roofline(kv, flops, dts, k_ms * 1e-3)
    print(f"[bench] prefill: S={w.S} T={pw.T} Hq={w.Hq} Hkv={w.Hkv} B={w.B} ctx={int(w.lens.sum())} "
          f"plan {plan}; kernel {k_ms * 1e3:.1f} us, combine {c_ms * 1e3:.1f} us, step {step_ms * 1e3:.1f} us",
          file=sys.stderr, flush=True)
    res = {
        "metric": "Paged causal multi-token attention (chunked prefill): TFLOP/s",
        "value": round(tf, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(step_ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": dts, "data": "synthetic",
        "config": {"workload": f"prefill_{name}", "S": w.S, "T": pw.T, "Hq": w.Hq, "Hkv": w.Hkv,
                   "D": w.D, "B": w.B, "context_tokens": int(w.lens.sum()),
                   "new_tokens_per_seq": int(pw.max_query_len), "flops": flops, "kernel": kname,
                   "partition_tokens": plan["partition_tokens"], "split": bool(plan["split"])},
        "kernel_us": {"partitions": round(k_ms * 1e3, 2), "combine": round(c_ms * 1e3, 2)},
        "roofline": {"bound": bound, "kernel": f"pa_prefill_{kname}", "achieved": round(achieved, 2),
                     "peak": peak, "unit": unit, "frac": round(achieved / peak, 4), "kv_bytes": kv,
                     "traffic": recorded_traffic(f"pa_prefill_{kname}", record_key(f"prefill_{name}", args), w.B,
                                                 plan["partition_tokens"])},
    }
    if not args.no_cpu_baseline:
        import oracle
        # the inputs on the host once, so the timing is the oracle's arithmetic
        host = [t.cpu() for t in (pw.query, w.key_cache, w.value_cache, w.block_tables,
                                  w.seq_lens, pw.query_start)]
        import numpy as np
        qs = host[5].numpy().astype(np.int64)
        lens = host[4].numpy().astype(np.int64)
        # tokens each query row attends (row k of sequence s sits at L_s - n_s + k)
        att = np.concatenate([np.arange(L - n + 1, L + 1) for L, n in zip(lens, np.diff(qs))])
        # size the sample on the first few rows (after one untimed call)
        probe = min(8, len(att))
        rows = list(range(probe * w.Hq))
        oracle.prefill(*host, w.scale, rows=rows)
        t0 = time.perf_counter()
        oracle.prefill(*host, w.scale, rows=rows)
        per_tok = max(time.perf_counter() - t0, 1e-6) / max(int(att[:probe].sum()), 1)
        cum = np.cumsum(att)

        def rows_for(seconds):
            return max(1, min(int(np.searchsorted(cum, seconds / per_tok)) + 1, len(att)))

        # a call has a fixed cost the probe overweights: re-estimate on a
        # quarter of the target before sizing the sample
        n1 = rows_for(args.cpu_seconds / 4)
        t0 = time.perf_counter()
        oracle.prefill(*host, w.scale, rows=list(range(n1 * w.Hq)))
        per_tok = max(time.perf_counter() - t0, 1e-6) / int(cum[n1 - 1])
        # sample: the first query rows, all heads, through as many sequences
        # as about cpu_seconds of work take
        nrows = rows_for(args.cpu_seconds)
        rows = list(range(nrows * w.Hq))
        t0 = time.perf_counter()
        oracle.prefill(*host, w.scale, rows=rows)
        dt = time.perf_counter() - t0
        toks = int(att[:nrows].sum())
        res["cpu_baseline"] = {"value": round(4 * w.D * w.Hq * toks / dt / 1e12, 6), "unit": "TFLOP/s",
                               "cores": oracle.num_threads(), "cpu": cpu_model(),
                               "kind": "oracle",
                               "sample": f"the first {nrows} of {len(att)} query rows, all heads",
                               "seconds": round(dt, 2)}
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.print_source_sha:
        print(json.dumps({k: source_sha256(k) for k in KERNEL_SOURCES}))
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(the hot path needs no cross-GPU exchange; see the sharding note in the design doc)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from paged_kv_cache_301_amd import binding, workloads

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.op == "prefill":
        bench_prefill(args, dev)
        return
    over = {}
    if args.block_size:
        over["B"] = args.block_size
    if args.q_heads:
        over["Hq"] = args.q_heads
    if args.seqs:
        over["S"] = args.seqs
    if args.fixed_len:
        S = args.seqs or workloads.SPECS[args.workload].S
        over["lens"] = ("fixed", (args.fixed_len,) * S)
        over["max_len"] = args.fixed_len
    t_gen = time.perf_counter()
    w = workloads.make_workload(args.workload, device=dev, poison=False, **over)
    torch.cuda.synchronize()
    print(f"[bench] workload {args.workload}: S={w.S} Hq={w.Hq} Hkv={w.Hkv} D={w.D} B={w.B} "
          f"NB={w.NB} max_blocks={w.max_blocks} tokens={int(w.lens.sum())} "
          f"kv={w.kv_bytes() / 1e9:.3f} GB (generated in {time.perf_counter() - t_gen:.1f}s)",
          file=sys.stderr, flush=True)

    if args.op != "decode":
        bench_write(args, w, dev)
        return

    kv_reuse = args.kv_reuse == "on"
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)   # cache eviction
    plan, t, (step, args_, kw) = measure_decode(w, args, dev, scratch, kernel=args.kernel,
                                                partition_tokens=args.partition_tokens,
                                                kv_reuse=kv_reuse, token_waves=args.token_waves)
    kname = KERNEL_NAMES[plan["kernel"]]
    uniq0 = w.unique_kv_bytes() if w.spec.prefix_tokens else w.kv_bytes()
    floor = None if args.no_read_peak else plain_read_floor(uniq0, args, dev, scratch)
    summ = decode_summary(w, plan, t, kname, floor)
    kv = w.kv_bytes()
    step_ms = t["cold"]["median_us"] * 1e-3
    gbs = kv / (step_ms * 1e-3) / 1e9
    part_avg = t["partitions"]["mean_us"] * 1e-3
    achieved = kv / (part_avg * 1e-3) / 1e9
    print(f"[bench] plan {plan}; cold: step median {t['cold']['median_us']:.1f} us, partition "
          f"kernel mean {t['partitions']['mean_us']:.1f} us, combine "
          f"{(t['combine'] or {}).get('mean_us', 0.0):.1f} us; warm step "
          f"{t['warm']['ms_per_step'] * 1e3:.1f} us", file=sys.stderr, flush=True)

    # the same step captured once in a HIP graph (both kernels) and replayed:
    # one host launch per step instead of two
    graph = None
    if args.graph:
        stream = kw["stream"]
        gstream = torch.cuda.Stream(dev)
        run_all = binding.prepare(*args_, stages=0, **{**kw, "stream": gstream})
        run_all()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=gstream):
            run_all()
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        g_step_ms, g_gpu_ms = time_loop(g.replay, args.steps, stream)
        graph = {"ms_per_step": round(g_step_ms, 5),
                 "value": round(kv / (g_step_ms * 1e-3) / 1e9, 2),
                 "gpu_us": round(g_gpu_ms * 1e3, 2)}
        del g

    # the other decode configurations, measured the same way (automatic plan)
    extra = None
    if not args.no_extra_configs and not (args.block_size or args.q_heads or args.seqs
                                          or args.fixed_len or args.kernel != "auto"
                                          or args.partition_tokens or args.token_waves):
        extra = {}
        for key, name, over in (("mha_small", "mha_small", {}), ("gqa_70b", "gqa_70b", {}),
                                ("gqa_long_B16", "gqa_long", {"B": 16})):
            if name == args.workload and over.get("B", w.B) == w.B:
                continue
            wx = workloads.make_workload(name, device=dev, poison=False, **over)
            torch.cuda.synchronize()
            px, tx, _ = measure_decode(wx, args, dev, scratch, kv_reuse=kv_reuse)
            ux = wx.unique_kv_bytes() if wx.spec.prefix_tokens else wx.kv_bytes()
            fx = None if args.no_read_peak else plain_read_floor(ux, args, dev, scratch)
            extra[key] = decode_summary(wx, px, tx, KERNEL_NAMES[px["kernel"]], fx)
            e = extra[key]
            print(f"[bench] {key}: cold step {e['step_cold_us']['median_us']:.1f} us "
                  f"({e['gbs']:.0f} GB/s logical, {e['unique_hbm_frac'] * 100:.1f} % of 8 TB/s "
                  f"on unique bytes), kernel {e['kernel_cold_us']['mean_us']:.1f} us, plain read "
                  f"of the same bytes {(e.get('plain_read_floor') or {}).get('median_us', 0):.1f} us",
                  file=sys.stderr, flush=True)
            del wx
    del scratch

    esz = w.esz
    unique = summ["unique_kv_bytes"] if w.spec.prefix_tokens else None
    n_blocks = int(((w.lens + w.B - 1) // w.B).sum())
    alg_total = kv + 2 * w.S * w.Hq * w.D * esz + 4 * n_blocks + 4 * w.S

    res = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {torch.bfloat16: "bf16", torch.float16: "f16", torch.float32: "f32"}[w.dtype],
        "data": "synthetic",
        "config": {"workload": args.workload, "S": w.S, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D,
                   "B": w.B, "tokens": int(w.lens.sum()), "kv_bytes": kv,
                   "unique_kv_bytes": unique or kv,
                   "kernel": kname, "partition_tokens": plan["partition_tokens"],
                   "token_waves": plan["token_waves"], "kv_reuse": kv_reuse, "fixed_len": args.fixed_len,
                   "split": bool(plan["split"]), "timing": "cold cache, median step"},
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "seqs_per_s": round(w.S / (step_ms * 1e-3), 1),
        # with a prefix shared by the batch, the rate on the bytes stored once
        # (each shared block counted once): the conservative figure
        "unique_gbs": round(unique / (step_ms * 1e-3) / 1e9, 2) if unique else None,
        "unique_hbm_frac": round(unique / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
                           if unique else None,
        "step_cold_us": t["cold"],
        "plain_read_floor": summ.get("plain_read_floor"),
        "step_vs_floor": summ.get("step_vs_floor"),
        "kernel_us": {"partitions": t["partitions"], "combine": t["combine"]},
        "warm": {**t["warm"], "value": round(kv / (t["warm"]["ms_per_step"] * 1e-3) / 1e9, 2)},
        "graph": graph,
        "alg_bytes_total": alg_total,
        "workspace_bytes": plan["workspace_bytes"],
        "flops_alg": int(w.lens.sum()) * w.Hq * 4 * w.D,
        "roofline": {"bound": "hbm", "kernel": f"pa_{kname}_partitions",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic(f"pa_{kname}_partitions", record_key(args.workload, args), w.B,
                                                 plan["partition_tokens"], plan["token_waves"])},
        "configs": extra,
    }
    if not args.no_read_peak:
        peak = measured_read_peak(dev)
        peak["step_frac"] = round(gbs / peak["gbs"], 4)
        res["read_peak_measured"] = peak
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
