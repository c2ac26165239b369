"""Benchmark: paged-KV decode on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config NAME] [--partition-size PS]

One step is one pass of the whole hot path over one batch: the cache write of
every sequence's new token, the block-table-driven decode partitions, and the
split-K reduce.  Where every sequence gains one token at position L - 1 of
a bf16 or fp8 cache (the static bf16 and fp8 decode workloads) the measured
step is the fused form, paged_attention_decode_append(_fp8), whose decode
launch stores the new tokens itself (bit for bit the result of the two
calls); the two-call form, reshape_and_cache(_fp8) then
paged_attention_decode(_fp8), is timed beside it and reported under
``two_call`` (``--two-call`` makes it the measured step).  Other workloads
(fp32, continuous batching with prompt writes) take the two calls.  The default workload is the
Llama-3-8B-shaped decode layer (64 sequences, 32 q / 8 KV heads, head_dim 128,
bf16 KV, context lengths uniform on [128, 4096]).  Inputs are resident in HBM
before timing starts, and before the W warmup steps the step runs untimed for
at least --settle-ms (default 200 ms) so that the timed steps see the GPU's
steady clock (with 20 warmup steps alone, about 1 ms of work, the fp8 decode
step measured about 4 % slower).  To keep the 256 MB Infinity Cache from serving KV
across steps, several copies of the pool are used in rotation, so a step never
reads data a recent step read.

Printed: one JSON line with the KV-read bandwidth (algorithmic KV bytes per
step / wall time per step, over K steps with nothing else on the stream),
decode tokens/s, the dominant kernel's roofline (HIP events around its
launches in a second pass of K steps), and the CPU oracle's rate on a
bounded sample of the same workload.
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

PEAK_HBM_GBS = 8000.0
METRIC = "paged-attn decode: achieved KV-read HBM GB/s (% of peak) + decode tokens/s"
PEAK_BF16_TFLOPS = 2500.0
PREFILL_METRIC = "paged-attn chunked prefill: attention TFLOP/s (causal flops) + prefill tokens/s"
PREFILL_CONFIGS = ("chunked_prefill", "chunked_prefill_fp8")
COPY_CONFIGS = ("block_copy", "swap")
PEAK_HOST_LINK_GBS = 64.0   # PCIe 5.0 x16, one direction
COPY_METRIC = "whole-block KV copies: GB/s moved (copy-on-write in HBM: read + write; swap: over the host link)"


def family(workload: str) -> str:
    if workload in PREFILL_CONFIGS:
        return "prefill"
    if workload in COPY_CONFIGS:
        return "copy"
    return "decode"


# static bf16 and fp8 decode workloads whose step can take the fused append
FUSABLE_CONFIGS = ("llama3_8b_decode", "shared_prefix", "long_context", "llama3_8b_decode_fp8", "long_context_fp8")


def settle(step, ms: float) -> None:
    """Run ``step()`` untimed for at least ``ms`` milliseconds of wall time, the GPU kept busy, so that
    what is timed next runs at the GPU's steady clock rather than while it ramps up."""
    import torch
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(8):
            step()
        torch.cuda.synchronize()


def traffic_file(workload: str, fused: bool = False) -> str:
    tag = "_fused" if fused else ""
    return os.path.join(ROOT, "profiles", f"{family(workload)}_traffic_{workload}{tag}.json")


def kernel_sources(workload: str):
    """Sources whose code decides the kernel's traffic: the kernel, the
    internal header, and (decode) the launch planning in the ABI layer."""
    if family(workload) == "prefill":
        files = ("prefill_wide.hip", "prefill_common.h", "prefill.h", "kernels.h")
    else:
        main = "copy_blocks.hip" if family(workload) == "copy" else "decode_mfma.hip"
        files = (main, "kernels.h", "pagedkv_abi.hip") if family(workload) == "decode" else (main, "kernels.h")
    return [os.path.join(ROOT, "paged_kv_cache_372_amd", "csrc", f) for f in files]


def _code_only(text: str) -> str:
    """C++ source with comments removed and whitespace collapsed, so that an
    edit to comments alone keeps the counters taken on the same code."""
    import re
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":  # string or character literal, kept whole
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return re.sub(r"\s+", " ", "".join(out)).strip()


def kernel_source_hash(workload: str = "llama3_8b_decode") -> str:
    h = hashlib.sha256()
    for p in kernel_sources(workload):
        h.update(_code_only(open(p).read()).encode())
    return h.hexdigest()


def measured_traffic(workload: str, partition_size: int, fused: bool = False):
    """Per-launch HBM bytes of the decode kernel from committed rocprofv3 counters.

    Null unless the counters were taken on this exact kernel source and
    workload configuration (and the same form of the step: fused or not).
    """
    try:
        rec = json.load(open(traffic_file(workload, fused)))
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != kernel_source_hash(workload):
        return None
    if rec.get("workload") != workload or rec.get("partition_size") != partition_size:
        return None
    fetch = rec["fetch_kib_per_dispatch"] * 1024 * rec["fetch_copy_factor"]
    write = rec["write_kib_per_dispatch"] * 1024 * rec["write_copy_factor"]
    return int(round(fetch + write))


def build_workload(name: str, ps: int):
    """(batch, steps): a static DecodeBatch and None, or, for the
    continuous-batching run, a DecodeBatch describing its first step (pools
    before any write) and the list of its ten steps."""
    import workloads as W
    if name == "long_context":
        return W.long_context(partition_size=ps if ps >= 0 else 512), None
    if name == "long_context_fp8":
        return W.fp8_variant(W.long_context(partition_size=ps if ps >= 0 else 512)), None
    ps = max(ps, 0)
    if name == "continuous_batching":
        sim = W.ContinuousBatching(partition_size=ps)
        k_pool, v_pool = sim.initial_pools()
        steps = [sim.step(i) for i in range(sim.steps)]
        st = steps[0]
        b = W.DecodeBatch(name=sim.name, seed=sim.seed, dtype=sim.dtype, num_q_heads=sim.Hq, num_kv_heads=sim.Hkv,
                          head_dim=sim.D, block_size=sim.bs, num_blocks=sim.num_blocks, q=st.q, k_new=st.k_write,
                          v_new=st.v_write, slot_mapping=st.slot_mapping, k_pool=k_pool, v_pool=v_pool,
                          block_tables=st.block_tables, context_lens=st.context_lens, scale=sim.scale,
                          partition_size=ps)
        return b, steps
    if name == "llama3_8b_decode":
        return W.llama3_8b_decode(partition_size=ps), None
    if name == "llama3_8b_decode_fp8":
        return W.fp8_variant(W.llama3_8b_decode(partition_size=ps)), None
    if name == "shared_prefix":
        return W.shared_prefix(partition_size=ps), None
    if name == "tiny_fp32":
        return W.tiny_fp32(), None
    raise SystemExit(f"unknown --config {name}")


def cpu_baseline(b, budget_s: float = 12.0):
    """The oracle, as it stands, over the same workload, one (sequence, KV
    head) at a time -- each call covers the query heads of that KV head's
    group -- pass after pass, until about ``budget_s`` seconds of CPU work
    are done."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    fp8 = b.dtype == "fp8"
    if fp8:
        ks, vs = b.info["k_scale"], b.info["v_scale"]
        kp, vp = oracle.ref_reshape_and_cache_fp8(b.k_new, b.v_new, b.slot_mapping, b.k_pool, b.v_pool, ks, vs,
                                                  "bf16")
    else:
        ks = vs = None
        kp, vp = oracle.ref_reshape_and_cache(b.k_new, b.v_new, b.slot_mapping, b.k_pool, b.v_pool)
    G = b.num_q_heads // b.num_kv_heads
    units = [(s, g) for s in range(b.num_seqs) for g in range(b.num_kv_heads)]
    t0 = time.perf_counter()
    done, kv_bytes, passes = 0, 0, 0
    es = {"bf16": 2, "f32": 4, "fp8": 1}[b.dtype]
    while time.perf_counter() - t0 < budget_s:
        for s, g in units:
            oracle.ref_paged_attention_decode(b.q, kp, vp, b.block_tables, b.context_lens, b.scale, b.dtype, seqs=[s],
                                              q_heads=list(range(g * G, (g + 1) * G)), k_scale=ks, v_scale=vs)
            done += 1
            kv_bytes += int(b.context_lens[s]) * 2 * b.head_dim * es
            if time.perf_counter() - t0 >= budget_s:
                break
        passes += 1
    dt = time.perf_counter() - t0
    return {"value": round(kv_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} (sequence, KV head) decodes of the {b.name} workload ({len(units)} per pass, "
                      f"{passes} pass(es) begun; each over its {G} query heads, float64, after the oracle's cache "
                      f"write), {dt:.1f} s",
            "tokens_per_s": round(done / b.num_kv_heads / dt, 3), "cpu_model": _cpu_model(),
            "os_cpu_count": os.cpu_count()}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def host_pack_ms(b, reps: int = 20):
    """Time to pack the step's tables on the host and copy them to the GPU (pinned, async + sync)."""
    import numpy as np
    import torch
    from paged_kv_cache_372_amd.blocks import pack_block_tables, Sequence
    seqs = []
    for s in range(b.num_seqs):
        L = int(b.context_lens[s])
        n = -(-L // b.block_size)
        seqs.append(Sequence(s, b.block_tables[s, :n].tolist(), L))
    width = b.block_tables.shape[1]
    pin_bt = torch.empty((b.num_seqs, width), dtype=torch.int32, pin_memory=True)
    pin_len = torch.empty((b.num_seqs,), dtype=torch.int32, pin_memory=True)
    pin_slot = torch.empty((b.num_seqs,), dtype=torch.int64, pin_memory=True)
    d_bt = torch.empty_like(pin_bt, device="cuda")
    d_len = torch.empty_like(pin_len, device="cuda")
    d_slot = torch.empty_like(pin_slot, device="cuda")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        pin_bt.numpy()[:] = pack_block_tables(seqs, width, b.pad_block if b.pad_block >= 0 else 0)
        pin_len.numpy()[:] = [s.num_tokens for s in seqs]
        pin_slot.numpy()[:] = [s.slot_of(s.num_tokens - 1, b.block_size) for s in seqs]
        d_bt.copy_(pin_bt, non_blocking=True)
        d_len.copy_(pin_len, non_blocking=True)
        d_slot.copy_(pin_slot, non_blocking=True)
        torch.cuda.synchronize()
    return (time.perf_counter() - t0) / reps * 1e3


def calibrate_copy(mib: int, reps: int):
    """A plain device copy of known size, for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE."""
    import torch
    n = mib * 1024 * 1024 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read": n * 4, "bytes_written": n * 4, "reps": reps}))


DECODE_KERNEL_PREFIX = "void pkv::(anonymous namespace)::decode_bf16_balanced_kernel"
PREFILL_KERNEL_PREFIX = "void pkv::(anonymous namespace)::prefill_wide_kernel"
COPY_KERNEL_PREFIX = "pkv::(anonymous namespace)::copy_blocks_kernel"


def _read_counter(dirpath: str, counter: str):
    """Mean per-dispatch value of ``counter`` for each kernel in a rocprofv3 csv run."""
    import csv
    import glob
    sums = {}
    for f in glob.glob(os.path.join(dirpath, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            sums.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in sums.items()}


def _short_kernel_name(k: str) -> str:
    k = k[5:] if k.startswith("void ") else k
    return k.replace("pkv::(anonymous namespace)::", "").split("(")[0]


def summarize_profile(prefix: str, workload: str, partition_size, copy_mib: int, out_md: str, out_json: str,
                      commands: str, fused: bool = False) -> None:
    """Turn rocprofv3 csv output (``<prefix>_trace``, ``_fetch``, ``_write``,
    ``_cal_fetch``, ``_cal_write``) into a short markdown summary and the
    per-launch traffic record ``measured_traffic`` reads."""
    import csv
    import glob
    stats = []
    for f in glob.glob(os.path.join(prefix + "_trace", "**", "*kernel_stats.csv"), recursive=True):
        stats += list(csv.DictReader(open(f)))
    fetch = _read_counter(prefix + "_fetch", "FETCH_SIZE")
    write = _read_counter(prefix + "_write", "WRITE_SIZE")
    copy_kib = copy_mib * 1024.0
    cal_f = _read_counter(prefix + "_cal_fetch", "FETCH_SIZE")
    cal_w = _read_counter(prefix + "_cal_write", "WRITE_SIZE")
    copy_name = "__amd_rocclr_copyBuffer"
    f_factor = copy_kib / cal_f[copy_name]
    w_factor = copy_kib / cal_w[copy_name]
    prefix_k = {"prefill": PREFILL_KERNEL_PREFIX,
                "copy": COPY_KERNEL_PREFIX}.get(family(workload), DECODE_KERNEL_PREFIX)
    short_k = prefix_k.split("::")[-1]
    dec = [k for k in fetch if short_k in k][0]
    form = " (fused append step)" if fused else ""
    lines = [f"# rocprofv3: {family(workload)} kernels on the {workload} workload{form}", "",
             "Commands (run from the repository root; `cd /tmp && export TMPDIR=/tmp` first):", "", "```",
             commands.strip(), "```", "", "## Kernel trace (`--kernel-trace --stats`)", "",
             "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    for r in stats:
        name = _short_kernel_name(r["Name"])
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    lines += ["", "## HBM traffic per dispatch (`--pmc FETCH_SIZE`, then `--pmc WRITE_SIZE`)", "",
              f"Calibration: a {copy_mib} MiB device copy (`{copy_name}`) reads FETCH_SIZE = {cal_f[copy_name]:.0f} KiB "
              f"and WRITE_SIZE = {cal_w[copy_name]:.0f} KiB, so the counters are scaled by {f_factor:.4f} (fetch) and "
              f"{w_factor:.4f} (write).", "",
              "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled read MB | scaled write MB |", "|---|---|---|---|---|"]
    for k in fetch:
        if k.startswith("__amd_rocclr"):
            continue
        name = _short_kernel_name(k)
        lines.append(f"| `{name}` | {fetch[k]:.0f} | {write.get(k, 0):.0f} | {fetch[k] * 1024 * f_factor / 1e6:.1f} | "
                     f"{write.get(k, 0) * 1024 * w_factor / 1e6:.2f} |")
    bench_log = prefix + "_bench.log"
    if os.path.exists(bench_log):
        last = [ln for ln in open(bench_log).read().splitlines() if ln.startswith("{")]
        if last:
            flag = "" if fused or workload not in FUSABLE_CONFIGS else " --two-call"
            lines += ["", f"## Bench line of the same build (`python bench.py --config {workload}{flag}`)", "", "```",
                      last[-1], "```"]
    rec = {"source_sha256": kernel_source_hash(workload), "workload": workload, "partition_size": partition_size,
           "kernel": dec, "fetch_kib_per_dispatch": fetch[dec], "write_kib_per_dispatch": write.get(dec, 0.0),
           "fetch_copy_factor": f_factor, "write_copy_factor": w_factor}
    os.makedirs(os.path.dirname(out_md), exist_ok=True)
    open(out_md, "w").write("\n".join(lines) + "\n")
    json.dump(rec, open(out_json, "w"), indent=1)
    print(f"wrote {out_md} and {out_json}")


def cpu_baseline_prefill(b, budget_s: float = 12.0):
    """The prefill oracle, as it stands, request after request of the same
    workload, until about ``budget_s`` seconds of CPU work are done."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    fp8 = b.dtype == "fp8"
    if fp8:
        ks, vs = b.info["k_scale"], b.info["v_scale"]
        kp, vp = oracle.ref_reshape_and_cache_fp8(b.k_new, b.v_new, b.slot_mapping, b.k_pool, b.v_pool, ks, vs,
                                                  b.info["src_dtype"])
        scales = dict(k_scale=ks, v_scale=vs)
    else:
        kp, vp = oracle.ref_reshape_and_cache(b.k_new, b.v_new, b.slot_mapping, b.k_pool, b.v_pool)
        scales = {}
    n = b.query_lens()
    L = b.context_lens.astype(np.int64)
    t0 = time.perf_counter()
    done, flops, tokens = 0, 0, 0
    for s in range(b.num_seqs):
        oracle.ref_paged_attention_prefill(b.q, kp, vp, b.block_tables, b.context_lens, b.query_start_loc, b.scale,
                                           b.dtype, seqs=[s], **scales)
        done += 1
        tokens += int(n[s])
        flops += 4 * b.head_dim * b.num_q_heads * int(n[s] * (L[s] - n[s]) + n[s] * (n[s] + 1) // 2)
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} of the {b.num_seqs} requests of the {b.name} workload ({tokens} query tokens, "
                      f"float64, all {b.num_q_heads} q heads, after the oracle's cache write), {dt:.1f} s",
            "tokens_per_s": round(tokens / dt, 3), "cpu_model": _cpu_model(), "os_cpu_count": os.cpu_count()}


def run_prefill(args):
    """Chunked-prefill step: the cache write of every new token, then the
    multi-token-query attention.  Value = algorithmic (causal) attention
    flops per step / wall time per step."""
    import numpy as np
    import torch
    from paged_kv_cache_372_amd import ops
    import workloads as W

    fp8 = args.config == "chunked_prefill_fp8"
    t_gen = time.perf_counter()
    b = W.chunked_prefill()
    if fp8:  # the same step over an fp8 (E4M3) cache with per-KV-head scales
        b = W.fp8_variant(b)
    gen_s = time.perf_counter() - t_gen

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)

    def ints(a, dt):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=dt)).cuda()

    q, k_new, v_new = dev(b.q), dev(b.k_new), dev(b.v_new)
    if fp8:
        kc, vc = ints(b.k_pool, np.uint8), ints(b.v_pool, np.uint8)
        ks, vs = ints(b.info["k_scale"], np.float32), ints(b.info["v_scale"], np.float32)
    else:
        kc, vc = dev(b.k_pool), dev(b.v_pool)
    slots = ints(b.slot_mapping, np.int64)
    bt, lens, qsl = ints(b.block_tables, np.int32), ints(b.context_lens, np.int32), ints(b.query_start_loc, np.int32)
    out = torch.empty_like(q)
    flops = b.flops()

    def step(ev=None):
        if fp8:
            ops.reshape_and_cache_fp8(k_new, v_new, slots, kc, vc, ks, vs)
        else:
            ops.reshape_and_cache(k_new, v_new, slots, kc, vc)
        if ev is not None:
            ev[0].record()
        if fp8:
            ops.paged_attention_prefill_fp8(q, kc, vc, ks, vs, bt, lens, qsl, b.scale, out,
                                            max_context_len=b.max_context_len)
        else:
            ops.paged_attention_prefill(q, kc, vc, bt, lens, qsl, b.scale, out, max_context_len=b.max_context_len)
        if ev is not None:
            ev[1].record()

    settle(step, args.settle_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    k_ms = sum(e[0].elapsed_time(e[1]) for e in events) / args.steps
    ms = wall / args.steps * 1e3
    value = flops / (ms / 1e3) / 1e12
    achieved = flops / (k_ms / 1e3) / 1e12
    traffic = measured_traffic(b.name, "none")
    rec = {
        "metric": PREFILL_METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "settle_ms": args.settle_ms, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": b.name, "seed": b.seed, "num_seqs": b.num_seqs, "num_tokens": b.num_tokens,
                   "num_q_heads": b.num_q_heads, "num_kv_heads": b.num_kv_heads, "head_dim": b.head_dim,
                   "block_size": b.block_size, "chunk": int(b.query_lens().max()),
                   "cached_mean": round(float(np.mean(b.info["cached"])), 1),
                   "context_len_max": b.max_context_len, "flops_per_step": flops,
                   "kv_dtype": "fp8_e4m3" if fp8 else "bf16"},
        "frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "tokens_per_s": round(b.num_tokens / (ms / 1e3), 1),
        "prefill_kernel_ms": round(k_ms, 5),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "kernel": "prefill_wide_kernel", "flops_per_launch": flops},
        "input_generation_s": round(gen_s, 2),
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline_prefill(b, args.cpu_budget)
    print(json.dumps(rec), flush=True)


def run_copy(args):
    """Whole-block copies on the Llama-3-8B shape (8 KV heads x 128 dims,
    bf16: 32 KiB per block per pool).  block_copy: 4096 copy-on-write pairs
    inside a 16384-block device pool (random distinct blocks).  swap: 1024
    blocks out to a pinned host pool, then back into other device blocks;
    one step is the round trip."""
    import numpy as np
    import torch
    from paged_kv_cache_372_amd import ops
    import oracle

    rng = np.random.default_rng(3727)
    hkv, D, nb = 8, 128, 16384
    block_bytes = hkv * D * 16 * 2
    kp = torch.randn((nb, hkv, D // 8, 16, 8), dtype=torch.bfloat16, device="cuda")
    vp = torch.randn((nb, hkv, D, 16), dtype=torch.bfloat16, device="cuda")
    perm = rng.permutation(nb)
    if args.config == "block_copy":
        n = 4096
        pairs = torch.from_numpy(np.stack([perm[:n], perm[n:2 * n]], axis=1).astype(np.int64)).cuda()
        moved = n * 2 * block_bytes                      # bytes copied (K and V)
        hbm = 2 * moved                                  # read + write

        def step(ev=None):
            if ev is not None:
                ev[0].record()
            ops.copy_blocks(kp, vp, pairs)
            if ev is not None:
                ev[1].record()
        launches = 1
    else:
        n = 1024
        hk = torch.empty((n,) + tuple(kp.shape[1:]), dtype=kp.dtype).pin_memory()
        hv = torch.empty((n,) + tuple(vp.shape[1:]), dtype=vp.dtype).pin_memory()
        out_pairs = torch.from_numpy(np.stack([perm[:n], np.arange(n)], axis=1).astype(np.int64)).cuda()
        in_pairs = torch.from_numpy(np.stack([np.arange(n), perm[n:2 * n]], axis=1).astype(np.int64)).cuda()
        moved = 2 * n * 2 * block_bytes                  # out and back, K and V
        hbm = moved

        def step(ev=None):
            if ev is not None:
                ev[0].record()
            ops.swap_blocks(kp, vp, hk, hv, out_pairs)
            ops.swap_blocks(hk, hv, kp, vp, in_pairs)
            if ev is not None:
                ev[1].record()
        launches = 2
    settle(step, args.settle_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    k_ms = sum(e[0].elapsed_time(e[1]) for e in events) / args.steps
    ms = wall / args.steps * 1e3
    value = moved / (ms / 1e3) / 1e9
    if args.config == "block_copy":
        roof = {"bound": "hbm", "achieved": round(hbm / (k_ms / 1e3) / 1e9, 2), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(hbm / (k_ms / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
                "traffic": measured_traffic(args.config, "none"), "kernel": "copy_blocks_kernel",
                "bytes_per_launch": hbm}
    else:
        per_dir = moved / 2 / (k_ms / 2 / 1e3) / 1e9
        roof = {"bound": "host-link", "achieved": round(per_dir, 2), "peak": PEAK_HOST_LINK_GBS, "unit": "GB/s",
                "frac": round(per_dir / PEAK_HOST_LINK_GBS, 4), "traffic": None, "kernel": "copy_blocks_kernel",
                "bytes_per_launch": moved // 2}
    rec = {"metric": COPY_METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "settle_ms": args.settle_ms, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": args.config, "pairs_per_launch": n, "launches_per_step": launches,
                      "num_kv_heads": hkv, "head_dim": D, "block_bytes_per_pool": block_bytes,
                      "bytes_copied_per_step": moved},
           "kernel_ms": round(k_ms, 5), "roofline": roof}
    if not args.no_cpu_baseline:
        ks = (64, hkv, D // 8, 16, 8)
        vs = (64, hkv, D, 16)
        hk0 = rng.integers(0, 65535, size=ks, dtype=np.uint16)
        hv0 = rng.integers(0, 65535, size=vs, dtype=np.uint16)
        p = np.stack([np.arange(32), np.arange(32, 64)], axis=1)
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < min(args.cpu_budget, 3.0):
            oracle.ref_copy_blocks(hk0, hv0, hk0, hv0, p)
            reps += 1
        dt = time.perf_counter() - t0
        rec["cpu_baseline"] = {"value": round(reps * 32 * 2 * block_bytes / dt / 1e9, 3), "unit": "GB/s", "cores": 1,
                               "kind": "oracle", "sample": f"{reps} oracle calls of 32 block copies in a 64-block "
                                                           f"pool ({dt:.1f} s, numpy, one thread)"}
    print(json.dumps(rec), flush=True)


def identity_table_comparison(b, kcs, vcs, g, ps, steps, warmup, permuted_ms):
    """Cost of the indirection: the same tokens laid out with identity block
    tables (each sequence's blocks consecutive and in order), decode launch
    timed by events against the permuted layout's."""
    import numpy as np
    import torch
    from paged_kv_cache_372_amd import ops
    block_map, tables, slots = identity_layout(b)
    bm = torch.from_numpy(block_map).cuda()
    kid = [k.index_select(0, bm) for k in kcs]
    vid = [v.index_select(0, bm) for v in vcs]
    bt = torch.from_numpy(tables).cuda()
    sl = torch.from_numpy(slots).cuda()
    out = torch.empty_like(g["out"])
    R = len(kid)
    ws = torch.empty(max(1, ops.decode_workspace_bytes(b.num_seqs, b.num_q_heads, b.num_kv_heads, b.head_dim,
                                                       g["max_ctx"], ps)), dtype=torch.uint8, device="cuda")
    plans = [ops.prepare_decode(g["q"], kid[r], vid[r], bt, g["lens"], b.scale, out, partition_size=ps,
                                max_context_len=g["max_ctx"], workspace=ws) for r in range(R)]

    def step(i, ev=None):
        r = i % R
        ops.reshape_and_cache(g["k_new"], g["v_new"], sl, kid[r], vid[r])
        if ev is not None:
            ev[0].record()
        ops.run_partitions(plans[r])
        if ev is not None:
            ev[1].record()
        ops.run_reduce(plans[r])
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    same = bool(torch.equal(out.view(torch.int16), g["out"].view(torch.int16)))
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for i in range(steps):
        step(warmup + i, events[i])
    torch.cuda.synchronize()
    t = [e[0].elapsed_time(e[1]) for e in events]
    ident = sum(t) / steps
    return {"identity_decode_kernel_ms": round(ident, 5), "permuted_decode_kernel_ms": round(permuted_ms, 5),
            "identity_over_permuted": round(ident / permuted_ms, 4), "identity_decode_kernel_ms_median":
            round(float(np.median(t)), 5), "outputs_bit_identical": same,
            "layout": "each sequence's blocks consecutive, in table order, same pool replicas"}


def vector_alu_comparison(b, kcs, vcs, g, ps, plans, steps, warmup):
    """The same decode (the two launches: decode and split-K reduce) on the
    vector ALU and on the matrix cores, each timed by events over K calls,
    alternating pool replicas as the main loop does."""
    import numpy as np
    import torch
    from paged_kv_cache_372_amd import ops
    R = len(kcs)
    need = ops.decode_workspace_bytes(b.num_seqs, b.num_q_heads, b.num_kv_heads, b.head_dim, g["max_ctx"], ps,
                                      torch.float32)
    ws = torch.empty(max(1, need), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(g["out"])

    def valu(i):
        r = i % R
        ops.paged_attention_decode_vector_alu(g["q"], kcs[r], vcs[r], g["bt"], g["lens"], b.scale, out,
                                              partition_size=ps, max_context_len=g["max_ctx"], workspace=ws)

    def mfma(i):
        ops.run_partitions(plans[0, i % R])
        ops.run_reduce(plans[0, i % R])

    res = {}
    for name, fn in (("vector_alu", valu), ("matrix_core", mfma)):
        for i in range(warmup):
            fn(i)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        torch.cuda.synchronize()
        for i in range(steps):
            ev[i][0].record()
            fn(i)
            ev[i][1].record()
        torch.cuda.synchronize()
        t = [e[0].elapsed_time(e[1]) for e in ev]
        res[name + "_ms"] = round(sum(t) / steps, 5)
        res[name + "_ms_median"] = round(float(np.median(t)), 5)
    torch.cuda.synchronize()
    res["vector_alu_over_matrix_core"] = round(res["vector_alu_ms"] / res["matrix_core_ms"], 4)
    res["max_abs_diff"] = float((out.float() - g["out"].float()).abs().max().item())
    res["what"] = "decode + split-K reduce launches, HIP events, same inputs and pool replicas"
    return res


HBM_READ_METRIC = "plain HBM read ceiling: GB/s of 16-byte loads (contiguous, and random tiles)"


def run_hbm_read(args):
    """Read-only microbenchmark: a 4 GiB buffer (16x the Infinity Cache) read
    front to back, and as random whole tiles of 4, 16 and 32 KiB (every tile
    once, in a seeded random order), with streaming and with ordinary loads.
    Each launch is timed by HIP events; the headline is the contiguous
    streaming read."""
    import numpy as np
    import torch
    from paged_kv_cache_372_amd import ops
    nbytes = 4 << 30
    src = torch.full((nbytes // 4,), 0x01010101, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1024, dtype=torch.int32, device="cuda")
    rng = np.random.default_rng(3729)
    cases = [("contiguous", None, 0)]
    for tb in (4096, 16384, 32768):
        perm = torch.from_numpy(rng.permutation(nbytes // tb).astype(np.int32)).cuda()
        cases.append((f"tiles_{tb // 1024}k", perm, tb))
    # the KV bytes of one Llama-3-8B-shaped decode step (seed 3722: 578.3 MB)
    # as random 32 KiB tiles, one K or V block of 8 heads each: a plain read
    # of the same size, launch and drain included
    c2_tiles = 578277376 // 32768
    perm = torch.from_numpy(rng.permutation(nbytes // 32768)[:c2_tiles].astype(np.int32)).cuda()
    cases.append(("tiles_32k_c2_bytes", perm, 32768))
    out = {}
    for name, tiles, tb in cases:
        for streaming in (True, False):
            def launch():
                ops.hbm_read_bench(src, sink, tiles, tb, streaming)
            for _ in range(args.warmup):
                launch()
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
            torch.cuda.synchronize()
            for i in range(args.steps):
                ev[i][0].record()
                launch()
                ev[i][1].record()
            torch.cuda.synchronize()
            t = [e[0].elapsed_time(e[1]) for e in ev]
            key = f"{name}_{'streaming' if streaming else 'ordinary'}"
            nb = nbytes if tiles is None else tiles.numel() * tb
            out[key] = {"gbs": round(nb / (sum(t) / len(t) / 1e3) / 1e9, 1),
                        "gbs_median": round(nb / (float(np.median(t)) / 1e3) / 1e9, 1),
                        "ms_mean": round(sum(t) / len(t), 5), "bytes": nb}
            print(json.dumps({"case": key, **out[key]}), flush=True)
    head = out["contiguous_streaming"]
    rec = {"metric": HBM_READ_METRIC, "value": head["gbs"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": head["ms_mean"], "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "u8", "data": "synthetic",
           "config": {"workload": "hbm_read", "buffer_bytes": nbytes, "tile_bytes": [4096, 16384, 32768],
                      "loads": "16-byte, 8 in flight per thread, 8 workgroups of 256 threads per CU"},
           "frac_of_peak": round(head["gbs"] / PEAK_HBM_GBS, 4),
           "roofline": {"bound": "hbm", "achieved": head["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(head["gbs"] / PEAK_HBM_GBS, 4), "traffic": None, "kernel": "hbm_read_kernel",
                        "bytes_per_launch": nbytes},
           "cases": out}
    print(json.dumps(rec), flush=True)


ISSUE_RATE_METRIC = "instruction issue rates: matrix-core TFLOP/s, vector ALU cycles per instruction, LDS bytes per cycle"


def run_issue_rates(args):
    """Issue-rate microbenchmark (library aid pkv_issue_rate_bench): each
    pattern with one and with two waves per SIMD, one workgroup per compute
    unit, timed by HIP events on the launching stream.  Cycles are at the
    nominal 2.4 GHz.  The headline is mfma_f32_32x32x16_bf16 into four
    accumulators, one wave per SIMD."""
    import torch
    from paged_kv_cache_372_amd import ops
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.zeros(512, dtype=torch.int32, device="cuda")
    iters = {0: 4000, 1: 4000, 2: 2000, 3: 2000, 4: 20000, 5: 10000, 6: 10000}
    flops = {0: 16384, 1: 16384, 2: 32768, 3: 32768}
    clk = 2.4e9
    cases = {}
    for wps in (1, 2):
        for pat, name in enumerate(ops.ISSUE_RATE_PATTERNS):
            n = iters[pat]
            for _ in range(max(1, args.warmup // 10)):
                ops.issue_rate_bench(pat, wps, max(1, n // 10), sink)
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(3)]
            for e in ev:
                e[0].record()
                ops.issue_rate_bench(pat, wps, n, sink)
                e[1].record()
            torch.cuda.synchronize()
            ms = min(e[0].elapsed_time(e[1]) for e in ev)
            waves = cus * 4 * wps
            insts = waves * n * 16  # per pattern instruction (EXP: each v_exp_f32 with its v_add_f32)
            key = f"{name}_wps{wps}"
            rec = {"case": key, "ms": round(ms, 4), "instructions": insts}
            if pat in flops:
                rec["tflops"] = round(insts * flops[pat] / (ms / 1e3) / 1e12, 1)
                rec["frac_of_bf16_peak"] = round(rec["tflops"] / PEAK_BF16_TFLOPS, 4)
            elif pat in (4, 5):
                # one SIMD's instructions per cycle, all its waves together
                per_simd = insts / (cus * 4)
                rec["cycles_per_instruction_per_simd"] = round((ms / 1e3) * clk / per_simd, 2)
            else:
                nbytes = insts * 64 * 16
                rec["lds_bytes_per_cycle_per_cu"] = round(nbytes / (ms / 1e3) / clk / cus, 1)
            cases[key] = rec
            print(json.dumps(rec), flush=True)
    head = cases["mfma_32x32x16_bf16_4acc_wps1"]
    out = {"metric": ISSUE_RATE_METRIC, "value": head["tflops"], "unit": "TFLOP/s", "n_gpus": 1, "steps": 3,
           "warmup": args.warmup, "ms_per_step": head["ms"], "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "issue_rates", "compute_units": cus, "grid": "one workgroup per CU",
                      "instructions_per_wave_and_iteration": 16},
           "frac_of_peak": head["frac_of_bf16_peak"],
           "roofline": {"bound": "mfma", "achieved": head["tflops"], "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                        "frac": head["frac_of_bf16_peak"], "traffic": None, "kernel": "rate_mfma32"},
           "cases": cases}
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="untimed run of the step before the warmup steps, in ms of wall time (0: none)")
    ap.add_argument("--config", default="llama3_8b_decode")
    ap.add_argument("--partition-size", type=int, default=-1,
                    help="0 = the library's balanced split; default: the workload's own (512 for long_context)")
    ap.add_argument("--replicas", type=int, default=0, help="pool copies in rotation (0 = enough for >= 2 GiB of KV)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB")
    ap.add_argument("--summarize-profile", metavar="PREFIX", help="summarize rocprofv3 csv runs <PREFIX>_trace, "
                    "_fetch, _write, _cal_fetch, _cal_write into profiles/ (no GPU needed)")
    ap.add_argument("--profile-copy-mib", type=int, default=1024)
    ap.add_argument("--profile-commands", default="")
    ap.add_argument("--no-compare", action="store_true",
                    help="run only the measured form of the step (for profiles: the kernel counts one form)")
    ap.add_argument("--no-long-context", action="store_true",
                    help="skip the long_context record the default Llama-3-8B run carries beside its own")
    ap.add_argument("--cold", action="store_true",
                    help="also time each decode launch after a 512 MiB write that flushes L2 and the Infinity Cache")
    ap.add_argument("--vector-alu", action="store_true",
                    help="also time the bf16 decode with every product on the vector ALU (a measurement aid)")
    ap.add_argument("--identity-table", action="store_true",
                    help="also time the decode on the same tokens laid out with identity block tables")
    ap.add_argument("--two-call", action="store_true",
                    help="measure the two-call step (reshape_and_cache, then paged_attention_decode) where the fused "
                         "one applies")
    ap.add_argument("--fused", action="store_true",
                    help="(default where it applies) measure the fused step (paged_attention_decode_append: the cache "
                         "write inside the decode "
                         "launch) where it applies")
    args = ap.parse_args()

    if args.summarize_profile:
        # the partition the bench resolves for this workload (its own default
        # when --partition-size is not given: 512 for the long contexts)
        ps = args.partition_size
        if ps < 0:
            ps = 512 if args.config in ("long_context", "long_context_fp8") else 0
        ps = ps if ps > 0 else "balanced"
        if family(args.config) != "decode":
            ps = "none"
        fused = args.config in FUSABLE_CONFIGS and not args.two_call
        tag = "_fused" if fused else ""
        summarize_profile(args.summarize_profile, args.config, ps, args.profile_copy_mib,
                          os.path.join(ROOT, "profiles", f"{family(args.config)}_{args.config}{tag}.md"),
                          traffic_file(args.config, fused),
                          open(args.profile_commands).read() if args.profile_commands else "", fused)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from paged_kv_cache_372_amd import ops
    from paged_kv_cache_372_amd.blocks import tables_share_blocks

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    ops.load_library()
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy, max(1, args.steps))
        return

    if args.config == "hbm_read":
        run_hbm_read(args)
        return
    if args.config == "issue_rates":
        run_issue_rates(args)
        return
    if family(args.config) == "prefill":
        run_prefill(args)
        return
    if family(args.config) == "copy":
        run_copy(args)
        return

    rec = run_decode(args, args.config, args.partition_size, args.steps, args.warmup, not args.two_call,
                     not args.no_compare, args.identity_table, args.cpu_budget, args.vector_alu)
    if args.config == "llama3_8b_decode" and args.partition_size < 0 and not args.no_long_context:
        # the second configuration with a bandwidth target: 8 x 128k tokens,
        # 64 q / 8 KV heads, split-K at partition 512, on the same clock
        import gc
        import torch
        gc.collect()
        torch.cuda.empty_cache()
        lc = run_decode(args, "long_context", 512, args.steps, args.warmup, not args.two_call, True, False,
                        args.cpu_budget)
        keep = ("value", "unit", "ms_per_step", "step_ms_median", "step_ms_p10", "step_ms_p90", "frac_of_peak",
                "host_enqueue_ms_per_step", "two_call", "fused", "host_pack_h2d_ms", "tokens_per_s_with_host",
                "tokens_per_s", "decode_kernel_ms", "decode_kernel_ms_median", "roofline", "step", "config",
                "cpu_baseline", "input_generation_s")
        rec["long_context"] = {k: lc[k] for k in keep if k in lc}
    print(json.dumps(rec), flush=True)


def identity_layout(b):
    """The same cached tokens re-laid so that each sequence's blocks are
    consecutive physical blocks in table order (an identity block table per
    sequence, offset by the blocks of the sequences before it), plus one NaN
    block at the end for table padding.  Returns (block_map, tables, slots):
    new pool block i holds old block block_map[i]."""
    import numpy as np
    lens = np.asarray(b.context_lens, dtype=np.int64)
    nblk = -(-lens // b.block_size)
    off = np.concatenate([[0], np.cumsum(nblk)])
    T = int(off[-1])
    block_map = np.empty(T + 1, dtype=np.int64)
    tables = np.full(b.block_tables.shape, T, dtype=np.int32)
    for s in range(b.num_seqs):
        n = int(nblk[s])
        block_map[off[s]:off[s] + n] = b.block_tables[s, :n]
        tables[s, :n] = np.arange(off[s], off[s] + n, dtype=np.int32)
    block_map[T] = b.pad_block if b.pad_block >= 0 else int(b.block_tables[0, 0])
    pos = lens - 1
    slots = (tables[np.arange(b.num_seqs), pos // b.block_size].astype(np.int64) * b.block_size
             + pos % b.block_size)
    return block_map, tables, slots


def run_decode(args, config, partition_arg, steps, warmup, fused_flag, compare_forms, identity, cpu_budget,
               vector_alu=False):
    """One decode workload: K timed steps of the whole hot path, then the
    decode launch by events, a per-step event pass for the median and spread,
    and the CPU oracle on a bounded sample.  Returns the bench record."""
    import numpy as np
    import torch
    from paged_kv_cache_372_amd import ops
    from paged_kv_cache_372_amd.blocks import tables_share_blocks

    t_gen = time.perf_counter()
    b, batching_steps = build_workload(config, partition_arg)
    gen_s = time.perf_counter() - t_gen
    fp8 = b.dtype == "fp8"
    dtype = torch.float32 if b.dtype == "f32" else torch.bfloat16   # q / out (bf16 over an fp8 cache)
    pool_dtype = torch.uint8 if fp8 else dtype

    def dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:      # bf16 bit patterns
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()

    def ints(a):
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    # The inputs of every distinct step, resident on the GPU: one for a
    # static batch, ten for the continuous-batching run (cycled in order).
    if batching_steps is None:
        host_steps = [(b.k_new, b.v_new, b.slot_mapping, b.q, b.block_tables, b.context_lens)]
    else:
        host_steps = [(st.k_write, st.v_write, st.slot_mapping, st.q, st.block_tables, st.context_lens)
                      for st in batching_steps]
    es = {"bf16": 2, "f32": 4, "fp8": 1}[b.dtype]
    step_kv = [int(np.asarray(h[5], dtype=np.int64).sum()) * 2 * b.num_kv_heads * b.head_dim * es for h in host_steps]
    kv_bytes = sum(step_kv) / len(step_kv)  # per step, averaged over the distinct steps
    pool_bytes = b.k_pool.nbytes + b.v_pool.nbytes
    # pool copies in rotation, so that no step reads what a recent step left
    # in the 256 MB Infinity Cache (a continuous-batching step reads > 1 GB)
    R = args.replicas or (1 if batching_steps is not None else max(2, math.ceil(2 * 2**30 / max(1, kv_bytes))))
    k0, v0 = dev(b.k_pool), dev(b.v_pool)
    kcs = [k0] + [k0.clone() for _ in range(R - 1)]
    vcs = [v0] + [v0.clone() for _ in range(R - 1)]
    ps = b.partition_size if partition_arg < 0 else partition_arg
    gpu_steps = []
    for (kw, vw, sm, qh, bth, lh) in host_steps:
        q = dev(qh)
        gpu_steps.append(dict(k_new=dev(kw), v_new=dev(vw), slots=ints(sm), q=q, bt=ints(bth), lens=ints(lh),
                              max_ctx=int(np.max(lh)), out=torch.empty(q.shape, dtype=dtype, device="cuda"),
                              shared=tables_share_blocks(bth, lh, b.block_size)))
    ws_bytes = max(ops.decode_workspace_bytes(b.num_seqs, b.num_q_heads, b.num_kv_heads, b.head_dim, g["max_ctx"], ps,
                                              pool_dtype) for g in gpu_steps)
    if fp8:
        k_scale = torch.from_numpy(np.asarray(b.info["k_scale"], dtype=np.float32)).cuda()
        v_scale = torch.from_numpy(np.asarray(b.info["v_scale"], dtype=np.float32)).cuda()
    else:
        k_scale = v_scale = None
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    n_in = len(gpu_steps)
    plans = {}
    for j, g in enumerate(gpu_steps):
        for r in range(R):
            plans[j, r] = ops.prepare_decode(g["q"], kcs[r], vcs[r], g["bt"], g["lens"], b.scale, g["out"],
                                             partition_size=ps, max_context_len=g["max_ctx"], workspace=ws,
                                             shared_blocks=g["shared"], k_scale=k_scale, v_scale=v_scale)
    resolved_ps = ps if ps else ("auto" if b.dtype == "f32" else "balanced")

    # The fused step applies when each sequence gains exactly one token, into
    # a bf16 or fp8 cache at position L - 1 of its table (the static decode
    # workloads).
    def append_slots(bt, lens):
        lens = np.asarray(lens, dtype=np.int64)
        pos = lens - 1
        return np.asarray(bt, dtype=np.int64)[np.arange(len(lens)), pos // b.block_size] * b.block_size \
            + pos % b.block_size
    fusable = (b.dtype in ("bf16", "fp8") and b.num_q_heads // b.num_kv_heads <= 16 and
               all(len(h[2]) == len(h[5]) and int(np.min(h[5])) >= 1 and
                   np.array_equal(np.asarray(h[2], dtype=np.int64), append_slots(h[4], h[5])) for h in host_steps))
    fused = fusable and fused_flag
    compare = fusable and compare_forms
    fplans = {}
    if fusable:
        for j, g in enumerate(gpu_steps):
            for r in range(R):
                fplans[j, r] = ops.prepare_decode(g["q"], kcs[r], vcs[r], g["bt"], g["lens"], b.scale, g["out"],
                                                  partition_size=ps, max_context_len=g["max_ctx"], workspace=ws,
                                                  shared_blocks=g["shared"], k_scale=k_scale, v_scale=v_scale,
                                                  k_new=g["k_new"], v_new=g["v_new"])

    def step_two_call(i, ev=None):
        j, r = i % n_in, i % R
        g = gpu_steps[j]
        if fp8:
            ops.reshape_and_cache_fp8(g["k_new"], g["v_new"], g["slots"], kcs[r], vcs[r], k_scale, v_scale)
        else:
            ops.reshape_and_cache(g["k_new"], g["v_new"], g["slots"], kcs[r], vcs[r])
        if ev is not None:
            ev[0].record()
        ops.run_partitions(plans[j, r])
        if ev is not None:
            ev[1].record()
        ops.run_reduce(plans[j, r])

    def step_fused(i, ev=None):
        j, r = i % n_in, i % R
        if ev is not None:
            ev[0].record()
        ops.run_partitions(fplans[j, r])
        if ev is not None:
            ev[1].record()
        ops.run_reduce(fplans[j, r])

    step = step_fused if fused else step_two_call

    n_settle = [0]

    def settle_step():
        step(n_settle[0])
        if compare:
            (step_two_call if fused else step_fused)(n_settle[0])
        n_settle[0] += 1
    settle(settle_step, args.settle_ms)
    for i in range(warmup):
        step(i)
        if compare:
            (step_two_call if fused else step_fused)(i)
    torch.cuda.synchronize()

    # timed region 1: K whole steps, nothing but the kernels on the stream
    t0 = time.perf_counter()
    for i in range(steps):
        step(warmup + i)
    t_enq = time.perf_counter() - t0   # host time to enqueue the K steps
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    timed_kv = sum(step_kv[(warmup + i) % n_in] for i in range(steps))

    # the other form of the same steps, for comparison: wall time, then the
    # decode launch by events
    other_wall = other_dec = None
    if compare:
        other = step_two_call if fused else step_fused
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for i in range(steps):
            other(warmup + i)
        torch.cuda.synchronize()
        other_wall = time.perf_counter() - t1
        oev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        for i in range(steps):
            other(warmup + i, oev[i])
        torch.cuda.synchronize()
        other_dec = sum(e[0].elapsed_time(e[1]) for e in oev) / steps

    # timed region 2: the same K steps with HIP events around each decode
    # launch (on the launch stream), for the decode kernel's own duration
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        step(warmup + steps + i, events[i])
    torch.cuda.synchronize()
    dec_times = [e[0].elapsed_time(e[1]) for e in events]
    dec = sum(dec_times) / steps
    dec_kv = sum(step_kv[(warmup + steps + i) % n_in] for i in range(steps))
    ms_per_step = wall / steps * 1e3
    value = timed_kv / wall / 1e9
    achieved = dec_kv / (sum(dec_times) / 1e3) / 1e9
    traffic = measured_traffic(b.name, resolved_ps, fused)

    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "settle_ms": args.settle_ms,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if fp8 else b.dtype,   # an fp8 cache is decoded to bf16 for the products
        "data": "synthetic",
        "config": {"workload": b.name, "seed": b.seed, "num_seqs": b.num_seqs, "num_q_heads": b.num_q_heads,
                   "num_kv_heads": b.num_kv_heads, "head_dim": b.head_dim, "block_size": b.block_size,
                   "context_len_mean": round(float(b.context_lens.mean()), 1),
                   "context_len_max": b.max_context_len, "partition_size": resolved_ps,
                   "kv_bytes_per_step": int(round(kv_bytes)), "distinct_steps": n_in, "pool_bytes": pool_bytes,
                   "pool_replicas": R, "shared_blocks": any(g["shared"] for g in gpu_steps),
                   "kv_dtype": "fp8_e4m3" if fp8 else b.dtype},
        "step": "fused append + decode + reduce" if fused else "cache write + decode + reduce",
        "frac_of_peak": round(value / PEAK_HBM_GBS, 4),
        "tokens_per_s": round(b.num_seqs / (ms_per_step / 1e3), 1),
        "decode_kernel_ms": round(dec, 5),
        "host_enqueue_ms_per_step": round(t_enq / steps * 1e3, 5),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                     "kernel": "decode_valu_kernel" if b.dtype == "f32" else "decode_bf16_balanced_kernel",
                     "bytes_per_launch": int(round(kv_bytes))},
        "input_generation_s": round(gen_s, 2),
    }
    if other_wall is not None:
        key = "two_call" if fused else "fused"
        rec[key] = {"ms_per_step": round(other_wall / steps * 1e3, 5),
                    "value": round(timed_kv / other_wall / 1e9, 2),
                    "decode_kernel_ms": round(other_dec, 5)}
    # per-step spread: each whole step bracketed by events (the timed region
    # above has no events in it)
    sev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        sev[i][0].record()
        step(warmup + 2 * steps + i)
        sev[i][1].record()
    torch.cuda.synchronize()
    step_times = sorted(e[0].elapsed_time(e[1]) for e in sev)
    rec["step_ms_median"] = round(float(np.median(step_times)), 5)
    rec["step_ms_p10"] = round(float(np.percentile(step_times, 10)), 5)
    rec["step_ms_p90"] = round(float(np.percentile(step_times, 90)), 5)
    rec["decode_kernel_ms_median"] = round(float(np.median(dec_times)), 5)
    if args.cold:
        # each decode launch after a 512 MiB write that evicts L2 and the
        # Infinity Cache: cold caches, against the warm rotation above
        flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        cev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        torch.cuda.synchronize()
        for i in range(steps):
            flush.fill_(i & 0xFF)
            step(warmup + 3 * steps + i, cev[i])
        torch.cuda.synchronize()
        ct = [e[0].elapsed_time(e[1]) for e in cev]
        rec["cold"] = {"decode_kernel_ms": round(sum(ct) / steps, 5),
                       "decode_kernel_ms_median": round(float(np.median(ct)), 5),
                       "flush_bytes": 512 << 20,
                       "kv_gbs": round(kv_bytes / (sum(ct) / steps / 1e3) / 1e9, 2)}
        del flush
    if vector_alu and b.dtype == "bf16" and batching_steps is None:
        rec["vector_alu"] = vector_alu_comparison(b, kcs, vcs, gpu_steps[0], ps, plans, steps, warmup)
    if identity and batching_steps is None:
        rec["identity_table"] = identity_table_comparison(b, kcs, vcs, gpu_steps[0], ps, steps, warmup, dec)
    try:
        rec["host_pack_h2d_ms"] = round(host_pack_ms(b), 4)
        # with the host's packing and copies done before each step and not
        # overlapped with the GPU (the serial case)
        rec["tokens_per_s_with_host"] = round(b.num_seqs / ((ms_per_step + rec["host_pack_h2d_ms"]) / 1e3), 1)
    except Exception as e:  # aux figure only
        rec["host_pack_h2d_ms"] = f"unavailable: {e}"
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(b, cpu_budget)
    return rec


if __name__ == "__main__":
    main()
