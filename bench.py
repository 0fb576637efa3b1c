#!/usr/bin/env python3
"""Benchmark of paged single-token decode attention on one MI355X.

One step = one decode call over every sequence of one layer (one kernel
launch: a persistent grid that splits the batch's tiles evenly over its waves
and merges shared sequences in-kernel), on synthetic inputs already resident
in HBM.  Layers are rotated
(distinct pool buffers with the same contents) so the 256 MB Infinity Cache
cannot serve a layer from the previous step.

Prints ONE JSON line: value = algorithmic HBM bytes per step / time per step
(GB/s), with the roofline of the decode kernel (timed with HIP events on the
stream it runs on) and the fp64 oracle timed on this host's cores as a
baseline.

    python bench.py [--steps K] [--warmup W] [--config NAME]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
COPY_CALIBRATION_MIB = 1024   # size of the plain copy the counters are calibrated on
WARMUP_SECONDS = 1.0          # minimum untimed warm-up after the W warm-up steps
DEFAULT_CONFIG = "llama3_8b_gqa"


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default=None,
                    help="one decode workload (default: every decode workload, headline first, in one line)")
    ap.add_argument("--flush-check", action="store_true",
                    help="with --config: also time one layer with a 512 MiB scratch write between launches")
    ap.add_argument("--graph", action="store_true",
                    help="with --config: also time the launches replayed from a HIP graph")
    ap.add_argument("--num-splits", type=int, default=0,
                    help="waves sharing the batch's tiles (0 = library default)")
    ap.add_argument("--rotate", type=int, default=0,
                    help="distinct layer buffers cycled through (0 = enough for >= 1 GB of KV)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--stream-reference", action="store_true",
                    help="time a plain 2 GiB device copy and a read-only reduction (HBM reference)")
    ap.add_argument("--op", choices=["decode", "append", "serve", "prefill"], default="decode",
                    help="decode: the decode step (default); append: write every token of the workload "
                         "into the pools with pkv_write_kv (quantising f16/bf16 rows for int8/fp8 pools); "
                         "serve: the continuous-batching loop (scheduler step, K/V appends, decode of the "
                         "mixed batch) over a backlog of requests of the workload's shape; prefill: one "
                         "chunked-prefill step (a 512-token chunk per sequence) of the workload's shape")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum wall time of the oracle baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of COPY_CALIBRATION_MIB MiB (counter calibration)")
    ap.add_argument("--summarize-counters", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV",
                                                              "COPY_WRITE_CSV"),
                    help="turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE counter CSVs of this benchmark and "
                         "of the copy calibration into profiles/paged_decode_<config>_counters.json")
    ap.add_argument("--sq-counters", nargs="*", metavar="CSV", default=[],
                    help="with --summarize-counters: further rocprofv3 --pmc CSVs of the same workload (SQ_*, "
                         "GRBM_* and derived counters such as VALUBusy), averaged per decode dispatch")
    return ap.parse_args()


def source_digest() -> str:
    h = hashlib.sha256()
    for f in ("decode.hip", "api.cpp"):
        with open(os.path.join(ROOT, "paged_kv_cache_266_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile(workload: str):
    """HBM bytes per launch of the partition kernel from the committed counter
    summary, or None when there is none or the kernel source changed since."""
    path = os.path.join(ROOT, "profiles", f"paged_decode_{workload}_counters.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_digest") != source_digest():
        return None
    return rec.get("hbm_bytes_per_launch")


def decode_kernel_name(workload: str) -> str:
    from synth import CONFIGS

    cfg = CONFIGS[workload]
    return "paged_decode_fp8_mfma_kernel" if cfg.kv_dtype == "fp8" and cfg.head_dim == 128 \
        else "paged_decode_kernel"


def _counter_rows(path, counter):
    import csv

    with open(path, newline="") as f:
        return [r for r in csv.DictReader(f) if r["Counter_Name"] == counter]


def _per_dispatch(rows, match):
    """Counter value (KiB) per dispatch of kernels whose name contains match."""
    vals = {}
    for r in rows:
        if match in r["Kernel_Name"]:
            vals[r["Dispatch_Id"]] = vals.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return list(vals.values())


def summarize_counters(workload: str, files, copy_bytes: int) -> dict:
    """HBM bytes per launch of the decode kernel (paged_decode_kernel, or
    paged_decode_fp8_mfma_kernel) from FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch), each divided by what the same counter reads per byte for a
    plain device copy of copy_bytes bytes."""
    fetch_csv, write_csv, cfetch_csv, cwrite_csv = files
    fetch = _per_dispatch(_counter_rows(fetch_csv, "FETCH_SIZE"), "paged_decode_")
    write = _per_dispatch(_counter_rows(write_csv, "WRITE_SIZE"), "paged_decode_")
    # the copy kernel is the largest dispatch of the calibration run
    cf = max(_per_dispatch(_counter_rows(cfetch_csv, "FETCH_SIZE"), ""))
    cw = max(_per_dispatch(_counter_rows(cwrite_csv, "WRITE_SIZE"), ""))
    f_factor = cf * 1024 / copy_bytes
    w_factor = cw * 1024 / copy_bytes
    fetch_b = sum(fetch) / len(fetch) * 1024 / f_factor
    write_b = sum(write) / len(write) * 1024 / w_factor
    return {
        "workload": workload,
        "kernel": decode_kernel_name(workload),
        "source_digest": source_digest(),
        "dispatches": {"fetch": len(fetch), "write": len(write)},
        "fetch_kib_per_dispatch": round(sum(fetch) / len(fetch), 1),
        "write_kib_per_dispatch": round(sum(write) / len(write), 1),
        "copy_bytes": copy_bytes,
        "copy_factor": {"fetch": round(f_factor, 4), "write": round(w_factor, 4)},
        "hbm_fetch_bytes_per_launch": int(fetch_b),
        "hbm_write_bytes_per_launch": int(write_b),
        "hbm_bytes_per_launch": int(fetch_b + write_b),
    }


def summarize_sq(files) -> dict:
    """Per-dispatch means of every counter in the given rocprofv3 --pmc CSVs
    for the decode kernel's dispatches, and the ratios read from them: the
    fraction of wave cycles spent waiting for an instruction's operands
    (SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES), vector-ALU and vector-memory
    instructions per wave, and the matrix-core instruction count."""
    import csv

    sums, counts = {}, {}
    for path in files:
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                if "paged_decode_" not in r["Kernel_Name"]:
                    continue
                k = r["Counter_Name"]
                sums[k] = sums.get(k, 0.0) + float(r["Counter_Value"])
                counts[k] = counts.get(k, 0) + 1
    mean = {k: sums[k] / counts[k] for k in sums}
    out = {"per_dispatch_mean": {k: round(v, 3) for k, v in sorted(mean.items())},
           "dispatches": {k: counts[k] for k in sorted(counts)}}
    waves = mean.get("SQ_WAVES")
    ratios = {}
    if "SQ_WAIT_INST_ANY" in mean and mean.get("SQ_WAVE_CYCLES"):
        ratios["wait_inst_any_over_wave_cycles"] = round(mean["SQ_WAIT_INST_ANY"] / mean["SQ_WAVE_CYCLES"], 4)
    if waves:
        for k in ("SQ_INSTS_VALU", "SQ_INSTS_VMEM_RD", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU"):
            if k in mean:
                ratios[k.lower().replace("sq_insts_", "insts_") + "_per_wave"] = round(mean[k] / waves, 1)
    out["ratios"] = ratios
    return out


def copy_calibration(mib: int) -> None:
    import torch

    n = mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)


def stream_reference(mib: int, reps: int = 20) -> None:
    """What plain streams reach on this GPU, as a practical reference for the
    HBM roofline: a device-to-device copy (bytes read + written) and a
    read-only reduction (torch's sum of a bf16 buffer into fp32), timed with
    HIP events over `reps` launches each."""
    import torch

    n = mib * (1 << 20)
    src = torch.ones(n // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    res = {}
    for name, fn, moved in (("copy", lambda: dst.copy_(src), 2 * n),
                            ("read (sum)", lambda: torch.sum(src, dtype=torch.float32), n)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        res[name] = {"us": round(us, 1), "GB/s": round(moved / (us * 1e-6) / 1e9, 1)}
    print(json.dumps({"stream_reference_bytes": n, "results": res}), flush=True)


def cpu_baseline(case, min_seconds: float, got, tol: float):
    """The cpu_baseline leg: the fp64 oracle on the whole workload, timed on
    this host's cores.  Its first (untimed) pass also gives the reference
    output that the GPU's first launch is checked against (the parity of the
    benchmarked launch configuration)."""
    import numpy as np
    import oracle

    threads = oracle.default_threads()
    ref = oracle.paged_decode(case, n_threads=threads)    # warm-up, and the parity reference
    max_err = float(np.abs(got - ref).max())
    parity = {"max_abs_err": max_err, "tol": tol, "ok": bool(max_err <= tol)}
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.paged_decode(case, n_threads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return parity, {
        "value": round(case.bytes_alg() * reps / el / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"the whole {case.cfg.name} workload (seed {case.seed}), "
                  f"{reps} fp64 layer-steps in {el:.1f} s, {el / reps * 1e6:.0f} us per layer-step; "
                  f"{cpu_model}",
    }


def cpu_baseline_append(rows_f32, kind: str, got_codes, got_scales, min_seconds: float):
    """The cpu_baseline leg of the append benchmark: the oracle's quantiser
    over every appended row (its first pass is also the parity reference:
    codes and scales must match bit for bit), timed on this host."""
    import numpy as np
    import oracle

    codes, sc = oracle.quantize_rows(rows_f32, kind)
    parity = {"rows": int(sc.size), "bit_exact": bool(
        np.array_equal(np.asarray(got_codes).view(np.uint8), codes.view(np.uint8))
        and np.array_equal(np.asarray(got_scales).view(np.uint32), sc.view(np.uint32)))}
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.quantize_rows(rows_f32, kind)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    moved = rows_f32.size * (2 + 1) + sc.size * 4
    return parity, {"value": round(moved * reps / el / 1e9, 4), "unit": "GB/s", "cores": 1,
                    "kind": "oracle", "sample": f"{sc.size} rows of one pool (K), {reps} passes in {el:.1f} s"}


def bench_append(args) -> None:
    """Throughput of pkv_write_kv over a whole workload's tokens (a prefill's
    worth of K/V, every KV head): rows in the query type, quantised on the
    device when the pool is int8 / fp8, else copied.  Also times
    pkv_copy_pages (the copy-on-write page copy) over a batch of pages."""
    import numpy as np
    import torch

    import paged_kv_cache_266_amd as pkv
    from synth import CONFIGS
    from synth.device import torch_dtype
    from synth.make import _to_bits, draw_context_lens

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    cfg = CONFIGS[args.config]
    rng = np.random.default_rng(cfg.seed)
    lens = draw_context_lens(cfg, rng)
    n = int(lens.sum())
    Hkv, D, PS = cfg.num_kv_heads, cfg.head_dim, cfg.page_size
    src_t, kv_t = cfg.q_dtype, cfg.kv_dtype
    byte = kv_t in ("i8", "fp8")
    if not byte and kv_t != src_t:
        raise SystemExit("a 16-bit pool takes rows of its own type")
    e = 1 if byte else 2
    dev = "cuda"
    with pkv.KVPool(cfg.num_pages, PS, initial_free_order=rng.permutation(cfg.num_pages)) as pool:
        slots = np.concatenate([pool.allocate(b, int(m)) for b, m in enumerate(lens)])
    bits = [_to_bits(rng.standard_normal((n, Hkv, D)).astype(np.float32), src_t) for _ in range(2)]
    new = [torch.from_numpy(b.view(np.int16)).view(torch_dtype(src_t)).to(dev) for b in bits]
    shape = (cfg.num_pages, Hkv, PS, D)
    if byte:
        pools = [torch.zeros(shape, dtype=torch.uint8, device=dev).view(torch_dtype(kv_t)) for _ in range(2)]
        scales = [torch.zeros(shape[:3], dtype=torch.float32, device=dev) for _ in range(2)]
    else:
        pools = [torch.zeros(shape, dtype=torch_dtype(kv_t), device=dev) for _ in range(2)]
        scales = [None, None]
    slots_d = torch.from_numpy(slots).to(dev)
    stream = torch.cuda.current_stream()

    def step():
        pkv.write_kv(new[0], new[1], slots_d, pools[0], pools[1], k_scale=scales[0], v_scale=scales[1])

    step()
    torch.cuda.synchronize()
    pg, off = slots // PS, slots % PS
    got = [p.view(torch.uint8 if byte else torch.int16).cpu().numpy()[pg, :, off, :] for p in pools]
    parity, baseline = None, None
    if byte:
        if not args.no_cpu_baseline:
            rows = ((bits[0].astype(np.uint32) << 16).view(np.float32) if src_t == "bf16"
                    else bits[0].view(np.float16).astype(np.float32))
            parity, baseline = cpu_baseline_append(rows, kv_t, got[0], scales[0].cpu().numpy()[pg, :, off],
                                                   args.cpu_seconds)
    else:
        parity = {"rows": n * Hkv * 2, "bit_exact": bool(all(
            np.array_equal(g.view(np.uint16), b) for g, b in zip(got, bits)))}
    del got

    def timed(fn, steps):
        fn()
        t_w = time.perf_counter()
        while time.perf_counter() - t_w < WARMUP_SECONDS:
            fn()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        t0 = time.perf_counter()
        ev[0].record(stream)
        for _ in range(steps):
            fn()
        ev[1].record(stream)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps, ev[0].elapsed_time(ev[1]) / steps

    ms, ev_ms = timed(step, args.steps)
    moved = 2 * n * Hkv * D * (2 + e) + (2 * n * Hkv * 4 if byte else 0)

    # page copies: the used pages' first half copied onto free pages
    used = np.unique(pg)
    free = np.setdiff1d(np.arange(cfg.num_pages), used)
    ncopy = int(min(len(used), len(free), 4096))
    pairs = torch.from_numpy(np.stack([used[:ncopy], free[:ncopy]], 1).astype(np.int32)).to(dev)

    def copy_step():
        pkv.copy_pages(pairs, pools[0], pools[1], k_scale=scales[0], v_scale=scales[1])

    copy_step()
    torch.cuda.synchronize()
    src_i, dst_i = pairs[:, 0].long(), pairs[:, 1].long()
    copy_ok = all(bool(torch.equal(t[dst_i], t[src_i]))
                  for t in [p.view(torch.uint8) for p in pools] + [x for x in scales if x is not None])
    cms, cev_ms = timed(copy_step, args.steps)
    page_bytes = Hkv * PS * D * e + (Hkv * PS * 4 if byte else 0)
    cmoved = 2 * 2 * ncopy * page_bytes

    rec = {
        "metric": "K/V append (pkv_write_kv) HBM GB/s (% of 8 TB/s peak)",
        "value": round(moved / (ms * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "dtype": f"{src_t}->{kv_t}", "data": "synthetic",
        "config": {"workload": f"append_{cfg.name}", "tokens": n, "num_kv_heads": Hkv, "head_dim": D,
                   "page_size": PS, "bytes_alg_per_step": moved, "quantise": byte},
        "pct_of_peak": round(100 * moved / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 2),
        "event_us": round(ev_ms * 1e3, 2),
        "parity": parity,
        "copy_pages": {"pages": ncopy, "bytes_alg": cmoved, "us": round(cms * 1e3, 2),
                       "event_us": round(cev_ms * 1e3, 2),
                       "GB/s": round(cmoved / (cms * 1e-3) / 1e9, 2), "bit_exact": copy_ok},
    }
    if baseline is not None:
        rec["cpu_baseline"] = baseline
    print(json.dumps(rec), flush=True)


def bench_serve(args) -> None:
    """The serving loop over one layer's pools, one native call per step
    (pkv_serve_step): the scheduler step (retire, admit, one token per
    running sequence), the staging of its slots, context lengths and block
    tables, the admitted prompts' and the new tokens' K/V appends, and the
    decode of the mixed batch.  Requests: a backlog whose prompt lengths
    follow the workload's length law and which generate 32..256 tokens each
    (uniform, 144 on average), all arrived at step 0, at most `batch`
    running; batch x (steps / 144 + 4) requests, so that the batch stays full
    through the warm-up and both timed passes.  K steps are timed after W warm-up steps: once as issued (the
    host runs ahead of the GPU), once with HIP events around each step's
    device work, which give the GPU's busy time per step and the gaps between
    steps."""
    import numpy as np
    import torch

    import paged_kv_cache_266_amd as pkv
    from synth import CONFIGS
    from synth.device import torch_dtype
    from synth.make import draw_context_lens

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    cfg = CONFIGS[args.config]
    rng = np.random.default_rng(cfg.seed)
    B, Hq, Hkv, D, PS = cfg.batch, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.page_size
    byte = cfg.kv_dtype in ("i8", "fp8")
    src_t = cfg.q_dtype if byte else cfg.kv_dtype
    rounds = -(-(args.warmup + 2 * args.steps) // 144) + 4
    n_req = rounds * B
    prompts = np.concatenate([draw_context_lens(cfg, rng) for _ in range(rounds)])[:n_req]
    new_tok = rng.integers(32, 257, size=n_req)
    cap = int(prompts.max() + new_tok.max())
    max_blocks = -(-cap // PS)
    dev = "cuda"
    shape = (cfg.num_pages, Hkv, PS, D)
    if byte:
        pools = [torch.zeros(shape, dtype=torch.uint8, device=dev).view(torch_dtype(cfg.kv_dtype)) for _ in range(2)]
        scales = [torch.zeros(shape[:3], dtype=torch.float32, device=dev) for _ in range(2)]
    else:
        pools = [torch.zeros(shape, dtype=torch_dtype(cfg.kv_dtype), device=dev) for _ in range(2)]
        scales = [None, None]
    gen = torch.Generator(device=dev)
    gen.manual_seed(cfg.seed)
    # every admitted prompt's rows come from one buffer of the largest
    # step's size (all B sequences admitted at once with the longest prompt)
    max_prompt_tokens = B * int(prompts.max())
    rows_prompt = [torch.randn((max_prompt_tokens, Hkv, D), generator=gen, device=dev).to(torch_dtype(src_t))
                   for _ in range(2)]
    rows_new = [torch.randn((B, Hkv, D), generator=gen, device=dev).to(torch_dtype(src_t)) for _ in range(2)]
    q = torch.randn((B, Hq, D), generator=gen, device=dev).to(torch_dtype(cfg.q_dtype))
    pool = pkv.KVPool(cfg.num_pages, PS, initial_free_order=rng.permutation(cfg.num_pages))
    sch = pkv.Scheduler(pool, B, pkv.CONTINUOUS)
    for i in range(n_req):
        sch.submit(i, int(prompts[i]), int(new_tok[i]), 0)
    stream = torch.cuda.current_stream()
    loop = pkv.ServeLoop(sch, q, pools[0], pools[1], cfg.scale, k_new=rows_new[0], v_new=rows_new[1],
                         k_prompt=rows_prompt[0], v_prompt=rows_prompt[1], max_blocks=max_blocks,
                         k_scale=scales[0], v_scale=scales[1], ring=8, stream=stream)
    e_kv = 1 if byte else 2
    for _ in range(args.warmup):
        loop.step()
    torch.cuda.synchronize()

    # Python's collector stays off while the steps are issued (a collection
    # would show as a gap between steps that the loop itself does not cause);
    # the event pairs of pass 2 are made beforehand for the same reason
    import gc

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    gc_on = gc.isenabled()
    gc.disable()
    try:
        # pass 1: as issued
        tokens = 0
        t0 = time.perf_counter()
        host = wait = 0.0
        for _ in range(args.steps):
            h0 = time.perf_counter()
            r = loop.step()
            host += time.perf_counter() - h0
            wait += r.slot_wait_us * 1e-6
            tokens += r.sched.n_running
        t_issue = time.perf_counter() - t0
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        # pass 2: events around each step's device work
        for ev in evs:
            ev[0].record(stream)
            loop.step()
            ev[1].record(stream)
        torch.cuda.synchronize()
    finally:
        if gc_on:
            gc.enable()
    busy = [e[0].elapsed_time(e[1]) * 1e3 for e in evs]
    gaps = [a_[1].elapsed_time(b_[0]) * 1e3 for a_, b_ in zip(evs, evs[1:])]
    st_ = sch.stats()
    loop.close()
    sch.close()
    pool.close()
    print(json.dumps({
        "metric": "continuous-batching decode loop, sequences decoded per second (one layer)",
        "value": round(tokens / el, 1), "unit": "sequence-steps/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(el * 1e3 / args.steps, 4), "higher_is_better": True,
        "dtype": cfg.kv_dtype, "data": "synthetic",
        "config": {"workload": f"serve_{cfg.name}", "max_batch": B, "requests": n_req,
                   "prompt_law": cfg.lens_kind, "new_tokens": "uniform 32..256", "page_size": PS,
                   "kv_bytes_per_token_per_layer": 2 * Hkv * D * e_kv},
        "avg_batch": round(tokens / args.steps, 2),
        "host_us_per_step": round((host - wait) * 1e6 / args.steps, 1),
        "host_slot_wait_us_per_step": round(wait * 1e6 / args.steps, 1),
        "host_issue_us_per_step": round(t_issue * 1e6 / args.steps, 1),
        # steps that admit requests also write their prompts, so the mean
        # sits above the median
        "gpu_busy_us_per_step": {"mean": round(float(np.mean(busy)), 2),
                                 "median": round(float(np.median(busy)), 2),
                                 "max": round(float(np.max(busy)), 2)},
        "gpu_idle_us_between_steps": {"mean": round(float(np.mean(gaps)), 2),
                                      "median": round(float(np.median(gaps)), 2),
                                      "p90": round(float(np.percentile(gaps, 90)), 2)},
        "scheduler": {"now": st_["now"], "finished": st_["finished"], "waiting": st_["waiting"]},
    }), flush=True)


PEAK_MFMA_TFLOPS_16BIT = 2500.0   # MI355X dense bf16 / f16


def bench_prefill(args) -> None:
    """One chunked-prefill step: every sequence of the workload processes a
    chunk of 512 new tokens at the end of its context (lengths from the
    workload's law, at least 512), the workload's K/V type.  FLOPs counted causally:
    4 * head_dim per (query row, query head, visible key).  The cpu_baseline
    leg runs the fp64 oracle on the last 64 rows of every chunk (16 for an
    E4M3 cache; about 10 s on 16 host cores), which is also the parity check
    of those rows."""
    import numpy as np
    import torch

    import paged_kv_cache_266_amd as pkv
    from synth import CONFIGS, make_case
    from synth.configs import get_config
    from synth.device import torch_dtype, upload
    from synth.make import _to_bits, draw_context_lens

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    base = CONFIGS[args.config]
    if base.head_dim != 128:
        raise SystemExit("prefill: head_dim 128 only")
    chunk = 512
    rng = np.random.default_rng(base.seed)
    lens = np.maximum(draw_context_lens(base, rng), chunk).astype(np.int32)
    cfg = get_config(base.name, lens_kind="fixed", lens_args=tuple(int(x) for x in lens))
    case = make_case(cfg)
    dev = upload(case, "cuda")
    B, Hq, D = cfg.batch, cfg.num_q_heads, cfg.head_dim
    qrng = np.random.default_rng(cfg.seed + 1)
    q_bits = _to_bits(qrng.standard_normal((B * chunk, Hq, D)).astype(np.float32), cfg.q_dtype)
    q = torch.from_numpy(q_bits.view(np.int16)).view(torch_dtype(cfg.q_dtype)).cuda()
    q_start = np.arange(0, B * chunk + 1, chunk, dtype=np.int32)
    qs = torch.from_numpy(q_start).cuda()
    out = torch.empty_like(q)

    def step():
        pkv.paged_prefill(q, dev.k_pool, dev.v_pool, dev.block_tables, qs, dev.context_lens, case.scale,
                          max_context_len=cfg.max_context_len, max_q_len=chunk, out=out,
                          k_scale=dev.k_scale, v_scale=dev.v_scale)

    step()
    torch.cuda.synchronize()
    got = out.to(torch.float64).cpu().numpy()
    tol = {"f16": 4e-3, "bf16": 1.6e-2, "i8": 2.5e-2, "fp8": 2.5e-2}[cfg.kv_dtype]
    parity, baseline = {"ok": None, "note": "not checked: --no-cpu-baseline"}, None
    if not args.no_cpu_baseline:
        import dataclasses

        import oracle

        # about 10 s of fp64 work on 16 cores (E4M3 decoding makes the oracle ~4x slower per row)
        nb, rows = B, 16 if cfg.kv_dtype == "fp8" else 64
        sub = dataclasses.replace(case, cfg=get_config(cfg.name, batch=nb, lens_kind="fixed",
                                                       lens_args=tuple(int(x) for x in lens[:nb])),
                                  context_lens=case.context_lens[:nb], block_tables=case.block_tables[:nb])
        sel = np.concatenate([np.arange(q_start[b + 1] - rows, q_start[b + 1]) for b in range(nb)])
        qs8 = np.arange(0, nb * rows + 1, rows, dtype=np.int32)
        threads = oracle.default_threads()
        t0 = time.perf_counter()
        ref = oracle.paged_prefill(sub, q_bits[sel], qs8, n_threads=threads)
        el = time.perf_counter() - t0
        err = float(np.abs(got[sel] - ref).max())
        parity = {"rows_checked": int(sel.size), "max_abs_err": err, "tol": tol, "ok": bool(err <= tol)}
        flops_s = 4.0 * D * Hq * sum(int(lens[b]) - rows + i + 1 for b in range(nb) for i in range(rows))
        baseline = {"value": round(flops_s / el / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
                    "sample": f"the last {rows} rows of each of the {nb} chunks, {el:.2f} s"}
    # causal FLOPs of the whole step
    flops = 0.0
    for b in range(B):
        n = int(lens[b])
        first = n - chunk + 1            # keys visible to the chunk's first row
        flops += 4.0 * D * Hq * (chunk * first + chunk * (chunk - 1) / 2)
    t_w = time.perf_counter()
    while time.perf_counter() - t_w < WARMUP_SECONDS:
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    kern_ms = e0.elapsed_time(e1) / args.steps
    achieved = flops / (kern_ms * 1e-3) / 1e12
    rec = {
        "metric": "chunked prefill attention TFLOP/s (causal), one layer",
        "value": round(flops / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "dtype": cfg.kv_dtype,
        "data": "synthetic",
        "config": {"workload": f"prefill_{cfg.name}", "batch": B, "chunk": chunk, "num_q_heads": Hq,
                   "q_dtype": cfg.q_dtype, "kv_dtype": cfg.kv_dtype,
                   "num_kv_heads": cfg.num_kv_heads, "head_dim": D, "page_size": cfg.page_size,
                   "context_tokens": int(lens.sum()), "flops_per_step": flops},
        "roofline": {"bound": "mfma", "kernel": "paged_prefill_kernel", "achieved": round(achieved, 2),
                     "peak": PEAK_MFMA_TFLOPS_16BIT, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_MFMA_TFLOPS_16BIT, 4), "traffic": None},
        "parity": parity,
    }
    if baseline is not None:
        rec["cpu_baseline"] = baseline
    print(json.dumps(rec), flush=True)


GATED = ("llama3_8b_gqa", "long_128k")     # >= 70 % of the HBM peak on one GPU
GATE_FRAC = 0.70
# the default run: the headline workload first, then the other gated one,
# the rest of the decode workloads, and the launch-bound tiny case
SUITE = ("llama3_8b_gqa", "long_128k", "llama2_7b_mha", "qwen_1p8b_int8", "llama3_8b_gqa_fp8", "tiny")
SECONDARY_CPU_SECONDS = 4.0                # oracle sample of each non-headline workload
FLUSH_MIB = 512                            # scratch written between launches in the cache-flush check
FLUSH_TOLERANCE = 0.03


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def decode_workload(name: str, args, cpu_seconds: float, flush_check: bool = False, graph: bool = False) -> dict:
    """Benchmark one decode workload: W warm-up steps, K timed steps (one
    library call, one kernel launch each) between synchronisations, layers
    rotated so that >= 1 GB of KV cycles.  Returns its record: wall time per
    step, the kernel's roofline (HIP events on the launch stream around the K
    launches), the parity of the first launch against the fp64 oracle and the
    oracle's own throughput on this host (cpu_seconds of work)."""
    import ctypes

    import numpy as np
    import torch

    import paged_kv_cache_266_amd as pkv
    from paged_kv_cache_266_amd._lib import check, lib
    from synth import CONFIGS, make_case
    from synth.device import upload

    L = lib()
    cfg = CONFIGS[name]
    t_set = time.perf_counter()
    case = make_case(cfg)
    bytes_alg = case.bytes_alg()

    # block tables through the library's own allocator, as a caller would
    with pkv.KVPool(cfg.num_pages, cfg.page_size, initial_free_order=case.free_order) as pool:
        for b, n in enumerate(case.context_lens):
            pool.allocate(b, int(n))
        bt, lens = pool.block_tables(list(range(cfg.batch)), cfg.max_blocks)
    assert (bt == case.block_tables).all() and (lens == case.context_lens).all()

    kv_bytes_layer = case.total_tokens * cfg.num_kv_heads * cfg.head_dim * 2 * \
        (1 if cfg.kv_dtype in ("i8", "fp8") else 2)
    rotate = args.rotate or max(1, -(-(1 << 30) // max(kv_bytes_layer, 1)))
    layers = [upload(case, "cuda") for _ in range(rotate)]
    q = layers[0].q
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    argv = []
    for dev in layers:
        a = pkv.decode_args(dev.q, dev.k_pool, dev.v_pool, dev.block_tables, dev.context_lens,
                            case.scale, max_context_len=cfg.max_context_len, out=out,
                            k_scale=dev.k_scale, v_scale=dev.v_scale,
                            num_splits=args.num_splits)
        argv.append(a)
    ws = pkv.alloc_workspace(argv[0], q.device)
    ctr = pkv.alloc_merge_counters(argv[0], q.device)
    for a in argv:
        a.workspace = 0 if ws is None else ws.data_ptr()
        a.workspace_bytes = 0 if ws is None else ws.numel()
        a.merge_counters = 0 if ctr is None else ctr.data_ptr()
        a.merge_counter_bytes = 0 if ctr is None else 4 * ctr.numel()
    num_splits = L.pkv_decode_num_splits(ctypes.byref(argv[0]))
    launch_bound = name == "tiny"

    def step(i):
        check(L.pkv_paged_attn_decode(ctypes.byref(argv[i % rotate]), sh))

    # the cpu_baseline leg (which also checks the first launch's output) runs
    # first: the oracle keeps the GPU idle for seconds, so it must not sit
    # between the warm-up and the timed region
    step(0)
    torch.cuda.synchronize()
    got = out.to(torch.float64).cpu().numpy()
    tol = {"f16": 4e-3, "bf16": 1.6e-2, "i8": 2.5e-2, "fp8": 2.5e-2}[cfg.kv_dtype]
    parity, baseline = {"ok": None, "note": "not checked: --no-cpu-baseline"}, None
    if not args.no_cpu_baseline:
        parity, baseline = cpu_baseline(case, cpu_seconds, got, tol)
    log(f"[{name}] set-up and oracle leg {time.perf_counter() - t_set:.1f} s")

    # W warm-up steps, then more (untimed) until the GPU has been busy for
    # WARMUP_SECONDS, so that clocks have settled before the timed region
    t_w = time.perf_counter()
    i = 0
    while i < args.warmup or time.perf_counter() - t_w < WARMUP_SECONDS:
        step(i)
        i += 1
        if i % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()

    # the timed region: K whole steps (one library call, one kernel launch
    # each), nothing else, bracketed by HIP events on the launch stream; their
    # span / K is the kernel's average duration for the roofline
    region = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    region[0].record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    region[1].record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    ms_per_step = wall_ms / args.steps
    value = bytes_alg / (ms_per_step * 1e-3) / 1e9
    launch_ms = region[0].elapsed_time(region[1]) / args.steps

    # a second pass of K steps with an event pair around each launch: the
    # spread of launch durations (each pair adds its own overhead, so these
    # read a little above the timed region's average)
    def per_launch_ms(n, between=None):
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]
        torch.cuda.synchronize()
        for k in range(n):
            if between is not None:
                between()
            evs[k][0].record(stream)
            step(args.warmup + args.steps + k)
            evs[k][1].record(stream)
        torch.cuda.synchronize()
        return np.array([e[0].elapsed_time(e[1]) for e in evs])

    kern_ms = per_launch_ms(args.steps)
    achieved = bytes_alg / (launch_ms * 1e-3) / 1e9
    rec = {
        "metric": "paged-attn decode HBM GB/s (% of 8 TB/s peak), us per layer-step",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.kv_dtype,
        "data": "synthetic",
        "config": {
            "workload": cfg.name,
            "batch": cfg.batch, "num_q_heads": cfg.num_q_heads, "num_kv_heads": cfg.num_kv_heads,
            "head_dim": cfg.head_dim, "page_size": cfg.page_size, "q_dtype": cfg.q_dtype,
            "kv_dtype": cfg.kv_dtype, "context_tokens": case.total_tokens,
            "max_context_len": cfg.max_context_len, "num_splits": num_splits,
            "layers_rotated": rotate, "seed": cfg.seed, "bytes_alg_per_step": bytes_alg,
        },
        "us_per_layer_step": round(ms_per_step * 1e3, 2),
        "pct_of_peak": round(100 * value / PEAK_HBM_GBPS, 2),
        "kernel_us_timed_region": round(launch_ms * 1e3, 2),
        "kernel_event_us": {
            "mean": round(float(kern_ms.mean()) * 1e3, 2),
            "median": round(float(np.median(kern_ms)) * 1e3, 2),
            "p10": round(float(np.percentile(kern_ms, 10)) * 1e3, 2),
            "p90": round(float(np.percentile(kern_ms, 90)) * 1e3, 2),
        },
        "roofline": None if launch_bound else {
            "bound": "hbm",
            "kernel": decode_kernel_name(cfg.name),
            "achieved": round(achieved, 2),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4),
            "traffic": traffic_from_profile(cfg.name),
        },
        "parity": parity,
    }
    if launch_bound:
        rec["note"] = "launch-bound: a few KB per step, no roofline claim"
    if baseline is not None:
        rec["cpu_baseline"] = baseline

    if flush_check:
        # Cross-check of the rotation: one layer only, with FLUSH_MIB of
        # scratch streamed through the caches between launches so no K/V byte
        # can come from them; per-launch event pairs on both sides (like with
        # like).  The flush READS the scratch (a reduction): a flush that
        # writes it leaves dirty lines whose write-back then competes with the
        # decode's reads, which times the write-back rather than the decode
        # (reported beside it for that reason).
        scratch = torch.ones((FLUSH_MIB << 20) // 4, dtype=torch.float32, device="cuda")
        one = argv[0]

        # The small per-step inputs (q, block tables, context lengths) stay
        # cached between layers in a real step (the block tables are shared by
        # all layers, q was just written) and under the rotation; after the
        # flush they are read again, so that only the K/V pools start cold.
        small = [layers[0].q.view(torch.uint8), layers[0].block_tables.view(torch.uint8),
                 layers[0].context_lens.view(torch.uint8)]

        def rewarm():
            for t_ in small:
                torch.sum(t_.reshape(-1), dim=0, dtype=torch.int64)

        def flushed(n, flush, warm=True):
            evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]
            torch.cuda.synchronize()
            for k in range(n):
                flush(k)
                if warm:
                    rewarm()
                evs[k][0].record(stream)
                check(L.pkv_paged_attn_decode(ctypes.byref(one), sh))
                evs[k][1].record(stream)
            torch.cuda.synchronize()
            return np.array([e[0].elapsed_time(e[1]) for e in evs])

        sink = torch.empty((), dtype=torch.float32, device="cuda")
        read_flush = lambda k: torch.sum(scratch, dim=0, out=sink)   # noqa: E731
        write_flush = lambda k: scratch.fill_(float(k))               # noqa: E731
        flushed(3, read_flush)
        med_r = float(np.median(kern_ms)) * 1e3
        med_f = float(np.median(flushed(args.steps, read_flush))) * 1e3
        med_c = float(np.median(flushed(args.steps, read_flush, warm=False))) * 1e3
        med_w = float(np.median(flushed(args.steps, write_flush))) * 1e3
        rec["flush_cross_check"] = {
            "flush_mib": FLUSH_MIB, "layers": 1, "flush": "read (reduction), then q / block tables / lengths re-read",
            "kernel_event_us_median": round(med_f, 2),
            "rotation_kernel_event_us_median": round(med_r, 2), "layers_rotated": rotate,
            "rel_diff": round(med_f / med_r - 1.0, 4),
            "flagged": bool(abs(med_f / med_r - 1.0) > FLUSH_TOLERANCE),
            "all_cold_kernel_event_us_median": round(med_c, 2),
            "write_flush_kernel_event_us_median": round(med_w, 2),
        }
        del scratch, sink

    if graph:
        # the launch overhead apart: the same launches captured in a HIP graph
        # (K decode launches, no memset nodes) and replayed; every replay's
        # output is checked against the eager output, bit for bit
        ref_out = out.clone()
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.graph(g, stream=cap):
            for k in range(args.steps):
                check(L.pkv_paged_attn_decode(ctypes.byref(argv[k % rotate]), cap.cuda_stream))
        stream.wait_stream(cap)
        torch.cuda.synchronize()
        same = True
        for _ in range(3):
            out.zero_()
            g.replay()
            torch.cuda.synchronize()
            same = same and bool(torch.equal(out.view(torch.int16), ref_out.view(torch.int16)))
            step(0)                                   # eager work between replays
            torch.cuda.synchronize()
        ge = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ge[0].record(stream)
        reps = 10
        for _ in range(reps):
            g.replay()
        ge[1].record(stream)
        torch.cuda.synchronize()
        rec["graph_replay"] = {"launches_per_graph": args.steps, "replays": reps,
                               "us_per_layer_step": round(ge[0].elapsed_time(ge[1]) * 1e3 / (reps * args.steps), 2),
                               "outputs_bit_exact": same,
                               "note": "beside the stream-launched number above, never in place of it"}
        del g
    del layers, argv, ws, ctr, out
    torch.cuda.empty_cache()
    return rec


def compact(rec: dict) -> dict:
    """A secondary workload's record inside the headline line."""
    keep = ("value", "unit", "ms_per_step", "us_per_layer_step", "pct_of_peak", "kernel_us_timed_region",
            "kernel_event_us", "roofline", "parity", "cpu_baseline", "graph_replay", "note")
    out = {k: rec[k] for k in keep if k in rec}
    c = rec["config"]
    out["config"] = {k: c[k] for k in ("batch", "num_q_heads", "num_kv_heads", "head_dim", "page_size", "q_dtype",
                                       "kv_dtype", "context_tokens", "num_splits", "layers_rotated", "seed",
                                       "bytes_alg_per_step")}
    return out


def main():
    args = parse()
    if args.summarize_counters:
        from synth import CONFIGS, make_case

        name = args.config or DEFAULT_CONFIG
        rec = summarize_counters(name, args.summarize_counters, COPY_CALIBRATION_MIB << 20)
        rec["bytes_alg_per_launch"] = make_case(CONFIGS[name]).bytes_alg()
        rec["traffic_over_alg"] = round(rec["hbm_bytes_per_launch"] / rec["bytes_alg_per_launch"], 4)
        if args.sq_counters:
            rec["sq"] = summarize_sq(args.sq_counters)
        path = os.path.join(ROOT, "profiles", f"paged_decode_{name}_counters.json")
        os.makedirs(os.path.dirname(path), exist_ok=True)
        with open(path, "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        print(json.dumps(rec))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        copy_calibration(COPY_CALIBRATION_MIB)
        return
    if args.stream_reference:
        stream_reference(2048)
        return
    if args.op != "decode" and args.config is None:
        args.config = DEFAULT_CONFIG
    if args.op == "append":
        bench_append(args)
        return
    if args.op == "serve":
        bench_serve(args)
        return
    if args.op == "prefill":
        bench_prefill(args)
        return

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.config is not None:
        # one workload (profiling runs, sweeps)
        rec = decode_workload(args.config, args, args.cpu_seconds, flush_check=args.flush_check,
                              graph=args.graph or args.config == "tiny")
        rec["source_digest"] = source_digest()
        print(json.dumps(rec), flush=True)
        return

    # the default run: every decode workload, the headline's record on top
    recs = {}
    for name in SUITE:
        head = name == DEFAULT_CONFIG
        recs[name] = decode_workload(name, args, args.cpu_seconds if head else min(args.cpu_seconds,
                                                                                  SECONDARY_CPU_SECONDS),
                                     flush_check=head, graph=name == "tiny")
        r = recs[name]
        log(f"[{name}] {r['us_per_layer_step']} us/step, {r['value']} GB/s"
            + (f", roofline frac {r['roofline']['frac']}" if r["roofline"] else "")
            + f", parity {r['parity'].get('ok')}")
    result = recs[DEFAULT_CONFIG]
    result["gate"] = {"threshold_frac": GATE_FRAC,
                      "workloads": {n: {"frac": recs[n]["roofline"]["frac"],
                                        "parity_ok": recs[n]["parity"].get("ok"),
                                        "pass": bool(recs[n]["roofline"]["frac"] >= GATE_FRAC
                                                     and recs[n]["parity"].get("ok"))} for n in GATED}}
    result["workloads"] = {n: compact(recs[n]) for n in SUITE if n != DEFAULT_CONFIG}
    result["source_digest"] = source_digest()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
