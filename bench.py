"""Benchmark: paged decode attention on one MI355X.

One step = one pass of the hot path over one batch: append the step's new
tokens into their pages, the decode partial pass over every sequence's paged
context, the log-sum-exp merge, and (mixed workload) chunked prefill.
Inputs are seeded synthetic data, resident in HBM before timing starts.

Default workload: Llama-2-13B-shaped MHA decode in bf16 (64 sequences,
40/40 heads, head_dim 128, page 64, context lengths uniform in [128, 4096]).
By default a step is one pkv_mixed_step call (append, then decode and, for
a mixed workload, prefill on a second stream); --launch selects separate
calls or HIP-graph replays instead.  Prints one JSON line: achieved HBM GB/s
of the whole step (algorithmic bytes / step time), seq-steps/s, the
decode-partial kernel's roofline (its own event-timed duration: inside the
timed loop with --launch calls, else in an eager loop after it) and the CPU
oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0


def measured_traffic(spec_name: str, split_tokens: int):
    """HBM bytes per launch of the decode-partial kernel from the committed
    counter records (profiles/traffic.json, one per workload), or None when
    no record is for this workload and context-range size, or the kernel's
    sources changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        recs = json.load(open(path))
    except (OSError, ValueError):
        return None
    for rec in recs if isinstance(recs, list) else [recs]:
        try:
            if rec.get("workload") != spec_name or rec.get("split_tokens") != split_tokens:
                continue
            h = hashlib.sha256()
            for f in rec["sources"]:
                h.update(open(os.path.join(ROOT, f), "rb").read())
            if h.hexdigest() != rec["sources_sha256"]:
                return None
            return int(rec["traffic_bytes_per_launch"])
        except (OSError, KeyError, ValueError):
            return None
    return None


def cpu_baseline(wl, budget_s: float = 12.0, budget_1thread_s: float = 4.0) -> dict:
    """The oracle, as it stands, over the workload's sequences in order
    (repeating the pass if it is short) until about `budget_s` seconds of
    decode work, scaled to GB/s of the same algorithmic bytes per sequence
    the GPU figure uses.

    The oracle handles one sequence at a time, so the baseline uses the
    host's cores by running it on disjoint sequences at once: one worker
    thread per core this process may run on (at most 16), each with its
    numerical library limited to one thread.  Sequences go in waves of one
    per worker; a wave's pages are filled by the oracle's append outside the
    timed region, then its decodes are timed together (wall clock).  A
    second, shorter run with a single worker gives the one-core figure."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    from oracle import attention as oa
    from paged_kv_cache_277_amd import workloads as wk

    s = wl.spec
    kp, vp = wl.poisoned_pool()
    filled = set()

    def fill(b):
        if b in filled:
            return
        owners = {("seq", b)}
        for batch in (wl.setup, wl.step):
            rows = [i for i, o in enumerate(batch.owners) if o in owners or o[0] == "prefix"]
            oa.kv_cache_append(kp, vp, s.kv_dtype, batch.k, batch.v, s.kv_in_dtype, batch.cu,
                               batch.start_pos, batch.block_tables, wl.k_scale, wl.v_scale,
                               rows=rows)
        filled.add(b)

    def decode(b):
        oa.paged_attn_decode(wl.q, s.q_dtype, kp, vp, s.kv_dtype, wl.block_tables,
                             wl.context_lens, wl.sm_scale, wl.k_scale, wl.v_scale,
                             seqs=np.array([b]))

    def run(budget, workers):
        order = [b for _ in range(50) for b in range(wl.num_seqs)]
        done, bytes_done, t_total, tokens = 0, 0, 0.0, 0
        with threadpool_limits(limits=1), ThreadPoolExecutor(workers) as ex:
            for w0 in range(0, len(order), workers):
                wave = order[w0:w0 + workers]
                list(ex.map(fill, sorted(set(wave) - filled)))
                t0 = time.perf_counter()
                list(ex.map(decode, wave))
                t_total += time.perf_counter() - t0
                done += len(wave)
                tokens += int(wl.context_lens[wave].sum())
                bytes_done += sum(wk.decode_bytes(s, wl.context_lens[[b]], unique_prefix=False)
                                  for b in wave)
                if t_total >= budget:
                    break
        return bytes_done / t_total / 1e9, done, tokens, t_total

    n = max(1, min(16, len(os.sched_getaffinity(0))))
    gbs, done, tokens, t_total = run(budget_s, n)
    gbs1, done1, tokens1, t1 = run(budget_1thread_s, 1)
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": n, "kind": "oracle",
            "sample": f"fp64 oracle decode of {done} sequence-queries in order ({tokens} context "
                      f"tokens) on {n} worker threads, one sequence each at a time, BLAS at one "
                      f"thread per worker, {t_total:.1f} s of wall-clock decode",
            "value_1thread": round(gbs1, 4),
            "sample_1thread": f"the same on one worker: {done1} sequence-queries ({tokens1} "
                              f"context tokens) in {t1:.1f} s"}


def copy_calibration(args) -> int:
    """A plain device-to-device copy of 1 GiB (torch's copy kernel): the known
    read and write volume against which HBM byte counters are scaled."""
    import torch
    n = 1 << 30
    a = torch.ones(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(args.warmup):
        b.copy_(a)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(args.steps):
        b.copy_(a)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / args.steps
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "ms_per_copy": round(ms, 5),
                      "copy_GBps_read_plus_write": round(2 * n / ms / 1e6, 1)}), flush=True)
    return 0


def chunk_sweep(args) -> int:
    """Prefill of long prompts in chunks of several sizes (P1 §5.3 leaves the
    chunk size to experiment) against one context-attention call over the
    whole prompts' contiguous K/V.  8B-shaped GQA (32/8 heads, head_dim 128,
    page 32), 4 prompts of 8192 tokens, bf16, seeded N(0,1) data.  Each chunk
    step appends the chunk's K/V and runs one chunked-prefill call for all
    four prompts; the sweep line reports the summed time per chunk size."""
    import torch

    from paged_kv_cache_277_amd import binding as B
    from paged_kv_cache_277_amd import device as dev
    from paged_kv_cache_277_amd import workloads as wk

    R, L, Hq, Hkv, D, P = 4, 8192, 32, 8, 128, 32
    scale = 1.0 / np.sqrt(D)
    rng = np.random.default_rng(20261202)
    T = R * L
    q = dev._dev(wk.bf16_bits_rne(rng.standard_normal((T, Hq, D), dtype=np.float32)), "bf16", "cuda")
    k = dev._dev(wk.bf16_bits_rne(rng.standard_normal((T, Hkv, D), dtype=np.float32)), "bf16", "cuda")
    v = dev._dev(wk.bf16_bits_rne(rng.standard_normal((T, Hkv, D), dtype=np.float32)), "bf16", "cuda")
    npg = L // P
    perm = rng.permutation(R * npg).astype(np.int32)
    bt = torch.from_numpy(perm.reshape(R, npg).copy()).cuda()
    cache = B.PagedCache(dev.poisoned_pool(R * npg, Hkv, P, D, "bf16", "cuda"),
                         dev.poisoned_pool(R * npg, Hkv, P, D, "bf16", "cuda"))
    flops = 4 * Hq * D * R * (L * (L + 1) // 2)
    qv = q.view(R, L, Hq, D)
    kv_, vv_ = k.view(R, L, Hkv, D), v.view(R, L, Hkv, D)
    results = []

    def timed(fn, reps):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    for C in (256, 512, 1024, 2048, 4096, 8192):
        steps = []
        for pos in range(0, L, C):
            c = min(C, L - pos)
            sq = qv[:, pos:pos + c].contiguous().view(R * c, Hq, D)
            sk = kv_[:, pos:pos + c].contiguous().view(R * c, Hkv, D)
            sv = vv_[:, pos:pos + c].contiguous().view(R * c, Hkv, D)
            cu = torch.arange(0, R * c + 1, c, dtype=torch.int32, device="cuda")
            ctx = torch.full((R,), pos, dtype=torch.int32, device="cuda")
            out = torch.empty_like(sq)
            sp = min(args.prefill_split, (pos + c + 63) // 64 * 64) if args.prefill_split else 0
            ws = B.prefill_workspace(cache, R, R * c, Hq, c, pos + c, sp)
            steps.append((sq, sk, sv, cu, ctx, out, ws, c, pos + c, sp))

        def run():
            for sq, sk, sv, cu, ctx, out, ws, c, tot, sp in steps:
                B.pkv_kv_cache_append(cache, sk, sv, cu, ctx, bt)
                B.pkv_paged_attn_chunked_prefill(cache, sq, out, cu, ctx, bt, c, tot, scale,
                                                 split_tokens=sp, workspace=ws)
        ms = timed(run, args.steps)
        results.append({"chunk": C, "steps": len(steps), "ms": round(ms, 3),
                        "tflops": round(flops / ms / 1e9, 1)})
        print(f"[sweep] chunk {C}: {ms:.3f} ms", file=sys.stderr, flush=True)
        del steps
    out = torch.empty_like(q)
    cu = torch.arange(0, T + 1, L, dtype=torch.int32, device="cuda")
    sp = min(args.prefill_split, (L + 63) // 64 * 64) if args.prefill_split else 0
    ws = B.context_workspace(R, T, Hq, Hkv, D, L, sp)
    ms = timed(lambda: B.pkv_context_fmha(q, k, v, out, cu, L, scale, split_tokens=sp,
                                          workspace=ws), args.steps)
    print(json.dumps({"chunk_sweep": results,
                      "context_fmha": {"ms": round(ms, 3), "tflops": round(flops / ms / 1e9, 1)},
                      "config": {"workload": "prefill of 4 x 8192-token prompts, 32/8 heads, "
                                             "head_dim 128, page 32, bf16",
                                 "causal_gflop": round(flops / 1e9, 1)},
                      "mfma_peak_tflops": MFMA_BF16_PEAK_TFS}), flush=True)
    return 0


def measure(spec, args, warmup, split_tokens: int, prefill_split: int):
    """Time `args.steps` steps of one workload (after `warmup` untimed ones)
    in the launch form `args.launch`; returns (JSON line without the CPU
    baseline, the generated workload)."""
    import torch

    from paged_kv_cache_277_amd import device as dev
    from paged_kv_cache_277_amd import workloads as wk

    t0 = time.perf_counter()
    wl = wk.make_workload(spec)
    print(f"[bench] workload {spec.name}: generated in {time.perf_counter() - t0:.1f} s",
          file=sys.stderr, flush=True)
    if warmup is None:
        warmup = 200 if wl.pf_block_tables is not None else 10
    dw = dev.upload(wl, "cuda", split_tokens=split_tokens, prefill_split=prefill_split)
    dw.setup()
    torch.cuda.synchronize()
    print(f"[bench] uploaded, split_tokens={dw.split_tokens}", file=sys.stderr, flush=True)

    side = torch.cuda.Stream() if args.launch.endswith("mixed_step") else None
    fused = args.launch == "decode_step"
    for _ in range(warmup):
        if side is not None:
            dw.mixed_step(side_stream=side)
        elif fused:
            dw.decode_step()
        else:
            dw.step()
    torch.cuda.synchronize()

    K = args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    graph = dw.capture_step(side_stream=side) if args.launch.startswith("graph") else None
    torch.cuda.synchronize()
    start.record()
    t_host = time.perf_counter()
    for i in range(K):
        if graph is not None:
            graph.replay()
            continue
        if side is not None:
            dw.mixed_step(side_stream=side)
            continue
        if fused:
            dw.decode_step()
            continue
        dw.append_step()
        if wl.num_seqs:
            ev[i][0].record()
            dw.decode_partial()
            ev[i][1].record()
            dw.merge()
        dw.prefill()
    host_us = (time.perf_counter() - t_host) / K * 1e6
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / K
    # Kernel durations: the decode partial (and the prefill call) timed alone
    # with events in an eager loop after the timed steps (inside a replay or a
    # fused call they cannot be bracketed; with --launch calls the partial's
    # events were recorded inside the timed loop already).
    # The partial is timed in the order the step's decode used: a one-call
    # step whose decode has the GPU to itself takes its items from a work
    # list (longest ranges first), built here once (the lengths do not
    # change between these calls) instead of inside each step's append.
    listed = args.launch.endswith("mixed_step") and not wl.num_prefill
    if listed and wl.num_seqs:
        dw.build_work_list()
    ev_pf = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(K)]
    for i in range(K):
        dw.append_step()
        if wl.num_seqs:
            if args.launch != "calls":
                ev[i][0].record()
            dw.decode_partial(listed=listed)
            if args.launch != "calls":
                ev[i][1].record()
            dw.merge()
        ev_pf[i][0].record()
        dw.prefill()
        ev_pf[i][1].record()
    torch.cuda.synchronize()
    part_times = [a.elapsed_time(b) for a, b in ev] if wl.num_seqs else [0.0]
    part_ms = float(np.mean(part_times))
    pf_times = [a.elapsed_time(b) for a, b in ev_pf] if wl.num_prefill else []

    # Cold-cache steps: a 1 GiB device write before each step (outside the
    # events) evicts L2 and the Infinity Cache; median / p10 / p90 reported.
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    cold = []
    for i in range(min(K, 20)):
        flush.fill_(i & 0xFF)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        if graph is not None:
            graph.replay()
        elif side is not None:
            dw.mixed_step(side_stream=side)
        elif fused:
            dw.decode_step()
        else:
            dw.step()
        b.record()
        torch.cuda.synchronize()
        cold.append(a.elapsed_time(b))
    del flush

    dec_bytes = wk.decode_bytes(spec, wl.context_lens) if wl.num_seqs else 0
    e_in = wk.DTYPE_BYTES[spec.kv_in_dtype]
    e_kv = wk.DTYPE_BYTES[spec.kv_dtype]
    app_bytes = wl.step.num_tokens * spec.num_kv_heads * spec.head_dim * 2 * (e_in + e_kv)
    pf_bytes = 0
    flops = 0
    if wl.num_prefill:
        flops = wk.prefill_flops(spec, wl.pf_ctx_before, wl.pf_cu)
    step_bytes = dec_bytes + app_bytes + pf_bytes
    value = step_bytes / (ms * 1e-3) / 1e9
    part_gbs = dec_bytes / (part_ms * 1e-3) / 1e9 if part_ms > 0 else 0.0
    cold_med = float(np.median(cold))

    line = {
        "metric": "paged decode attention: achieved HBM GB/s (% of peak) + seq-steps/s at 1 GPU",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "fp8": "bf16 q / fp8 e4m3 kv",
                  "int8": "bf16 q / int8 kv"}[spec.kv_dtype],
        "data": "synthetic (seeded N(0,1) K/V/Q, seeded page permutation)",
        "config": {"workload": spec.name, "num_seqs": spec.num_seqs,
                   "num_q_heads": spec.num_q_heads, "num_kv_heads": spec.num_kv_heads,
                   "head_dim": spec.head_dim, "page_size": spec.page_size,
                   "context_tokens": int(wl.context_lens.sum()),
                   "split_tokens": dw.split_tokens,
                   "prefill_split_tokens": dw.pf["split"] if dw.pf else None,
                   "parallelism": "single GPU",
                   "launch": args.launch,
                   "decode_order": "work list (longest ranges first) when the call is large "
                                   "enough" if listed else "grid"},
        "seq_steps_per_s": round((wl.num_seqs + wl.num_prefill) / (ms * 1e-3), 1),
        # host time to enqueue one step (the launch loop without its final
        # synchronisation): above ms_per_step the step is launch-bound
        "host_us_per_step": round(host_us, 2),
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "step_bytes": step_bytes,
        "cold_cache": {"ms_median": round(cold_med, 5),
                       "ms_p10": round(float(np.percentile(cold, 10)), 5),
                       "ms_p90": round(float(np.percentile(cold, 90)), 5),
                       "gbs_at_median": round(step_bytes / (cold_med * 1e-3) / 1e9, 2),
                       "steps": len(cold), "flush_bytes": 1 << 30},
        "roofline": {"bound": "hbm", "kernel": "decode_partial", "achieved": round(part_gbs, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(part_gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(spec.name, dw.split_tokens),
                     "kernel_ms": round(part_ms, 5),
                     "kernel_ms_p10_p50_p90": [round(float(np.percentile(part_times, q)), 5)
                                               for q in (10, 50, 90)],
                     "bytes_per_launch": dec_bytes},
    }
    if spec.shared_prefix_pages and wl.num_seqs:
        line["logical_step_bytes"] = (wk.decode_bytes(spec, wl.context_lens, unique_prefix=False)
                                      + app_bytes)
    if flops:
        pf_med = float(np.median(pf_times))
        line["prefill_flops"] = flops
        line["prefill"] = {"flops": flops, "call_ms_median": round(pf_med, 5),
                           "tflops": round(flops / (pf_med * 1e-3) / 1e12, 1),
                           "mfma_frac": round(flops / (pf_med * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS, 4),
                           "note": "kernel plus its range merge, timed alone"}
    return line, wl


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps first (default: 200 for a step with a prefill part, "
                         "whose matrix-core kernel reaches steady clocks only after ~20 ms of "
                         "work; 10 otherwise)")
    ap.add_argument("--workload", type=int, default=2, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--split-tokens", type=int, default=0,
                    help="decode context-range size in tokens (0: the library's default)")
    ap.add_argument("--prefill-split", type=int, default=0,
                    help="prefill key-range size in tokens (0: the library's default)")
    ap.add_argument("--kv-format", choices=("fp8", "int8"), default=None,
                    help="run the workload with this 8-bit KV format instead (a variant, "
                         "not one of the five workloads)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="default workload only: skip the 70B-shaped fp8 decode timed beside it")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--launch", choices=("mixed_step", "calls", "graph", "graph_mixed_step",
                                         "decode_step"),
                    default="mixed_step",
                    help="mixed_step: one pkv_mixed_step call per step, prefill on a second "
                         "stream; calls: append, decode and prefill calls one after another; "
                         "graph / graph_mixed_step: replays of those captured as a HIP graph; "
                         "decode_step: one pkv_decode_step call (the append inside the "
                         "attention launch; decode-only workloads)")
    ap.add_argument("--chunk-sweep", action="store_true",
                    help="instead of the step benchmark: chunked prefill of long prompts at "
                         "several chunk sizes against one context-attention call")
    ap.add_argument("--cpu-baseline-only", action="store_true",
                    help="only the CPU oracle baseline of the workload (no GPU): one JSON line")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="time a plain device copy of known size instead (counter scaling)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only (use --gpus 1): the decode path would shard by "
              "sequence or KV head with no exchange, so the throughput of N GPUs is N times "
              "that of one GPU's share.",
              file=sys.stderr)
        return 2

    from paged_kv_cache_277_amd import workloads as wk

    if args.cpu_baseline_only:
        spec = (wk.variant(f"{args.workload}-{args.kv_format}") if args.kv_format
                else wk.CONFIGS[args.workload])
        wl = wk.make_workload(spec)
        print(json.dumps({"workload": spec.name, "cpu_baseline": cpu_baseline(wl, args.cpu_budget)}),
              flush=True)
        return 0

    import torch

    from paged_kv_cache_277_amd import device as dev

    torch.cuda.set_device(0)
    if args.warmup is None and args.copy_calibration:
        args.warmup = 2
    if args.warmup is None and args.chunk_sweep:
        args.warmup = 10            # matrix-core work: steady clocks after ~20 ms
    if args.copy_calibration:
        return copy_calibration(args)
    if args.chunk_sweep:
        return chunk_sweep(args)
    spec = (wk.variant(f"{args.workload}-{args.kv_format}") if args.kv_format
            else wk.CONFIGS[args.workload])
    line, wl = measure(spec, args, args.warmup, args.split_tokens, args.prefill_split)
    if args.workload == 2 and not args.kv_format and not args.no_secondary:
        # The decode bar applies to the largest batch by bytes (this one) and
        # the largest by context, the 70B-shaped fp8 batch: timed the same way.
        second, _ = measure(wk.CONFIGS[4], args, None, 0, 0)
        keep = ("value", "unit", "ms_per_step", "hbm_frac", "seq_steps_per_s", "step_bytes",
                "config", "roofline", "cold_cache", "dtype")
        line["secondary"] = {k: second[k] for k in keep}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
