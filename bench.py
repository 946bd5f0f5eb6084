"""Benchmark: one cascade beam-decode attention step per layer on one MI355X.

A step is one bsp_decode_step launch over all B*W beams of one layer: the
current-token KV write, the shared prompt attended once per request and every
beam's tail, merged in one online softmax. The same step as four launches
(bsp_write_kv + bsp_prefix_attn + bsp_tail_attn + bsp_merge) and the per-beam
comparator are timed beside it. Consecutive timed steps rotate over
several layers, each with its own KV pool, query and new-token buffers, so
that at least 512 MB of other layers' reads pass between two steps on the same
layer and every step reads its prompt pages from HBM rather than from the
256 MB last-level cache (as consecutive layers of a model would). Inputs are
seeded synthetic draws already resident in HBM when the timed region starts.

The default workload is the wide-beam recommendation shape (128 requests x
beam 96, prompts of about 3k tokens: the largest single-GPU configuration);
``--config`` selects the others.

Prints one JSON line. The roofline entry is the step kernel: its algorithmic
bytes per launch over its average duration from HIP events recorded on the
launch stream around the timed launches; a second pass with an event between
consecutive launches gives the per-launch median, p10 and p90.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "beam-decode attention steps/s per layer + achieved HBM GB/s vs roofline"
HBM_PEAK_GBPS = 8000.0
EBYTES = {"f32": 4, "f16": 2, "bf16": 2}
WORKLOADS = {
    "qwen3_0p6b": "Qwen3-0.6B-like layer: 16 Q / 8 KV heads, head_dim 128, bf16, 32-token pages, "
                  "64 requests x beam 30, prompts U{400..600}, tails U{0..4}",
    "wide_beam": "wide-beam recommendation shape: 16 Q / 8 KV heads, head_dim 128, bf16, 32-token "
                 "pages shuffled, 128 requests x beam 96, prompts U{2800..3200}, tails U{0..8}",
    "qwen3_4b": "Qwen3-4B-like layer: 32 Q / 8 KV heads, head_dim 128, fp16, 32-token pages, "
                "64 requests x beam 30, prompts U{1600..2400}, tails U{1..4}",
    "qwen3_4b_d64": "Qwen3-4B-like layer at head_dim 64: 32 Q / 8 KV heads, fp16, 32-token pages, "
                    "64 requests x beam 30, prompts U{1600..2400}, tails U{1..4}",
    "qwen3_4b_d256": "Qwen3-4B-like layer at head_dim 256: 32 Q / 8 KV heads, fp16, 32-token pages, "
                     "64 requests x beam 30, prompts U{1600..2400}, tails U{1..4}",
    "nsample": "n-sample prefix sharing (parallel sampling): 16 Q / 8 KV heads, head_dim 128, bf16, "
               "32-token pages, 64 prompts x 16 samples, prompts U{400..600}, each sample's own "
               "tail U{8..32}",
    "prefill": "context phase of a mixed step alone: Qwen3-0.6B-like layer (16 Q / 8 KV heads, "
               "head_dim 128, bf16, 32-token pages shuffled), 8 fresh prompts U{1500..2500} "
               "as whole-prompt chunks, causal",
    "mixed": "mixed step: the qwen3_0p6b beam step (64 requests x beam 30, prompts U{400..600}, "
             "tails U{0..4}) plus 4 newly arrived requests whose prompts U{400..600} run as "
             "whole-prompt chunks (KV write, then causal prefill beside the beam step in one "
             "launch)",
    "cached_decode": "masked cached-prefix decode (beam 1): 24 Q / 8 KV heads, head_dim 128, fp16, "
                     "10368-row allocation with all 10368 rows valid, 1 new row; the key range is "
                     "split into chunks the plan picks (kv_split = -1) and merged",
    "cached_prefill": "masked cached-prefix prefill (beam 1): 24 Q / 8 KV heads, head_dim 128, "
                      "fp16, 10368 valid cached rows plus 2000 new prompt rows (causal)",
}
MFMA_BF16_PEAK_TFLOPS = 2500.0
MFMA_F16_PEAK_TFLOPS = 2500.0
CACHED_ROWS = 10368
CACHED_PREFILL_ROWS = 2000
PREFILL_SHAPE = dict(batch=8, chunk_range=(1500, 2500), cached_range=(0, 0))
MIXED_CTX_SHAPE = dict(batch=4, chunk_range=(400, 600), cached_range=(0, 0))
# Bytes of other layers' data that pass between two reads of the same layer's
# buffers: more than the 256 MB last-level cache, so that a timed step reads
# its KV from HBM.
FLUSH_BYTES = 512e6


def rotation_layers(bytes_per_step: float, forced: int = 0) -> int:
    """Layer copies to rotate over so that at least FLUSH_BYTES of other layers'
    reads pass between two steps on the same copy."""
    if forced:
        return forced
    return max(2, int(np.ceil(FLUSH_BYTES / max(bytes_per_step, 1.0))) + 1)


def launch_percentiles(torch, fn, n, stream):
    """Per-launch GPU durations (us) from HIP events recorded on the launch
    stream between consecutive launches: median, p10, p90 over n launches."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(n):
        fn(i)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    d = np.array([ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(n)])
    return {"median_us": float(np.median(d)), "p10_us": float(np.percentile(d, 10)),
            "p90_us": float(np.percentile(d, 90)), "launches": n}


KERNEL_SOURCES = ("beam_search_shared_amd/csrc/prefix_attn.hip",
                  "beam_search_shared_amd/csrc/tile_index.h",
                  "beam_search_shared_amd/csrc/device_common.h",
                  "beam_search_shared_amd/csrc/bsp_internal.h")


def kernel_source_hash() -> str:
    """sha256 over the sources of the fused kernel (ties counter records to a kernel version)."""
    import hashlib
    h = hashlib.sha256()
    root = os.path.dirname(os.path.abspath(__file__))
    for rel in KERNEL_SOURCES:
        with open(os.path.join(root, rel), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(config: str):
    """HBM bytes per launch of the fused kernel from the committed counter summaries
    (profiles/*.md, lines ``traffic-record: {json}``), if they were taken on the
    current kernel sources; otherwise None."""
    root = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles")
    want = kernel_source_hash()
    if not os.path.isdir(root):
        return None
    for name in sorted(os.listdir(root)):
        if not name.endswith(".md"):
            continue
        with open(os.path.join(root, name)) as fh:
            for line in fh:
                if line.startswith("traffic-record:"):
                    rec = json.loads(line.split(":", 1)[1])
                    if rec.get("config") == config and rec.get("kernel_source_sha256") == want:
                        return rec
    return None


def algorithmic_bytes(inp):
    """Bytes the method must move in one step, and those of the prefix kernel alone.

    step: shared prompt K+V once per request + distinct tail rows gathered + Q
    read + O written + current-token K/V written. prefix kernel: shared prompt
    K+V once per request + Q read + its fp32 partial (o and lse) written.
    """
    e = EBYTES[inp.dtype]
    Hkv, D, Hq = inp.num_kv_heads, inp.head_dim, inp.num_q_heads
    row = Hkv * D * e * 2                    # one position's K and V over all KV heads
    prefix = int(inp.prefix_len.astype(np.int64).sum()) * row
    uniq = 0
    ps = inp.page_size
    for b in range(inp.batch):
        P, S = int(inp.prefix_len[b]), int(inp.seq_len[b])
        seen = set()
        for j in range(P, S):
            for src in np.unique(inp.cache_indirection[b, :, j]):
                seen.add((int(inp.block_tables[b, src, j // ps]), j % ps))
        uniq += len(seen)
    rows = inp.batch * inp.beam
    q_bytes = rows * Hq * D * e
    o_bytes = rows * Hq * D * e
    write = len(inp.slots) * row
    step = prefix + uniq * row + q_bytes + o_bytes + write
    prefix_kernel = prefix + q_bytes + rows * Hq * (D + 1) * 4
    return step, prefix_kernel


def prefill_work(inp):
    """FLOPs of causal attention (2 products of 2 FLOPs per visible key, query
    head and dimension) and algorithmic bytes (K+V of every request read once
    per KV head, chunk K+V written, Q read, O written) of one context phase."""
    e = EBYTES[inp.dtype]
    Hq, Hkv, D = inp.num_q_heads, inp.num_kv_heads, inp.head_dim
    keys = 0
    for b in range(inp.batch):
        L, n = int(inp.cached_len[b]), int(inp.q_len[b])
        keys += n * L + n * (n + 1) // 2
    R = int(inp.q_len.sum())
    flops = 4 * keys * Hq * D
    kv_read = int((inp.cached_len + inp.q_len).sum()) * Hkv * D * e * 2
    nbytes = kv_read + R * Hkv * D * e * 2 + 2 * R * Hq * D * e
    return flops, nbytes, keys


def cpu_baseline_prefill(inp, budget_s: float):
    """The fp64 oracle on a bounded sample of rows of the same context phase,
    scaled to the whole phase by visible keys."""
    import oracle
    from threadpoolctl import threadpool_info

    rng = np.random.default_rng(0)
    _, _, keys_total = prefill_work(inp)
    done_keys, total, n = 0, 0.0, 0
    while total < budget_s / 2:
        b = int(rng.integers(0, inp.batch))
        i = int(rng.integers(0, int(inp.q_len[b])))
        t0 = time.perf_counter()
        oracle.prefill_attention_one(inp, b, i)
        total += time.perf_counter() - t0
        done_keys += int(inp.cached_len[b]) + i + 1
        n += 1
    threads = max([int(x.get("num_threads", 1)) for x in threadpool_info()] or [1])
    return total * keys_total / done_keys, threads, n


def cpu_baseline(config: str, seed: int, budget_s: float):
    """Time the fp64 oracle, as it stands, on a bounded sample of the same workload.

    The sample is the first n requests (n doubled until one pass takes about a
    quarter of the budget or covers the whole batch), repeated until about half
    the budget is spent; the rate is scaled to whole steps.
    """
    import oracle
    import synth
    from threadpoolctl import threadpool_info

    spec = synth.BEAM_CONFIGS[config]
    n = 1
    while True:
        inp = synth.make_beam_step(config, seed, batch=n, garbage="unit")
        kp, vp = oracle.write_kv(inp.k_pool, inp.v_pool, inp.slots, inp.k_new, inp.v_new,
                                 inp.page_size)
        inp.k_pool, inp.v_pool = kp, vp
        t0 = time.perf_counter()
        oracle.beam_decode_attention(inp)
        one = time.perf_counter() - t0
        if one * 4 > budget_s or n * 2 > spec.batch:
            break
        n *= 2
    reps, total = 1, one
    while total < budget_s / 2:
        t0 = time.perf_counter()
        oracle.beam_decode_attention(inp)
        total += time.perf_counter() - t0
        reps += 1
    threads = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    steps_per_s = reps * (n / spec.batch) / total
    return {"value": steps_per_s, "unit": "steps/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n} of {spec.batch} requests of the same workload (seed {seed}), "
                      f"{reps} passes in {total:.1f} s of fp64 numpy (BLAS threads {threads}), "
                      f"scaled to whole steps"}


def _timed_loop(torch, fn, steps, warmup, warm_seconds, stream, sync):
    t_end = time.perf_counter() + warm_seconds
    i = 0
    while time.perf_counter() < t_end:
        for _ in range(8):
            fn(i)
            i += 1
        torch.cuda.synchronize()
    for i in range(warmup):
        fn(i)
    sync()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    sec = time.perf_counter() - t0
    sync()
    return sec, e0.elapsed_time(e1) / steps


def _prefill_copies(S, inp, dev, layers):
    base = S.upload_prefill(inp, dev)
    copies = [base]
    for _ in range(layers - 1):
        c = S.PrefillDevice(**{**base.__dict__})
        c.k_pool = base.k_pool.clone()
        c.v_pool = base.v_pool.clone()
        c.q = base.q.clone()
        c.out = base.out.clone()
        copies.append(c)
    S.plan_prefill(base)
    return base, copies


def bench_prefill(args, torch, synth, B, S) -> dict:
    """Context phase alone: bsp_write_kv + bsp_prefill_attn per layer step."""
    dev = "cuda"
    inp = synth.make_prefill("qwen3_0p6b", args.seed, garbage="unit", **PREFILL_SHAPE)
    flops, nbytes, _ = prefill_work(inp)
    layers = rotation_layers(nbytes, args.layers)
    base, copies = _prefill_copies(S, inp, dev, layers)
    stream = torch.cuda.current_stream()
    sync = lambda: B.bsp_check(base.plan)  # noqa: E731
    sec, _ = _timed_loop(torch, lambda i: S.run_prefill(copies[i % layers], stream), args.steps,
                         args.warmup, args.warm_seconds, stream, sync)
    _, attn_ms = _timed_loop(torch, lambda i: S.run_prefill(copies[i % layers], stream,
                                                            write=False),
                             args.steps, args.warmup, 0.0, stream, sync)
    achieved = flops / (attn_ms * 1e-3) / 1e12
    res = {
        "metric": "context-phase (causal prefill) steps/s per layer + achieved TFLOP/s vs roofline",
        "value": args.steps / sec, "unit": "steps/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": sec / args.steps * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": inp.dtype, "data": "synthetic",
        "config": {"workload": WORKLOADS["prefill"], "name": "prefill",
                   "prompts": inp.q_len.tolist(), "layers_rotated": layers,
                   "step": "bsp_write_kv + bsp_prefill_attn", "flops": flops,
                   "alg_bytes": nbytes},
        "roofline": {"kernel": "prefix_mfma_kernel<MODE 3> (bsp_prefill_attn)", "bound": "mfma",
                     "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / MFMA_BF16_PEAK_TFLOPS, "traffic": None,
                     "avg_launch_us": attn_ms * 1e3,
                     "hbm_gbps_alg": nbytes / (attn_ms * 1e-3) / 1e9},
    }
    if not args.no_cpu_baseline:
        t, threads, n = cpu_baseline_prefill(inp, args.cpu_budget)
        res["cpu_baseline"] = {"value": 1.0 / t, "unit": "steps/s", "cores": threads,
                               "kind": "oracle",
                               "sample": f"{n} random rows of the same phase (seed {args.seed}) "
                                         f"in fp64 numpy, scaled to the whole phase by visible "
                                         f"keys"}
    return res


def bench_mixed(args, torch, synth, B, S) -> dict:
    """Mixed step: context phase on a second stream beside the fused beam step."""
    dev = "cuda"
    gen = synth.make_beam_step("qwen3_0p6b", args.seed, garbage="unit")
    ctx = synth.make_prefill("qwen3_0p6b", args.seed + 1, garbage="unit", **MIXED_CTX_SHAPE)
    step_bytes, _ = algorithmic_bytes(gen)
    flops, ctx_bytes, _ = prefill_work(ctx)
    gbase = S.upload_beam_step(gen, dev)
    layers = rotation_layers(step_bytes + ctx_bytes, args.layers)
    gcopies = [gbase]
    for _ in range(layers - 1):
        c = S.BeamStepDevice(**{**gbase.__dict__})
        c.q = gbase.q.clone()
        c.k_pool = gbase.k_pool.clone()
        c.v_pool = gbase.v_pool.clone()
        c.k_new_beams = gbase.k_new_beams.clone()
        c.v_new_beams = gbase.v_new_beams.clone()
        gcopies.append(c)
    S.plan_beam_step(gbase)
    cbase, ccopies = _prefill_copies(S, ctx, dev, layers)
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()

    def sync():
        B.bsp_check(gbase.plan)
        B.bsp_check(cbase.plan)

    res_t = {}
    for name, cs in (("one_stream", None), ("two_streams", side)):
        sec, _ = _timed_loop(torch, lambda i: S.run_mixed_step(ccopies[i % layers],
                                                               gcopies[i % layers], main, cs),
                             args.steps, args.warmup, args.warm_seconds, main, sync)
        res_t[name] = sec / args.steps * 1e3
    sec, _ = _timed_loop(torch, lambda i: S.run_mixed_step_fused(ccopies[i % layers],
                                                                 gcopies[i % layers], main),
                         args.steps, args.warmup, 0.0, main, sync)
    res_t["one_launch"] = sec / args.steps * 1e3
    sec_g, gen_ms = _timed_loop(torch, lambda i: S.run_decode_step(gcopies[i % layers], main),
                                args.steps, args.warmup, 0.0, main, sync)
    sec_c, _ = _timed_loop(torch, lambda i: S.run_prefill(ccopies[i % layers], main),
                           args.steps, args.warmup, 0.0, main, sync)
    ms = res_t["one_launch"]
    achieved = step_bytes / (gen_ms * 1e-3) / 1e9
    res = {
        "metric": "mixed steps/s per layer (context prefill + beam decode step)",
        "value": 1e3 / ms, "unit": "steps/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": gen.dtype, "data": "synthetic",
        "config": {"workload": WORKLOADS["mixed"], "name": "mixed",
                   "context_prompts": ctx.q_len.tolist(), "layers_rotated": layers,
                   "step": "bsp_write_kv (context rows) + bsp_mixed_step (context and beam-step "
                           "workgroups in one launch)",
                   "one_launch_ms_per_step": ms,
                   "separate_launches_one_stream_ms_per_step": res_t["one_stream"],
                   "separate_launches_two_streams_ms_per_step": res_t["two_streams"],
                   "decode_step_alone_ms": sec_g / args.steps * 1e3,
                   "context_phase_alone_ms": sec_c / args.steps * 1e3,
                   "context_flops": flops, "context_alg_bytes": ctx_bytes,
                   "decode_alg_bytes": step_bytes},
        "roofline": {"kernel": "prefix_mfma_kernel<FUSED> (bsp_decode_step)", "bound": "hbm",
                     "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": None,
                     "avg_launch_us": gen_ms * 1e3},
    }
    if not args.no_cpu_baseline:
        t_ctx, threads, n = cpu_baseline_prefill(ctx, args.cpu_budget / 2)
        gen_rate = cpu_baseline("qwen3_0p6b", args.seed, args.cpu_budget / 2)["value"]
        res["cpu_baseline"] = {"value": 1.0 / (t_ctx + 1.0 / gen_rate), "unit": "steps/s",
                               "cores": threads, "kind": "oracle",
                               "sample": f"{n} random context rows scaled by visible keys plus "
                                         f"the beam-step oracle on its first requests scaled "
                                         f"to the batch, fp64 numpy"}
    return res


def cached_work(L: int, Sq: int, Hq: int, Hkv: int, D: int, e: int):
    """FLOPs and algorithmic bytes of one cached-prefix call: L valid cached rows
    (K+V read once per KV head) and Sq new rows (written, read), each new row i
    attending L + i + 1 keys; Q read, O written, fp32 partials not counted."""
    keys = Sq * L + Sq * (Sq + 1) // 2
    flops = 4 * keys * Hq * D
    nbytes = (L + Sq) * Hkv * D * e * 2 + Sq * Hkv * D * e * 2 + 2 * Sq * Hq * D * e
    return flops, nbytes


def bench_cached(args, torch, synth, B, S, prefill: bool) -> dict:
    """The masked cached-prefix call, rotating over layer copies: bsp_write_kv +
    bsp_prefix_attn_two (cache chunks and new rows) + bsp_merge; for a one-row decode
    also bsp_prefix_attn (cache chunks) + bsp_cached_decode_merge (the headline there)
    and the one-launch bsp_cached_decode; beside them the same call with one
    bsp_prefix_attn per segment, and the cache chunks alone (the roofline entry)."""
    import oracle

    dev = "cuda"
    Sq = CACHED_PREFILL_ROWS if prefill else 1
    L = CACHED_ROWS
    inp = synth.make_cached_prefix(args.seed, valid_rows=L, q_len=Sq, garbage="unit")
    Hq, D = inp.q.shape[1], inp.q.shape[2]
    Hkv = inp.cache_k.shape[1]
    flops, nbytes = cached_work(L, Sq, Hq, Hkv, D, EBYTES[inp.dtype])

    def copies_for(split):
        base = S.upload_cached_prefix(inp, dev, kv_split=split)
        layers = rotation_layers(nbytes, args.layers)
        cs = [base]
        for _ in range(layers - 1):
            c = S.CachedPrefixDevice(**{**base.__dict__})
            c.k_pool = base.k_pool.clone()
            c.v_pool = base.v_pool.clone()
            c.q = base.q.clone()
            cs.append(c)
        S.plan_cached_prefix(base)
        for c in cs[1:]:
            c.o_part, c.lse_part, c.out, c.lse_out, c.n_split = (
                base.o_part.clone(), base.lse_part.clone(), base.out.clone(),
                base.lse_out.clone(), base.n_split)
        return base, cs, layers

    main_stream = torch.cuda.current_stream()
    res_t = {}
    for name, split in (("auto", -1), ("fixed_256", 256)):
        base, cs, layers = copies_for(split)

        def sync():
            B.bsp_check(base.plan_cache)

        # The four launches of a call, through the C entry points with their
        # arguments marshalled once per layer copy (the Python wrapper costs more
        # than the GPU work of a one-row call).
        lib = B.load_library()
        sh = main_stream.cuda_stream
        ns = base.n_split
        hd = base.num_kv_heads * base.head_dim
        rows = base.q_len
        calls, calls4 = [], []
        for c in cs:
            write = (lib.bsp_write_kv, (c.plan_new.handle, c.new_k.data_ptr(), c.new_v.data_ptr(),
                                        hd, c.slots.data_ptr(), rows, c.k_pool.data_ptr(),
                                        c.v_pool.data_ptr(), sh))
            cache = (lib.bsp_prefix_attn, (c.plan_cache.handle, c.q.data_ptr(), c.k_pool.data_ptr(),
                                           c.v_pool.data_ptr(), c.o_part.data_ptr(),
                                           c.lse_part.data_ptr(), sh))
            new = (lib.bsp_prefix_attn, (c.plan_new.handle, c.q.data_ptr(), c.k_pool.data_ptr(),
                                         c.v_pool.data_ptr(), c.o_part[ns].data_ptr(),
                                         c.lse_part[ns].data_ptr(), sh))
            both = (lib.bsp_prefix_attn_two, (c.plan_cache.handle, c.plan_new.handle,
                                              c.q.data_ptr(), c.k_pool.data_ptr(),
                                              c.v_pool.data_ptr(), c.o_part.data_ptr(),
                                              c.lse_part.data_ptr(), c.o_part[ns].data_ptr(),
                                              c.lse_part[ns].data_ptr(), sh))
            merge = (lib.bsp_merge, (rows, base.num_q_heads, base.head_dim, ns + 1,
                                     c.o_part.data_ptr(), c.lse_part.data_ptr(),
                                     rows * base.num_q_heads * base.head_dim,
                                     rows * base.num_q_heads, c.out.data_ptr(),
                                     B.DTYPE_CODE[base.dtype], c.lse_out.data_ptr(), sh))
            one = (lib.bsp_cached_decode, (c.plan_cache.handle, c.q.data_ptr(), c.new_k.data_ptr(),
                                           c.new_v.data_ptr(), hd, c.slots.data_ptr(),
                                           c.k_pool.data_ptr(), c.v_pool.data_ptr(),
                                           c.o_part.data_ptr(), c.lse_part.data_ptr(),
                                           c.out.data_ptr(), c.lse_out.data_ptr(), sh))
            mrow = (lib.bsp_cached_decode_merge, (c.plan_cache.handle, c.q.data_ptr(),
                                                  c.new_k.data_ptr(), c.new_v.data_ptr(), hd,
                                                  c.slots.data_ptr(), c.k_pool.data_ptr(),
                                                  c.v_pool.data_ptr(), c.o_part.data_ptr(),
                                                  c.lse_part.data_ptr(), c.out.data_ptr(),
                                                  c.lse_out.data_ptr(), sh))
            # the call: write, both key segments (one launch when their tiles
            # allow it), merge; the same as one bsp_prefix_attn per segment; and,
            # for a one-row decode, the cache chunks then their merge with the
            # new row (which also writes it), and the whole call in one launch
            calls.append((write, both, merge, cache, one, mrow))
            calls4.append((write, cache, new, merge))

        def runner(table, sel):
            def run(i):
                for fn, a in (table[i % layers][j] for j in sel):
                    if fn(*a) != 0:
                        raise RuntimeError(B.load_library().bsp_last_error().decode())
            return run

        sec, _ = _timed_loop(torch, runner(calls, (0, 1, 2)), args.steps, args.warmup,
                             args.warm_seconds if name == "auto" else 0.2, main_stream, sync)
        sec4, _ = _timed_loop(torch, runner(calls4, (0, 1, 2, 3)), args.steps, args.warmup, 0.0,
                              main_stream, sync)
        _, seg_ms = _timed_loop(torch, runner(calls, (3,)), args.steps, args.warmup, 0.0,
                                main_stream, sync)
        one_ms = one_gpu_ms = two_ms = None
        if not prefill:
            sec1, one_gpu_ms = _timed_loop(torch, runner(calls, (4,)), args.steps, args.warmup, 0.0,
                                           main_stream, sync)
            one_ms = sec1 / args.steps * 1e3
            sec2, _ = _timed_loop(torch, runner(calls, (3, 5)), args.steps, args.warmup, 0.0,
                                  main_stream, sync)
            two_ms = sec2 / args.steps * 1e3
        res_t[name] = dict(ms=sec / args.steps * 1e3, ms4=sec4 / args.steps * 1e3, seg_ms=seg_ms,
                           one_ms=one_ms, one_gpu_ms=one_gpu_ms, two_ms=two_ms,
                           n_split=base.n_split, split_keys=base.plan_cache.split_keys,
                           layers=layers)
        del cs, base
    a = res_t["auto"]
    seg_bytes = L * Hkv * D * EBYTES[inp.dtype] * 2 + Sq * Hq * D * EBYTES[inp.dtype]
    if prefill:
        seg_flops = 4 * Sq * L * Hq * D
        achieved = seg_flops / (a["seg_ms"] * 1e-3) / 1e12
        roof = {"kernel": "prefix_mfma_kernel<MODE 0> (bsp_prefix_attn, cache chunks)",
                "bound": "mfma", "achieved": achieved, "peak": MFMA_F16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / MFMA_F16_PEAK_TFLOPS, "traffic": None,
                "avg_launch_us": a["seg_ms"] * 1e3, "flops_per_launch": seg_flops}
    else:
        achieved = seg_bytes / (a["seg_ms"] * 1e-3) / 1e9
        roof = {"kernel": "prefix_mfma_kernel<MODE 0> (bsp_prefix_attn, cache chunks)",
                "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBPS, "traffic": None,
                "avg_launch_us": a["seg_ms"] * 1e3, "alg_bytes_per_launch": seg_bytes}
    cfg = "cached_prefill" if prefill else "cached_decode"
    # the headline: for the one-row decode the two-launch call (cache chunks, then
    # their merge with the new row, which also writes it), with the three-launch
    # call (write, both segments, merge) and the one-launch bsp_cached_decode
    # beside it; for the prefill the three-launch call
    call_ms = a["ms"] if prefill else a["two_ms"]
    step = ("bsp_write_kv + bsp_prefix_attn_two (cache chunks and new rows) + bsp_merge" if prefill
            else "bsp_prefix_attn (cache chunks) + bsp_cached_decode_merge (merge with the new "
                 "row, which it writes into its page)")
    res = {
        "metric": "masked cached-prefix calls/s per layer (write + cache chunks and new rows + merge)",
        "value": 1e3 / call_ms, "unit": "calls/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": call_ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": inp.dtype, "data": "synthetic",
        "config": {"workload": WORKLOADS[cfg], "name": cfg, "valid_rows": L, "new_rows": Sq,
                   "layers_rotated": a["layers"], "chunks": a["n_split"],
                   "chunk_keys": a["split_keys"], "flops": flops, "alg_bytes": nbytes,
                   "step": step,
                   "segments_one_launch_each_ms_per_step": a["ms4"],
                   "fixed_256_chunks": res_t["fixed_256"]["n_split"],
                   "fixed_256_ms_per_step": res_t["fixed_256"]["ms"],
                   "fixed_256_cache_segment_us": res_t["fixed_256"]["seg_ms"] * 1e3},
        "roofline": roof,
    }
    if not prefill:
        # bsp_cached_decode: the same one-row call as one launch (write, cache
        # chunks, new row and merge), host-timed per call and event-timed per launch
        res["config"]["three_launch_ms_per_step"] = a["ms"]
        res["config"]["one_launch_ms_per_step"] = a["one_ms"]
        res["config"]["one_launch_kernel_us"] = a["one_gpu_ms"] * 1e3
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_info
        n = Sq if Sq <= 16 else 16
        small = synth.make_cached_prefix(args.seed, valid_rows=L, q_len=n, garbage="unit")
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < args.cpu_budget / 2 or reps == 0:
            oracle.cached_prefix_attention(small)
            reps += 1
        t = (time.perf_counter() - t0) / reps * (Sq / n)
        threads = max([int(x.get("num_threads", 1)) for x in threadpool_info()] or [1])
        res["cpu_baseline"] = {"value": 1.0 / t, "unit": "calls/s", "cores": threads,
                               "kind": "oracle",
                               "sample": f"the first {n} of {Sq} new rows over the same "
                                         f"{L} cached rows, {reps} passes, scaled by rows"}
    return res


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="wide_beam", choices=sorted(WORKLOADS))
    ap.add_argument("--layers", type=int, default=0,
                    help="rotating layer copies (0: enough that 512 MB of other layers' reads "
                         "pass between two steps on the same copy)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-naive", action="store_true",
                    help="do not time the per-beam comparator beside the step")
    ap.add_argument("--naive-steps", type=int, default=5,
                    help="timed steps of the per-beam comparator (it re-reads the prompt per "
                         "beam and head: tens of ms per step on the wide-beam shape)")
    ap.add_argument("--skip-unfused", action="store_true",
                    help="do not time the four-launch (unfused) step beside the fused one")
    ap.add_argument("--warm-seconds", type=float, default=0.5,
                    help="untimed run of the step before the counted warmup steps, to reach "
                         "steady GPU clocks")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="before timing, copy a MIB-sized buffer 3 times (a plain copy kernel "
                         "of known size, to scale HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the step runs on a "
              "single MI355X; across GPUs each would run it on its own share of the requests.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    from beam_search_shared_amd import _binding as B
    from beam_search_shared_amd import step as S

    B.load_library()
    if args.config in ("prefill", "mixed"):
        fn = bench_prefill if args.config == "prefill" else bench_mixed
        print(json.dumps(fn(args, torch, synth, B, S)), flush=True)
        return
    if args.config in ("cached_decode", "cached_prefill"):
        res = bench_cached(args, torch, synth, B, S, args.config == "cached_prefill")
        print(json.dumps(res), flush=True)
        return
    dev = "cuda"
    inp = synth.make_beam_step(args.config, args.seed, garbage="unit")
    step_bytes, _ = algorithmic_bytes(inp)
    base = S.upload_beam_step(inp, dev)
    layers = rotation_layers(step_bytes, args.layers)
    copies = [base]
    for _ in range(layers - 1):
        c = S.BeamStepDevice(**{**base.__dict__})
        c.q = base.q.clone()
        c.k_pool = base.k_pool.clone()
        c.v_pool = base.v_pool.clone()
        c.k_new = base.k_new.clone()
        c.v_new = base.v_new.clone()
        c.k_new_beams = base.k_new_beams.clone()
        c.v_new_beams = base.v_new_beams.clone()
        copies.append(c)
    # Host planning time (once per step for all layers): median of several plans of
    # the same step, each after the previous plan's copy has completed.
    plan_s = []
    for _ in range(11):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        S.plan_beam_step(base)
        plan_s.append(time.perf_counter() - t0)
    torch.cuda.synchronize()
    t_plan = float(np.median(plan_s))

    stream = torch.cuda.current_stream()

    # The timed step calls the C entry point directly with its arguments
    # marshalled once per layer copy, so that the loop measures the GPU rather
    # than Python: bsp_decode_step, one launch per layer step.
    lib = B.load_library()
    decode = lib.bsp_decode_step
    stream_h = stream.cuda_stream
    row_stride = base.num_kv_heads * base.head_dim
    fused_args = [(c.plan.handle, c.q.data_ptr(), c.k_new_beams.data_ptr(), c.v_new_beams.data_ptr(),
                   row_stride, c.k_pool.data_ptr(), c.v_pool.data_ptr(), c.block_tables.data_ptr(),
                   c.cache_indirection.data_ptr(), c.out.data_ptr(),
                   c.lse_out.data_ptr() if c.lse_out is not None else None, stream_h)
                  for c in copies]

    def fused(i):
        if decode(*fused_args[i % layers]) != 0:
            B.bsp_check(base.plan)  # raises with the library's message
            raise RuntimeError("bsp_decode_step failed")

    def unfused(i):
        S.run_beam_step(copies[i % layers])

    def timed(fn, steps, warmup, warm_seconds=0.0):
        # Bring the GPU to its steady clocks first: a few dozen launches of a
        # 50-500 us kernel are too short for that, and the first timed
        # milliseconds after idle run about 15% slow.
        t_end = time.perf_counter() + warm_seconds
        i = 0
        while time.perf_counter() < t_end:
            for _ in range(16):
                fn(i)
                i += 1
            torch.cuda.synchronize()
        for i in range(warmup):
            fn(i)
        B.bsp_check(base.plan)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for i in range(steps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        sec = time.perf_counter() - t0
        B.bsp_check(base.plan)
        # GPU time per step on the launch stream (one kernel per fused step)
        return sec, e0.elapsed_time(e1) / steps

    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # the timed step: bsp_decode_step, one launch per layer step
    sec, fused_ms = timed(fused, args.steps, args.warmup, args.warm_seconds)
    ms_per_step = sec / args.steps * 1e3
    achieved = step_bytes / (fused_ms * 1e-3) / 1e9
    traffic = recorded_traffic(args.config)

    extra = {}
    if not args.skip_unfused:
        n_unf = max(10, args.steps // 4)
        usec, _ = timed(unfused, n_unf, 5)
        extra["unfused_4_launch_ms_per_step"] = usec / n_unf * 1e3
    # per-launch distribution of the step kernel (a separate pass with an event
    # between consecutive launches)
    pct = launch_percentiles(torch, fused, args.steps, stream)
    B.bsp_check(base.plan)
    if not args.no_naive:
        # the per-beam comparator over the same KV: current-token write, then every
        # beam attends its whole sequence, prompt re-read per beam and KV head
        out = torch.empty_like(base.out)

        def naive(i):
            c = copies[i % layers]
            S.write_current_tokens(c)
            B.bsp_naive_beam_attn(c.plan, c.q, c.k_pool, c.v_pool, c.block_tables,
                                  c.cache_indirection, out)
        n_naive = max(1, args.naive_steps)
        nsec, _ = timed(naive, n_naive, 1)
        extra["naive_per_beam_ms_per_step"] = nsec / n_naive * 1e3
        extra["naive_steps_timed"] = n_naive
        extra["cascade_speedup_vs_naive"] = extra["naive_per_beam_ms_per_step"] / ms_per_step

    result = {
        "metric": METRIC,
        "value": args.steps / sec,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": inp.dtype,
        "data": "synthetic",
        "config": {
            "workload": WORKLOADS[args.config],
            "name": args.config,
            "batch": inp.batch,
            "beam": inp.beam,
            "step": "bsp_decode_step (current-token write + shared prefix + tails, one launch)",
            "layers_rotated": layers,
            "bytes_between_reuses": (layers - 1) * step_bytes,
            "warm_seconds": args.warm_seconds,
            "step_alg_bytes": step_bytes,
            "step_alg_gbps": step_bytes / (ms_per_step * 1e-3) / 1e9,
            "plan_host_ms": t_plan * 1e3,
            **extra,
        },
        "roofline": {
            "kernel": "prefix_mfma_kernel<FUSED> (bsp_decode_step)",
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": traffic["traffic_bytes_per_launch"] if traffic else None,
            "traffic_unit": "HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "alg_bytes_per_launch": step_bytes,
            "avg_launch_us": fused_ms * 1e3,
            "launch_us_median": pct["median_us"],
            "launch_us_p10": pct["p10_us"],
            "launch_us_p90": pct["p90_us"],
        },
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args.config, args.seed, args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
