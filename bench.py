"""Benchmark: MoE decode tokens/s vs pool size of a pooled expert stack on one MI355X.

A step is one ubatch (default: one batch-1 decode token) through every layer of
the stack: per layer the slot manager (distinct ids, eviction policy, miss copies,
remap) and the forward (w13 + SwiGLU, w2 + top-k combine, residual added), issued as
one moe_pool_step call.  Inputs (routing trace, activations, gate weights) are
resident in HBM before the timed region; the experts live in the library's pinned
host store and stream into the slot pools on misses.

Prints one JSON line.  `value` is the headline workload (default: OLMoE-1B-7B shapes
in bf16, 16 layers x 64 experts, top-8, hidden 2048, intermediate 1024, 16 slots per
layer).  `sweep` is the pool-size curve of the large fan-out workload (48 layers x 512
INT4-g128 experts, top-10) at 0/16/32/48/64 slots per layer, on one filled store.
`link_calibration` is the host-link sweep (both copy engines, 2-256 MiB, 1-4
streams) whose best rate is `link_peak_gbps`; `roofline` is the dominant kernel's;
`cpu_baseline` is the oracle on the host cores (a bounded sample).
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

from expert_slot_cache_amd import synth  # noqa: E402

METRIC = "MoE decode tokens/s vs pool size; HBM GB/s on hits, link GB/s on misses"
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16
DECODE_MAX_TOKENS = 8            # larger ubatches take the grouped MFMA path (bf16)
GRAPH_WARM = 3                   # untimed replays after a capture (--graph)
PF_AFTER_LAYER, PF_AFTER_QUEUED, PF_AFTER_PREVIOUS = 0, 1, 2   # moe_pool_prefetch start points

# HBM bytes per launch of the dominant kernel from rocprofv3 --pmc FETCH_SIZE and
# WRITE_SIZE (KiB per dispatch), each scaled by the counter's reading for a plain
# copy of known size; valid only for the kernel source these were taken on.
PMC_TRAFFIC = {
    # per dispatch, median over the run's dispatches (all-hit steps for the fused step);
    # FETCH_SIZE scaled by the 256 MiB copy calibration (262144 / 131086.1 KiB)
    ("olmoe_bf16_e64", "aad76ee1c1c849c7"): {"fetch_kib": 32860.3, "fetch_scale": 1.9998,
                                             "write_kib": 64.7, "write_scale": 1.0},
    ("fanout_int4_e512", "aad76ee1c1c849c7"): {"fetch_kib": 8369.9, "fetch_scale": 1.9998,
                                               "write_kib": 25.0, "write_scale": 1.0},
}


def kernel_source_hash() -> str:
    """SHA-256 prefix of the sources of the timed decode kernels (the GEMVs and the fused
    step, which includes the device decision)."""
    import hashlib
    h = hashlib.sha256()
    for name in ("kernels.hip", "policy_dev.hpp"):
        with open(os.path.join(ROOT, "expert_slot_cache_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--workload", default="olmoe_bf16_e64", choices=sorted(synth.WORKLOADS))
    ap.add_argument("--slots", type=int, default=None, help="slots per layer (default: workload's)")
    ap.add_argument("--sweep", default="0,16,32,48,64",
                    help="comma-separated slot counts of the pool-size sweep ('' = none)")
    ap.add_argument("--sweep-steps", type=int, default=100,
                    help="timed steps of each sweep point (at least --steps)")
    ap.add_argument("--sweep-warmup", type=int, default=64,
                    help="untimed steps before each sweep point (at least --warmup): the pool's "
                         "steady state, not its cold start")
    ap.add_argument("--sweep-evictions", default="lru,fifo,lfu,slru,decay",
                    help="eviction policies of the pool-size sweep (the first gives its main points; "
                         "each policy runs every point on the same filled store)")
    ap.add_argument("--evict", default="lru", choices=["lru", "fifo", "lfu", "slru", "decay"],
                    help="eviction policy of the headline run")
    ap.add_argument("--sweep-workload", default="fanout_int4_e512", choices=sorted(synth.WORKLOADS),
                    help="workload of the pool-size sweep (one filled store serves every point)")
    ap.add_argument("--multi-tokens", default="8",
                    help="comma-separated tokens per step of extra decode points on the headline "
                         "workload with every expert resident (the kernels at several tokens, no "
                         "host link; '' = none)")
    ap.add_argument("--multi-steps", type=int, default=100,
                    help="timed steps of each multi-token point (untimed steps before it: 20)")
    ap.add_argument("--layers", type=int, default=None)
    ap.add_argument("--tokens", type=int, default=None, help="tokens per ubatch (default: workload's)")
    ap.add_argument("--rule", default="distinct", choices=["distinct", "static"])
    ap.add_argument("--resident", action="store_true", help="all experts resident (no pool)")
    ap.add_argument("--copy-streams", type=int, default=1)
    ap.add_argument("--copy-chunk-mib", type=int, default=0)
    ap.add_argument("--copy-engine", default="kernel", choices=["dma", "kernel"],
                    help="miss-path copies: DMA engine (hipMemcpyAsync) or a copy kernel reading the "
                         "mapped pinned store")
    ap.add_argument("--policy", default="device", choices=["host", "device"],
                    help="slot manager: LRU on the host (reads back the distinct ids) or in one GPU "
                         "workgroup (no host round trip on the decode path)")
    ap.add_argument("--read-through", type=int, default=-1, choices=[-1, 0, 1],
                    help="device policy, one token per step: the fused step (decision inside the w13 "
                         "launch, missed experts read through from the pinned store); -1 = the faster "
                         "form for the weight format (fused for bf16 / fp32, copying for INT4)")
    ap.add_argument("--graph", action="store_true",
                    help="device policy, one token per step: capture one decode token (every layer's "
                         "step) in a HIP graph and time its replays; the kernel and link figures then "
                         "come from event-timed eager warm-up steps (a capture cannot hold them)")
    ap.add_argument("--prefetch-accuracy", type=float, default=None,
                    help="cross-layer prefetch with a stand-in predictor that is right for this fraction of "
                         "(step, layer) id rows (default: no prefetch)")
    ap.add_argument("--prefetch-distance", type=int, default=1,
                    help="layers ahead that a layer's predicted experts are prefetched")
    ap.add_argument("--prefetch-slots", type=int, default=None,
                    help="prefetch entries per layer (default: 2 x top_k, at most 64)")
    ap.add_argument("--no-timing", action="store_true", help="no HIP events around kernels")
    ap.add_argument("--timing-every", type=int, default=7,
                    help="time every Nth forward / copy batch with HIP events (coprime with layers)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="budget for the oracle's CPU baseline (0 = skip)")
    ap.add_argument("--link-sweep", default="2,8,32,128,256",
                    help="transfer sizes (MiB) of the host-link calibration sweep, each with both copy "
                         "engines over 1, 2 and 4 streams")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of 256 MiB 4 times (for scaling the HBM "
                         "traffic counters) and exit")
    return ap.parse_args()


def copy_calibration(torch, dev):
    """A plain elementwise device copy of exactly 256 MiB (read 256 MiB, write 256 MiB),
    launched 4 times: the reference reading for FETCH_SIZE / WRITE_SIZE."""
    n = (256 << 20) // 4
    src = torch.full((n,), 7, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(4):
        torch.add(src, 0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "elementwise int32 copy", "bytes_read": n * 4, "bytes_written": n * 4,
                      "launches": 4}), flush=True)


def read_ceiling(torch, dev, binding, nbytes: int, achieved_gbps: float) -> dict:
    """What a plain streaming read of the dominant kernel's bytes per launch achieves
    on this GPU in one launch, timed like the kernel (events around the dispatch),
    rotating over 8 regions so no launch is served from the on-chip caches."""
    nbytes = max(16, nbytes // 16 * 16)
    buf = torch.empty(nbytes * 8, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    us = binding.read_calibration(buf, nbytes, reps=40)
    del buf
    gbps = nbytes / (us * 1e-6) / 1e9
    return {"gbps": round(gbps, 1), "bytes": nbytes, "avg_launch_us": round(us, 2),
            "frac_of_read_ceiling": round(achieved_gbps / gbps, 4),
            "method": "plain streaming read of the same bytes in one launch, event-timed, 8 rotating regions"}


def link_sweep(binding, sizes_mib, eb: int) -> dict:
    """Pinned host -> HBM rate of one transfer per size (MiB, plus one expert), with
    both copy engines (the library's calibration call: hipMemcpyAsync, or the copy
    kernel reading the device-mapped store), split over 1, 2 and 4 streams, each
    event-timed; the peak is the best of all."""
    sizes = sorted({int(m) << 20 for m in sizes_mib} | {(eb + 15) // 16 * 16})
    table = []
    for nbytes in sizes:
        for engine in ("dma", "kernel"):
            for streams in (1, 2, 4):
                us = binding.link_calibration(nbytes, engine=engine, reps=4, streams=streams)
                table.append({"bytes": nbytes, "engine": engine, "streams": streams,
                              "gbps": round(nbytes / (us * 1e-6) / 1e9, 2)})
    best = max(table, key=lambda r: r["gbps"])
    at_expert = max((r for r in table if r["bytes"] == sizes[0] or r["bytes"] == (eb + 15) // 16 * 16),
                    key=lambda r: r["gbps"])
    return {"peak": best["gbps"], "peak_at": {k: best[k] for k in ("bytes", "engine", "streams")},
            "best_at_one_expert": at_expert, "table": table}


def cpu_baseline(wl, experts_fn, trace, xs, ws, budget_s: float):
    """The oracle (LRU simulator + float64 MoE layer) on a bounded sample of steps,
    counted per layer so that slow configurations still give a rate."""
    from threadpoolctl import threadpool_info

    from oracle import lru as olru
    from oracle import moe as omoe

    L = trace.shape[1]
    T = trace.shape[2]
    stack = olru.StackLRU(L, wl.experts, wl.slots)
    t0 = time.perf_counter()
    layers_done = 0
    for s in range(trace.shape[0]):
        x = xs[s]
        for l in range(L):
            stack.step(l, trace[s, l])
            y = omoe.moe_layer(x, trace[s, l], ws[s, l], lambda e: experts_fn(l, e), wl.wtype,
                               wl.hidden, wl.inter, resid=x, atype=wl.atype)
            x = synth.f32_to_bf16_bits(y.astype(np.float32)) if wl.atype == "bf16" else y.astype(np.float32)
            layers_done += 1
            if time.perf_counter() - t0 > budget_s:
                break
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    tokens = layers_done / L * T
    return {"value": tokens / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{layers_done} layer-steps ({tokens:.2f} tokens of the {L}-layer stack) of the "
                      f"same workload: LRU simulator + float64 MoE layer, numpy BLAS threads={threads}, "
                      f"{dt:.1f} s"}


def read_through_for(args, wl) -> bool:
    """The fused one-token step (read-through misses) or the copying step."""
    if args.policy != "device" or wl.tokens != 1 or args.evict == "decay":
        return False
    if args.read_through >= 0:
        return bool(args.read_through)
    return wl.wtype != "int4"


def make_pool(args, binding, wl, slots, gen, resident, prefetch_slots=0, read_through=None):
    """A pool for the workload with its store (or, resident, its slots) filled."""
    if read_through is None:
        read_through = read_through_for(args, wl)
    L, E, K, H, I, T = wl.layers, wl.experts, wl.top_k, wl.hidden, wl.inter, wl.tokens
    t0 = time.perf_counter()
    pool = binding.MoePool(layers=L, experts=E, top_k=K, hidden=H, inter=I, slots=slots,
                           wtype=wl.wtype, atype=wl.atype, rule=args.rule, resident=resident,
                           max_tokens=T, copy_streams=args.copy_streams,
                           copy_chunk_bytes=args.copy_chunk_mib << 20, copy_engine=args.copy_engine,
                           policy=args.policy, read_through=read_through,
                           timing=0 if args.no_timing else args.timing_every, prefetch_slots=prefetch_slots,
                           evict=args.evict)
    eb = pool.expert_nbytes
    if resident:
        buf = np.empty(eb, np.uint8)
        for l in range(L):
            for e in range(E):
                pool.load_expert(l, e, gen.expert(l, e, buf))
    else:
        for l in range(L):
            for e in range(E):
                gen.expert(l, e, pool.store_view(l, e))
    log(f"[bench] {wl.name}: store filled, {L * E * eb / 2**30:.2f} GiB pinned, "
        f"{time.perf_counter() - t0:.1f} s")
    return pool


def run_point(args, torch, binding, wl, slots, trace, xs_d, ws_d, gen, resident, pool=None):
    """One timed run at `slots` slots per layer, on `pool` (set to that many slots and
    cold) or on a pool of its own; returns the result dict and the expert size.  With
    --graph the pool and everything around it run on a side stream, which a capture
    needs."""
    if not args.graph:
        return _run_point(args, torch, binding, wl, slots, trace, xs_d, ws_d, gen, resident, pool)
    if args.policy != "device" or resident or wl.tokens != 1:
        raise SystemExit("--graph needs the device policy, a pooled stack and one token per step")
    with torch.cuda.stream(torch.cuda.Stream()):
        return _run_point(args, torch, binding, wl, slots, trace, xs_d, ws_d, gen, resident, pool)


def _run_point(args, torch, binding, wl, slots, trace, xs_d, ws_d, gen, resident, shared=None):
    dev = torch.device("cuda:0")
    L, E, K, H, I, T = wl.layers, wl.experts, wl.top_k, wl.hidden, wl.inter, wl.tokens
    prefetch = args.prefetch_accuracy is not None and slots > 0 and not resident and shared is None
    pf_slots = (args.prefetch_slots or min(64, 2 * K)) if prefetch else 0
    if shared is not None:
        pool = shared
        pool.set_slots(slots)
        pool.reset_timing()
    else:
        pool = make_pool(args, binding, wl, slots, gen, resident, pf_slots)
    adt = torch.float32 if wl.atype == "f32" else torch.bfloat16
    slot_d = torch.empty((L, T, K), dtype=torch.int32, device=dev)
    bufs = [torch.empty((T, H), dtype=adt, device=dev) for _ in range(2)]
    ids_d = torch.from_numpy(trace).to(dev)
    ids_p, w_p, x_p, slot_p = ids_d.data_ptr(), ws_d.data_ptr(), xs_d.data_ptr(), slot_d.data_ptr()
    buf_p = [b.data_ptr() for b in bufs]
    ids_stride = T * K * 4
    x_stride = T * H * xs_d.element_size()
    L_ = binding.lib()
    h = pool._h

    if prefetch:
        pred_d = torch.from_numpy(synth.predictions(wl, trace, args.prefetch_accuracy)).to(dev)
        pred_p = pred_d.data_ptr()
        dist = max(1, args.prefetch_distance)

    def run(s0, n):
        for s in range(s0, s0 + n):
            x = x_p + s * x_stride
            if prefetch:
                # the first layers' predictions are issued at the start of the token; each
                # copy may start once its layer's last step is done
                for l in range(min(dist, L)):
                    st = L_.moe_pool_prefetch(h, l, pred_p + (s * L + l) * ids_stride, T, PF_AFTER_LAYER)
                    if st:
                        binding._check(st)
            for l in range(L):
                if prefetch and l + dist < L:
                    st = L_.moe_pool_prefetch(h, l + dist, pred_p + (s * L + l + dist) * ids_stride, T,
                                              PF_AFTER_LAYER)
                    if st:
                        binding._check(st)
                out = buf_p[l & 1]
                st = L_.moe_pool_step(h, l, ids_p + (s * L + l) * ids_stride, T, slot_p + l * ids_stride,
                                      x, w_p + (s * L + l) * ids_stride, x, out, None, 0, None, None)
                if st:
                    binding._check(st)
                x = out

    g = None
    if args.graph:
        # one token's steps, captured on the static input buffers below; a replay reads
        # the token's ids, gate weights and input copied there first
        ids_s = torch.empty((L, T, K), dtype=torch.int32, device=dev)
        w_s = torch.empty((L, T, K), dtype=torch.float32, device=dev)
        x_s = torch.empty((T, H), dtype=adt, device=dev)

        if prefetch:
            pred_s = torch.empty((L, T, K), dtype=torch.int32, device=dev)

        def record():
            x = x_s.data_ptr()
            if prefetch:
                # the capture forks the copy stream once, at its start; a replay runs after
                # the previous one has finished, so every later copy follows the previous one
                for l in range(min(dist, L)):
                    st = L_.moe_pool_prefetch(h, l, pred_s.data_ptr() + l * ids_stride, T,
                                              PF_AFTER_QUEUED if l == 0 else PF_AFTER_PREVIOUS)
                    if st:
                        binding._check(st)
            for l in range(L):
                if prefetch and l + dist < L:
                    st = L_.moe_pool_prefetch(h, l + dist, pred_s.data_ptr() + (l + dist) * ids_stride, T,
                                              PF_AFTER_PREVIOUS)
                    if st:
                        binding._check(st)
                out = buf_p[l & 1]
                st = L_.moe_pool_step(h, l, ids_s.data_ptr() + l * ids_stride, T, slot_p + l * ids_stride,
                                      x, w_s.data_ptr() + l * ids_stride, x, out, None, 0, None, None)
                if st:
                    binding._check(st)
                x = out

        def replay(s0, n):
            for s in range(s0, s0 + n):
                ids_s.copy_(ids_d[s])
                w_s.copy_(ws_d[s])
                x_s.copy_(xs_d[s])
                if prefetch:
                    pred_s.copy_(pred_d[s])
                g.replay()

    torch.cuda.synchronize()
    if args.graph:
        # warm-up eagerly; the kernel and link timings come from its second half
        run(0, args.warmup // 2)
        pool.sync()
        pool.reset_timing()
        run(args.warmup // 2, args.warmup - args.warmup // 2)
        pool.sync()
        tm = pool.timing()
        pool.set_timing(0)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=torch.cuda.current_stream()):
            record()
        replay(args.warmup, GRAPH_WARM)          # the first replays, untimed
        pool.sync()
        s0 = args.warmup + GRAPH_WARM
    else:
        run(0, args.warmup)
        pool.sync()
        s0 = args.warmup
    st0 = pool.stats()
    if not args.graph:
        pool.reset_timing()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    if args.graph:
        replay(s0, args.steps)
    else:
        run(s0, args.steps)
    pool.sync()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    st1 = pool.stats()
    if not args.graph:
        tm = pool.timing()
    else:
        g.reset()
    eb = pool.expert_nbytes
    if shared is None:
        pool.close()
    del ids_d, slot_d, bufs
    d = {k: st1[k] - st0[k] for k in st1}
    tokens = args.steps * T
    value = tokens / elapsed
    log(f"[bench] slots={slots}: {args.steps} steps in {elapsed:.3f} s: {value:.2f} tokens/s; {d}")

    # algorithmic work of one w13 / w2 launch, averaged over the timed layer-steps
    timed = trace[s0:s0 + args.steps]
    flat = timed.reshape(-1, T * K)
    D_mean = float(np.mean([len(np.unique(r)) for r in flat]))
    wbytes = {"f32": 4.0, "bf16": 2.0, "int4": 0.5}[wl.wtype]
    sbytes = 2.0 / 128 if wl.wtype == "int4" else 0.0      # bf16 scale per 128 weights
    xb = xs_d.element_size()
    actb = 4 if wl.wtype == "f32" else 2
    w13_bytes = D_mean * 2 * I * H * (wbytes + sbytes) + T * H * xb + T * K * I * actb
    w2_bytes = D_mean * H * I * (wbytes + sbytes) + T * K * I * actb + 2 * T * H * xb + T * K * 8
    w13_flops = 2.0 * 2 * I * H * T * K
    grouped = T > DECODE_MAX_TOKENS and wl.wtype == "bf16"
    res = {"slots": slots, "value": round(value, 3), "ms_per_step": round(elapsed / args.steps * 1e3, 4),
           # demanded experts served from the pool; staged ones (fallback steps, and the
           # host reads of decayed-count placement) count against it
           "hit_rate": round(d["hits"] / max(1, d["hits"] + d["misses"] + d["staged"]), 4),
           "misses_per_token": round(d["misses"] / tokens, 4),
           "fallback_steps": d["fallbacks"], "staged_experts": d["staged"],
           "h2d_gb": round(d["bytes_h2d"] / 1e9, 3),
           "readback_wait_ms_per_step": round(tm["sync_wait_ms"] / args.steps, 4)}
    if prefetch:
        res["prefetch"] = {"predictor_accuracy": args.prefetch_accuracy, "distance": max(1, args.prefetch_distance),
                           "slots": pf_slots, "served_from_prefetch_per_token": round(d["prefetched"] / tokens, 4),
                           "prefetch_gb": round(d["prefetch_bytes"] / 1e9, 3),
                           "predictor": "stand-in: the trace's own ids of the (step, layer) with this "
                                        "probability, else an independent trace's"}
    if tm["copy_ms"] > 0:
        res["link_gbps_misses"] = round(tm["copy_bytes"] / (tm["copy_ms"] * 1e-3) / 1e9, 2)
        res["miss_batch_bytes"] = int(tm["copy_bytes"] // max(1, tm["copy_calls"]))
    if not args.no_timing and tm["kernel_calls"] > 0:
        n = tm["kernel_calls"]
        w13_us = tm["w13_ms"] / n * 1e3
        w2_us = tm["w2_ms"] / n * 1e3
        ach = w13_bytes / (w13_us * 1e-6) / 1e9
        tflops = w13_flops / (w13_us * 1e-6) / 1e12
        fused = pool.read_through and not resident
        name = ("k_grouped_w13 (grouped MFMA w13 + SwiGLU)" if grouped else
                "k_step_w13 (decision + w13 + SwiGLU, fused step)" if fused else "k_w13_gemv (w13 + SwiGLU)")
        intensity = w13_flops / w13_bytes
        mfma_bound = grouped and intensity > MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
        if mfma_bound:
            roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4)}
        else:
            roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": round(ach / HBM_PEAK_GBPS, 4)}
        pmc = PMC_TRAFFIC.get((wl.name, kernel_source_hash())) if T == 1 and not resident else None
        traffic = None if pmc is None else int((pmc["fetch_kib"] * pmc["fetch_scale"] +
                                                pmc["write_kib"] * pmc["write_scale"]) * 1024)
        roof.update({"traffic": traffic, "kernel": name, "avg_launch_us": round(w13_us, 2),
                     "bytes_per_launch": int(w13_bytes), "flops_per_launch": int(w13_flops),
                     "timed_launches": n, "distinct_experts_per_launch": round(D_mean, 2),
                     "w2_stage_avg_us": round(w2_us, 2),
                     "w2_stage_achieved_gbps": round(w2_bytes / (w2_us * 1e-6) / 1e9, 1)})
        if grouped:
            roof["mfma_tflops"] = round(tflops, 2)
            roof["mfma_util"] = round(tflops / MFMA_BF16_PEAK_TFLOPS, 5)
            roof["hbm_gbps"] = round(ach, 1)
        if roof["bound"] == "hbm":
            roof["read_ceiling"] = read_ceiling(torch, dev, binding, int(w13_bytes), ach)
        if args.graph:
            roof["measured_in"] = "event-timed eager warm-up steps before the graph replays"
        res["roofline"] = roof
        res["hbm_gbps_hits"] = round((w13_bytes + w2_bytes) / ((w13_us + w2_us) * 1e-6) / 1e9, 1)
    torch.cuda.empty_cache()
    return res, eb


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the slot cache is a single-GPU path); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    import torch

    from expert_slot_cache_amd import binding

    dev = torch.device("cuda:0")
    if args.copy_calibration:
        copy_calibration(torch, dev)
        return
    wl = synth.WORKLOADS[args.workload]
    if args.layers:
        wl = wl.with_(layers=args.layers)
    if args.tokens:
        wl = wl.with_(tokens=args.tokens)
    points = [int(v) for v in args.sweep.split(",") if v.strip()] if args.sweep else []
    slots = wl.slots if args.slots is None else args.slots
    wl = wl.with_(slots=slots)
    L, E, K, H, I, T = wl.layers, wl.experts, wl.top_k, wl.hidden, wl.inter, wl.tokens
    S = args.warmup + args.steps + (GRAPH_WARM if args.graph else 0)
    log(f"[bench] workload {wl.name}: L={L} E={E} K={K} H={H} I={I} slots={slots} T={T} "
        f"steps={S} rule={args.rule} resident={args.resident}")

    def inputs(w, S=S):
        tr = synth.make_trace(w, steps=S)
        _, _, rx, rg = synth.streams(w)
        xs = synth.draw_activations(rx, (S, w.tokens, w.hidden), w.atype)
        ws = synth.draw_gate_weights(rg, (S, w.layers, w.tokens, w.top_k))
        if w.atype == "f32":
            xd = torch.from_numpy(xs).to(dev)
        else:
            xd = torch.from_numpy(xs.view(np.int16)).to(dev).view(torch.bfloat16)
        return tr, xs, ws, xd, torch.from_numpy(ws).to(dev)

    # the headline: the workload at its own slot count
    trace, xs, ws, xs_d, ws_d = inputs(wl)
    gen = synth.WindowedExperts(wl)
    main_res, eb = run_point(args, torch, binding, wl, slots, trace, xs_d, ws_d, gen, args.resident)
    del xs_d, ws_d
    torch.cuda.empty_cache()

    # decode at several tokens per step, every expert resident: the GEMVs' rate on the
    # distinct experts of a step (a shared expert's w13 rows are read once per step)
    multi = []
    for tm in [int(v) for v in args.multi_tokens.split(",") if v.strip()] if args.multi_tokens else []:
        if tm < 2 or tm > DECODE_MAX_TOKENS or args.graph:
            continue
        mwl = wl.with_(tokens=tm)
        margs = argparse.Namespace(**vars(args))
        margs.steps, margs.warmup = args.multi_steps, 20
        margs.prefetch_accuracy = None
        log(f"[bench] multi-token point: {tm} tokens per step, all experts resident")
        m_trace, _, _, m_xd, m_wd = inputs(mwl, margs.warmup + margs.steps)
        r, _ = run_point(margs, torch, binding, mwl, E, m_trace, m_xd, m_wd, gen, True)
        multi.append({"tokens_per_step": tm, "steps": margs.steps, "warmup": margs.warmup, "resident": True,
                      **{k: r[k] for k in ("value", "ms_per_step", "roofline") if k in r}})
        del m_xd, m_wd
        torch.cuda.empty_cache()

    # the pool-size sweep: one pool with the largest slot count, its store filled once,
    # set to each point's slot count (cold) in turn
    sweep = None
    if points:
        swl = synth.WORKLOADS[args.sweep_workload]
        swl = swl.with_(slots=max(points))
        sargs = argparse.Namespace(**vars(args))
        sargs.steps = max(args.steps, args.sweep_steps)
        sargs.warmup = max(args.warmup, args.sweep_warmup)
        log(f"[bench] sweep {swl.name}: slots {points}, {sargs.warmup} + {sargs.steps} steps per point")
        s_trace, _, _, s_xd, s_wd = inputs(swl, sargs.warmup + sargs.steps + (GRAPH_WARM if args.graph else 0))
        s_gen = synth.WindowedExperts(swl)
        # the copying step: every policy of the comparison runs on it
        s_pool = make_pool(args, binding, swl, max(points), s_gen, False, read_through=False)
        sweep = {"workload": swl.name, "steps": sargs.steps, "warmup": sargs.warmup,
                 "layers": swl.layers, "experts": swl.experts, "top_k": swl.top_k,
                 "hidden": swl.hidden, "inter": swl.inter, "weights": swl.wtype, "activations": swl.atype,
                 "expert_bytes": s_pool.expert_nbytes, "read_through": False, "points": []}
        evicts = [v.strip() for v in args.sweep_evictions.split(",") if v.strip()] or [args.evict]
        sweep["eviction"] = evicts[0]
        sweep["by_eviction"] = {}
        for ev in evicts:
            s_pool.set_eviction(ev)
            pts = []
            for n in points:
                r, _ = run_point(sargs, torch, binding, swl, n, s_trace, s_xd, s_wd, s_gen, False, pool=s_pool)
                pts.append(r)
            if ev == evicts[0]:
                sweep["points"] = pts
            sweep["by_eviction"][ev] = [
                {k: r.get(k) for k in ("slots", "value", "hit_rate", "misses_per_token", "staged_experts",
                                       "h2d_gb", "link_gbps_misses")} for r in pts]
        s_pool.close()
        del s_xd, s_wd
        torch.cuda.empty_cache()

    link = link_sweep(binding, [v for v in args.link_sweep.split(",") if v.strip()], eb)
    peak_link = link["peak"]
    line = {
        "metric": METRIC, "value": main_res["value"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.wtype if wl.wtype != "int4" else "int4-g128/bf16", "data": "synthetic",
        "config": {"workload": wl.name, "layers": L, "experts": E, "top_k": K, "hidden": H,
                   "inter": I, "slots": slots, "tokens_per_step": T, "weights": wl.wtype,
                   "activations": wl.atype, "expert_bytes": eb, "rule": args.rule,
                   "resident": args.resident, "copy_streams": args.copy_streams,
                   "copy_engine": args.copy_engine, "policy": args.policy, "evict": args.evict,
                   "read_through": read_through_for(args, wl) and not args.resident,
                   "graph": bool(args.graph), "prefetch_accuracy": args.prefetch_accuracy},
    }
    for k, v in main_res.items():
        if k not in ("value", "ms_per_step", "slots", "roofline"):
            line[k] = v
    line["link_peak_gbps"] = round(peak_link, 2)
    line["link_calibration"] = link
    if "link_gbps_misses" in main_res:
        line["link_frac"] = round(main_res["link_gbps_misses"] / peak_link, 4)
    line["roofline"] = main_res.get("roofline")
    if multi:
        line["multi_token"] = multi
    if sweep is not None:
        for r in sweep["points"]:
            if "link_gbps_misses" in r:
                r["link_frac"] = round(r["link_gbps_misses"] / peak_link, 4)
        line["sweep"] = sweep
    if args.cpu_seconds > 0:
        n_cpu = min(S, 64)
        line["cpu_baseline"] = cpu_baseline(wl, lambda l, e: gen.expert(l, e), trace[:n_cpu],
                                            xs[:n_cpu], ws[:n_cpu], args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
