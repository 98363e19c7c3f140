"""Benchmark: MoE decode tokens/s of a pooled expert stack on one MI355X.

A step is one batch-1 decode token through every layer of the stack: per layer,
prepare (distinct ids, LRU, miss copies, map upload, remap) then forward (w13 +
SwiGLU, w2 + top-k combine, residual added).  Inputs (routing trace, activations,
gate weights) are resident in HBM before the timed region; the experts live in the
library's pinned host store and stream into the slot pools on misses.

Prints one JSON line.  Default workload: OLMoE-1B-7B shapes in bf16, 16 layers x
64 experts, top-8, hidden 2048, intermediate 1024, 16 slots per layer.
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


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--workload", default="olmoe_bf16_e64", choices=sorted(synth.WORKLOADS))
    ap.add_argument("--slots", type=int, default=None, help="slots per layer (default: workload's)")
    ap.add_argument("--layers", type=int, default=None)
    ap.add_argument("--copy-streams", type=int, default=1)
    ap.add_argument("--copy-chunk-mib", type=int, default=0)
    ap.add_argument("--no-timing", action="store_true", help="no HIP events around kernels")
    ap.add_argument("--timing-every", type=int, default=7,
                    help="time every Nth forward / copy batch with HIP events (coprime with layers)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="budget for the oracle's CPU baseline (0 = skip)")
    return ap.parse_args()


def link_peak_gbps(torch, dev, nbytes: int) -> float:
    """Pinned host -> HBM hipMemcpyAsync rate for copies of `nbytes` (the expert size)."""
    h = torch.empty(max(nbytes, 1 << 20) * 8, dtype=torch.uint8, pin_memory=True)
    h.fill_(3)
    d = torch.empty_like(h, device=dev)
    n = max(nbytes, 1 << 20)
    best = 0.0
    for _ in range(3):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        reps = 0
        while reps < 64:
            for i in range(8):
                d[i * n:(i + 1) * n].copy_(h[i * n:(i + 1) * n], non_blocking=True)
            reps += 8
        torch.cuda.synchronize()
        best = max(best, reps * n / (time.perf_counter() - t0) / 1e9)
    del h, d
    return best


def cpu_baseline(wl, experts_fn, trace, xs, ws, budget_s: float):
    """The oracle (LRU simulator + float64 MoE layer) on a bounded sample of steps."""
    from threadpoolctl import threadpool_info

    from oracle import lru as olru
    from oracle import moe as omoe

    L = trace.shape[1]
    stack = olru.StackLRU(L, wl.experts, wl.slots)
    t0 = time.perf_counter()
    done = 0
    for s in range(trace.shape[0]):
        x = xs[s]
        for l in range(L):
            stack.step(l, trace[s, l])
            y = omoe.moe_layer(x, trace[s, l], ws[s, l], lambda e: experts_fn(l, e), wl.wtype,
                               wl.hidden, wl.inter, resid=x, atype=wl.atype)
            x = synth.f32_to_bf16_bits(y.astype(np.float32)) if wl.atype == "bf16" else y.astype(np.float32)
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": done / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} decode tokens x {L} layers of the same workload (LRU simulator + "
                      f"float64 MoE layer, numpy BLAS threads={threads}), {dt:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the slot cache is a single-GPU path); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    import torch

    from expert_slot_cache_amd import binding

    dev = torch.device("cuda:0")
    wl = synth.WORKLOADS[args.workload]
    if args.layers:
        wl = wl.with_(layers=args.layers)
    slots = wl.slots if args.slots is None else args.slots
    wl = wl.with_(slots=slots)
    L, E, K, H, I, T = wl.layers, wl.experts, wl.top_k, wl.hidden, wl.inter, wl.tokens
    S = args.warmup + args.steps
    log(f"[bench] workload {wl.name}: L={L} E={E} K={K} H={H} I={I} slots={slots} T={T} steps={S}")

    t0 = time.perf_counter()
    trace = synth.make_trace(wl, steps=S)
    _, _, rx, rg = synth.streams(wl)
    xs = synth.draw_activations(rx, (S, T, H), wl.atype)
    ws = synth.draw_gate_weights(rg, (S, L, T, K))
    gen = synth.WindowedExperts(wl)
    pool = binding.MoePool(layers=L, experts=E, top_k=K, hidden=H, inter=I, slots=slots,
                           wtype=wl.wtype, atype=wl.atype, max_tokens=T,
                           copy_streams=args.copy_streams,
                           copy_chunk_bytes=args.copy_chunk_mib << 20,
                           timing=0 if args.no_timing else args.timing_every)
    for l in range(L):
        for e in range(E):
            gen.expert(l, e, pool.store_view(l, e))
    eb = pool.expert_nbytes
    log(f"[bench] store filled: {L * E * eb / 2**30:.2f} GiB pinned, {time.perf_counter() - t0:.1f} s")

    ids_d = torch.from_numpy(trace).to(dev)                     # [S, L, T, K]
    adt = torch.float32 if wl.atype == "f32" else torch.bfloat16
    if wl.atype == "f32":
        x_d = torch.from_numpy(xs).to(dev)
    else:
        x_d = torch.from_numpy(xs.view(np.int16)).to(dev).view(torch.bfloat16)
    w_d = torch.from_numpy(ws).to(dev)                          # [S, L, T, K]
    slot_d = torch.empty((L, T, K), dtype=torch.int32, device=dev)
    bufs = [torch.empty((T, H), dtype=adt, device=dev) for _ in range(2)]
    ids_p = ids_d.data_ptr()
    w_p = w_d.data_ptr()
    x_p = x_d.data_ptr()
    slot_p = slot_d.data_ptr()
    buf_p = [b.data_ptr() for b in bufs]
    ids_stride = T * K * 4
    x_stride = T * H * x_d.element_size()
    L_ = binding.lib()
    h = pool._h

    def run(s0, n):
        for s in range(s0, s0 + n):
            x = x_p + s * x_stride
            for l in range(L):
                out = buf_p[l & 1]
                st = L_.moe_pool_step(h, l, ids_p + (s * L + l) * ids_stride, T, slot_p + l * ids_stride,
                                      x, w_p + (s * L + l) * ids_stride, x, out, None, 0, None, None)
                if st:
                    binding._check(st)
                x = out

    torch.cuda.synchronize()
    run(0, args.warmup)
    pool.sync()
    torch.cuda.synchronize()
    st0 = pool.stats()
    pool.reset_timing()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    run(args.warmup, args.steps)
    pool.sync()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    st1 = pool.stats()
    tm = pool.timing()
    d = {k: st1[k] - st0[k] for k in st1}
    tokens = args.steps * T
    value = tokens / elapsed
    log(f"[bench] timed {args.steps} steps in {elapsed:.3f} s: {value:.1f} tokens/s; stats {d}")

    # per-launch algorithmic bytes of the dominant kernel (w13 + SwiGLU), batch 1:
    # K distinct experts' w13 (2I x H weights) + x + the activations written
    wbytes = {"f32": 4.0, "bf16": 2.0, "int4": 0.5}[wl.wtype]
    sbytes = 2.0 / 128 if wl.wtype == "int4" else 0.0      # bf16 scale per 128 weights
    w13_bytes = K * 2 * I * H * (wbytes + sbytes) + T * H * x_d.element_size() + T * K * I * 4
    w2_bytes = (K * H * I * (wbytes + sbytes) + T * K * I * 4 + 2 * T * H * x_d.element_size()
                + T * K * 8)
    roof = None
    hbm_hits = None
    if not args.no_timing and tm["kernel_calls"] > 0:
        n_fwd = tm["kernel_calls"]
        w13_avg_ms = tm["w13_ms"] / n_fwd
        w2_avg_ms = tm["w2_ms"] / n_fwd
        ach = w13_bytes / (w13_avg_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": "k_w13_gemv (w13 + SwiGLU)", "achieved": round(ach, 1),
                "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4),
                "traffic": None, "avg_launch_us": round(w13_avg_ms * 1e3, 2),
                "bytes_per_launch": int(w13_bytes), "timed_launches": n_fwd,
                "w2_kernel_avg_us": round(w2_avg_ms * 1e3, 2),
                "w2_achieved_gbps": round(w2_bytes / (w2_avg_ms * 1e-3) / 1e9, 1)}
        hit_bytes = (w13_bytes + w2_bytes) * n_fwd
        hbm_hits = hit_bytes / ((tm["w13_ms"] + tm["w2_ms"]) * 1e-3) / 1e9
    peak_link = link_peak_gbps(torch, dev, eb)
    link = None
    if tm.get("copy_ms", 0) > 0:
        link = tm["copy_bytes"] / (tm["copy_ms"] * 1e-3) / 1e9
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.wtype if wl.wtype != "int4" else "int4-g128/bf16", "data": "synthetic",
        "config": {"workload": wl.name, "layers": L, "experts": E, "top_k": K, "hidden": H,
                   "inter": I, "slots": slots, "tokens_per_step": T, "weights": wl.wtype,
                   "activations": wl.atype, "expert_bytes": eb, "copy_streams": args.copy_streams},
        "hit_rate": round(d["hits"] / max(1, d["hits"] + d["misses"]), 4),
        "misses_per_token": round(d["misses"] / tokens, 3),
        "fallback_steps": d["fallbacks"],
        "hbm_gbps_hits": None if hbm_hits is None else round(hbm_hits, 1),
        "link_gbps_misses": None if link is None else round(link, 2),
        "link_peak_gbps": round(peak_link, 2),
        "link_frac": None if link is None else round(link / peak_link, 4),
        "readback_wait_ms_per_step": round(tm["sync_wait_ms"] / args.steps, 4),
        "roofline": roof,
    }
    pool.close()
    del ids_d, x_d, w_d
    torch.cuda.empty_cache()
    if args.cpu_seconds > 0:
        n_cpu = min(S, 64)
        line["cpu_baseline"] = cpu_baseline(wl, lambda l, e: gen.expert(l, e), trace[:n_cpu],
                                            xs[:n_cpu], ws[:n_cpu], args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
