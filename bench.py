#!/usr/bin/env python3
"""Benchmark of the DFlash block draft-and-verify step on one MI355X.

One step = dflash_draft_step -> target stand-in (planted target tokens) ->
dflash_fuse_inject(commit = 0) -> dflash_verify_commit over the whole batch, with
synthetic seeded inputs already resident in HBM.  With --temperature T > 0 the step
samples instead: dflash_draft_step_sampled (Gumbel-max drafts, logits and
log-sum-exps out) -> target stand-in (planted target logits) -> dflash_fuse_inject
-> dflash_verify_sampled (rejection sampling over the full vocabulary).  Steps are
captured as HIP graphs and replayed.  Prints one JSON line:
  value         block steps/s of the headline workload (all B sequences per step)
  roofline      its dominant kernel (fused final-norm + LM head + argmax), timed with
                HIP events on the stream it runs on, against the MFMA peak (batches of
                >= 128 block rows) or the 8 TB/s HBM peak (smaller batches)
  cpu_baseline  the fp64 oracle timed on this host on a bounded sample
  also          the other bf16 workloads, measured the same way in the same run
Default headline workload: batch 256, block 8, SWA window 128 at logical position
262144 (the long-context throughput configuration); --only skips the others.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def parse():
    from block_diffusion_speculative_dflash_amd import configs
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default=configs.C5.name, choices=sorted(configs.WORKLOADS))
    p.add_argument("--only", action="store_true",
                   help="measure the chosen workload alone (default: also the other bf16 workloads)")
    p.add_argument("--accept-q", type=float, default=None,
                   help="override the planted geometric q (sub-runs of the SWA workload)")
    p.add_argument("--head-launches", type=int, default=50)
    p.add_argument("--head-warmup", type=int, default=3,
                   help="untimed eager draft steps before the timed LM-head launches (the first "
                        "eager launches after the graph replays run up to 30 %% slower)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-steps", type=int, default=8)
    p.add_argument("--pmc-probe", action="store_true",
                   help="for hardware-counter runs: 5 draft steps, then 5 copies of 1 GiB "
                        "(the copy calibrates FETCH_SIZE / WRITE_SIZE against known bytes)")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--temperature", type=float, default=0.0,
                   help="0: greedy drafting and verification; > 0: sampled drafting and "
                        "rejection-sampling verification at this temperature")
    p.add_argument("--adaptive", action="store_true",
                   help="per-sequence block lengths chosen every step by the block-size controller "
                        "(dflash_adapt_block_len, default thresholds) from the accepted lengths")
    p.add_argument("--persistent", action="store_true",
                   help="greedy draft step as one persistent kernel per layer (dflash_draft_step_persistent; "
                        "bf16 drafters with <= 64 block rows)")
    p.add_argument("--sink", type=int, default=0,
                   help="attention sink: positions 0..S-1 stay visible beside the window "
                        "(adds S cache slots; the sink rows are injected before the prefill)")
    return p.parse_args()


class HipEvents:
    """hipEvent_t pairs through the HIP runtime (the library records them on the
    stream its kernels run on)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self) -> int:
        e = ctypes.c_void_p()
        if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e.value

    def elapsed_ms(self, a: int, b: int) -> float:
        f = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(f), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return f.value

    def destroy(self, e: int) -> None:
        self.hip.hipEventDestroy(ctypes.c_void_p(e))


def main() -> int:
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this library runs the DFlash step on one GPU only (the data-parallel "
                          "shard of one GPU is the whole measurement); run with --gpus 1",
                          "n_gpus": args.gpus}), flush=True)
        return 2
    import torch
    from block_diffusion_speculative_dflash_amd import configs

    torch.cuda.init()
    wl = configs.WORKLOADS[args.workload]
    res = measure(args, wl, headline=True)
    if res is None:  # --pmc-probe
        return 0
    if not args.only:
        also = {}
        for other in configs.ALL:
            if other.name == wl.name or other.dims.dtype != configs.BF16:
                continue
            torch.cuda.empty_cache()
            r = measure(args, other, headline=False)
            also[other.name] = {key: r[key] for key in ("value", "unit", "ms_per_step", "committed_tok_s",
                                                        "accepted_tok_s", "mean_accept",
                                                        "planted_accept_matches", "step_roofline",
                                                        "roofline", "dev_error")}
        res["also"] = also
    print(json.dumps(res), flush=True)
    return 0


def measure(args, wl, headline: bool):
    """Prefill, capture and time one workload; returns its result record (None for
    a hardware-counter probe run)."""
    import torch
    from block_diffusion_speculative_dflash_amd import binding as bd
    from block_diffusion_speculative_dflash_amd import configs, harness, synth
    from block_diffusion_speculative_dflash_amd.roofline import (HBM_PEAK_GBS, MFMA_BF16_PEAK_TFLOPS,
                                                                  measured_head_traffic, step_cost)

    d = wl.dims
    if args.sink:
        from dataclasses import replace
        d = replace(d, sink=args.sink, cache_slots=d.cache_slots + args.sink)
    B, k, V = d.batch, d.block_k, d.vocab
    dev = "cuda"
    log(f"[bench] workload {wl.name}: {wl.description}")
    W = bd.pack_weights(d, synth.make_weights(d, seed=args.seed, device=dev))
    ctx = synth.make_context_lengths(wl, seed=args.seed)
    pre = np.minimum(ctx, wl.prefill)
    anchors = synth.make_anchors(d, seed=args.seed)
    cache = bd.alloc_cache(d, device=dev, ctx_len=ctx - pre, anchor=anchors)
    ws = bd.alloc_workspace(d, device=dev)

    # prefill: inject the committed context (all of it, or the last W for SWA); with
    # an attention sink, positions 0..S-1 first when the prefill starts past them
    n_max = d.max_inject_rows
    if d.sink and int((ctx - pre).min()) >= d.sink:
        cache["ctx_len"].zero_()
        sr = torch.full((B,), d.sink, dtype=torch.int32, device=dev)
        bd.dflash_fuse_inject(d, W, sink_taps(d, args.seed), sr, d.sink, True, cache, ws)
        cache["ctx_len"].copy_(torch.as_tensor(ctx - pre, dtype=torch.int32))
    n_pre = int(pre.max())
    for r0 in range(0, n_pre, n_max):
        taps = prefill_taps(d, n_pre, r0, args.seed)
        n_rows = torch.as_tensor(np.clip(pre - r0, 0, taps.shape[1]), dtype=torch.int32, device=dev)
        bd.dflash_fuse_inject(d, W, taps, n_rows, taps.shape[1], True, cache, ws)
    torch.cuda.synchronize()
    assert np.array_equal(cache["ctx_len"].cpu().numpy(), ctx), "prefill did not reach the context"
    log(f"[bench] prefilled {n_pre} rows; context {int(ctx.min())}..{int(ctx.max())}")

    if args.pmc_probe:
        draft = torch.zeros((B, k), dtype=torch.int32, device=dev)
        for _ in range(5):
            bd.dflash_draft_step(d, W, cache, draft, None, ws)
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] pmc probe done: 5 draft steps, 5 copies of 1073741824 bytes")
        return None

    # planted acceptance and the target stand-in tables
    kind, q = wl.accept
    if args.accept_q is not None:
        kind, q = "geometric", args.accept_q
    n_tab = args.warmup + args.steps + 8
    a_tab = synth.planted_accept(kind, q, k, n_tab, B, seed=args.seed)
    fill = synth.target_fill(k, n_tab, B, seed=args.seed)
    pool = [synth.make_taps(d, k + 1, seed=args.seed, stream=1 + i, device=dev) for i in range(4)]
    saved_ctx = cache["ctx_len"].clone()
    sampled = args.temperature > 0
    adaptive = args.adaptive
    loop = harness.RoundLoop(d, W, cache, ws, a_tab, fill, seed=args.seed, temperature=args.temperature,
                             adaptive=adaptive, persistent=args.persistent, device=dev)

    # eager warm-up of every code path, then capture one graph per taps slot
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        loop.round(pool[0])
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graphs = []
    for taps in pool:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            loop.round(taps)
        graphs.append(g)
    # the eager warm-up and the captures consumed table entries; restart the tables
    loop.restart(saved_ctx)
    torch.cuda.synchronize()
    acc_total, accept = loop.acc_total, loop.accept
    if adaptive:
        kb_total, aparams = loop.kb_total, loop.aparams
    if sampled:
        smp, logits, lse = loop.smp, loop.logits, loop.lse
    draft = loop.draft

    def run(n, s0):
        for s in range(s0, s0 + n):
            graphs[s % len(graphs)].replay()
            if wl.rewind and (s + 1) % wl.rewind == 0:
                cache["ctx_len"].copy_(saved_ctx)

    run(args.warmup, 0)
    torch.cuda.synchronize()
    tot0, acc0 = int(acc_total.item()), accept.clone()
    kb0 = int(kb_total.item()) if adaptive else 0
    t0 = time.perf_counter()
    run(args.steps, args.warmup)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    tot1 = int(acc_total.item())
    accepted = tot1 - tot0 - int(acc0.sum().item()) + int(accept.sum().item())
    elapsed = t1 - t0
    planted = int(a_tab[args.warmup:args.warmup + args.steps].sum())
    adapt_info = None
    if adaptive:
        final = cache["block_len"].cpu().numpy()
        adapt_info = {"mean_block_len": round((int(kb_total.item()) - kb0) / (args.steps * B), 4),
                      "final_block_len_hist": {str(v): int((final == v).sum()) for v in sorted(set(final.tolist()))},
                      "params": {"alpha": aparams.alpha, "theta_down": aparams.theta_down,
                                 "theta_off": aparams.theta_off, "theta_up": aparams.theta_up,
                                 "cooldown": aparams.cooldown}}
    err = int(cache["dev_error"].item())
    steps_per_s = args.steps / elapsed
    committed = accepted + args.steps * B
    log(f"[bench] {args.steps} steps in {elapsed * 1e3:.2f} ms: {steps_per_s:.1f} steps/s, "
        f"accepted {accepted} (planted {planted}), dev_error {err}")

    # dominant kernel: final norm + LM head + argmax, timed with HIP events around its
    # launch in eager draft steps, after --head-warmup untimed ones
    ev = HipEvents()
    pairs = [(ev.create(), ev.create()) for _ in range(args.head_launches)]

    def head_step(e0, e1):
        if sampled:
            bd.dflash_draft_step_sampled_timed(d, W, cache, smp, draft, logits, lse, ws, e0, e1)
        else:
            bd.dflash_draft_step_timed(d, W, cache, draft, None, ws, e0, e1)

    for _ in range(args.head_warmup if pairs else 0):
        head_step(*pairs[0])
    for e0, e1 in pairs:
        head_step(e0, e1)
    torch.cuda.synchronize()
    head_ms = float(np.mean([ev.elapsed_ms(e0, e1) for e0, e1 in pairs]))
    for e0, e1 in pairs:
        ev.destroy(e0)
        ev.destroy(e1)
    cost = step_cost(d, float(ctx.mean()), sampled=sampled)
    head_epi = "EPI_SAMPLE" if sampled else "EPI_ARGMAX"
    head_what = "LM head + Gumbel-max draw + logits/lse out" if sampled else "LM head + argmax"
    head_traffic = None if sampled else measured_head_traffic(wl.name)
    head_gbs = cost.head_bytes / (head_ms * 1e-3) / 1e9
    step_gbs = cost.bytes_total * steps_per_s / 1e9
    head_tfs = cost.head_flops / (head_ms * 1e-3) / 1e12
    step_tfs = cost.flops_total * steps_per_s / 1e12
    log(f"[bench] head kernel {head_ms * 1e3:.1f} us = {head_gbs:.0f} GB/s, {head_tfs:.1f} TFLOP/s; "
        f"step {step_gbs:.0f} GB/s, {step_tfs:.1f} TFLOP/s ({cost.bytes_total / 1e9:.3f} GB/step)")
    # batch x block >= 128 rows: the projections run on the tiled MFMA GEMM and the
    # step is compute-bound (bf16-class MFMA peak); below that it streams weights
    mfma_bound = d.dtype == configs.BF16 and B * k >= 128
    if mfma_bound:
        step_roof = {"bound": "mfma", "flops_per_step": cost.flops_total,
                     "achieved_TFLOPs": round(step_tfs, 1), "peak_TFLOPs": MFMA_BF16_PEAK_TFLOPS,
                     "frac": round(step_tfs / MFMA_BF16_PEAK_TFLOPS, 4)}
        head_roof = {"kernel": f"gemm_tiled_kernel<{head_epi}> (final norm + {head_what})",
                     "bound": "mfma", "achieved": round(head_tfs, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(head_tfs / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": head_traffic,
                     "avg_us": round(head_ms * 1e3, 2), "flops_per_launch": cost.head_flops}
    else:
        step_roof = {"bound": "hbm", "bytes_per_step": cost.bytes_total,
                     "achieved_GBs": round(step_gbs, 1), "peak_GBs": HBM_PEAK_GBS,
                     "frac": round(step_gbs / HBM_PEAK_GBS, 4)}
        head_roof = {"kernel": f"gemm_kernel<{head_epi}> (final norm + {head_what})",
                     "bound": "hbm", "achieved": round(head_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(head_gbs / HBM_PEAK_GBS, 4),
                     "traffic": head_traffic,
                     "avg_us": round(head_ms * 1e3, 2), "bytes_per_launch": cost.head_bytes}

    cpu = None
    if headline and not args.no_cpu_baseline:
        cpu = cpu_baseline(args, d, W, ctx, pre, anchors, a_tab)

    res = {
        "metric": "draft+verify block steps/s & accepted tok/s at batch B; % of HBM/MFMA roofline",
        "value": round(steps_per_s, 3),
        "unit": "block steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # a bf16 drafter's matrix-core operands, q/k/v and K/V cache are fp16 (its
        # weights and taps arrive as bf16, accumulation and residual are fp32)
        "dtype": "fp16" if d.dtype == configs.BF16 else "f32",
        "precision": ("bf16 weights and taps; fp16 MFMA operands, q/k/v and K/V cache; fp32 accumulation, "
                      "residual and softmax" if d.dtype == configs.BF16 else "fp32 throughout"),
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) taps, planted targets"
                + (", N(0,4) target logits with planted acceptance)" if sampled else ")"),
        "config": {"workload": wl.name},
        "options": {"accept": [kind, q], "temperature": args.temperature, "adaptive": adaptive,
                    "persistent": bool(args.persistent),
                    "sink": d.sink, "context": [int(ctx.min()), int(ctx.max())]},
        "accepted_tok_s": round(accepted / elapsed, 1),
        "committed_tok_s": round(committed / elapsed, 1),
        "mean_accept": round(accepted / (args.steps * B), 4),
        "planted_accept_matches": (accepted == planted) if not adaptive else None,
        "adaptive": adapt_info,
        "step_roofline": step_roof,
        "roofline": head_roof,
        "cpu_baseline": cpu,
        "dev_error": err,
    }
    return res


def prefill_taps(d, n_pre: int, r0: int, seed: int):
    """Taps of prefill rows r0 .. r0 + n_max of every sequence (one seeded draw per chunk)."""
    from block_diffusion_speculative_dflash_amd import synth
    return synth.make_taps(d, min(d.max_inject_rows, n_pre - r0), seed=seed, stream=10_000 + r0,
                           device="cuda")


def sink_taps(d, seed: int):
    """Taps of the attention-sink positions 0..S-1 of every sequence."""
    from block_diffusion_speculative_dflash_amd import synth
    return synth.make_taps(d, d.sink, seed=seed, stream=9_999, device="cuda")


def cpu_baseline(args, d, W, ctx, pre, anchors, a_tab):
    """The fp64 oracle, as it stands, on this host: a bounded sample of the same
    workload (sequence 0's block steps; at batch 1 that is the whole batch)."""
    import torch
    from block_diffusion_speculative_dflash_amd import synth
    from oracle import dflash_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        threads = max([t.get("num_threads", 1) for t in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = None
    k = d.block_k
    cores = len(os.sched_getaffinity(0))
    log(f"[bench] cpu baseline: oracle on sequence 0, {args.cpu_steps} block steps, {cores} cores")
    Wn = {n: t.float().cpu().numpy() for n, t in W.items() if n != "packed"}
    st = orc.new_state(d, batch=1, ctx_len=[int(ctx[0] - pre[0])], anchor=[int(anchors[0])])
    n_pre, n_all = int(pre[0]), int(pre.max())
    if d.sink and int((ctx - pre).min()) >= d.sink:
        st.ctx_len[0] = 0
        orc.fuse_inject(d, Wn, st, sink_taps(d, args.seed)[:1].float().cpu().numpy(), [d.sink], commit=True)
        st.ctx_len[0] = int(ctx[0] - pre[0])
    if n_pre:
        rows = [prefill_taps(d, n_all, r0, args.seed)[:1] for r0 in range(0, n_all, d.max_inject_rows)]
        taps = torch.cat(rows, dim=1)[:, :n_pre].float().cpu().numpy()
        orc.fuse_inject(d, Wn, st, taps, [n_pre], commit=True)
    taps_step = synth.make_taps(d, k + 1, seed=args.seed, stream=1, device="cuda")[:1].float().cpu().numpy()
    fill = synth.target_fill(k, 1, 1, seed=args.seed + 1)[0]
    temp = args.temperature
    if temp > 0:
        from oracle import sampling as sp
        fill_logits = synth.make_logits((1, k + 1, d.vocab), seed=args.seed, stream=31_337)
    t0 = time.perf_counter()
    committed = 0
    for s in range(args.cpu_steps):
        if temp > 0:
            # sampled round: Gumbel-max drafts, planted target logits, rejection sampling
            o = orc.draft_step(d, Wn, st, want_logits=True)
            sd = sp.sample_drafts(o["logits"], temp, args.seed + 1, s)
            tl = synth.plant_target_logits(torch.as_tensor(o["logits"], dtype=torch.float32), sd["draft"],
                                           a_tab[s, :1], fill_logits)
            orc.fuse_inject(d, Wn, st, taps_step, [k + 1], commit=False)
            r = sp.verify_sampled(sd["draft"], o["logits"], tl.double().numpy(), temp, args.seed + 1, s)
            sp.commit_sampled(d, st, r)
        else:
            o = orc.draft_step(d, Wn, st, want_logits=False)
            T = synth.plant_targets(o["draft"], a_tab[s, :1], fill, d.vocab)
            orc.fuse_inject(d, Wn, st, taps_step, [k + 1], commit=False)
            r = orc.verify_commit(d, st, o["draft"], T)
        committed += int(r["accept_len"][0]) + 1
    dt = time.perf_counter() - t0
    per_seq_step = dt / args.cpu_steps
    steps_per_s = 1.0 / (per_seq_step * d.batch)   # a full-batch block step costs B sequence steps
    return {"value": round(steps_per_s, 6), "unit": "block steps/s", "cores": cores,
            "blas_threads": threads, "kind": "oracle",
            "committed_tok_s": round(committed / dt, 4),
            "seconds": round(dt, 2),
            "sample": f"{args.cpu_steps} block steps of sequence 0 (of {d.batch}), fp64 numpy"
                      + (f", sampled at T={temp}" if temp > 0 else "")
                      + f"; full-batch rate = per-sequence rate / {d.batch}"}


if __name__ == "__main__":
    sys.exit(main())
