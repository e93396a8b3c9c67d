"""The draft step as one persistent kernel per layer (dflash_draft_step_persistent:
QKV -> attention -> key-split merge -> O -> gate/up -> down inside one launch, grid
barriers between the phases) against the separate-kernel draft step and the fp64
oracle.

Where every sequence's keys are in one piece or split into at least 8 (the merge
then sums in the separate kernel's order) the persistent step must give the same
drafts and logits bitwise; elsewhere it must meet the oracle parity rules.  The
full-size Qwen3-8B-shaped batch-1 drafter (context 4096, 17 key splits) and the
MiMo-shaped batch-8 SWA drafter run bitwise over several decode rounds through the
benchmark's round loop, which replays the persistent step inside a HIP graph."""
from dataclasses import replace

import numpy as np
import pytest
import torch

from block_diffusion_speculative_dflash_amd import binding as bd
from block_diffusion_speculative_dflash_amd import configs, harness, synth
from block_diffusion_speculative_dflash_amd.configs import BF16
from tests.parity import ParityRun, say

pytestmark = pytest.mark.gpu


def _small(**kw):
    base = dict(batch=2, n_q_heads=4, n_kv_heads=2, head_dim=128, hidden=512, tap_dim=128, ffn=1000,
                vocab=2000, window=64, cache_slots=72, dtype=BF16)
    base.update(kw)
    return replace(configs.C1.dims, **base)


def _both(d, ctx, pre):
    """Drafts and logits of the separate-kernel step and of the persistent step on the
    same prefilled state."""
    W = bd.pack_weights(d, synth.make_weights(d, seed=0, device="cuda"))
    cache = bd.alloc_cache(d, ctx_len=np.asarray(ctx) - np.asarray(pre), anchor=synth.make_anchors(d))
    ws = bd.alloc_workspace(d)
    n = int(max(pre))
    for r0 in range(0, n, d.max_inject_rows):
        m = min(d.max_inject_rows, n - r0)
        taps = synth.make_taps(d, m, seed=0, stream=40_000 + r0, device="cuda")
        rows = torch.as_tensor(np.clip(np.asarray(pre) - r0, 0, m), dtype=torch.int32, device="cuda")
        bd.dflash_fuse_inject(d, W, taps, rows, m, True, cache, ws)
    out = []
    for fn in (bd.dflash_draft_step, bd.dflash_draft_step_persistent):
        dr = torch.empty((d.batch, d.block_k), dtype=torch.int32, device="cuda")
        z = torch.empty((d.batch, d.block_k, d.vocab), dtype=torch.float32, device="cuda")
        fn(d, W, cache, dr, z, ws)
        torch.cuda.synchronize()
        out.append((dr.cpu(), z.cpu()))
    assert int(cache["dev_error"].item()) == 0
    return out


@pytest.mark.parametrize("case", ["b2_no_split", "b4_k16_no_split", "b1_k8_nine_splits", "b8_k8_rows64"])
def test_persistent_step_equals_separate_kernels_bitwise(case):
    if case == "b2_no_split":
        d, ctx, pre = _small(), [70, 64], [64, 64]
    elif case == "b4_k16_no_split":
        d = _small(batch=4, block_k=16, cache_slots=80, max_inject_rows=64)
        ctx, pre = [40, 50, 60, 64], [40, 50, 60, 64]
    elif case == "b1_k8_nine_splits":
        d = _small(batch=1, window=2300, cache_slots=2308, max_inject_rows=64)
        ctx, pre = [2200], [2200]
    else:
        d, ctx, pre = _small(batch=8, window=128, cache_slots=136), [300] * 8, [128] * 8
    say(f"[persistent] {case}: {d}")
    (d0, z0), (d1, z1) = _both(d, ctx, pre)
    assert torch.equal(d0, d1), f"{case}: drafts differ"
    assert torch.equal(z0, z1), f"{case}: logits differ (max {float((z0 - z1).abs().max())})"
    say(f"[persistent] {case}: drafts and logits bitwise equal to the separate kernels")


def test_persistent_step_matches_the_oracle():
    """Key splits of 2..7 pieces (merge order differs from the separate kernels): the
    oracle parity rules, several rounds, GQA, ragged contexts."""
    d = _small(batch=3, block_k=4, window=1300, cache_slots=1304, max_inject_rows=64)
    say(f"[persistent] oracle parity {d}")
    W = synth.make_weights(d, seed=0, device="cuda")
    ctx = [1290, 700, 1050]
    run = ParityRun(d, W, ctx, synth.make_anchors(d), ctx, seed=0, persistent=True)
    for s, a in enumerate([[4, 0, 2], [1, 3, 4], [2, 2, 0]]):
        r = run.step(a)
        assert r.ok, f"step {s}: {r}"
    assert run.dev_error() == 0


def test_persistent_rejects_what_it_does_not_cover():
    d = configs.C1.dims  # fp32, head_dim 64
    W = bd.pack_weights(d, synth.make_weights(d, seed=0, device="cuda"))
    cache = bd.alloc_cache(d)
    ws = bd.alloc_workspace(d)
    dr = torch.empty((d.batch, d.block_k), dtype=torch.int32, device="cuda")
    with pytest.raises(bd.DFlashError) as e:
        bd.dflash_draft_step_persistent(d, W, cache, dr, None, ws)
    assert e.value.status == bd.DFLASH_E_UNSUPPORTED


@pytest.mark.timeout(900)
@pytest.mark.parametrize("wl", [configs.C2, configs.C3], ids=lambda w: w.name)
def test_persistent_rounds_in_graphs_bitwise(wl):
    """The benchmark's round loop (draft, target stand-in, injection, verification) with
    the persistent draft step, eager and replayed from HIP graphs, against the same
    rounds with the separate-kernel draft step: every round bitwise equal."""
    d = wl.dims
    say(f"[persistent] rounds {wl.name}")
    W = bd.pack_weights(d, synth.make_weights(d, seed=0, device="cuda"))
    ctx = synth.make_context_lengths(wl, seed=0)
    pre = np.minimum(ctx, wl.prefill)
    rounds = 6
    kind, q = wl.accept
    a_tab = synth.planted_accept(kind, q, d.block_k, rounds + 8, d.batch, seed=0)
    fill = synth.target_fill(d.block_k, rounds + 8, d.batch, seed=0)
    pool = [synth.make_taps(d, d.block_k + 1, seed=0, stream=1 + i, device="cuda") for i in range(4)]
    recs = {}
    for mode in ("separate", "persistent", "persistent_graph"):
        cache = bd.alloc_cache(d, ctx_len=ctx - pre, anchor=synth.make_anchors(d))
        ws = bd.alloc_workspace(d)
        n_pre, n_max = int(pre.max()), d.max_inject_rows
        for r0 in range(0, n_pre, n_max):
            taps = synth.make_taps(d, min(n_max, n_pre - r0), seed=0, stream=10_000 + r0, device="cuda")
            rows = torch.as_tensor(np.clip(pre - r0, 0, taps.shape[1]), dtype=torch.int32, device="cuda")
            bd.dflash_fuse_inject(d, W, taps, rows, taps.shape[1], True, cache, ws)
        torch.cuda.synchronize()
        loop = harness.RoundLoop(d, W, cache, ws, a_tab, fill, persistent=mode != "separate")
        graphs = None
        if mode == "persistent_graph":
            saved = cache["ctx_len"].clone()
            snap = {n: t.clone() for n, t in cache.items()}
            graphs = []
            for taps in pool:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    loop.round(taps)
                graphs.append(g)
            for n, t in snap.items():
                cache[n].copy_(t)
            loop.restart(saved)
            torch.cuda.synchronize()
        out = []
        for r in range(rounds):
            if graphs is None:
                loop.round(pool[r % 4])
            else:
                graphs[r % 4].replay()
            torch.cuda.synchronize()
            out.append([t.cpu().clone() for t in (loop.draft, loop.accept, loop.out_tok, cache["ctx_len"],
                                                  cache["anchor"])])
        out.append([cache["k"].cpu(), cache["v"].cpu()])
        assert int(cache["dev_error"].item()) == 0, f"{mode}: dev_error {int(cache['dev_error'].item())}"
        recs[mode] = out
        del cache, ws, loop, graphs
        torch.cuda.empty_cache()
    for mode in ("persistent", "persistent_graph"):
        for r, (a, b) in enumerate(zip(recs["separate"], recs[mode])):
            for x, y in zip(a, b):
                assert torch.equal(x, y), f"{mode}: round {r} differs from the separate kernels"
    say(f"[persistent] {wl.name}: {rounds} rounds bitwise equal (eager and graph replays); "
        f"accepted {[int(x[1].sum()) for x in recs['persistent'][:rounds]]}")
