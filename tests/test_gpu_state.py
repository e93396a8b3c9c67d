"""The caller-owned decode state and the library's scratch memory.

* Snapshot / resume: the whole decode state (K/V rings, committed lengths, anchors)
  copied to host memory mid-decode and restored into freshly allocated buffers,
  with a fresh workspace, continues bitwise as the original does (the zhihu
  answer's §5.2: the injected context features persist in the drafter's KV cache,
  so that cache is the state a serving runtime would checkpoint).
* NaN poisoning (dflash_debug_poison): the workspace's scratch filled with NaN
  before every call and the rolled-back ring rows after every verification leave
  every result bitwise unchanged and parity with the oracle green, so no kernel
  reads memory that an earlier call left behind or a rolled-back row.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

from block_diffusion_speculative_dflash_amd import binding as bd
from block_diffusion_speculative_dflash_amd import configs, synth
from block_diffusion_speculative_dflash_amd.configs import BF16, F32
from tests.parity import ParityRun, say

pytestmark = pytest.mark.gpu

STATE_KEYS = ("k", "v", "ctx_len", "anchor")


def _rounds(d, W, cache, ws, n, start, seed=0):
    """n greedy rounds from round index `start`: draft, targets planted from the
    drafts (a* from a seeded table), tentative injection, verification.  Returns the
    per-round drafts, accepted lengths, emitted tokens and committed state."""
    k = d.block_k
    a_tab = synth.planted_accept("uniform", None, k, start + n, d.batch, seed=seed)
    fill = synth.target_fill(k, start + n, d.batch, seed=seed)
    out = []
    for r in range(start, start + n):
        draft = torch.empty((d.batch, k), dtype=torch.int32, device="cuda")
        bd.dflash_draft_step(d, W, cache, draft, None, ws)
        T = synth.plant_targets(draft.cpu().numpy(), a_tab[r], fill[r], d.vocab)
        taps = synth.make_taps(d, k + 1, seed=seed, stream=500 + r, device="cuda")
        bd.dflash_fuse_inject(d, W, taps, torch.full((d.batch,), k + 1, dtype=torch.int32, device="cuda"),
                              k + 1, False, cache, ws)
        acc = torch.empty(d.batch, dtype=torch.int32, device="cuda")
        emitted = torch.empty((d.batch, k + 1), dtype=torch.int32, device="cuda")
        bd.dflash_verify_commit(d, draft, torch.as_tensor(T).cuda(), cache, acc, emitted)
        torch.cuda.synchronize()
        out.append({"draft": draft.cpu().numpy(), "accept": acc.cpu().numpy(), "out": emitted.cpu().numpy(),
                    "ctx": cache["ctx_len"].cpu().numpy(), "anchor": cache["anchor"].cpu().numpy()})
    return out


def _prefilled(d, ctx, seed=0):
    W = bd.pack_weights(d, synth.make_weights(d, seed=seed, device="cuda"))
    cache = bd.alloc_cache(d, ctx_len=np.zeros(d.batch, np.int64), anchor=synth.make_anchors(d, seed=seed))
    ws = bd.alloc_workspace(d)
    n = int(max(ctx))
    for r0 in range(0, n, d.max_inject_rows):
        m = min(d.max_inject_rows, n - r0)
        taps = synth.make_taps(d, m, seed=seed, stream=20_000 + r0, device="cuda")
        rows = torch.as_tensor(np.clip(np.asarray(ctx) - r0, 0, m), dtype=torch.int32, device="cuda")
        bd.dflash_fuse_inject(d, W, taps, rows, m, True, cache, ws)
    torch.cuda.synchronize()
    return W, cache, ws


@pytest.mark.parametrize("case", ["gqa_swa_ring_bf16", "mimo_swa_b8"])
def test_snapshot_resume_is_bitwise_identical(case):
    if case == "gqa_swa_ring_bf16":
        d = replace(configs.C1.dims, batch=3, block_k=4, n_q_heads=4, n_kv_heads=2, window=16,
                    cache_slots=20, dtype=BF16, max_inject_rows=16)
        ctx = [40, 17, 5]
    else:
        d = configs.C3.dims
        ctx = [128] * d.batch
    say(f"[state] snapshot/resume {case}: {d}")
    W, cache, ws = _prefilled(d, ctx)
    _rounds(d, W, cache, ws, 2, 0)
    snap = {n: cache[n].cpu().clone() for n in STATE_KEYS}       # host copy mid-decode
    ref = _rounds(d, W, cache, ws, 3, 2)
    kv_ref = (cache["k"].cpu(), cache["v"].cpu())

    fresh = bd.alloc_cache(d)
    for n in STATE_KEYS:
        fresh[n].copy_(snap[n])
    ws2 = bd.alloc_workspace(d)
    got = _rounds(d, W, fresh, ws2, 3, 2)
    for r, (a, b) in enumerate(zip(ref, got)):
        for key in a:
            assert np.array_equal(a[key], b[key]), f"round {r}: {key} differs after resume"
    assert torch.equal(fresh["k"].cpu(), kv_ref[0]) and torch.equal(fresh["v"].cpu(), kv_ref[1])
    assert int(cache["dev_error"].item()) == 0 and int(fresh["dev_error"].item()) == 0
    say(f"[state] {case}: 3 rounds after resume bitwise equal (accept {[list(x['accept']) for x in got]})")


POISON_CASES = {
    "tiny_fp32": (configs.C1.dims, [128], [128], [[8], [3], [0], [5]], None),
    "gqa_swa_ring_bf16": (replace(configs.C1.dims, batch=3, block_k=4, n_q_heads=4, n_kv_heads=2, window=16,
                                  cache_slots=20, dtype=BF16, max_inject_rows=16),
                          [40, 17, 5], [40, 17, 5], [[4, 0, 2], [1, 4, 3], [2, 2, 4]], None),
    "sink_fp32": (replace(configs.C1.dims, batch=2, block_k=4, n_layers=1, window=12, sink=2,
                          cache_slots=2 + 12 + 4 + 3, max_inject_rows=64),
                  [45, 33], [45, 33], [[2, 4], [4, 1], [0, 3]], None),
    "tiled_b32_bf16": (replace(configs.C1.dims, batch=32, block_k=8, n_q_heads=4, n_kv_heads=2, window=48,
                               cache_slots=56, dtype=BF16, max_inject_rows=16),
                       [60] * 32, [48] * 32, [[(3 * b + s) % 9 for b in range(32)] for s in range(2)], None),
    "ffn_pad_sampled_bf16": (replace(configs.C1.dims, batch=2, block_k=6, dtype=BF16), [70, 64], [70, 64],
                             [[6, 2], [1, 6]], 1.0),
    # per-sequence block lengths on the tiled GEMMs: the compacted rows
    "compacted_b32_bf16": (replace(configs.C1.dims, batch=32, block_k=8, n_q_heads=4, n_kv_heads=2, window=48,
                                   cache_slots=56, dtype=BF16, max_inject_rows=16),
                           [60] * 32, [48] * 32, [[(3 * b + s) % 7 for b in range(32)] for s in range(2)], None,
                           [[(5 * b + 2 * s) % 9 for b in range(32)] for s in range(2)]),
}


@pytest.mark.parametrize("case", list(POISON_CASES))
def test_nan_poison_leaves_results_unchanged(case):
    d, ctx, pre, steps, temp = POISON_CASES[case][:5]
    lens = POISON_CASES[case][5] if len(POISON_CASES[case]) > 5 else [None] * len(steps)
    say(f"[state] poison {case}: {d}")
    runs = []
    for poison in (False, True):
        W = synth.make_weights(d, seed=0, device="cuda")
        run = ParityRun(d, W, ctx, synth.make_anchors(d), pre, seed=0, poison=poison)
        recs = []
        for a, kb in zip(steps, lens):
            rep = run.step_sampled(a, temp, seed=9) if temp else run.step(a, block_len=kb)
            assert rep.ok, f"poison={poison}: {rep}"
            rec = {n: t.cpu() for n, t in run.last.items()}
            if kb is not None:  # logits rows past a block are not written: compare the live ones
                live = torch.arange(d.block_k)[None, :] < torch.as_tensor(kb)[:, None]
                rec["logits"][~live] = 0.0
            assert bool(torch.isfinite(rec["logits"]).all())
            recs.append(rec)
        assert run.dev_error() == 0
        runs.append(recs)
    for r, (a, b) in enumerate(zip(*runs)):
        for key in a:
            assert torch.equal(a[key], b[key]), f"step {r}: {key} changed under poisoning"
    say(f"[state] poison {case}: {len(steps)} steps bitwise equal with and without poisoning")
