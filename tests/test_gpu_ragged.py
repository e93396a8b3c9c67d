"""GPU parity of per-sequence block lengths and of the runtime block-size
controller (through the C ABI) against the fp64 oracle.

* ragged rounds: every sequence drafts its own k_b in [0, k] (0 = speculation off),
  greedy and sampled, streaming and tiled LM heads, fp32 and bf16, with the parity
  gates of ParityRun; drafts past a block must read -1;
* the controller kernel against oracle/adaptive.py over long random trajectories:
  block lengths, cool-down counters and the float32 moving average bit-exact;
* closed loop: the controller chooses each round's block lengths from the accepted
  lengths of the round before, on both sides.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

from block_diffusion_speculative_dflash_amd import binding as bd
from block_diffusion_speculative_dflash_amd import configs, synth
from block_diffusion_speculative_dflash_amd.configs import BF16
from oracle import adaptive as ad
from tests.parity import ParityRun, say

pytestmark = pytest.mark.gpu


def _assert_ok(reps, min_checked=0.5):
    for i, r in enumerate(reps):
        assert r.logits_ok, f"round {i}: logit error {r.logit_err}"
        assert r.draft_mismatch == 0, f"round {i}: {r.draft_mismatch} draft mismatches"
        assert r.state_mismatch == 0, f"round {i}: {r.state_mismatch} state mismatches"
        assert r.kv_ok, f"round {i}: kv error {r.kv_err}"
    # bf16 greedy gates at the fixed 0.1 margin: the tiny model's logits span only ~1.2
    assert sum(r.seqs_checked for r in reps) >= min_checked * sum(r.seqs_checked + r.seqs_excluded for r in reps)


def _ragged_run(d, ctx, lens, a_stars, sampled_T=None, seed=0):
    W = synth.make_weights(d, seed=seed, device="cuda")
    run = ParityRun(d, W, ctx, synth.make_anchors(d, seed=seed), [min(c, d.window) for c in ctx], seed=seed)
    reps = []
    for s, (kb, a) in enumerate(zip(lens, a_stars)):
        if sampled_T is None:
            reps.append(run.step(a, block_len=kb))
        else:
            reps.append(run.step_sampled(a, sampled_T, seed=99, soft=0.2, block_len=kb))
    assert run.dev_error() == 0
    return reps


def test_ragged_blocks_greedy_fp32():
    d = replace(configs.C1.dims, batch=4, window=24, cache_slots=32, max_inject_rows=16)
    say(f"[ragged] greedy fp32 {d}")
    lens = [[8, 3, 0, 1], [1, 8, 5, 0], [0, 0, 8, 4], [4, 2, 1, 8]]
    _assert_ok(_ragged_run(d, [40, 9, 0, 25], lens, [[8, 2, 0, 1], [1, 8, 3, 0], [0, 0, 8, 4], [2, 2, 1, 6]]))


def test_ragged_blocks_greedy_bf16_gqa():
    d = replace(configs.C1.dims, batch=3, n_q_heads=4, n_kv_heads=2, window=16, cache_slots=24, dtype=BF16,
                max_inject_rows=16)
    say(f"[ragged] greedy bf16 {d}")
    lens = [[8, 4, 0], [4, 0, 8], [0, 8, 4]]
    _assert_ok(_ragged_run(d, [30, 17, 5], lens, [[8, 1, 0], [3, 0, 5], [0, 8, 4]]), min_checked=0.25)


def test_ragged_blocks_sampled_bf16():
    d = replace(configs.C1.dims, batch=3, dtype=BF16, window=32, cache_slots=40)
    say(f"[ragged] sampled bf16 {d}")
    lens = [[8, 4, 0], [0, 8, 4], [4, 0, 8]]
    reps = _ragged_run(d, [50, 20, 33], lens, [[8, 2, 0], [0, 8, 4], [1, 0, 8]], sampled_T=1.0)
    for i, r in enumerate(reps):
        assert r.lse_ok, f"round {i}: lse error {r.lse_err}"
    _assert_ok(reps)


def test_ragged_blocks_tiled_bf16():
    """160 block rows: the tiled LM head and GEMMs with per-sequence block lengths."""
    d = replace(configs.C1.dims, batch=20, block_k=8, n_layers=2, n_q_heads=4, n_kv_heads=2, ffn=1100,
                vocab=40003, window=32, cache_slots=40, dtype=BF16, max_inject_rows=16)
    say(f"[ragged] tiled {d}")
    ctx = [40 + (7 * b) % 23 for b in range(d.batch)]
    lens = [[(3 * b + s) % 9 for b in range(d.batch)] for s in range(2)]
    _assert_ok(_ragged_run(d, ctx, lens, [[(5 * b + s) % 9 for b in range(d.batch)] for s in range(2)]),
               min_checked=0.25)


@pytest.mark.parametrize("k", [8, 1, 10])
def test_adapt_kernel_matches_the_oracle(k):
    """300 sequences, 80 rounds of random accepted lengths (a <= k_b): block lengths,
    cool-downs and the float32 averages bit-exact every round."""
    B = 300
    d = replace(configs.C1.dims, batch=B, block_k=k, window=32, cache_slots=32 + k, max_inject_rows=max(16, k + 1))
    params = ad.AdaptParams(alpha=0.3, theta_down=4.0, theta_off=2.0, theta_up=6.0, cooldown=5)
    cp = bd.adapt_params(params.alpha, params.theta_down, params.theta_off, params.theta_up, params.cooldown)
    cache = bd.alloc_cache(d, ctx_len=np.zeros(B, np.int64))
    rng = np.random.default_rng(k)
    kb = rng.choice([0, k // 2 if k > 1 else 0, k], size=B).astype(np.int64)
    off = np.where(kb == 0, rng.integers(1, 6, size=B), 0).astype(np.int64)
    m = rng.uniform(1.0, 9.0, size=B).astype(np.float32)
    cache["block_len"] = torch.as_tensor(kb, dtype=torch.int32, device="cuda")
    ema = torch.as_tensor(m, device="cuda")
    off_d = torch.as_tensor(off, dtype=torch.int32, device="cuda")
    say(f"[ragged] adapt kernel k={k} B={B}")
    for rnd in range(80):
        # acceptance that drifts: good phases and bad phases per sequence
        good = ((np.arange(B) + rnd // 10) % 3) != 0
        acc = np.array([rng.integers(0, int(x) + 1) if x > 0 else rng.integers(0, k + 1) for x in kb])
        acc = np.where(good & (kb > 0), kb, acc)
        acc_d = torch.as_tensor(acc, dtype=torch.int32, device="cuda")
        bd.dflash_adapt_block_len(d, cp, acc_d, cache, ema, off_d)
        torch.cuda.synchronize()
        kb, m, off = ad.adapt(params, k, kb, m, off, acc)
        assert np.array_equal(cache["block_len"].cpu().numpy(), kb), f"round {rnd}: block lengths"
        assert np.array_equal(off_d.cpu().numpy(), off), f"round {rnd}: cool-downs"
        assert np.array_equal(ema.cpu().numpy().view(np.uint32), m.view(np.uint32)), f"round {rnd}: averages"
    assert int(cache["dev_error"].item()) == 0
    if k > 1:
        assert len(set(kb.tolist())) > 1


def test_controller_closes_the_loop():
    """The controller picks every round's block lengths from the previous round's
    accepted lengths on both sides (planted low acceptance drives sequences down the
    ladder, high acceptance back up)."""
    d = replace(configs.C1.dims, batch=4, dtype=BF16, window=32, cache_slots=40)
    params = ad.AdaptParams(alpha=0.5, theta_down=4.0, theta_off=2.0, theta_up=6.0, cooldown=2)
    cp = bd.adapt_params(params.alpha, params.theta_down, params.theta_off, params.theta_up, params.cooldown)
    W = synth.make_weights(d, seed=3, device="cuda")
    ctx = [40, 33, 50, 21]
    run = ParityRun(d, W, ctx, synth.make_anchors(d, seed=3), [min(c, 32) for c in ctx], seed=3)
    B, k = d.batch, d.block_k
    kb = np.full(B, k, np.int64)
    m = np.full(B, 6.0, np.float32)
    off = np.zeros(B, np.int64)
    ema = torch.as_tensor(m, device="cuda")
    off_d = torch.zeros(B, dtype=torch.int32, device="cuda")
    seen = set()
    for rnd in range(12):
        plan = np.where((np.arange(B) + (rnd >= 6)) % 2 == 0, 0, k)       # poor then good acceptance
        rep = run.step(plan, block_len=kb)
        assert rep.state_mismatch == 0 and rep.draft_mismatch == 0
        acc = torch.as_tensor(rep.accept, dtype=torch.int32, device="cuda")
        bd.dflash_adapt_block_len(d, cp, acc, run.cache, ema, off_d)
        torch.cuda.synchronize()
        kb, m, off = ad.adapt(params, k, kb, m, off, np.asarray(rep.accept))
        assert np.array_equal(run.cache["block_len"].cpu().numpy(), kb), f"round {rnd}"
        seen |= set(kb.tolist())
    assert run.dev_error() == 0
    assert {0, k // 2, k} <= seen
