"""Full-size workloads on the GPU, checked against the fp64 oracle on sampled
sequences (every sequence's computation is independent of the others, so the
oracle runs only the sampled ones while the GPU runs the whole batch in the
launch configuration the benchmark times).  Two block steps each, with planted
acceptance drawn from the workload's distribution."""
from dataclasses import replace

import numpy as np
import pytest

from block_diffusion_speculative_dflash_amd import configs, synth
from tests.parity import ParityRun, say

pytestmark = pytest.mark.gpu

CASES = {
    configs.C2.name: [0],
    configs.C3.name: [0, 5],
    configs.C4.name: [0, 37],
    configs.C5.name: [0, 255],
}


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", list(CASES))
def test_fullsize_parity(name):
    w = configs.WORKLOADS[name]
    d = w.dims
    say(f"[fullsize] {name}: B={d.batch} k={d.block_k} L={d.n_layers} V={d.vocab} sample={CASES[name]}")
    W = synth.make_weights(d, seed=0, device="cuda")
    ctx = synth.make_context_lengths(w, seed=0)
    pre = np.minimum(ctx, w.prefill)
    kind, q = w.accept
    a_tab = synth.planted_accept(kind, q, d.block_k, 2, d.batch, seed=0)
    run = ParityRun(d, W, ctx, synth.make_anchors(d), pre, sample=CASES[name], seed=0)
    for s in range(2):
        r = run.step(a_tab[s])
        assert r.logits_ok, f"step {s}: max |dz| {r.logit_err} > 0.05"
        assert r.draft_mismatch == 0
        assert r.state_mismatch == 0
        assert r.kv_ok, f"step {s}: kv error {r.kv_err}"
    assert run.dev_error() == 0


@pytest.mark.timeout(900)
def test_fullsize_swa_with_attention_sink():
    """The MiMo-shaped SWA workload (batch 8, window 128, logical position 65536) with
    an attention sink of 4: positions 0..3 stay visible beside the window."""
    w = configs.C3
    d = replace(w.dims, sink=4, cache_slots=w.dims.cache_slots + 4)
    say(f"[fullsize] sink: B={d.batch} k={d.block_k} sink={d.sink} W={d.window} C={d.cache_slots}")
    W = synth.make_weights(d, seed=0, device="cuda")
    ctx = synth.make_context_lengths(w, seed=0)
    pre = np.minimum(ctx, w.prefill)
    kind, q = w.accept
    a_tab = synth.planted_accept(kind, q, d.block_k, 2, d.batch, seed=0)
    run = ParityRun(d, W, ctx, synth.make_anchors(d), pre, sample=[0, 5], seed=0)
    for s in range(2):
        r = run.step(a_tab[s])
        assert r.logits_ok, f"step {s}: max |dz| {r.logit_err} > 0.05"
        assert r.draft_mismatch == 0
        assert r.state_mismatch == 0
        assert r.kv_ok, f"step {s}: kv error {r.kv_err}"
    assert run.dev_error() == 0


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,sample", [(configs.C2.name, [0]), (configs.C5.name, [0, 100, 255])])
def test_fullsize_sampled_round(name, sample):
    """One sampled round (temperature 1) at full size: Gumbel-max drafts from the
    fused LM head, rejection-sampling verification over the full vocabulary."""
    w = configs.WORKLOADS[name]
    d = w.dims
    say(f"[fullsize] sampled {name}: B={d.batch} k={d.block_k} V={d.vocab} sample={sample}")
    W = synth.make_weights(d, seed=0, device="cuda")
    ctx = synth.make_context_lengths(w, seed=0)
    pre = np.minimum(ctx, w.prefill)
    kind, q = w.accept
    a_tab = synth.planted_accept(kind, q, d.block_k, 1, d.batch, seed=0)
    run = ParityRun(d, W, ctx, synth.make_anchors(d), pre, sample=sample, seed=0)
    r = run.step_sampled(a_tab[0], 1.0, seed=5)
    assert r.logits_ok, f"max |dz| {r.logit_err} > 0.05"
    assert r.lse_ok, f"lse error {r.lse_err}"
    assert r.draft_mismatch == 0
    assert r.state_mismatch == 0
    assert r.kv_ok, f"kv error {r.kv_err}"
    assert run.dev_error() == 0
