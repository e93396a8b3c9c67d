"""Full-size workloads on the GPU, checked against the fp64 oracle on sampled
sequences (every sequence's computation is independent of the others, so the
oracle runs only the sampled ones while the GPU runs the whole batch in the
launch configuration the benchmark times).

Every step compares, for every sampled sequence and with no margin gate, the
GPU's verify/commit of its own drafts against the oracle's verify_commit of the
same drafts and target tokens (integer work: bit-exact), besides the logits, the
margin-gated drafts and the K/V window.  The planted acceptance alternates
between draws from the workload's distribution and a* = 0: a round that accepts
nothing is decided by row 0 alone, so the margin-gated comparison of the oracle's
whole trajectory (accepted length, emitted tokens, committed state) admits a
sizeable share of sequence-steps, and each test asserts a minimum of them."""
from dataclasses import replace

import numpy as np
import pytest

from block_diffusion_speculative_dflash_amd import configs, synth
from tests.parity import ParityRun, say

pytestmark = pytest.mark.gpu

def _spread(ctx, n):
    """n sequences whose context lengths span the batch's range (ragged workloads)."""
    order = np.argsort(ctx, kind="stable")
    return sorted(int(order[i]) for i in np.linspace(0, len(ctx) - 1, n).round().astype(int))


# sampled sequences, steps, and the least number of margin-gated sequence-steps
CASES = {
    configs.C2.name: (lambda ctx: [0], 6, 1),
    configs.C3.name: (lambda ctx: list(range(8)), 4, 4),
    configs.C4.name: (lambda ctx: _spread(ctx, 8), 4, 4),
    configs.C5.name: (lambda ctx: [0, 37, 73, 110, 146, 183, 219, 255], 4, 4),
}


def planted_schedule(w, steps):
    """Planted a*: the workload's distribution on even steps, 0 on odd steps."""
    kind, q = w.accept
    a_tab = synth.planted_accept(kind, q, w.dims.block_k, steps, w.dims.batch, seed=0)
    a_tab[1::2] = 0
    return a_tab


def run_steps(name, run, a_tab, min_gated, block_lens=None):
    checked = excluded = 0
    for s in range(len(a_tab)):
        r = run.step(a_tab[s]) if block_lens is None else run.step(a_tab[s], block_len=block_lens[s])
        assert r.logits_ok, f"step {s}: max |dz| {r.logit_err} > 0.05"
        assert r.draft_mismatch == 0
        assert r.seqs_verified == len(run.sample) and r.verify_mismatch == 0, \
            f"step {s}: verify/commit of the GPU drafts differs from the oracle's for {r.verify_mismatch} sequences"
        assert r.state_mismatch == 0
        assert r.kv_ok, f"step {s}: kv error {r.kv_err}"
        checked += r.seqs_checked
        excluded += r.seqs_excluded
    say(f"[fullsize] {name}: {len(a_tab)} steps x {len(run.sample)} sequences; verify/commit on the GPU's "
        f"drafts exact for all; oracle trajectory margin-gated in {checked}, excluded {excluded}")
    assert checked >= min_gated, f"only {checked} sequence-steps passed the margin gate"
    assert run.dev_error() == 0


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", list(CASES))
def test_fullsize_parity(name):
    w = configs.WORKLOADS[name]
    d = w.dims
    ctx = synth.make_context_lengths(w, seed=0)
    pick, steps, min_gated = CASES[name]
    sample = pick(ctx)
    say(f"[fullsize] {name}: B={d.batch} k={d.block_k} L={d.n_layers} V={d.vocab} sample={sample} "
        f"contexts={[int(ctx[b]) for b in sample]}")
    W = synth.make_weights(d, seed=0, device="cuda")
    pre = np.minimum(ctx, w.prefill)
    run = ParityRun(d, W, ctx, synth.make_anchors(d), pre, sample=sample, seed=0)
    run_steps(name, run, planted_schedule(w, steps), min_gated)


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
    run = ParityRun(d, W, ctx, synth.make_anchors(d), pre, sample=[0, 3, 5, 7], seed=0)
    run_steps("sink", run, planted_schedule(w, 4), 2)


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


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", [configs.C4.name, configs.C5.name])
def test_fullsize_compacted_blocks(name):
    """Per-sequence block lengths (the runtime block size) at the two large batches,
    where the draft step compacts the live rows of shrunken blocks before the GEMMs:
    every sequence draws its own k_b in [0, k] each step (about half the rows live),
    the sampled sequences cover k_b = 0, k and values between."""
    w = configs.WORKLOADS[name]
    d = w.dims
    k, B = d.block_k, d.batch
    ctx = synth.make_context_lengths(w, seed=0)
    sample = CASES[name][0](ctx)
    rng = np.random.default_rng(11)
    steps = 3
    lens = rng.integers(0, k + 1, size=(steps, B)).astype(np.int64)
    for s in range(steps):  # the sampled sequences: 0, k and intermediate lengths
        lens[s, sample] = [(j * (k + 1) // len(sample) + 3 * s) % (k + 1) for j in range(len(sample))]
    a_tab = np.minimum(planted_schedule(w, steps), lens)
    say(f"[fullsize] compacted {name}: B={B} k={k} live rows per step {lens.sum(axis=1).tolist()} of {B * k}; "
        f"sample={sample} block lengths {[lens[s, sample].tolist() for s in range(steps)]}")
    W = synth.make_weights(d, seed=0, device="cuda")
    pre = np.minimum(ctx, w.prefill)
    run = ParityRun(d, W, ctx, synth.make_anchors(d), pre, sample=sample, seed=0)
    run_steps(f"compacted {name}", run, a_tab, 2, block_lens=lens)


@pytest.mark.timeout(900)
def test_fullsize_split_transposed_tiles():
    """The MiMo-shaped SWA drafter at batch 32 (256 block rows): the tile planner takes
    256 x 128 tiles for the projections and splits O and down 8 ways, so their
    transposed residual products go through the split-K reduction; SwiGLU runs
    transposed (unsplit) and the LM head persistent on the same tile shape."""
    w = replace(configs.C3, dims=replace(configs.C3.dims, batch=32))
    d = w.dims
    ctx = synth.make_context_lengths(w, seed=0)
    sample = [0, 11, 22, 31]
    say(f"[fullsize] split tiles: B={d.batch} k={d.block_k} L={d.n_layers} V={d.vocab} sample={sample}")
    W = synth.make_weights(d, seed=0, device="cuda")
    pre = np.minimum(ctx, w.prefill)
    run = ParityRun(d, W, ctx, synth.make_anchors(d), pre, sample=sample, seed=0)
    run_steps("split tiles", run, planted_schedule(w, 4), 2)


@pytest.mark.timeout(900)
def test_fullsize_persistent_tiles_k_steps_not_multiple_of_four():
    """The same drafter with hidden 4032: the projections that read the hidden state
    take 126 K steps, not a whole number of groups of four, so the persistent LM head
    and SwiGLU issue each next tile's first stages after the K loop rather than during
    its last steps; O, down and the fusion GEMM end in a half-filled 128-column tile
    (63 column tiles), and the RMSNorm partial sums (63 per row) take the scalar sum."""
    w = replace(configs.C3, dims=replace(configs.C3.dims, batch=32, hidden=4032))
    d = w.dims
    ctx = synth.make_context_lengths(w, seed=1)
    sample = [3, 16, 29]
    say(f"[fullsize] hidden 4032: B={d.batch} k={d.block_k} L={d.n_layers} V={d.vocab} sample={sample}")
    W = synth.make_weights(d, seed=1, device="cuda")
    pre = np.minimum(ctx, w.prefill)
    run = ParityRun(d, W, ctx, synth.make_anchors(d), pre, sample=sample, seed=1)
    run_steps("hidden 4032", run, planted_schedule(w, 4), 2)
