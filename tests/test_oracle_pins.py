"""Pins of the fp64 oracle against things other than itself (CPU only).

* library special cases (torch fp64 RMSNorm / SiLU / linear / SDPA);
* the RoFormer complex-rotation form of RoPE and its invariants;
* the scalar brute-force twin (no ring, committed history only) on tiny shapes;
* invariants: window >= context is full attention, block of 1 is a decode step,
  a global position shift leaves logits unchanged, ring rotation leaves logits
  unchanged, the block is bidirectional, tentative rows + rollback equal
  injecting only the committed rows, exhaustive greedy verification;
* the attention sink (first s positions stay visible): brute force with its own
  visibility rule, over steps with rollback; a sink inside the window changes
  nothing; a block of one with a sink is a decode step.
"""
import itertools
from dataclasses import replace

import numpy as np
import pytest
import torch

from block_diffusion_speculative_dflash_amd import synth
from oracle import bruteforce as bf
from oracle import dflash_oracle as orc
from tests.helpers import prefilled, random_taps, tiny_dims, tiny_weights, with_sink, with_window

RNG = np.random.default_rng(1234)


# ---------------------------------------------------------------- I1 library
def test_rms_norm_matches_torch():
    x, g = RNG.normal(size=(3, 5, 16)), RNG.normal(size=16)
    ref = torch.nn.functional.rms_norm(torch.tensor(x), (16,), weight=torch.tensor(g), eps=1e-6)
    np.testing.assert_allclose(orc.rms_norm(x, g, 1e-6), ref.numpy(), rtol=1e-13, atol=1e-13)


def test_silu_and_linear_match_torch():
    x, W = RNG.normal(size=(7, 9)), RNG.normal(size=(5, 9))
    np.testing.assert_allclose(orc.silu(x), torch.nn.functional.silu(torch.tensor(x)).numpy(),
                               rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(orc.linear(x, W),
                               torch.nn.functional.linear(torch.tensor(x), torch.tensor(W)).numpy(),
                               rtol=1e-13, atol=1e-13)


def test_linear_chunking_is_exact():
    x, W = RNG.normal(size=(3, 8)), RNG.normal(size=(20000, 8))
    np.testing.assert_allclose(orc.linear(x, W), x @ W.T, rtol=1e-13, atol=1e-13)


def test_attend_matches_sdpa_with_explicit_mask():
    q, k, v = RNG.normal(size=(6, 16)), RNG.normal(size=(11, 16)), RNG.normal(size=(11, 16))
    mask = torch.ones(6, 11, dtype=torch.bool)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q)[None], torch.tensor(k)[None], torch.tensor(v)[None], attn_mask=mask)
    np.testing.assert_allclose(orc.attend(q, k, v), ref[0].numpy(), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- RoPE
@pytest.mark.parametrize("pos", [0, 1, 17, 65535, 262151])
def test_rope_is_complex_rotation(pos):
    x = RNG.normal(size=128)
    ref = bf.rotate(list(x), pos, 1e6)
    np.testing.assert_allclose(orc.rope(x, pos, 1e6), ref, rtol=0, atol=1e-9)


def test_rope_norm_identity_and_relative_position():
    q, k = RNG.normal(size=(4, 64)), RNG.normal(size=(4, 64))
    np.testing.assert_allclose(orc.rope(q, np.zeros(4), 1e6), q, atol=0)
    rq = orc.rope(q, np.full(4, 1000), 1e6)
    np.testing.assert_allclose(np.linalg.norm(rq, axis=-1), np.linalg.norm(q, axis=-1), rtol=1e-13)
    for m, n, shift in [(5, 3, 100), (0, 7, 65536), (262144, 262100, -262000)]:
        a = np.sum(orc.rope(q, np.full(4, m), 1e6) * orc.rope(k, np.full(4, n), 1e6), -1)
        b = np.sum(orc.rope(q, np.full(4, m + shift), 1e6) * orc.rope(k, np.full(4, n + shift), 1e6), -1)
        np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-9)


# ---------------------------------------------------------------- brute force
SCENARIOS = [
    dict(ctx=[5, 3], window=6, k=4),      # context shorter than the window
    dict(ctx=[9, 14], window=6, k=4),     # ring wrap, window saturated
    dict(ctx=[0, 2], window=6, k=4),      # empty context: block only
    dict(ctx=[7, 7], window=6, k=1),      # block of one
    dict(ctx=[11, 4], window=3, k=3),     # window smaller than the block
]


@pytest.mark.parametrize("sc", SCENARIOS, ids=lambda s: f"ctx{s['ctx']}_w{s['window']}_k{s['k']}")
def test_draft_step_matches_bruteforce(sc):
    d = with_window(tiny_dims(block_k=sc["k"], batch=len(sc["ctx"])), sc["window"])
    W = tiny_weights(d, seed=3)
    st, hist = prefilled(d, W, sc["ctx"], seed=4, anchors=[3, 29])
    out = orc.draft_step(d, W, st)
    for b, P in enumerate(sc["ctx"]):
        ref = np.array(bf.block_logits(d, W, hist[b], P, int(st.anchor[b])))
        np.testing.assert_allclose(out["logits"][b], ref, rtol=1e-10, atol=1e-10)
        assert np.all(np.isfinite(out["logits"][b]))
    assert np.array_equal(out["draft"], np.argmax(out["logits"], -1))


def test_block_is_bidirectional():
    d = with_window(tiny_dims(batch=1), 6)
    W = tiny_weights(d, seed=5)
    st, hist = prefilled(d, W, [6], seed=6)
    z = orc.draft_step(d, W, st)["logits"][0]
    causal = np.array(bf.block_logits(d, W, hist[0], 6, int(st.anchor[0]), causal_block=True))
    assert np.max(np.abs(z[0] - causal[0])) > 1e-3        # row 0 sees the mask rows
    W2 = dict(W, mask_embed=W["mask_embed"] + 0.5)
    z2 = orc.draft_step(d, W2, st)["logits"][0]
    assert np.max(np.abs(z2[0] - z[0])) > 1e-3


# ---------------------------------------------------------------- invariants
def test_window_at_least_context_is_full_attention():
    base = tiny_dims(batch=2)
    W = tiny_weights(base, seed=7)
    ctx = [8, 5]
    outs = []
    for window in (8, 9, 40):
        d = with_window(base, window)
        st, _ = prefilled(d, W, ctx, seed=8)
        outs.append(orc.draft_step(d, W, st)["logits"])
    np.testing.assert_allclose(outs[0], outs[1], rtol=0, atol=1e-12)
    np.testing.assert_allclose(outs[0], outs[2], rtol=0, atol=1e-12)
    d = with_window(base, 7)                        # smaller than one context: differs
    st, _ = prefilled(d, W, ctx, seed=8)
    assert np.max(np.abs(orc.draft_step(d, W, st)["logits"][0] - outs[0][0])) > 1e-6


def test_block_of_one_is_a_decode_step():
    d = with_window(tiny_dims(block_k=1, batch=2), 6)
    W = tiny_weights(d, seed=9)
    st, _ = prefilled(d, W, [9, 3], seed=10, anchors=[1, 30])
    z = orc.draft_step(d, W, st)["logits"][:, 0]
    np.testing.assert_allclose(z, orc.decode_step(d, W, st), rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("shift", [1, 65536 - 9, 262144 - 9])
def test_global_position_shift_leaves_logits_unchanged(shift):
    d = with_window(tiny_dims(batch=1, rope_theta=1e6), 6)
    W = tiny_weights(d, seed=11)
    st0, _ = prefilled(d, W, [9], seed=12, offset=0)
    st1, _ = prefilled(d, W, [9], seed=12, offset=shift)
    np.testing.assert_allclose(orc.draft_step(d, W, st1)["logits"],
                               orc.draft_step(d, W, st0)["logits"], rtol=1e-8, atol=1e-8)


def test_ring_rotation_leaves_logits_unchanged():
    base = tiny_dims(batch=1)
    W = tiny_weights(base, seed=13)
    ref = None
    for extra in (0, 3, 7, 13):
        d = with_window(base, 6, extra_slots=extra)
        st, _ = prefilled(d, W, [17], seed=14)
        z = orc.draft_step(d, W, st)["logits"]
        ref = z if ref is None else ref
        np.testing.assert_allclose(z, ref, rtol=0, atol=1e-12)


def test_fused_feature_has_unit_mean_square():
    d = tiny_dims()
    W = dict(tiny_weights(d, seed=15), fuse_norm=np.ones(d.hidden))
    taps = random_taps(d, 1, 3, seed=16)[0]
    u = orc.linear(taps.reshape(3, -1), W["fuse_w"])
    c = orc.fuse(d, W, taps)
    mu = np.mean(u * u, -1)
    np.testing.assert_allclose(np.mean(c * c, -1), mu / (mu + d.rms_eps), rtol=1e-12)
    np.testing.assert_allclose(c[1], bf.fused_feature(d, W, taps[1]), rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------- verify
@pytest.mark.parametrize("k", range(1, 11))
def test_verify_exhaustive_match_patterns(k):
    d = replace(tiny_dims(block_k=k, batch=1), vocab=1000)
    for bits in range(2 ** k):
        draft = np.arange(k)[None] + 5
        match = np.array([(bits >> i) & 1 for i in range(k)], bool)
        target = np.concatenate([np.where(match, draft[0], draft[0] + 100), [777]])[None]
        st = orc.new_state(d, batch=1, ctx_len=[40], anchor=[1])
        r = orc.verify_commit(d, st, draft, target)
        a = int(r["accept_len"][0])
        assert a == bf.first_mismatch(draft[0], target[0], k)
        assert 0 <= a <= k
        assert list(r["out_tokens"][0]) == list(target[0, :a + 1]) + [-1] * (k - a)
        assert st.ctx_len[0] == 40 + a + 1 and st.anchor[0] == target[0, a]


def test_planting_recovers_every_length_and_means():
    V, k, B = 50, 8, 4
    rng = np.random.default_rng(0)
    d = tiny_dims(block_k=k, batch=B, vocab=V)
    for a_star in range(k + 1):
        draft = rng.integers(0, V, size=(B, k))
        fill = synth.target_fill(k, 1, B, seed=a_star)[0]
        T = synth.plant_targets(draft, np.full(B, a_star), fill, V)
        st = orc.new_state(d, batch=B, ctx_len=np.zeros(B))
        assert np.all(orc.verify_commit(d, st, draft, T)["accept_len"] == a_star)
    for kind, q, kk, mean in [("geometric", 0.87072, 16, 6.0), ("geometric", 0.94664, 8, 6.30),
                              ("geometric", 0.91846, 8, 5.56), ("geometric", 0.85920, 8, 4.29),
                              ("geometric", 0.84772, 10, 4.5), ("uniform", None, 8, 4.0)]:
        a = synth.planted_accept(kind, q, kk, 4000, 8)
        se = a.std() / np.sqrt(a.size)
        assert abs(a.mean() - mean) < 4 * se + 0.005, (kind, q, a.mean())
        assert a.min() >= 0 and a.max() <= kk


# ---------------------------------------------------------------- commit / rollback
def test_tentative_rows_and_rollback_equal_committed_only_history():
    d = with_window(tiny_dims(batch=2, block_k=4), 6)
    W = tiny_weights(d, seed=17)
    st, hist = prefilled(d, W, [6, 2], seed=18, anchors=[4, 9])
    planted = [[0, 4], [4, 1], [2, 0], [3, 3], [1, 2], [0, 0]]
    for step, a_star in enumerate(planted):
        out = orc.draft_step(d, W, st)
        for b in range(2):
            ref = np.array(bf.block_logits(d, W, hist[b], int(st.ctx_len[b]), int(st.anchor[b])))
            np.testing.assert_allclose(out["logits"][b], ref, rtol=1e-10, atol=1e-10)
        fill = synth.target_fill(d.block_k, 1, 2, seed=100 + step)[0]
        T = synth.plant_targets(out["draft"], np.array(a_star), fill, d.vocab)
        taps = random_taps(d, 2, d.block_k + 1, seed=200 + step)
        P = st.ctx_len.copy()
        orc.fuse_inject(d, W, st, taps, np.full(2, d.block_k + 1), commit=False)
        r = orc.verify_commit(d, st, out["draft"], T)
        for b in range(2):
            a = int(r["accept_len"][b])
            assert a == a_star[b]
            assert st.ctx_len[b] == P[b] + a + 1
            for j in range(a + 1):                     # only committed rows enter history
                hist[b][int(P[b]) + j] = taps[b, j]


def test_oracle_is_deterministic():
    d = with_window(tiny_dims(batch=2), 6)
    W = tiny_weights(d, seed=19)
    z = []
    for _ in range(2):
        st, _ = prefilled(d, W, [9, 5], seed=20)
        z.append(orc.draft_step(d, W, st)["logits"])
    assert np.array_equal(z[0], z[1])


# ---------------------------------------------------------------- attention sink
SINK_SCENARIOS = [
    dict(ctx=[1, 5], sink=2, window=4, k=3),     # fewer committed positions than the sink; inside the window
    dict(ctx=[6, 7], sink=2, window=4, k=3),     # window about to leave the sink behind
    dict(ctx=[15, 23], sink=2, window=4, k=3),   # ring wrapped several times, sink kept
    dict(ctx=[12, 9], sink=3, window=2, k=4),    # window smaller than the block and the sink
]


@pytest.mark.parametrize("sc", SINK_SCENARIOS, ids=lambda s: f"ctx{s['ctx']}_s{s['sink']}_w{s['window']}_k{s['k']}")
def test_sink_draft_step_matches_bruteforce(sc):
    d = with_sink(tiny_dims(block_k=sc["k"], batch=2), sc["sink"], sc["window"], extra_slots=1)
    W = tiny_weights(d, seed=31)
    st, hist = prefilled(d, W, sc["ctx"], seed=32, anchors=[5, 21])
    out = orc.draft_step(d, W, st)
    for b, P in enumerate(sc["ctx"]):
        ref = np.array(bf.block_logits(d, W, hist[b], P, int(st.anchor[b])))
        np.testing.assert_allclose(out["logits"][b], ref, rtol=1e-10, atol=1e-10)
        assert np.all(np.isfinite(out["logits"][b]))


def test_sink_rows_survive_rounds_and_rollbacks():
    d = with_sink(tiny_dims(batch=2, block_k=4), 2, 5)
    W = tiny_weights(d, seed=33)
    st, hist = prefilled(d, W, [3, 8], seed=34, anchors=[6, 11])
    planted = [[4, 0], [1, 4], [3, 2], [0, 3], [4, 4], [2, 1], [0, 0]]
    for step, a_star in enumerate(planted):
        out = orc.draft_step(d, W, st)
        for b in range(2):
            ref = np.array(bf.block_logits(d, W, hist[b], int(st.ctx_len[b]), int(st.anchor[b])))
            np.testing.assert_allclose(out["logits"][b], ref, rtol=1e-10, atol=1e-10)
        fill = synth.target_fill(d.block_k, 1, 2, seed=300 + step)[0]
        T = synth.plant_targets(out["draft"], np.array(a_star), fill, d.vocab)
        taps = random_taps(d, 2, d.block_k + 1, seed=400 + step)
        P = st.ctx_len.copy()
        orc.fuse_inject(d, W, st, taps, np.full(2, d.block_k + 1), commit=False)
        r = orc.verify_commit(d, st, out["draft"], T)
        for b in range(2):
            a = int(r["accept_len"][b])
            for j in range(a + 1):
                hist[b][int(P[b]) + j] = taps[b, j]
    assert min(st.ctx_len) > d.sink + d.window + d.block_k   # the ring wrapped past the sink


def test_sink_inside_the_window_changes_nothing():
    base = tiny_dims(batch=2)
    W = tiny_weights(base, seed=35)
    ctx = [6, 4]
    z0 = orc.draft_step(with_window(base, 6), W, prefilled(with_window(base, 6), W, ctx, seed=36)[0])["logits"]
    d = with_sink(base, 3, 6)
    z1 = orc.draft_step(d, W, prefilled(d, W, ctx, seed=36)[0])["logits"]
    np.testing.assert_allclose(z1, z0, rtol=0, atol=1e-12)
    d2 = with_sink(base, 3, 3)                         # window alone would drop positions 0..2
    z2 = orc.draft_step(d2, W, prefilled(d2, W, ctx, seed=36)[0])["logits"]
    np.testing.assert_allclose(z2[0], z0[0], rtol=0, atol=1e-12)   # sink + window = all 6


def test_sink_block_of_one_is_a_decode_step():
    d = with_sink(tiny_dims(block_k=1, batch=2), 2, 4)
    W = tiny_weights(d, seed=37)
    st, _ = prefilled(d, W, [11, 5], seed=38, anchors=[2, 19])
    z = orc.draft_step(d, W, st)["logits"][:, 0]
    np.testing.assert_allclose(z, orc.decode_step(d, W, st), rtol=1e-11, atol=1e-11)
