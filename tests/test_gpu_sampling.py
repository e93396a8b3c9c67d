"""GPU parity of sampled drafting and rejection-sampling verification (through the
C ABI) against the fp64 oracle.

* dflash_verify_sampled alone, on identical seeded inputs (fp32 logits, the
  oracle's drafts and log-sum-exps): accepted lengths, emitted tokens, committed
  lengths and anchors bit-exact wherever every decision is >= 1e-3 from its
  threshold; vocabularies with a ragged tail, not a multiple of 4 (scalar loads),
  exactly one chunk and several chunks; k = 1 .. 16; two rounds on one workspace.
* whole sampled rounds (draft forward + Gumbel-max drafts + injection + verify)
  through every GEMM path of the LM head: weight-streaming with 16, 32 and 64-row
  blocks, fp32 and bf16, and the tiled 256 x 256 kernel, with the gates of
  ParityRun.step_sampled.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

from block_diffusion_speculative_dflash_amd import binding as bd
from block_diffusion_speculative_dflash_amd import configs, synth
from block_diffusion_speculative_dflash_amd.configs import BF16
from oracle import sampling as sp
from tests.parity import ParityRun, say

pytestmark = pytest.mark.gpu

GATE = 1e-3  # fp32 inputs on both sides: the kernel's own rounding stays far below this


def _verify_rounds(V, B, k, T, soft, seed=0, rounds=2, planted=None):
    d = replace(configs.C1.dims, batch=B, block_k=k, vocab=V, window=32, cache_slots=32 + k,
                max_inject_rows=max(16, k + 1))
    ctx = (100 + 3 * np.arange(B)).astype(np.int64)
    anchors = synth.make_anchors(d, seed=seed)
    cache = bd.alloc_cache(d, ctx_len=ctx, anchor=anchors)
    ws = bd.alloc_workspace(d)
    checked = total = 0
    accepts = []
    for st in range(rounds):
        say(f"[sampling] verify V={V} B={B} k={k} T={T} soft={soft} round {st}")
        z = synth.make_logits((B, k, V), seed=seed, stream=2 * st + 1, device="cuda")
        z64 = z.double().cpu().numpy()
        x = sp.sample_drafts(z64, T, seed, st)["draft"]
        lse = torch.as_tensor(sp.logsumexp(z64, T), dtype=torch.float32, device="cuda")
        a_star = planted[st] if planted is not None else \
            synth.planted_accept("uniform", None, k, 1, B, seed=seed + st)[0]
        fill = synth.make_logits((B, k + 1, V), seed=seed, stream=2 * st + 2, device="cuda")
        t = synth.plant_target_logits(z, x, np.asarray(a_star), fill, soft=soft, seed=st).contiguous()
        smp = bd.sampling_struct(T, seed, st)
        acc = torch.full((B,), -7, dtype=torch.int32, device="cuda")
        out = torch.full((B, k + 1), -7, dtype=torch.int32, device="cuda")
        xd = torch.as_tensor(x, dtype=torch.int32, device="cuda")
        bd.dflash_verify_sampled(d, smp, xd, z, lse, t, cache, acc, out, ws)
        torch.cuda.synchronize()
        r = sp.verify_sampled(x, z64, t.double().cpu().numpy(), T, seed, st)
        acc_g, out_g = acc.cpu().numpy(), out.cpu().numpy()
        ctx_g, anc_g = cache["ctx_len"].cpu().numpy(), cache["anchor"].cpu().numpy()
        for b in range(B):
            total += 1
            new_ctx = int(ctx[b]) + int(r["accept_len"][b]) + 1
            if r["accept_margin"][b] >= GATE and r["emit_gap"][b] >= GATE * (1 + r["emit_slack"][b]):
                checked += 1
                assert acc_g[b] == r["accept_len"][b], (st, b, acc_g[b], r["accept_len"][b])
                assert np.array_equal(out_g[b], r["out_tokens"][b]), (st, b, out_g[b], r["out_tokens"][b])
                assert ctx_g[b] == new_ctx and anc_g[b] == r["emitted"][b], (st, b)
            ctx[b] = new_ctx
        accepts.append(acc_g.copy())
        cache["ctx_len"].copy_(torch.as_tensor(ctx, dtype=torch.int32))
        cache["anchor"].copy_(torch.as_tensor(r["emitted"], dtype=torch.int32))
    assert int(cache["dev_error"].item()) == 0
    assert checked >= 0.75 * total, f"only {checked}/{total} sequences passed the gates"
    return accepts


@pytest.mark.parametrize("V,B,k,T,soft", [
    (1000, 6, 5, 1.0, 0.5),     # one chunk, ragged
    (1001, 3, 7, 0.7, 0.3),     # vocabulary not a multiple of 4: scalar loads
    (20000, 4, 4, 1.5, 0.0),    # ten 2048-entry chunks, ragged tail
    (20000, 4, 16, 1.2, 0.3),   # 4096-entry chunks in the log-sum-exp kernel
    (8192, 2, 1, 0.3, 1.0),     # exactly one chunk, block of one
    (3000, 2, 16, 2.0, 0.5),    # long block
])
def test_verify_sampled_matches_oracle(V, B, k, T, soft):
    _verify_rounds(V, B, k, T, soft)


def test_verify_sampled_planted_lengths_exact():
    """soft = 0: rows before a* copy the draft (always accepted), row a* gives the
    draft zero probability (always rejected), so the accepted length is a* exactly."""
    k, B = 6, 7
    planted = [np.arange(B) % (k + 1), (np.arange(B) * 3 + 1) % (k + 1)]
    accepts = _verify_rounds(2000, B, k, 0.9, 0.0, seed=3, planted=planted)
    for a_star, got in zip(planted, accepts):
        assert np.array_equal(got, a_star)


def _sampled_run(dims, ctx, prefill, a_stars, temps, soft=0.0, seed=0):
    W = synth.make_weights(dims, seed=seed, device="cuda")
    anchors = synth.make_anchors(dims, seed=seed)
    run = ParityRun(dims, W, ctx, anchors, prefill, seed=seed)
    reps = [run.step_sampled(a, T, seed=77, soft=soft) for a, T in zip(a_stars, temps)]
    assert run.dev_error() == 0
    for i, r in enumerate(reps):
        assert r.logits_ok, f"round {i}: logit error {r.logit_err} (ref max {r.logit_ref_max})"
        assert r.lse_ok, f"round {i}: lse error {r.lse_err}"
        assert r.draft_mismatch == 0, f"round {i}: {r.draft_mismatch} gated draft mismatches"
        assert r.state_mismatch == 0, f"round {i}: {r.state_mismatch} state mismatches"
        assert r.kv_ok, f"round {i}: kv error {r.kv_err}"
    checked = sum(r.seqs_checked for r in reps)
    assert checked >= 0.5 * sum(r.seqs_checked + r.seqs_excluded for r in reps), "too few sequences gated in"
    return reps


def test_sampled_rounds_tiny_fp32():
    w = configs.C1
    d = w.dims
    say(f"[test] sampled tiny fp32 {d}")
    reps = _sampled_run(d, [w.context], [w.prefill], [[a] for a in (8, 0, 3, 5, 8)],
                        [1.0, 0.6, 1.0, 2.0, 0.8])
    assert sum(r.drafts_checked for r in reps) > 0.8 * sum(r.drafts_total for r in reps)


def test_sampled_rounds_bf16_streaming_row_blocks():
    """bf16 with 8, 24, 40 and 80 block rows: the LM head streams with 16-, 32- and
    64-row blocks (80 rows: two 64-row tiles)."""
    for B in (1, 3, 5, 10):
        d = replace(configs.C1.dims, batch=B, dtype=BF16, window=32, cache_slots=40)
        say(f"[test] sampled bf16 streaming B={B}")
        ctx = [60 + 11 * b for b in range(B)]
        _sampled_run(d, ctx, [min(c, 32) for c in ctx],
                     [[(b + s) % 9 for b in range(B)] for s in range(2)], [1.0, 0.7], soft=0.3)


def test_sampled_rounds_tiled_bf16():
    """160 block rows take the tiled LM head (256 x 256 tiles, vocabulary tail)."""
    d = replace(configs.C1.dims, batch=20, block_k=8, n_layers=2, n_q_heads=4, n_kv_heads=2,
                ffn=1100, vocab=40003, window=32, cache_slots=40, dtype=BF16, max_inject_rows=16)
    say(f"[test] sampled tiled {d}")
    ctx = [40 + (7 * b) % 23 for b in range(d.batch)]
    _sampled_run(d, ctx, [min(c, d.window) for c in ctx],
                 [[(3 * b + s) % 9 for b in range(d.batch)] for s in range(2)], [1.0, 1.3], soft=0.2)


def test_sampled_draws_are_reproducible_and_step_dependent():
    d = replace(configs.C1.dims, batch=2, dtype=BF16, window=32, cache_slots=40)
    W = synth.make_weights(d, seed=1, device="cuda")
    bd.pack_weights(d, W)
    cache = bd.alloc_cache(d, ctx_len=[0, 0], anchor=synth.make_anchors(d, seed=1))
    ws = bd.alloc_workspace(d)
    B, k, V = d.batch, d.block_k, d.vocab
    outs = []
    for step in (5, 5, 6):
        dr = torch.empty((B, k), dtype=torch.int32, device="cuda")
        z = torch.empty((B, k, V), dtype=torch.float32, device="cuda")
        lse = torch.empty((B, k), dtype=torch.float32, device="cuda")
        bd.dflash_draft_step_sampled(d, W, cache, bd.sampling_struct(3.0, 9, step), dr, z, lse, ws)
        torch.cuda.synchronize()
        outs.append((dr.cpu().numpy(), z.cpu().numpy(), lse.cpu().numpy()))
    assert all(np.array_equal(a, b) for a, b in zip(outs[0], outs[1]))
    assert np.array_equal(outs[0][1], outs[2][1])          # same logits
    assert not np.array_equal(outs[0][0], outs[2][0])      # new step, new draws (T = 3)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("V,B,k", [(151936, 8, 16), (128256, 8, 10), (151936, 3, 12), (151936, 1, 16)])
def test_verify_sampled_full_vocabulary(V, B, k):
    """The verify kernels at full vocabulary on identical inputs, so every decision is
    compared at the 1e-3 gate; the shapes take 8192-, 4096- and 2048-entry chunks
    (the last is the batch-1, block-16 launch of the Qwen3-8B-shaped workload)."""
    _verify_rounds(V, B, k, 1.0, 0.3, seed=11, rounds=1)


def test_sampled_rounds_large_vocab_lm_head():
    """The 16-row LM head over 1025 column tiles (bf16, hidden 1024) with the sampled
    epilogue: draws, logits and log-sum-exps across many tiles and a ragged tail."""
    d = replace(configs.C1.dims, batch=1, block_k=16, hidden=1024, n_q_heads=8, n_kv_heads=2, head_dim=128,
                ffn=2048, vocab=65600, tap_dim=512, window=32, cache_slots=48, dtype=BF16, max_inject_rows=17)
    say(f"[test] sampled large-vocabulary head {d}")
    _sampled_run(d, [40], [32], [[16], [4], [9]], [1.0, 0.8, 1.5], soft=0.2)
