"""GPU parity of the HIP library against the fp64 oracle, through the C ABI.

Small shapes that the oracle finishes in seconds but that still span several
GEMM tiles, split-K, ragged tails (ffn 683, vocab tails), ring wrap, GQA, both
head sizes, k = 1 and empty contexts.  The full-size workloads are in
test_gpu_fullsize.py.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

from block_diffusion_speculative_dflash_amd import binding as bd
from block_diffusion_speculative_dflash_amd import configs, synth
from block_diffusion_speculative_dflash_amd.configs import BF16, F32
from oracle import dflash_oracle as orc
from tests.parity import ParityRun, say

pytestmark = pytest.mark.gpu


def _run(dims, ctx, prefill, a_stars, seed=0, sample=None, anchors=None):
    W = synth.make_weights(dims, seed=seed, device="cuda")
    if anchors is None:
        anchors = synth.make_anchors(dims, seed=seed)
    run = ParityRun(dims, W, ctx, anchors, prefill, sample=sample, seed=seed)
    reps = [run.step(a) for a in a_stars]
    assert run.dev_error() == 0
    return reps


def _assert_ok(reps):
    for i, r in enumerate(reps):
        assert r.logits_ok, f"step {i}: logit error {r.logit_err} (ref max {r.logit_ref_max})"
        assert r.draft_mismatch == 0, f"step {i}: {r.draft_mismatch} gated draft mismatches"
        assert r.state_mismatch == 0, f"step {i}: {r.state_mismatch} state mismatches"
        assert r.verify_mismatch == 0, f"step {i}: verify/commit of the GPU drafts differs for {r.verify_mismatch}"
        assert r.kv_ok, f"step {i}: kv error {r.kv_err}"


def test_tiny_fp32_every_planted_length():
    """Tiny fp32 drafter (batch 1, context 128, block 8): planted a* = 0..8."""
    w = configs.C1
    d = w.dims
    say(f"[test] tiny fp32 {d}")
    planted = list(range(9))
    reps = _run(d, [w.context], [w.prefill], [[a] for a in planted])
    _assert_ok(reps)
    for a, r in zip(planted, reps):
        if r.seqs_checked:
            assert r.accept[0] == a
    assert sum(r.drafts_checked for r in reps) > 0.9 * sum(r.drafts_total for r in reps)


def test_tiny_bf16():
    d = replace(configs.C1.dims, dtype=BF16)
    say(f"[test] tiny bf16 {d}")
    _assert_ok(_run(d, [128], [128], [[8], [3], [0], [5]]))


def test_gqa_swa_ring_wrap_ragged_bf16():
    """GQA 4/2, window 16 over contexts longer than the ring, ragged batch."""
    d = replace(configs.C1.dims, batch=3, block_k=4, n_q_heads=4, n_kv_heads=2, window=16,
                cache_slots=20, dtype=BF16, max_inject_rows=16)
    say(f"[test] gqa swa ring {d}")
    _assert_ok(_run(d, [40, 17, 5], [40, 17, 5], [[4, 0, 2], [1, 4, 3], [2, 2, 4], [0, 1, 1], [3, 3, 0]]))


def test_gqa_swa_fp32():
    d = replace(configs.C1.dims, batch=2, block_k=5, n_q_heads=4, n_kv_heads=1, window=24,
                cache_slots=29, max_inject_rows=16)
    say(f"[test] gqa swa fp32 {d}")
    _assert_ok(_run(d, [50, 23], [30, 23], [[5, 2], [0, 5], [3, 1]]))


def test_head_dim_128_bf16():
    d = replace(configs.C1.dims, batch=2, n_q_heads=4, n_kv_heads=2, head_dim=128, hidden=512,
                tap_dim=128, ffn=1000, vocab=2000, window=64, cache_slots=72, dtype=BF16)
    say(f"[test] head_dim 128 {d}")
    _assert_ok(_run(d, [70, 64], [64, 64], [[8, 1], [2, 7], [4, 4]]))


def test_two_row_tiles_streaming():
    """Just over one 64-row streaming tile: 8 x 9 injected rows (fusion and injection
    over two row tiles, the second nearly empty) with 64 block rows, then 80 block rows
    (every draft projection and the LM head over two row tiles) with 90 injected rows;
    bf16 GQA and fp32."""
    for B, dtype in ((8, BF16), (10, BF16), (9, F32)):
        d = replace(configs.C1.dims, batch=B, block_k=8, n_layers=2, n_q_heads=4, n_kv_heads=2,
                    window=32, cache_slots=40, dtype=dtype)
        say(f"[test] two row tiles, streaming {d}")
        ctx = [40 + (5 * b) % 19 for b in range(B)]
        pre = [min(c, d.window) for c in ctx]
        steps = [[(2 * b + s) % 9 for b in range(B)] for s in range(2)]
        _assert_ok(_run(d, ctx, pre, steps))


def test_ragged_long_windows_balanced_attention():
    """64 sequences with ragged full-attention contexts of 200..1100 keys over a window
    above 1024, keys unsplit: the attention places sequences by context-length rank
    (a permutation), fp32 and bf16."""
    for dtype in (F32, BF16):
        d = replace(configs.C1.dims, batch=64, block_k=4, n_layers=1, window=1100, cache_slots=1104,
                    dtype=dtype)
        say(f"[test] balanced attention {d}")
        ctx = [200 + (37 * b) % 901 for b in range(d.batch)]
        steps = [[(b + s) % 5 for b in range(d.batch)] for s in range(2)]
        _assert_ok(_run(d, ctx, ctx, steps))


def test_round_touches_only_tentative_ring_slots():
    """Cache traffic of one round, bitwise: the draft step writes no K/V byte; the
    injection of n rows at committed length P writes exactly the ring slots of
    positions P .. P+n-1 (sink slots fixed, ring wrap) in every layer and kv head and
    leaves every other byte alone; the verify moves ctx_len by a+1 and the anchor to
    the bonus token without touching K/V (rollback = the committed pointer)."""
    for dtype, sink in ((BF16, 0), (F32, 2)):
        d = replace(configs.C1.dims, batch=5, block_k=6, n_layers=2, n_q_heads=4, n_kv_heads=2,
                    window=24, cache_slots=24 + 6 + sink, sink=sink, dtype=dtype)
        say(f"[test] ring slots of one round {d}")
        W = bd.pack_weights(d, synth.make_weights(d, seed=3, device="cuda"))
        B, k, C = d.batch, d.block_k, d.cache_slots
        ctx = np.array([0, 5, 23, 40, 77], dtype=np.int32)  # empty, short, full window, wrapped
        cache = bd.alloc_cache(d, device="cuda", ctx_len=ctx, anchor=synth.make_anchors(d, seed=3))
        g = torch.Generator(device="cuda").manual_seed(11)
        cache["k"].copy_(torch.randn(cache["k"].shape, generator=g, device="cuda").to(cache["k"].dtype))
        cache["v"].copy_(torch.randn(cache["v"].shape, generator=g, device="cuda").to(cache["v"].dtype))
        ws = bd.alloc_workspace(d, device="cuda")
        k0, v0 = cache["k"].clone(), cache["v"].clone()

        draft = torch.zeros((B, k), dtype=torch.int32, device="cuda")
        bd.dflash_draft_step(d, W, cache, draft, None, ws)
        torch.cuda.synchronize()
        assert torch.equal(cache["k"], k0) and torch.equal(cache["v"], v0)

        n = np.array([k + 1, 1, k + 1, 3, k + 1], dtype=np.int32)  # rows injected per sequence
        taps = synth.make_taps(d, k + 1, seed=3, stream=7, device="cuda")
        bd.dflash_fuse_inject(d, W, taps, torch.as_tensor(n, device="cuda"), k + 1, False, cache, ws)
        torch.cuda.synchronize()
        written = np.zeros((B, C), dtype=bool)
        for b in range(B):
            for p in range(int(ctx[b]), int(ctx[b]) + int(n[b])):
                written[b, orc.slot_of(d, p)] = True
        changed_k = (cache["k"] != k0).any(dim=-1).cpu().numpy()  # [L, B, Hkv, C]
        changed_v = (cache["v"] != v0).any(dim=-1).cpu().numpy()
        for ch in (changed_k, changed_v):
            assert np.array_equal(ch, np.broadcast_to(written[None, :, None, :], ch.shape))
        np.testing.assert_array_equal(cache["ctx_len"].cpu().numpy(), ctx)  # commit = 0

        target = torch.as_tensor(np.concatenate([draft.cpu().numpy(), np.zeros((B, 1), np.int32)], 1) + 0,
                                 device="cuda")
        a_plant = [0, 2, k, 4, 1]
        for b, a in enumerate(a_plant):
            if a < k:
                target[b, a] = (draft[b, a] + 1) % d.vocab
        k1, v1 = cache["k"].clone(), cache["v"].clone()
        acc = torch.zeros(B, dtype=torch.int32, device="cuda")
        out = torch.zeros((B, k + 1), dtype=torch.int32, device="cuda")
        bd.dflash_verify_commit(d, draft, target, cache, acc, out)
        torch.cuda.synchronize()
        assert torch.equal(cache["k"], k1) and torch.equal(cache["v"], v1)
        np.testing.assert_array_equal(acc.cpu().numpy(), a_plant)
        np.testing.assert_array_equal(cache["ctx_len"].cpu().numpy(), ctx + np.array(a_plant) + 1)
        tg = target.cpu().numpy()
        np.testing.assert_array_equal(cache["anchor"].cpu().numpy(), [tg[b, a] for b, a in enumerate(a_plant)])
        assert int(cache["dev_error"].item()) == 0


def test_tiled_gemm_path_bf16():
    """Batch x block >= 128 rows takes the tiled MFMA GEMM for every projection: row
    tails (160 draft rows, 180 and 320 injected rows), ragged SwiGLU width and
    vocabulary, K split over workgroups in the fusion and down projections, and a
    vocabulary large enough that the 256 x 256 tile wins the plan."""
    d = replace(configs.C1.dims, batch=20, block_k=8, n_layers=2, n_q_heads=4, n_kv_heads=2,
                ffn=1100, vocab=40003, window=32, cache_slots=40, dtype=BF16, max_inject_rows=16)
    say(f"[test] tiled GEMM path {d}")
    ctx = [40 + (7 * b) % 23 for b in range(d.batch)]
    pre = [min(c, d.window) for c in ctx]
    steps = [[(3 * b + s) % 9 for b in range(d.batch)] for s in range(3)]
    _assert_ok(_run(d, ctx, pre, steps))


def test_attention_sink_fp32_ring_wrap():
    """Attention sink of 4 beside a window of 24: one sequence far past the sink
    (ring wrapped), one still inside the window."""
    d = replace(configs.C1.dims, batch=2, sink=4, window=24, cache_slots=4 + 24 + 8 + 3, max_inject_rows=16)
    say(f"[test] sink fp32 {d}")
    _assert_ok(_run(d, [60, 13], [60, 13], [[8, 3], [2, 8], [5, 0], [0, 4]]))


def test_attention_sink_gqa_bf16():
    d = replace(configs.C1.dims, batch=3, block_k=4, n_q_heads=4, n_kv_heads=2, sink=3, window=16,
                cache_slots=3 + 16 + 4, dtype=BF16, max_inject_rows=16)
    say(f"[test] sink gqa bf16 {d}")
    _assert_ok(_run(d, [40, 17, 2], [40, 17, 2], [[4, 0, 2], [1, 4, 3], [2, 2, 4], [0, 1, 1], [3, 3, 0]]))


def test_key_splits_fp32_sink_ragged():
    """Key lists past 1024 over few workgroups are split (>= 256 keys per split) and
    the fp32 partials merged: a ring wrapped behind a 4-position sink (6 splits), a
    shorter context (3 splits) and one that fits a single split, in one launch."""
    d = replace(configs.C1.dims, batch=3, sink=4, window=1500, cache_slots=4 + 1500 + 8 + 5,
                max_inject_rows=256)
    say(f"[test] key splits fp32 {d}")
    ctx = [1700, 700, 90]
    _assert_ok(_run(d, ctx, ctx, [[8, 3, 0], [2, 8, 5], [5, 0, 8]]))


def test_key_splits_gqa_bf16_head_dim_128_block_lengths():
    """64 query rows per kv head (GQA 4/1, block 16, head size 128: the batch-1
    Qwen3-8B attention shape) over 2016 keys in 256-key splits, with per-sequence
    block lengths masking block keys inside the last split."""
    d = replace(configs.C1.dims, batch=2, block_k=16, n_q_heads=4, n_kv_heads=1, head_dim=128, hidden=512,
                tap_dim=128, ffn=1000, vocab=2000, window=2000, cache_slots=2000 + 16 + 8, dtype=BF16,
                max_inject_rows=512)
    say(f"[test] key splits gqa bf16 {d}")
    ctx = [2100, 1100]
    W = synth.make_weights(d, seed=2, device="cuda")
    run = ParityRun(d, W, ctx, synth.make_anchors(d, seed=2), [min(c, d.window) for c in ctx], seed=2)
    reps = [run.step([16, 4]), run.step([3, 5], block_len=[16, 7]), run.step([0, 2], block_len=[5, 16])]
    assert run.dev_error() == 0
    _assert_ok(reps)


def test_balanced_k_pieces_qkv_bf16():
    """Hidden 4096 with 16/4 heads: the QKV projection (48 column tiles, 128 K steps)
    would split 8 ways into 384 workgroups, so it takes balanced pieces instead,
    10 or 11 per tile (512 workgroups, pieces of 11 and 12 K steps)."""
    d = replace(configs.C1.dims, batch=1, block_k=16, n_layers=1, hidden=4096, n_q_heads=16, n_kv_heads=4,
                head_dim=128, ffn=1024, vocab=3000, tap_dim=512, window=64, cache_slots=64 + 16 + 8, dtype=BF16,
                max_inject_rows=17)
    say(f"[test] balanced K pieces {d}")
    _assert_ok(_run(d, [70], [64], [[16], [5], [0]], seed=4))


def test_block_of_one_and_empty_context():
    d = replace(configs.C1.dims, batch=2, block_k=1, window=32, cache_slots=33, max_inject_rows=8)
    say(f"[test] k=1, empty context {d}")
    _assert_ok(_run(d, [0, 9], [0, 9], [[1, 0], [0, 1], [1, 1], [1, 0]]))


def test_empty_context_bf16_block():
    d = replace(configs.C1.dims, batch=2, dtype=BF16, window=32, cache_slots=40)
    _assert_ok(_run(d, [0, 0], [0, 0], [[8, 2], [3, 8]]))


def test_verify_exhaustive_patterns_on_gpu():
    """All 2^10 match patterns of a k = 10 block in one batch, plus planted lengths."""
    k = 10
    B = 2 ** k
    d = replace(configs.C1.dims, batch=B, block_k=k, vocab=50000, cache_slots=configs.C1.dims.window + k)
    rng = np.random.default_rng(5)
    draft = rng.integers(0, 40000, size=(B, k))
    bits = (np.arange(B)[:, None] >> np.arange(k)[None, :]) & 1
    target = np.concatenate([np.where(bits == 1, draft, draft + 1), rng.integers(0, 40000, (B, 1))], 1)
    ctx0 = rng.integers(0, 100000, B)
    anchors = rng.integers(0, 40000, B)
    cache = bd.alloc_cache(d, ctx_len=ctx0, anchor=anchors)
    acc = torch.empty(B, dtype=torch.int32, device="cuda")
    out = torch.empty((B, k + 1), dtype=torch.int32, device="cuda")
    say("[test] verify exhaustive 2^10")
    bd.dflash_verify_commit(d, torch.as_tensor(draft, dtype=torch.int32).cuda(),
                            torch.as_tensor(target, dtype=torch.int32).cuda(), cache, acc, out)
    torch.cuda.synchronize()
    # verification only touches integers; a one-slot ring stands in for the cache
    st = orc.State(np.zeros((1, B, 1, 1, 1)), np.zeros((1, B, 1, 1, 1)),
                   ctx0.astype(np.int64), anchors.astype(np.int64))
    ref = orc.verify_commit(replace(d, cache_slots=1), st, draft, target)
    assert np.array_equal(acc.cpu().numpy(), ref["accept_len"])
    assert np.array_equal(out.cpu().numpy(), ref["out_tokens"])
    assert np.array_equal(cache["ctx_len"].cpu().numpy(), st.ctx_len)
    assert np.array_equal(cache["anchor"].cpu().numpy(), st.anchor)
    assert int(cache["dev_error"].item()) == 0


def test_out_of_range_tokens_set_the_error_word():
    d = replace(configs.C1.dims, batch=2, block_k=4, vocab=100)
    cache = bd.alloc_cache(d, ctx_len=[5, 5], anchor=[3, 4])
    draft = torch.tensor([[1, 2, 3, 4], [1, 2, 3, 4]], dtype=torch.int32, device="cuda")
    target = torch.tensor([[1, 2, 500, 4, 5], [1, 2, 3, 4, 5]], dtype=torch.int32, device="cuda")
    acc = torch.empty(2, dtype=torch.int32, device="cuda")
    out = torch.empty((2, 5), dtype=torch.int32, device="cuda")
    bd.dflash_verify_commit(d, draft, target, cache, acc, out)
    torch.cuda.synchronize()
    assert int(cache["dev_error"].item()) & bd.DEVERR_TOKEN
    assert acc.cpu().tolist() == [2, 4]
    assert out.cpu().tolist()[0] == [1, 2, 99, -1, -1]     # clamped into [0, vocab)


def test_draft_is_deterministic_and_logits_optional():
    d = replace(configs.C1.dims, batch=2, dtype=BF16)
    W = bd.pack_weights(d, synth.make_weights(d, device="cuda"))
    cache = bd.alloc_cache(d, ctx_len=[0, 0], anchor=[5, 6])
    ws = bd.alloc_workspace(d)
    taps = synth.make_taps(d, 40, device="cuda")
    bd.dflash_fuse_inject(d, W, taps, torch.tensor([40, 33], dtype=torch.int32, device="cuda"), 40, True, cache, ws)
    outs = []
    for with_logits in (True, True, False):
        dr = torch.empty((2, d.block_k), dtype=torch.int32, device="cuda")
        lg = torch.empty((2, d.block_k, d.vocab), device="cuda") if with_logits else None
        bd.dflash_draft_step(d, W, cache, dr, lg, ws)
        torch.cuda.synchronize()
        outs.append((dr.cpu(), None if lg is None else lg.cpu()))
    assert torch.equal(outs[0][1], outs[1][1])          # bitwise reproducible
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][0], outs[2][0])
    assert cache["ctx_len"].cpu().tolist() == [40, 33]


def _large_vocab_dims(batch, block_k):
    """bf16, hidden 1024 (32 K steps) and a 65 600-token vocabulary (1025 column tiles,
    the last ragged): the 16-row weight-streaming LM head over many more tiles than
    the GPU has workgroup slots."""
    return replace(configs.C1.dims, batch=batch, block_k=block_k, hidden=1024, n_q_heads=8, n_kv_heads=2,
                   head_dim=128, ffn=2048, vocab=65600, tap_dim=512, window=32, cache_slots=32 + block_k,
                   dtype=BF16, max_inject_rows=max(16, block_k + 1))


def test_large_vocab_lm_head_bf16():
    d = _large_vocab_dims(1, 16)
    say(f"[test] large-vocabulary LM head {d}")
    _assert_ok(_run(d, [40], [32], [[16], [5], [0], [9]]))


def test_large_vocab_lm_head_partial_rows_and_block_lengths():
    """9 of 16 rows, per-sequence block lengths (drafts past a block read -1)."""
    d = _large_vocab_dims(3, 3)
    say(f"[test] large-vocabulary LM head, 9 rows {d}")
    W = synth.make_weights(d, seed=2, device="cuda")
    run = ParityRun(d, W, [20, 33, 7], synth.make_anchors(d, seed=2), [20, 32, 7], seed=2)
    reps = [run.step([3, 1, 0], block_len=[3, 2, 0]), run.step([2, 3, 1], block_len=[1, 3, 3]),
            run.step([0, 2, 3])]
    assert run.dev_error() == 0
    _assert_ok(reps)


def test_prefill_chunk_longer_than_ring():
    """One fuse_inject call carrying more rows per sequence than the ring holds: the
    cache must end as if the rows were written in position order (each ring slot
    keeps the last of its rows), for a plain ring (bf16 GQA) and with an attention
    sink whose positions arrive in the same call (fp32)."""
    d = replace(configs.C1.dims, batch=3, block_k=4, n_layers=2, n_q_heads=4, n_kv_heads=2, window=16,
                cache_slots=20, dtype=BF16, max_inject_rows=64)
    say(f"[test] prefill chunk > ring {d}")
    _assert_ok(_run(d, [50, 61, 21], [50, 61, 21], [[4, 0, 2], [1, 3, 4]]))
    d = replace(configs.C1.dims, batch=2, block_k=4, n_layers=1, window=12, sink=2, cache_slots=2 + 12 + 4,
                max_inject_rows=64)
    say(f"[test] prefill chunk > ring, sink in the same call {d}")
    _assert_ok(_run(d, [45, 33], [45, 33], [[2, 4], [4, 1]]))


def test_fp16_overflow_saturates_and_sets_the_error_word():
    """bf16 drafter whose SwiGLU products exceed the fp16 range (gate/up weights
    scaled up): the kernels finish, the stored values saturate (finite logits) and
    dev_error carries the overflow bit; the same drafter at the normal scale leaves
    the word clear."""
    d = replace(configs.C1.dims, dtype=BF16)
    for scale, expect in ((1.0, 0), (2000.0, bd.DEVERR_OVERFLOW)):
        W = synth.make_weights(d, seed=0, device="cuda")
        W["w_gate_up"] = (W["w_gate_up"].float() * scale).to(torch.bfloat16)
        bd.pack_weights(d, W)
        cache = bd.alloc_cache(d, ctx_len=[0], anchor=[3])
        ws = bd.alloc_workspace(d)
        taps = synth.make_taps(d, 32, seed=0, device="cuda")
        bd.dflash_fuse_inject(d, W, taps, torch.tensor([32], dtype=torch.int32, device="cuda"), 32, True, cache, ws)
        draft = torch.empty((1, d.block_k), dtype=torch.int32, device="cuda")
        logits = torch.empty((1, d.block_k, d.vocab), dtype=torch.float32, device="cuda")
        bd.dflash_draft_step(d, W, cache, draft, logits, ws)
        torch.cuda.synchronize()
        err = int(cache["dev_error"].item())
        say(f"[test] gate/up x{scale}: dev_error {err}, max |logit| {float(logits.abs().max()):.3g}")
        assert err == expect
        assert bool(torch.isfinite(logits).all())
