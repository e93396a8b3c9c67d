"""The benchmark's decode round (harness.RoundLoop: draft step, target stand-in
planted on the device, tentative injection, verification) captured into HIP graphs
and replayed the way bench.py times it, checked against the same rounds launched
eagerly (bitwise: drafts, target tokens, accepted lengths, emitted tokens,
committed lengths, anchors, and the whole K/V cache) and against the fp64 oracle
under the parity rules (drafts where the oracle's margin is >= 0.1, verify/commit
of the GPU's drafts bit-exact, the committed K/V window within 0.05).

Workloads: the Qwen3-8B-shaped batch-1 drafter over 10 rounds, which includes the
context rewind after round 8, and the batch-256 long-context SWA drafter, greedy
and sampled (the sampled rounds read their random-number step from a device word
the stand-in advances, so every replay of a graph draws new numbers; a graph that
had frozen the step would differ from the eager rounds)."""
import numpy as np
import pytest
import torch

from block_diffusion_speculative_dflash_amd import binding as bd
from block_diffusion_speculative_dflash_amd import configs, harness, synth
from oracle import dflash_oracle as orc
from tests.parity import integer_state, oracle_weights, say

pytestmark = pytest.mark.gpu


def _prefill(wl, d, W, seed=0):
    """The benchmark's prefill: the committed context in chunks of max_inject_rows
    rows, each chunk's taps one seeded draw (stream 10000 + first row)."""
    ctx = synth.make_context_lengths(wl, seed=seed)
    pre = np.minimum(ctx, wl.prefill)
    anchors = synth.make_anchors(d, seed=seed)
    cache = bd.alloc_cache(d, ctx_len=ctx - pre, anchor=anchors)
    ws = bd.alloc_workspace(d)
    n_pre, n_max = int(pre.max()), d.max_inject_rows
    chunks = []
    for r0 in range(0, n_pre, n_max):
        taps = synth.make_taps(d, min(n_max, n_pre - r0), seed=seed, stream=10_000 + r0, device="cuda")
        n_rows = torch.as_tensor(np.clip(pre - r0, 0, taps.shape[1]), dtype=torch.int32, device="cuda")
        bd.dflash_fuse_inject(d, W, taps, n_rows, taps.shape[1], True, cache, ws)
        chunks.append(taps)
    torch.cuda.synchronize()
    return cache, ws, ctx, pre, anchors, chunks


def _snapshot(cache):
    return {n: t.clone() for n, t in cache.items()}


def _restore(cache, snap):
    for n, t in snap.items():
        cache[n].copy_(t)


def _record(loop, cache):
    torch.cuda.synchronize()
    return {"draft": loop.draft.cpu().numpy().copy(), "target": loop.target.cpu().numpy().copy(),
            "accept": loop.accept.cpu().numpy().copy(), "out": loop.out_tok.cpu().numpy().copy(),
            "ctx": cache["ctx_len"].cpu().numpy().copy(), "anchor": cache["anchor"].cpu().numpy().copy()}


def _graph_vs_eager(wl, rounds, temperature=0.0, oracle_seqs=()):
    d = wl.dims
    B, k = d.batch, d.block_k
    say(f"[graph] {wl.name}: {rounds} rounds, temperature {temperature}, oracle on {list(oracle_seqs)}")
    W = bd.pack_weights(d, synth.make_weights(d, seed=0, device="cuda"))
    cache, ws, ctx, pre, anchors, chunks = _prefill(wl, d, W)
    kind, q = wl.accept
    n_tab = rounds + 8
    a_tab = synth.planted_accept(kind, q, k, n_tab, B, seed=0)
    fill = synth.target_fill(k, n_tab, B, seed=0)
    pool = [synth.make_taps(d, k + 1, seed=0, stream=1 + i, device="cuda") for i in range(4)]
    saved_ctx = cache["ctx_len"].clone()
    snap = _snapshot(cache)
    loop = harness.RoundLoop(d, W, cache, ws, a_tab, fill, seed=0, temperature=temperature)

    def rewind(r):
        if wl.rewind and (r + 1) % wl.rewind == 0:
            cache["ctx_len"].copy_(saved_ctx)

    # eager rounds
    loop.restart(saved_ctx)
    eager = []
    for r in range(rounds):
        loop.round(pool[r % 4])
        eager.append(_record(loop, cache))
        rewind(r)
    kv_eager = (cache["k"].clone(), cache["v"].clone())

    # the benchmark's sequence: an eager round on a side stream, one graph per taps
    # slot, the tables restarted; the decode state goes back to the snapshot
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
    _restore(cache, snap)
    loop.restart(saved_ctx)
    torch.cuda.synchronize()

    replays = []
    for r in range(rounds):
        graphs[r % 4].replay()
        rec = _record(loop, cache)
        for key in rec:
            assert np.array_equal(rec[key], eager[r][key]), f"round {r}: replayed {key} differs from eager"
        replays.append(rec)
        rewind(r)
    torch.cuda.synchronize()
    assert torch.equal(cache["k"], kv_eager[0]) and torch.equal(cache["v"], kv_eager[1]), \
        "K/V cache after the replays differs from the eager rounds"
    assert int(cache["dev_error"].item()) == 0
    if temperature > 0:
        assert int(loop.rng_step.item()) == rounds
    say(f"[graph] {wl.name}: {rounds} replays bitwise equal to eager rounds; "
        f"accepted per round {[int(r['accept'].sum()) for r in replays]}")

    if oracle_seqs:
        _oracle_check(wl, d, W, ctx, pre, anchors, chunks, pool, replays, oracle_seqs, saved_ctx, cache)


def _oracle_check(wl, d, W, ctx, pre, anchors, chunks, pool, replays, seqs, saved_ctx, cache):
    """The replayed rounds of sequences `seqs` against the fp64 oracle.  The oracle
    follows the GPU's accepted lengths (its verify_commit runs on the GPU's drafts
    and target tokens), so both sides keep the same context every round."""
    s = list(seqs)
    k = d.block_k
    Wn = oracle_weights(W)
    st = orc.new_state(d, batch=len(s), ctx_len=(ctx - pre)[s], anchor=anchors[s])
    taps = torch.cat(chunks, dim=1)[s].float().cpu().numpy()
    orc.fuse_inject(d, Wn, st, taps, pre[s], commit=True)
    saved = saved_ctx[s].cpu().numpy().astype(np.int64)
    gated = total = 0
    for r, rec in enumerate(replays):
        o = orc.draft_step(d, Wn, st, want_logits=False)
        gate = o["margin"] >= 0.1
        dg = rec["draft"][s].astype(np.int64)
        assert np.all((dg == o["draft"]) | ~gate), f"round {r}: a draft differs where the oracle margin >= 0.1"
        gated += int(gate.sum())
        total += gate.size
        orc.fuse_inject(d, Wn, st, pool[r % 4][s].float().cpu().numpy(), np.full(len(s), k + 1), commit=False)
        ist = integer_state(st.ctx_len, st.anchor, d)
        res = orc.verify_commit(d, st, dg, rec["target"][s])
        orc.verify_commit(d, ist, dg, rec["target"][s])
        assert np.array_equal(res["accept_len"], rec["accept"][s]), f"round {r}: accepted lengths"
        assert np.array_equal(res["out_tokens"], rec["out"][s]), f"round {r}: emitted tokens"
        assert np.array_equal(st.ctx_len, rec["ctx"][s]) and np.array_equal(st.anchor, rec["anchor"][s])
        if wl.rewind and (r + 1) % wl.rewind == 0:
            st.ctx_len[:] = saved
    # committed K/V window after the last round
    kc = cache["k"][:, s].float().cpu().numpy()
    vc = cache["v"][:, s].float().cpu().numpy()
    err = 0.0
    for j in range(len(s)):
        slots = np.array([orc.slot_of(d, int(p)) for p in orc.window_positions(d, int(st.ctx_len[j]))])
        err = max(err, float(np.max(np.abs(kc[:, j][:, :, slots] - st.k_ring[:, j][:, :, slots]))),
                  float(np.max(np.abs(vc[:, j][:, :, slots] - st.v_ring[:, j][:, :, slots]))))
    say(f"[graph] oracle: drafts {gated}/{total} margin-gated and equal; verify/commit exact; kv err {err:.3g}")
    assert err <= 0.05
    assert gated > 0


@pytest.mark.timeout(900)
def test_graph_replay_qwen3_8b_b1_with_rewind():
    _graph_vs_eager(configs.C2, rounds=10, oracle_seqs=(0,))


@pytest.mark.timeout(900)
def test_graph_replay_longctx_b256():
    _graph_vs_eager(configs.C5, rounds=5, oracle_seqs=(0, 255))


@pytest.mark.timeout(900)
def test_graph_replay_longctx_b256_sampled():
    _graph_vs_eager(configs.C5, rounds=5, temperature=1.0)
