"""Pins of the per-sequence block length (CPU only, oracle).

* a sequence drafting k_b < k rows gets exactly the rows of a block of k_b: the
  brute-force twin run with block size k_b (k_b = 1 is one decode step; k_b = 0
  drafts nothing);
* greedy verification over k_b rows: all 2^k_b match patterns, the bonus from
  target[k_b] after a full accept, rollback up to P + k_b only;
* sampled verification over k_b rows: its T -> 0 limit is the ragged greedy rule.
"""
from dataclasses import replace

import numpy as np
import pytest

from oracle import bruteforce as bf
from oracle import dflash_oracle as orc
from oracle import sampling as sp
from tests.helpers import prefilled, tiny_dims, tiny_weights, with_window


@pytest.mark.parametrize("lens", [[4, 1], [2, 3], [0, 4], [1, 0], [3, 2]])
def test_ragged_rows_equal_a_block_of_that_length(lens):
    d = with_window(tiny_dims(block_k=4, batch=2), 5)
    W = tiny_weights(d, seed=31)
    ctx = [9, 6]
    st, hist = prefilled(d, W, ctx, seed=32, anchors=[3, 11])
    out = orc.draft_step(d, W, st, block_len=lens)
    for b, kb in enumerate(lens):
        assert np.all(out["draft"][b, kb:] == -1) and np.all(np.isnan(out["logits"][b, kb:]))
        if kb == 0:
            continue
        ref = np.array(bf.block_logits(replace(d, block_k=kb), W, hist[b], ctx[b], int(st.anchor[b])))
        assert np.allclose(out["logits"][b, :kb], ref, rtol=1e-9, atol=1e-9)
        assert np.array_equal(out["draft"][b, :kb], np.argmax(ref, axis=-1))


def test_block_of_one_is_a_decode_step_per_sequence():
    d = with_window(tiny_dims(block_k=4, batch=2), 6)
    W = tiny_weights(d, seed=33)
    st, _ = prefilled(d, W, [7, 12], seed=34, anchors=[5, 9])
    z = orc.draft_step(d, W, st, block_len=[1, 1])["logits"][:, 0]
    assert np.allclose(z, orc.decode_step(d, W, st), rtol=1e-9, atol=1e-9)


def test_full_length_list_equals_the_default():
    d = tiny_dims(block_k=4, batch=2)
    W = tiny_weights(d, seed=35)
    st, _ = prefilled(d, W, [8, 3], seed=36)
    a = orc.draft_step(d, W, st)
    b = orc.draft_step(d, W, st, block_len=[4, 4])
    assert np.array_equal(a["draft"], b["draft"]) and np.array_equal(a["logits"], b["logits"])


def test_block_length_out_of_range_is_rejected():
    d = tiny_dims(block_k=4, batch=2)
    st = orc.new_state(d, batch=2, ctx_len=[3, 3])
    with pytest.raises(ValueError):
        orc.draft_step(d, tiny_weights(d), st, block_len=[5, 1])
    with pytest.raises(ValueError):
        orc.verify_commit(d, st, np.zeros((2, 4)), np.zeros((2, 5)), block_len=[-1, 2])


@pytest.mark.parametrize("kb", [0, 1, 3, 6])
def test_ragged_verify_every_pattern(kb):
    k = 6
    d = tiny_dims(block_k=k, batch=1, vocab=100, window=8)
    for bits in range(2 ** kb):
        draft = (np.arange(k)[None] + 1)
        tgt = np.array([[1 + i if i < kb and (bits >> i) & 1 else 50 + i for i in range(k)] + [70]])
        st = orc.new_state(d, batch=1, ctx_len=[20])
        st.k_ring[:] = 0.0
        r = orc.verify_commit(d, st, draft, tgt, block_len=[kb])
        a = bf.first_mismatch(draft[0], tgt[0], kb)
        assert r["accept_len"][0] == a <= kb
        assert list(r["out_tokens"][0, :a + 1]) == list(tgt[0, :a + 1])
        assert np.all(r["out_tokens"][0, a + 1:] == -1)
        assert st.ctx_len[0] == 20 + a + 1 and st.anchor[0] == tgt[0, a]
        # rows P+a+1 .. P+kb rolled back, nothing beyond P+kb touched
        dead = {orc.slot_of(d, p) for p in range(20 + a + 1, 20 + kb + 1)}
        for s in range(d.cache_slots):
            assert np.isnan(st.k_ring[0, 0, 0, s, 0]) == (s in dead)


def test_sampled_ragged_zero_temperature_is_ragged_greedy():
    rng = np.random.default_rng(12)
    n, k, V, T = 5, 4, 10, 1e-5
    z = np.round(rng.normal(0, 2, (n, k, V)), 2) + rng.permutation(V) * 1e-3
    t = np.round(rng.normal(0, 2, (n, k + 1, V)), 2) + rng.permutation(V) * 1e-3
    kb = np.array([0, 1, 2, 4, 3])
    for j in range(n):
        for i in range(j % (k + 1)):
            t[j, i] = z[j, i]
    d = sp.sample_drafts(z, T, 3, 2, block_len=kb)
    assert all(np.all(d["draft"][j, kb[j]:] == -1) for j in range(n))
    r = sp.verify_sampled(d["draft"], z, t, T, 3, 2, block_len=kb)
    dims = tiny_dims(block_k=k, batch=n, vocab=V)
    st = orc.new_state(dims, batch=n, ctx_len=[30] * n)
    g = orc.verify_commit(dims, st, np.where(d["draft"] < 0, 0, d["draft"]), np.argmax(t, axis=-1),
                          block_len=kb)
    assert np.array_equal(r["accept_len"], g["accept_len"])
    assert np.array_equal(r["out_tokens"], g["out_tokens"])
    assert np.all(r["accept_len"] <= kb)
