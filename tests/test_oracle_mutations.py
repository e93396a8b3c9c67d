"""Plant plausible mistakes into the oracle (CPU only) and check that its pins fail.

Each mutation replaces one oracle helper with a subtly wrong version; the pin
battery (brute-force twin on tiny scenarios + exhaustive verification) must
reject every one of them.  This shows the pins are strong enough to trust the
oracle, not that the oracle is wrong.
"""
import numpy as np
import pytest

from oracle import bruteforce as bf
from oracle import dflash_oracle as orc
from tests.helpers import prefilled, tiny_dims, tiny_weights, with_sink, with_window

_rope, _rms, _attend, _silu, _linear = orc.rope, orc.rms_norm, orc.attend, orc.silu, orc.linear
_window, _accepted, _slot = orc.window_positions, orc.accepted_length, orc.slot_of


def battery() -> bool:
    """True iff the oracle agrees with the brute force and the verify definition."""
    try:
        for ctx, window, k, sink in [([9, 3], 6, 4, 0), ([4, 12], 5, 3, 0), ([15, 4], 4, 3, 2)]:
            d = with_window(tiny_dims(block_k=k, batch=2), window) if sink == 0 else \
                with_sink(tiny_dims(block_k=k, batch=2), sink, window)
            W = tiny_weights(d, seed=21)
            st, hist = prefilled(d, W, ctx, seed=22, anchors=[2, 17])
            z = orc.draft_step(d, W, st)["logits"]
            for b in range(2):
                ref = np.array(bf.block_logits(d, W, hist[b], ctx[b], int(st.anchor[b])))
                if not np.allclose(z[b], ref, rtol=1e-9, atol=1e-9):
                    return False
        d = tiny_dims(block_k=4, batch=1, vocab=100)
        for bits in range(16):
            draft = np.arange(4)[None] + 1
            tgt = np.array([[1 + i if (bits >> i) & 1 else 50 for i in range(4)] + [60]])
            st = orc.new_state(d, batch=1, ctx_len=[10])
            if orc.verify_commit(d, st, draft, tgt)["accept_len"][0] != bf.first_mismatch(draft[0], tgt[0], 4):
                return False
        return True
    except (ValueError, IndexError):
        return False


def _rope_neg(x, pos, theta):
    return _rope(x, -np.asarray(pos), theta)


def _rope_interleaved(x, pos, theta):
    x = np.asarray(x, dtype=np.float64)
    dh = x.shape[-1]
    perm = np.concatenate([np.arange(0, dh, 2), np.arange(1, dh, 2)])
    inv = np.argsort(perm)
    return _rope(x[..., perm], pos, theta)[..., inv]


def _rope_slot(x, pos, theta):
    return _rope(x, np.asarray(pos) % 10, theta)


def _rms_no_eps(x, g, eps):
    return _rms(x, g, 0.0)


def _rms_sum(x, g, eps):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, -1, keepdims=True) + eps) * np.asarray(g)


def _rms_no_gain(x, g, eps):
    return _rms(x, np.ones_like(np.asarray(g, dtype=np.float64)), eps)


def _attend_unscaled(q, keys, vals):
    return orc.softmax(np.asarray(q) @ np.asarray(keys).T, -1) @ np.asarray(vals)


def _attend_causal_block(q, keys, vals):
    q, keys, vals = (np.asarray(a, dtype=np.float64) for a in (q, keys, vals))
    nq, nk = q.shape[0], keys.shape[0]
    s = q @ keys.T / np.sqrt(q.shape[-1])
    n_ctx = nk - nq
    for i in range(nq):
        s[i, n_ctx + i + 1:] = -np.inf
    return orc.softmax(s, -1) @ vals


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-np.asarray(x, dtype=np.float64)))


def _linear_t(x, W):
    return np.asarray(x, dtype=np.float64) @ np.asarray(W, dtype=np.float64)


def _window_short(dims, P):
    return np.arange(max(0, P - dims.window + 1), P)


def _window_long(dims, P):
    return np.arange(max(0, P - dims.window - 1), P)


def _window_sink_twice(dims, P):
    s = min(dims.sink, P)
    return np.concatenate([np.arange(0, s), np.arange(max(0, P - dims.window), P)])


def _window_sink_ignored(dims, P):
    return np.arange(max(0, P - dims.window), P)


def _slot_sink_in_ring(dims, p):
    return int(p) % dims.cache_slots


def _accept_count_all(draft_row, target_row, k):
    return int(sum(int(draft_row[i]) == int(target_row[i]) for i in range(k)))


MUTATIONS = {
    "rope_negative_angle": ("rope", _rope_neg),
    "rope_interleaved_pairs": ("rope", _rope_interleaved),
    "rope_at_ring_slot": ("rope", _rope_slot),
    "rmsnorm_without_eps": ("rms_norm", _rms_no_eps),
    "rmsnorm_sum_not_mean": ("rms_norm", _rms_sum),
    "rmsnorm_gain_dropped": ("rms_norm", _rms_no_gain),
    "attention_unscaled": ("attend", _attend_unscaled),
    "attention_causal_block": ("attend", _attend_causal_block),
    "silu_is_sigmoid": ("silu", _sigmoid),
    "linear_transposed": ("linear", _linear_t),
    "window_one_short": ("window_positions", _window_short),
    "window_one_long": ("window_positions", _window_long),
    "accept_counts_all_matches": ("accepted_length", _accept_count_all),
    "sink_counted_twice": ("window_positions", _window_sink_twice),
    "sink_ignored": ("window_positions", _window_sink_ignored),
    "sink_slots_in_the_ring": ("slot_of", _slot_sink_in_ring),
}


def test_battery_passes_unmutated():
    assert battery()


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(orc, attr, fn)
    assert not battery(), f"pins did not catch {name}"


def _kv_head_modulo(hq, n_q_heads, n_kv_heads):
    return hq % n_kv_heads


def test_gqa_grouping_mutation_is_caught(monkeypatch):
    """Query head h reads kv head h // (Hq/Hkv); h % Hkv is a plausible slip."""
    monkeypatch.setattr(orc, "kv_head_of", _kv_head_modulo)
    assert not battery()
