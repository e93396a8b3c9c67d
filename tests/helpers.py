"""Tiny shapes and scenario builders shared by the CPU oracle tests."""
from __future__ import annotations

from dataclasses import replace

import numpy as np

from block_diffusion_speculative_dflash_amd.configs import Dims, F32
from oracle import dflash_oracle as orc


def tiny_dims(**kw) -> Dims:
    """hidden 16 = Hq*dh (so w_o is square and a transposed operand shows),
    GQA 4 query heads over 2 kv heads, window 6, ring of window + k slots."""
    base = dict(batch=2, block_k=4, n_layers=2, hidden=16, n_q_heads=4, n_kv_heads=2,
                head_dim=4, ffn=12, vocab=32, n_taps=5, tap_dim=8, window=6,
                cache_slots=10, dtype=F32, max_inject_rows=8, rms_eps=1e-6,
                rope_theta=10000.0)
    base.update(kw)
    if "cache_slots" not in kw:
        base["cache_slots"] = base["window"] + base["block_k"]
    return Dims(**base)


def tiny_weights(d: Dims, seed: int = 0, std: float = 0.5, gain_jitter: float = 0.2):
    """Random weights large enough that logits spread (std 0.5) and non-unit gains
    (so a dropped gain shows)."""
    rng = np.random.default_rng(seed)
    L, D = d.n_layers, d.hidden

    def m(*shape):
        return rng.normal(0.0, std, size=shape)

    def g(*shape):
        return 1.0 + gain_jitter * rng.normal(size=shape)

    return {
        "fuse_w": m(D, d.n_taps * d.tap_dim) / np.sqrt(d.n_taps),
        "fuse_norm": g(D),
        "embed": m(d.vocab, D) * 2,
        "mask_embed": m(D) * 2,
        "attn_norm": g(L, D),
        "w_qkv": m(L, d.qkv_rows, D),
        "w_o": m(L, D, d.n_q_heads * d.head_dim),
        "mlp_norm": g(L, D),
        "w_gate_up": m(L, 2 * d.ffn, D),
        "w_down": m(L, D, d.ffn),
        "final_norm": g(D),
        "lm_head": m(d.vocab, D),
    }


def random_taps(d: Dims, B: int, n: int, seed: int):
    return np.random.default_rng(seed).normal(size=(B, n, d.n_taps, d.tap_dim))


def prefilled(d: Dims, W, ctx_lens, seed: int = 1, anchors=None, offset: int = 0):
    """Oracle state after committing ctx_lens[b] positions (starting at ``offset``),
    plus the committed history {position: taps} of every sequence."""
    B = len(ctx_lens)
    n_max = max(max(ctx_lens), 1)
    taps = random_taps(d, B, n_max, seed)
    st = orc.new_state(d, batch=B, ctx_len=np.full(B, offset),
                       anchor=anchors if anchors is not None else np.arange(B) % d.vocab)
    orc.fuse_inject(d, W, st, taps, np.asarray(ctx_lens), commit=True)
    hist = [{offset + p: taps[b, p] for p in range(ctx_lens[b])} for b in range(B)]
    return st, hist


def with_window(d: Dims, window: int, extra_slots: int = 0) -> Dims:
    return replace(d, window=window, cache_slots=window + d.block_k + extra_slots)


def with_sink(d: Dims, sink: int, window: int, extra_slots: int = 0) -> Dims:
    """Attention sink of `sink` positions plus a window of `window`: sink slots, then
    a ring of window + k (+ extra) slots."""
    return replace(d, sink=sink, window=window, cache_slots=sink + window + d.block_k + extra_slots)
