"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

This module only draws numbers: weights, target-layer taps, anchors, context
lengths, planted acceptance lengths and the planted target tokens that stand in
for the target model's greedy verification.  It holds none of the drafter's
arithmetic, and it imports neither the oracle nor the HIP library.

Recipe (seed 0 unless a caller says otherwise):
  * weight matrices and the mask embedding: N(0, 0.02^2), drawn in fp32 and, for
    bf16 drafters, rounded to bf16 (round to nearest even);
  * RMSNorm gains: 1;
  * taps (hidden states of the 5 target layers): N(0, 1), same rounding;
  * anchors and filler target tokens: uniform integers;
  * planted accepted length a*: min(G, k) with P(G >= j) = q^j (truncated
    geometric), or uniform on 0..k;
  * logits standing in for the target's (sampled verification): N(0, s^2) fp32
    filler, with planted rows (see plant_target_logits).
Every tensor has its own generator seeded from (seed, tensor id, ...), so any
tensor can be regenerated alone.  Tensors are drawn with torch on the device that
will hold them; the oracle receives host copies of exactly those values.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np
import torch

from .configs import BF16, Dims, Workload

WEIGHT_NAMES = ("fuse_w", "fuse_norm", "embed", "mask_embed", "attn_norm", "w_qkv",
                "w_o", "mlp_norm", "w_gate_up", "w_down", "final_norm", "lm_head")
_GAINS = ("fuse_norm", "attn_norm", "mlp_norm", "final_norm")
WEIGHT_STD = 0.02

# tensor ids of the non-weight streams
_TAPS, _ANCHOR, _CTX, _ACCEPT, _FILL, _LOGITS = 100, 101, 102, 103, 104, 105


def stream_seed(seed: int, *ids: int) -> int:
    """A 63-bit generator seed derived from (seed, ids) by numpy's SeedSequence."""
    st = np.random.SeedSequence([int(seed)] + [int(i) for i in ids]).generate_state(2, np.uint32)
    return int((int(st[0]) << 31) ^ int(st[1])) & 0x7FFF_FFFF_FFFF_FFFF


def torch_dtype(dims: Dims) -> torch.dtype:
    return torch.bfloat16 if dims.dtype == BF16 else torch.float32


def weight_shapes(d: Dims) -> Dict[str, tuple]:
    """nn.Linear layout [out, in] for every matrix; per-layer tensors lead with L."""
    L, D = d.n_layers, d.hidden
    return {
        "fuse_w": (D, d.n_taps * d.tap_dim),
        "fuse_norm": (D,),
        "embed": (d.vocab, D),
        "mask_embed": (D,),
        "attn_norm": (L, D),
        "w_qkv": (L, d.qkv_rows, D),
        "w_o": (L, D, d.n_q_heads * d.head_dim),
        "mlp_norm": (L, D),
        "w_gate_up": (L, 2 * d.ffn, D),
        "w_down": (L, D, d.ffn),
        "final_norm": (D,),
        "lm_head": (d.vocab, D),
    }


def _normal(shape, seed: int, ids: Sequence[int], std: float, dtype: torch.dtype,
            device) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(stream_seed(seed, *ids))
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def make_weights(d: Dims, seed: int = 0, device="cpu") -> Dict[str, torch.Tensor]:
    """All drafter weights, in the drafter's dtype, on ``device``."""
    dt = torch_dtype(d)
    out = {}
    for tid, (name, shape) in enumerate(weight_shapes(d).items()):
        if name in _GAINS:
            out[name] = torch.ones(shape, dtype=dt, device=device)
        elif len(shape) == 3:
            # one generator per layer so a layer can be regenerated alone
            out[name] = torch.stack([_normal(shape[1:], seed, (tid, l), WEIGHT_STD, dt, device)
                                     for l in range(shape[0])])
        else:
            out[name] = _normal(shape, seed, (tid,), WEIGHT_STD, dt, device)
    return out


def make_taps(d: Dims, n_rows: int, seed: int = 0, stream: int = 0, device="cpu",
              batch: Optional[int] = None) -> torch.Tensor:
    """Target hidden states of the 5 tapped layers: [B, n_rows, n_taps, tap_dim]."""
    B = d.batch if batch is None else batch
    return _normal((B, n_rows, d.n_taps, d.tap_dim), seed, (_TAPS, stream), 1.0,
                   torch_dtype(d), device)


def make_anchors(d: Dims, seed: int = 0) -> np.ndarray:
    rng = np.random.default_rng(stream_seed(seed, _ANCHOR))
    return rng.integers(0, d.vocab, size=d.batch, dtype=np.int64).astype(np.int32)


def make_context_lengths(w: Workload, seed: int = 0) -> np.ndarray:
    """Committed length of every sequence at the first block step."""
    B = w.dims.batch
    if w.context_lo is None:
        return np.full(B, w.context, dtype=np.int32)
    rng = np.random.default_rng(stream_seed(seed, _CTX))
    return rng.integers(w.context_lo, w.context + 1, size=B).astype(np.int32)


def planted_accept(kind: str, q: Optional[float], k: int, steps: int, batch: int,
                   seed: int = 0) -> np.ndarray:
    """Planted accepted lengths a* in 0..k, shape [steps, batch]."""
    if kind == "each":
        return np.tile((np.arange(steps) % (k + 1))[:, None], (1, batch)).astype(np.int32)
    rng = np.random.default_rng(stream_seed(seed, _ACCEPT, int(1e6 * (q or 0))))
    if kind == "uniform":
        return rng.integers(0, k + 1, size=(steps, batch)).astype(np.int32)
    if kind == "geometric":
        # G = number of leading successes of Bernoulli(q) trials; P(G >= j) = q^j
        u = rng.random((steps, batch, k))
        lead = np.cumprod(u < q, axis=2).sum(axis=2)
        return lead.astype(np.int32)
    raise ValueError(kind)


def target_fill(k: int, steps: int, batch: int, seed: int = 0) -> np.ndarray:
    """Uniform filler integers in [0, 2^31) for the planted targets, [steps, B, k+1]."""
    rng = np.random.default_rng(stream_seed(seed, _FILL))
    return rng.integers(0, 2 ** 31 - 1, size=(steps, batch, k + 1)).astype(np.int32)


def plant_targets(draft: np.ndarray, a_star: np.ndarray, fill: np.ndarray,
                  vocab: int) -> np.ndarray:
    """Target stand-in: tokens that accept exactly a* drafts of each sequence.

    T[i] = draft[i] for i < a*; if a* < k, T[a*] differs from draft[a*]; every
    other entry (and the bonus T[k] when a* = k) is filler.
    """
    draft = np.asarray(draft, dtype=np.int64)
    B, k = draft.shape
    T = (np.asarray(fill, dtype=np.int64) % vocab).copy()
    for b in range(B):
        a = int(a_star[b])
        T[b, :a] = draft[b, :a]
        if a < k:
            T[b, a] = (draft[b, a] + 1 + int(fill[b, a]) % (vocab - 1)) % vocab
    return T.astype(np.int32)


def make_logits(shape, seed: int = 0, stream: int = 0, scale: float = 2.0, device="cpu") -> torch.Tensor:
    """N(0, scale^2) fp32 logits of the given shape."""
    return _normal(tuple(shape), seed, (_LOGITS, stream), scale, torch.float32, device)


def plant_target_logits(draft_logits: torch.Tensor, draft: np.ndarray, a_star: np.ndarray,
                        fill: torch.Tensor, soft: float = 0.0, seed: int = 0) -> torch.Tensor:
    """Target-logit stand-in for sampled verification, [B, k+1, V] fp32.

    Rows i < a*: the draft's own logits (so p_i = q_i and the draft is accepted),
    plus N(0, soft^2) noise when soft > 0 (then acceptance is likely, not certain);
    row a* < k: filler with the drafted token's logit at -1e4 (p(x) = 0: rejected);
    every other row, and the bonus row k: filler."""
    z = draft_logits.float()
    B, k, V = z.shape
    t = fill.float().clone()
    dr = np.asarray(draft, dtype=np.int64)
    for b in range(B):
        a = int(a_star[b])
        if a > 0:
            t[b, :a] = z[b, :a]
            if soft > 0:
                t[b, :a] += _normal((a, V), seed, (_LOGITS, 10_000 + b), soft, torch.float32, z.device)
        if a < k and dr[b, a] >= 0:  # a draft past a shorter block (-1) has nothing to reject
            t[b, a, int(dr[b, a])] = -1.0e4
    return t
