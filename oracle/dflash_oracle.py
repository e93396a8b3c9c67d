"""Plain float64 CPU oracle of the DFlash block draft-and-verify step.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's CPU
baseline may import this module; the product path (the HIP library and its
binding) never does, and this module imports nothing from it.

What it computes, step by step, in the order the pages give it:

* Feature fusion (zhihu answer on MiMo-V2.5-Pro-UltraSpeed, §5.1): the hidden
  states of 5 target layers for one position are concatenated (ascending depth),
  projected by one linear map and RMS-normalised into the context feature c.
* KV injection (same answer, §5.2): c goes through every draft layer's K and V
  projections and is kept in that layer's KV cache, so every layer attends to the
  target context.  The cache is a ring of C slots per (layer, sequence, kv head);
  logical position p lives in slot p mod C (hotdry blog, "draft scheduling: SWA
  alignment": the drafter is all sliding-window attention with a 128-token window).
* Block drafting (hotdry blog, "from autoregressive to block-level prediction";
  zhihu answer §4 block diffusion and §5.3): a block of k positions, the visible
  anchor token followed by k-1 mask positions, runs through the draft transformer
  in one forward pass; attention inside the block is bidirectional and every block
  query also sees the last W committed positions.  Row i's argmax proposes the
  token at position P+i+1.
* Greedy verification (zhihu answer §2, the draft/verify/accept steps; lossless
  acceptance in §6): drafts are accepted up to the first one that differs from the
  target's token; the target's token at that point is the bonus token.  The
  committed length grows by accepted + 1, and cache rows past it are rolled back.

Everything is float64 numpy on whatever values the caller passes (the exact
bf16/fp32 values the GPU receives).  Where the pages are silent this module takes
one reading and says so at the point of use:
  - no biases; RMSNorm eps from the dims (1e-6 by default);
  - RoPE: rotate-half pairs (i, i + dh/2), base theta from the dims, applied to q
    and k at absolute logical positions, including injected context keys;
  - the mask position uses a dedicated embedding vector, not a vocabulary row;
  - the injected K/V use the same per-layer K/V projections as the block's own keys;
  - ties in argmax go to the smallest token id.
Every function here is pinned by the CPU tests (brute force on tiny inputs,
library special cases, invariants); none is "parity unpinned".

Precision study only: fuse_inject and draft_step take an optional `act_round`
function, applied to the values an implementation stores between its matrix
products (the normalised matrix inputs, q/k/v, the injected K/V rows, the attention
output, the SwiGLU product).  With the default None nothing is rounded and the
computation is the exact float64 one above; a test passes bf16 or fp16 rounding to
measure what storing those values in 16 bits costs in logit error.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Optional, Sequence

import numpy as np

_ROW_CHUNK = 8192  # rows of a weight matrix upcast to float64 at a time (memory only)


def f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# ----------------------------------------------------------------------------
# elementary operations
# ----------------------------------------------------------------------------

def linear(x, W) -> np.ndarray:
    """y = x W^T for W in nn.Linear layout [out, in]; no bias (reading)."""
    x = f64(x)
    W = np.asarray(W)
    out = np.empty(x.shape[:-1] + (W.shape[0],), dtype=np.float64)
    for r0 in range(0, W.shape[0], _ROW_CHUNK):
        out[..., r0:r0 + _ROW_CHUNK] = x @ f64(W[r0:r0 + _ROW_CHUNK]).T
    return out


def rms_norm(x, g, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * g over the last axis (zhihu answer §5.1 names RMSNorm)."""
    x = f64(x)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * f64(g)


def silu(x) -> np.ndarray:
    x = f64(x)
    return x / (1.0 + np.exp(-x))


def rope_inv_freq(head_dim: int, theta: float) -> np.ndarray:
    return float(theta) ** (-(2.0 * np.arange(head_dim // 2, dtype=np.float64)) / head_dim)


def rope(x, pos, theta: float) -> np.ndarray:
    """Rotate-half rotary embedding of x [..., dh] at integer positions pos [...]."""
    x = f64(x)
    dh = x.shape[-1]
    half = dh // 2
    ang = np.asarray(pos, dtype=np.float64)[..., None] * rope_inv_freq(dh, theta)
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def softmax(s, axis: int = -1) -> np.ndarray:
    s = f64(s)
    e = np.exp(s - np.max(s, axis=axis, keepdims=True))
    return e / np.sum(e, axis=axis, keepdims=True)


def kv_head_of(hq: int, n_q_heads: int, n_kv_heads: int) -> int:
    """Grouped-query attention: consecutive groups of Hq/Hkv query heads share a kv head."""
    return hq // (n_q_heads // n_kv_heads)


def attend(q, keys, vals) -> np.ndarray:
    """softmax(q keys^T / sqrt(dh)) vals for one head: q [n_q, dh], keys/vals [n_k, dh]."""
    q, keys, vals = f64(q), f64(keys), f64(vals)
    return softmax(q @ keys.T / np.sqrt(q.shape[-1]), axis=-1) @ vals


# ----------------------------------------------------------------------------
# decode state
# ----------------------------------------------------------------------------

@dataclass
class State:
    """Per-sequence decode state: K/V rings, committed length P and anchor token.

    k_ring / v_ring: [L, B, Hkv, C, dh] float64; slot_of(dims, p) holds position p.
    Slots that hold no committed position are NaN, so reading one poisons logits.
    """
    k_ring: np.ndarray
    v_ring: np.ndarray
    ctx_len: np.ndarray
    anchor: np.ndarray


def new_state(dims, batch: Optional[int] = None, ctx_len=None, anchor=None) -> State:
    B = dims.batch if batch is None else batch
    shape = (dims.n_layers, B, dims.n_kv_heads, dims.cache_slots, dims.head_dim)
    ctx = np.zeros(B, np.int64) if ctx_len is None else np.array(ctx_len, dtype=np.int64)
    anc = np.zeros(B, np.int64) if anchor is None else np.array(anchor, dtype=np.int64)
    return State(np.full(shape, np.nan), np.full(shape, np.nan), ctx, anc)


def _kv_rows(dims):
    """Row ranges of the K and V projections inside the fused [q | k | v] weight."""
    q_end = dims.n_q_heads * dims.head_dim
    k_end = q_end + dims.n_kv_heads * dims.head_dim
    return (q_end, k_end), (k_end, k_end + dims.n_kv_heads * dims.head_dim)


# ----------------------------------------------------------------------------
# feature fusion + KV injection
# ----------------------------------------------------------------------------

def fuse(dims, W: Dict[str, np.ndarray], taps) -> np.ndarray:
    """Fused context feature c for taps [..., n_taps, tap_dim] (zhihu answer §5.1).

    The n_taps hidden states are concatenated along features in ascending target
    depth (reading), projected by fuse_w and RMS-normalised with gain fuse_norm.
    """
    taps = f64(taps)
    x = taps.reshape(taps.shape[:-2] + (dims.n_taps * dims.tap_dim,))
    u = linear(x, W["fuse_w"])
    return rms_norm(u, W["fuse_norm"], dims.rms_eps)


def inject_kv(dims, W, layer: int, c, pos):
    """K/V rows that the fused feature c contributes to one draft layer (§5.2).

    Uses that layer's own K and V projections (reading); K gets RoPE at its
    logical position.  Returns K, V of shape [..., Hkv, dh].
    """
    (k0, k1), (v0, v1) = _kv_rows(dims)
    wq = W["w_qkv"][layer]
    K = linear(c, wq[k0:k1]).reshape(np.shape(c)[:-1] + (dims.n_kv_heads, dims.head_dim))
    V = linear(c, wq[v0:v1]).reshape(np.shape(c)[:-1] + (dims.n_kv_heads, dims.head_dim))
    K = rope(K, np.asarray(pos)[..., None], dims.rope_theta)
    return K, V


def _exact(a):
    return a


def fuse_inject(dims, W, st: State, taps, n_rows, commit: bool, act_round=None) -> None:
    """Fuse the taps of n_rows[b] new positions starting at ctx_len[b] and write
    their K/V rows into every layer's ring; with commit, advance ctx_len.
    act_round: precision study only (see the module notes); None = exact."""
    R = act_round or _exact
    taps = f64(taps)
    B = st.ctx_len.shape[0]
    n_rows = np.asarray(n_rows, dtype=np.int64)
    c = R(fuse(dims, W, taps))                               # [B, n_max, d]
    for b in range(B):
        n = int(n_rows[b])
        if n == 0:
            continue
        pos = st.ctx_len[b] + np.arange(n)
        for l in range(dims.n_layers):
            K, V = inject_kv(dims, W, l, c[b, :n], pos)     # [n, Hkv, dh]
            K, V = R(K), R(V)
            for r in range(n):                               # in position order
                slot = slot_of(dims, int(pos[r]))
                st.k_ring[l, b, :, slot, :] = K[r]
                st.v_ring[l, b, :, slot, :] = V[r]
        if commit:
            st.ctx_len[b] += n


def slot_of(dims, p: int) -> int:
    """Cache slot of position p: the first s positions (the attention sink) keep
    slots 0..s-1; later positions share a ring of C - s slots after them.  With
    s = 0 this is p mod C (hotdry blog, SWA section: sliding-window cache; aufer
    article, micro-op section, names the attention sink as this drafter's knob)."""
    s = int(getattr(dims, "sink", 0))
    if p < s:
        return int(p)
    return s + (int(p) - s) % (dims.cache_slots - s)


def window_positions(dims, P: int) -> np.ndarray:
    """Committed positions every block query sees: the sink positions 0..s-1 that
    exist, then the last W positions before P that are not sink positions (no
    position is listed twice)."""
    s = min(int(getattr(dims, "sink", 0)), P)
    return np.concatenate([np.arange(0, s), np.arange(max(s, P - dims.window), P)]).astype(np.int64)


# ----------------------------------------------------------------------------
# block draft
# ----------------------------------------------------------------------------

def block_lengths(dims, batch: int, block_len=None) -> np.ndarray:
    """Per-sequence block length k_b in [0, k] (None: every sequence drafts k rows).
    k_b = 0 means speculation is off for that sequence this round (hotdry blog,
    acceptance-rate section: the dynamic fallback may shrink the block or turn
    speculative decoding off)."""
    k = dims.block_k
    kb = np.full(batch, k, np.int64) if block_len is None else np.asarray(block_len, dtype=np.int64)
    if kb.shape != (batch,) or np.any(kb < 0) or np.any(kb > k):
        raise ValueError("block_len must hold one length in [0, k] per sequence")
    return kb


def block_logits(dims, W, st: State, b: int, kb: int, act_round=None) -> np.ndarray:
    """Logits [kb, V] of sequence b's block of kb rows: the anchor at position P,
    then kb - 1 mask positions; every row sees the committed window and all kb
    block keys (bidirectional inside the block).  act_round: precision study only."""
    R = act_round or _exact
    Hq, Hkv, dh, D, F = dims.n_q_heads, dims.n_kv_heads, dims.head_dim, dims.hidden, dims.ffn
    eps, theta = dims.rms_eps, dims.rope_theta
    P = int(st.ctx_len[b])

    # block construction: anchor at P, mask embedding at P+1 .. P+kb-1
    h = np.empty((kb, D), dtype=np.float64)
    h[0] = f64(np.asarray(W["embed"])[st.anchor[b]])
    h[1:] = f64(W["mask_embed"])
    pos = P + np.arange(kb)
    slots = np.array([slot_of(dims, int(p)) for p in window_positions(dims, P)], dtype=np.int64)

    for l in range(dims.n_layers):
        x = R(rms_norm(h, W["attn_norm"][l], eps))
        qkv = linear(x, W["w_qkv"][l])
        q = qkv[:, :Hq * dh].reshape(kb, Hq, dh)
        kk = qkv[:, Hq * dh:(Hq + Hkv) * dh].reshape(kb, Hkv, dh)
        vv = R(qkv[:, (Hq + Hkv) * dh:].reshape(kb, Hkv, dh))
        q = R(rope(q, pos[:, None], theta))
        kk = R(rope(kk, pos[:, None], theta))

        o = np.empty((kb, Hq, dh), dtype=np.float64)
        for hq in range(Hq):
            g = kv_head_of(hq, Hq, Hkv)
            keys = np.concatenate([st.k_ring[l, b, g, slots], kk[:, g]], axis=0)
            vals = np.concatenate([st.v_ring[l, b, g, slots], vv[:, g]], axis=0)
            o[:, hq] = attend(q[:, hq], keys, vals)           # no mask inside the block
        h = h + linear(R(o.reshape(kb, Hq * dh)), W["w_o"][l])

        y = R(rms_norm(h, W["mlp_norm"][l], eps))
        gu = linear(y, W["w_gate_up"][l])
        h = h + linear(R(silu(gu[:, :F]) * gu[:, F:]), W["w_down"][l])

    return linear(R(rms_norm(h, W["final_norm"], eps)), W["lm_head"])   # [kb, V]


def draft_step(dims, W, st: State, want_logits: bool = True, block_len=None,
               act_round=None) -> Dict[str, np.ndarray]:
    """One forward of the draft transformer over the block of every sequence.

    block_len: per-sequence block length k_b (default k for all).  Returns draft
    [B, k] (argmax, smallest id on ties; -1 past k_b), logits [B, k, V] (NaN past
    k_b) and margin [B, k] (top-1 minus top-2 logit; inf past k_b).
    act_round: precision study only (see the module notes); None = exact.
    """
    B, k, V = st.ctx_len.shape[0], dims.block_k, dims.vocab
    kb = block_lengths(dims, B, block_len)
    z = np.full((B, k, V), np.nan)
    draft = np.full((B, k), -1, np.int64)
    margin = np.full((B, k), np.inf)
    for b in range(B):
        n = int(kb[b])
        if n == 0:
            continue
        zb = block_logits(dims, W, st, b, n, act_round=act_round)
        z[b, :n] = zb
        draft[b, :n] = np.argmax(zb, axis=-1)                       # first max = smallest id
        top2 = np.sort(zb, axis=-1)[:, -2:]
        margin[b, :n] = top2[:, 1] - top2[:, 0]
    out = {"draft": draft, "margin": margin}
    if want_logits:
        out["logits"] = z
    return out


# ----------------------------------------------------------------------------
# greedy verification + commit / rollback
# ----------------------------------------------------------------------------

def accepted_length(draft_row: Sequence[int], target_row: Sequence[int], k: int) -> int:
    """Number of leading drafts equal to the target's tokens (accept until the first error)."""
    a = 0
    while a < k and int(draft_row[a]) == int(target_row[a]):
        a += 1
    return a


def verify_commit(dims, st: State, draft, target, block_len=None) -> Dict[str, np.ndarray]:
    """Greedy longest-prefix verify, bonus token, commit or roll back (in place).

    target[b] holds k+1 tokens: the target's greedy token for positions P+1..P+k+1
    given the anchor and the drafts before it.  With a block of k_b rows only
    draft[b, :k_b] is tested and target[b, k_b] is the bonus after a full accept.
    Emits target[b, 0..a]; the new committed length is P + a + 1 and the new anchor
    is target[b, a].  Rows written for positions past the new committed length are
    rolled back (poisoned with NaN here, since their content is never read again).
    """
    B, k = st.ctx_len.shape[0], dims.block_k
    kb = block_lengths(dims, B, block_len)
    draft = np.asarray(draft, dtype=np.int64)
    target = np.asarray(target, dtype=np.int64)
    acc = np.zeros(B, np.int64)
    out = np.full((B, k + 1), -1, np.int64)
    for b in range(B):
        n = int(kb[b])
        a = accepted_length(draft[b], target[b], n)
        acc[b] = a
        out[b, :a + 1] = target[b, :a + 1]
        P = int(st.ctx_len[b])
        dead = np.array([slot_of(dims, p) for p in range(P + a + 1, P + n + 1)], dtype=np.int64)
        st.k_ring[:, b][:, :, dead, :] = np.nan
        st.v_ring[:, b][:, :, dead, :] = np.nan
        st.ctx_len[b] = P + a + 1
        st.anchor[b] = target[b, a]
    return {"accept_len": acc, "out_tokens": out}


# ----------------------------------------------------------------------------
# one-token decode (used to pin the block path at k = 1)
# ----------------------------------------------------------------------------

def decode_step(dims, W, st: State) -> np.ndarray:
    """Textbook one-token decode of the anchor at position P: causal attention over
    the sink positions, the last W committed positions and the token itself.
    Returns logits [B, V]."""
    B = st.ctx_len.shape[0]
    Hq, Hkv, dh = dims.n_q_heads, dims.n_kv_heads, dims.head_dim
    logits = np.empty((B, dims.vocab))
    for b in range(B):
        P = int(st.ctx_len[b])
        t = f64(np.asarray(W["embed"])[int(st.anchor[b])])
        for l in range(dims.n_layers):
            a_in = rms_norm(t, W["attn_norm"][l], dims.rms_eps)
            proj = f64(W["w_qkv"][l]) @ a_in
            heads_q = proj[:Hq * dh].reshape(Hq, dh)
            own_k = proj[Hq * dh:(Hq + Hkv) * dh].reshape(Hkv, dh)
            own_v = proj[(Hq + Hkv) * dh:].reshape(Hkv, dh)
            heads_q = rope(heads_q, np.full(Hq, P), dims.rope_theta)
            own_k = rope(own_k, np.full(Hkv, P), dims.rope_theta)
            sink = int(getattr(dims, "sink", 0))
            past = [p for p in range(P) if p < sink or p >= P - dims.window]
            ctx = np.zeros(Hq * dh)
            for hq in range(Hq):
                g = (hq * Hkv) // Hq
                ks = [st.k_ring[l, b, g, slot_of(dims, p)] for p in past] + [own_k[g]]
                vs = [st.v_ring[l, b, g, slot_of(dims, p)] for p in past] + [own_v[g]]
                sc = np.array([heads_q[hq] @ kk for kk in ks]) / np.sqrt(dh)
                wts = np.exp(sc - sc.max())
                wts /= wts.sum()
                ctx[hq * dh:(hq + 1) * dh] = sum(w_ * v_ for w_, v_ in zip(wts, vs))
            t = t + f64(W["w_o"][l]) @ ctx
            m_in = rms_norm(t, W["mlp_norm"][l], dims.rms_eps)
            gu = f64(W["w_gate_up"][l]) @ m_in
            t = t + f64(W["w_down"][l]) @ (silu(gu[:dims.ffn]) * gu[dims.ffn:])
        logits[b] = f64(W["lm_head"]) @ rms_norm(t, W["final_norm"], dims.rms_eps)
    return logits
