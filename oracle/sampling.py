"""Sampled (temperature > 0) drafting and verification: the plain fp64 definition.

TEST INFRASTRUCTURE ONLY (same rules as dflash_oracle: only the tests, the smoke
check and the bench's CPU baseline use it; the HIP library never does).

The method.  The pages name the target's check of a drafted block "rejection
sampling" (aufer article, data-flow section); the zhihu answer lays out the
draft / verify / accept loop (§2) and states that the target's output
distribution is preserved (§6).  Written out for one sequence whose block has
draft rows i = 0..k-1 and target rows i = 0..k:

* the drafter's distribution at row i is q_i = softmax(z_i / T) and the draft x_i
  is a sample of q_i; the target's is p_i = softmax(t_i / T) (row k follows the
  whole block);
* for i = 0, 1, ..: x_i is accepted when u_i * q_i(x_i) <= p_i(x_i), u_i uniform
  on (0, 1); at the first rejection (row a) the emitted token is a sample of the
  residual max(0, p_a - q_a) (normalised); if all k drafts are accepted (a = k) it
  is a sample of p_k;
* the committed length grows by a + 1 and the emitted token becomes the anchor, as
  in greedy verification, which is the T -> 0 limit of this rule.

Random numbers.  Every draw comes from the counter-based generator Philox4x64-10
(Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3",
SC 2011): a block maps a 4-word counter and a 2-word key to 4 words of 64 bits,
read here as eight 32-bit values, low half of word 0 first.  A 32-bit value h
gives the uniform (h + 1/2) 2^-32 on (0, 1) and the Gumbel variate
-log(-log(u)).  Sampling from softmax(s) takes argmax_v (s_v + g_v) (the
Gumbel-max identity); ties go to the smallest index.  The key is (seed, stream);
the counters are:

  stream 1, draft noise of flattened block row m = b*k + i and token v:
      counter (16 * (v >> 5) + (v & 15), m >> 2, step, 0),
      value 2 * (m & 3) + ((v >> 4) & 1)
      (one block serves 4 consecutive rows times the token pair v, v + 16);
  stream 2, acceptance uniform of row i of sequence b: counter (i, b, step, 0), value 0;
  stream 3, noise of the emitted (residual or bonus) draw of sequence b, token v:
      counter (v >> 3, b, step, 0), value v & 7.

Readings where the pages are silent (each is a choice of this implementation):
the drafter and the target share one temperature; the residual draw ranges over
the tokens with p > q; if rounding left no such token, the draw is from p_a.
Every function here is pinned by the CPU tests (numpy's own Philox, the
Gumbel-max law, the losslessness of the whole rule on a tiny model, the T -> 0
limit, closed-form acceptance rates); none is "parity unpinned".
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

# Philox4x64 multipliers and Weyl key increments (the generator's published constants)
PHILOX_M = (0xD2E7470EE14C6C93, 0xCA5A826395121157)
PHILOX_W = (0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B)
_MASK64 = (1 << 64) - 1
_M32 = np.uint64(0xFFFFFFFF)

STREAM_DRAFT = 1
STREAM_ACCEPT = 2
STREAM_EMIT = 3


# ----------------------------------------------------------------------------
# Philox4x64-10
# ----------------------------------------------------------------------------

def philox4x64(ctr: Sequence[int], key: Sequence[int]):
    """One block, Python integers: 10 rounds of two 64x64 -> 128-bit products,
    the key bumped by the Weyl increments between rounds."""
    c = [int(x) & _MASK64 for x in ctr]
    k0, k1 = int(key[0]) & _MASK64, int(key[1]) & _MASK64
    for rnd in range(10):
        p0 = PHILOX_M[0] * c[0]
        p1 = PHILOX_M[1] * c[2]
        c = [(p1 >> 64) ^ c[1] ^ k0, p1 & _MASK64, (p0 >> 64) ^ c[3] ^ k1, p0 & _MASK64]
        if rnd < 9:
            k0 = (k0 + PHILOX_W[0]) & _MASK64
            k1 = (k1 + PHILOX_W[1]) & _MASK64
    return c


def _mulhilo(a: np.ndarray, m: int):
    """(high, low) 64-bit halves of the 128-bit products a * m, uint64 arrays."""
    a_lo, a_hi = a & _M32, a >> np.uint64(32)
    m_lo, m_hi = np.uint64(m & 0xFFFFFFFF), np.uint64(m >> 32)
    ll, lh, hl, hh = a_lo * m_lo, a_lo * m_hi, a_hi * m_lo, a_hi * m_hi
    mid = (ll >> np.uint64(32)) + (lh & _M32) + (hl & _M32)
    lo = (ll & _M32) | ((mid & _M32) << np.uint64(32))
    hi = hh + (lh >> np.uint64(32)) + (hl >> np.uint64(32)) + (mid >> np.uint64(32))
    return hi, lo


def philox4x64_np(c0, c1, c2, c3, key: Sequence[int]) -> np.ndarray:
    """The same block for arrays of counters (broadcast); returns [..., 4] uint64."""
    c = [np.asarray(x, dtype=np.uint64) for x in np.broadcast_arrays(c0, c1, c2, c3)]
    k0, k1 = int(key[0]) & _MASK64, int(key[1]) & _MASK64
    with np.errstate(over="ignore"):
        for rnd in range(10):
            hi0, lo0 = _mulhilo(c[0], PHILOX_M[0])
            hi1, lo1 = _mulhilo(c[2], PHILOX_M[1])
            c = [hi1 ^ c[1] ^ np.uint64(k0), lo1, hi0 ^ c[3] ^ np.uint64(k1), lo0]
            if rnd < 9:
                k0 = (k0 + PHILOX_W[0]) & _MASK64
                k1 = (k1 + PHILOX_W[1]) & _MASK64
    return np.stack(c, axis=-1)


def u32_of(block: np.ndarray, e) -> np.ndarray:
    """32-bit value e (0..7) of blocks [..., 4]: word e // 2, low half when e is even."""
    e = np.asarray(e)
    shape = np.broadcast_shapes(block.shape[:-1], e.shape)
    block = np.broadcast_to(block, shape + (4,))
    e = np.broadcast_to(e, shape)
    w = np.take_along_axis(block, (e // 2)[..., None].astype(np.int64), axis=-1)[..., 0]
    return np.where(e % 2 == 0, w & _M32, w >> np.uint64(32))


def uniform(h) -> np.ndarray:
    return (np.asarray(h, dtype=np.float64) + 0.5) * 2.0 ** -32


def gumbel(h) -> np.ndarray:
    return -np.log(-np.log(uniform(h)))


# ----------------------------------------------------------------------------
# the three draw families
# ----------------------------------------------------------------------------

def draft_noise(seed: int, step: int, m: int, V: int) -> np.ndarray:
    """Gumbel noise [V] of flattened block row m."""
    v = np.arange(V, dtype=np.uint64)
    blk = philox4x64_np(((v >> np.uint64(5)) << np.uint64(4)) | (v & np.uint64(15)),
                        np.uint64(m >> 2), np.uint64(step), np.uint64(0), (seed, STREAM_DRAFT))
    e = 2 * (m & 3) + ((v >> np.uint64(4)) & np.uint64(1)).astype(np.int64)
    return gumbel(u32_of(blk, e))


def accept_uniform(seed: int, step: int, b: int, i: int) -> float:
    blk = philox4x64_np(np.uint64(i), np.uint64(b), np.uint64(step), np.uint64(0), (seed, STREAM_ACCEPT))
    return float(uniform(u32_of(blk, 0)))


def emit_noise(seed: int, step: int, b: int, V: int) -> np.ndarray:
    v = np.arange(V, dtype=np.uint64)
    blk = philox4x64_np(v >> np.uint64(3), np.uint64(b), np.uint64(step), np.uint64(0), (seed, STREAM_EMIT))
    return gumbel(u32_of(blk, (v & np.uint64(7)).astype(np.int64)))


# ----------------------------------------------------------------------------
# sampling
# ----------------------------------------------------------------------------

def log_softmax(z, temperature: float) -> np.ndarray:
    s = np.asarray(z, dtype=np.float64) / temperature
    m = np.max(s, axis=-1, keepdims=True)
    return s - (m + np.log(np.sum(np.exp(s - m), axis=-1, keepdims=True)))


def logsumexp(z, temperature: float) -> np.ndarray:
    s = np.asarray(z, dtype=np.float64) / temperature
    m = np.max(s, axis=-1)
    return m + np.log(np.sum(np.exp(s - m[..., None]), axis=-1))


def gumbel_max(scores, noise):
    """(argmax of scores + noise, gap between the two largest perturbed scores);
    -inf scores never win while a finite one exists; smallest index on ties."""
    v = np.asarray(scores, dtype=np.float64) + np.asarray(noise, dtype=np.float64)
    top = int(np.argmax(v))
    rest = np.delete(v, top)
    gap = float(v[top] - np.max(rest)) if rest.size else np.inf
    return top, gap


def _ids(n: int, seq_ids: Optional[Sequence[int]]) -> np.ndarray:
    return np.arange(n) if seq_ids is None else np.asarray(seq_ids, dtype=np.int64)


def _lengths(n: int, k: int, block_len) -> np.ndarray:
    kb = np.full(n, k, np.int64) if block_len is None else np.asarray(block_len, dtype=np.int64)
    if kb.shape != (n,) or np.any(kb < 0) or np.any(kb > k):
        raise ValueError("block_len must hold one length in [0, k] per sequence")
    return kb


def sample_drafts(draft_logits, temperature: float, seed: int, step: int,
                  seq_ids: Optional[Sequence[int]] = None, block_len=None) -> Dict[str, np.ndarray]:
    """Drafts x[b, i] ~ softmax(z[b, i] / T) by Gumbel-max with stream 1.

    seq_ids: the batch index of each given sequence (the noise of row m = b*k + i
    depends on it); block_len: rows drafted per sequence (default k).  Returns
    draft [n, k] (-1 past the block), gap [n, k] (top-2 gap of the perturbed scores,
    i.e. how far the draw is from a tie; inf past the block) and lse [n, k] =
    log-sum-exp of z / T (NaN past the block)."""
    z = np.asarray(draft_logits, dtype=np.float64)
    n, k, V = z.shape
    ids = _ids(n, seq_ids)
    kb = _lengths(n, k, block_len)
    x = np.full((n, k), -1, np.int64)
    gap = np.full((n, k), np.inf)
    lse = np.full((n, k), np.nan)
    for j in range(n):
        for i in range(int(kb[j])):
            x[j, i], gap[j, i] = gumbel_max(z[j, i] / temperature,
                                            draft_noise(seed, step, int(ids[j]) * k + i, V))
            lse[j, i] = logsumexp(z[j, i], temperature)
    return {"draft": x, "gap": gap, "lse": lse}


def accept_score(lp_x: float, lq_x: float, u: float) -> float:
    """log p(x) - log q(x) - log u: the draft is accepted iff this is >= 0
    (u * q(x) <= p(x))."""
    return lp_x - lq_x - np.log(u)


def residual_scores(lp_row, lq_row) -> np.ndarray:
    """log max(0, p - q) per token (-inf where p <= q); when no token has p > q
    (possible only through rounding) the draw falls back to p itself."""
    r = np.exp(lp_row) - np.exp(lq_row)
    if not np.any(r > 0):
        return np.asarray(lp_row, dtype=np.float64)
    s = np.full(r.shape, -np.inf)
    s[r > 0] = np.log(r[r > 0])
    return s


def verify_sampled(draft, draft_logits, target_logits, temperature: float, seed: int, step: int,
                   seq_ids: Optional[Sequence[int]] = None, block_len=None) -> Dict[str, np.ndarray]:
    """Rejection-sampling verification of each sequence's block (of block_len[b]
    rows, default k: rows past it are not tested and the bonus row is k_b).

    Returns accept_len [n], emitted [n] (the residual or bonus token), out_tokens
    [n, k+1] (the accepted drafts, the emitted token, then -1), accept_margin [n]
    (the smallest |accept_score| over the acceptance tests made: how far each
    decision was from its threshold), emit_gap [n] (top-2 gap of the emitted
    draw's perturbed scores) and emit_slack [n] (for a residual draw, the largest
    q / (p - q) of those two tokens: how strongly an error in log q moves their
    scores; 0 for a draw from p)."""
    x = np.asarray(draft, dtype=np.int64)
    with np.errstate(invalid="ignore"):               # rows past a block may be NaN
        lq = log_softmax(draft_logits, temperature)   # [n, k, V]
        lp = log_softmax(target_logits, temperature)  # [n, k+1, V]
    n, k, V = lq.shape
    ids = _ids(n, seq_ids)
    kb = _lengths(n, k, block_len)
    acc = np.zeros(n, np.int64)
    emitted = np.zeros(n, np.int64)
    out = np.full((n, k + 1), -1, np.int64)
    margin = np.full(n, np.inf)
    egap = np.zeros(n)
    slack = np.zeros(n)
    for j in range(n):
        b = int(ids[j])
        nb = int(kb[j])
        a = 0
        while a < nb:
            d = accept_score(lp[j, a, x[j, a]], lq[j, a, x[j, a]], accept_uniform(seed, step, b, a))
            margin[j] = min(margin[j], abs(d))
            if d < 0:
                break
            a += 1
        s = residual_scores(lp[j, a], lq[j, a]) if a < nb else lp[j, nb]
        noise = emit_noise(seed, step, b, V)
        y, egap[j] = gumbel_max(s, noise)
        if a < nb and np.any(np.exp(lp[j, a]) > np.exp(lq[j, a])):
            pert = s + noise
            pert[y] = -np.inf
            for v in (y, int(np.argmax(pert))):
                pv, qv = np.exp(lp[j, a, v]), np.exp(lq[j, a, v])
                if pv > qv:
                    slack[j] = max(slack[j], qv / (pv - qv))
        acc[j], emitted[j] = a, y
        out[j, :a] = x[j, :a]
        out[j, a] = y
    return {"accept_len": acc, "emitted": emitted, "out_tokens": out,
            "accept_margin": margin, "emit_gap": egap, "emit_slack": slack}


def commit_sampled(dims, st, result, block_len=None) -> None:
    """Advance the decode state exactly as greedy verification does: P += a + 1,
    anchor = emitted token; rows past the new length (up to P + k_b) are rolled
    back (NaN here)."""
    from oracle import dflash_oracle as orc
    kb = _lengths(st.ctx_len.shape[0], dims.block_k, block_len)
    for j in range(st.ctx_len.shape[0]):
        a = int(result["accept_len"][j])
        P = int(st.ctx_len[j])
        dead = np.array([orc.slot_of(dims, p) for p in range(P + a + 1, P + int(kb[j]) + 1)], dtype=np.int64)
        st.k_ring[:, j][:, :, dead, :] = np.nan
        st.v_ring[:, j][:, :, dead, :] = np.nan
        st.ctx_len[j] = P + a + 1
        st.anchor[j] = int(result["emitted"][j])
