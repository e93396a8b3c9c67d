"""Scalar brute-force twin of the DFlash draft step, for tiny shapes only.

TEST INFRASTRUCTURE ONLY (same rule as dflash_oracle: tests, smoke and the CPU
baseline may use it; the product path never does).

It pins dflash_oracle by computing the same quantities a different way:
  * pure Python floats and explicit loops, no numpy arithmetic;
  * no ring buffer: the context keys of a block are rebuilt from the committed
    history (position -> target taps), so ring indexing, tentative writes and
    rollback in the oracle are checked against "only committed rows exist";
  * rotary embedding as multiplication of the complex number x_i + j x_{i+dh/2}
    by exp(j * pos * theta^(-2i/dh)) (the RoFormer formulation);
  * an explicit (window + k) x (window + k) visibility matrix, with a switch to
    make the block causal, so bidirectionality inside the block can be tested;
  * the kv head of query head h as floor(h * Hkv / Hq).
Shapes must stay tiny (hidden <= 32, vocab <= 64): it is O(everything) in Python.
"""
from __future__ import annotations

import cmath
import math
from typing import Dict, List, Sequence


def _rows(m) -> List[List[float]]:
    return [[float(v) for v in row] for row in m]


def _vec(v) -> List[float]:
    return [float(x) for x in v]


def matvec(w_rows: List[List[float]], x: List[float]) -> List[float]:
    """out[o] = sum_i W[o][i] * x[i] (nn.Linear, no bias)."""
    return [sum(w * xi for w, xi in zip(row, x)) for row in w_rows]


def rmsnorm(x: List[float], g: List[float], eps: float) -> List[float]:
    ms = sum(v * v for v in x) / len(x)
    r = 1.0 / math.sqrt(ms + eps)
    return [v * r * gi for v, gi in zip(x, g)]


def rotate(vec: List[float], pos: int, theta: float) -> List[float]:
    dh = len(vec)
    half = dh // 2
    out = [0.0] * dh
    for i in range(half):
        z = complex(vec[i], vec[i + half]) * cmath.exp(1j * pos * theta ** (-2.0 * i / dh))
        out[i], out[i + half] = z.real, z.imag
    return out


def swish(v: float) -> float:
    return v / (1.0 + math.exp(-v))


def fused_feature(dims, W, taps_pos) -> List[float]:
    """Concatenate the n_taps hidden states of one position, project, RMSNorm."""
    x: List[float] = []
    for j in range(dims.n_taps):
        x.extend(_vec(taps_pos[j]))
    return rmsnorm(matvec(_rows(W["fuse_w"]), x), _vec(W["fuse_norm"]), dims.rms_eps)


def block_logits(dims, W, history: Dict[int, Sequence], P: int, anchor: int,
                 causal_block: bool = False) -> List[List[float]]:
    """Logits [k][V] of the block at position P whose committed context is history.

    history maps every committed position p < P to its taps [n_taps][tap_dim];
    the block sees the last W of them and, with an attention sink of s, also
    positions 0..s-1.
    """
    k, D = dims.block_k, dims.hidden
    Hq, Hkv, dh, F = dims.n_q_heads, dims.n_kv_heads, dims.head_dim, dims.ffn
    eps, th = dims.rms_eps, dims.rope_theta
    sink = int(getattr(dims, "sink", 0))
    ctx_pos = [p for p in range(P) if p < sink or P - p <= dims.window]
    n_ctx = len(ctx_pos)
    feats = {p: fused_feature(dims, W, history[p]) for p in ctx_pos}

    # explicit visibility: block query i sees every context key and every block key
    n = n_ctx + k
    visible = [[True] * n for _ in range(k)]
    if causal_block:
        for i in range(k):
            for j in range(k):
                visible[i][n_ctx + j] = j <= i

    hs = [_vec(W["embed"][anchor])] + [_vec(W["mask_embed"]) for _ in range(k - 1)]
    q0 = Hq * dh
    k0 = q0 + Hkv * dh
    for l in range(dims.n_layers):
        wqkv = _rows(W["w_qkv"][l])
        w_q, w_k, w_v = wqkv[:q0], wqkv[q0:k0], wqkv[k0:]
        # context keys/values of this layer, rebuilt from the committed features
        ck, cv = [], []
        for p in ctx_pos:
            kk = matvec(w_k, feats[p])
            vv = matvec(w_v, feats[p])
            ck.append([rotate(kk[g * dh:(g + 1) * dh], p, th) for g in range(Hkv)])
            cv.append([vv[g * dh:(g + 1) * dh] for g in range(Hkv)])
        bq, bk, bv = [], [], []
        for i in range(k):
            x = rmsnorm(hs[i], _vec(W["attn_norm"][l]), eps)
            qq, kk, vv = matvec(w_q, x), matvec(w_k, x), matvec(w_v, x)
            bq.append([rotate(qq[h * dh:(h + 1) * dh], P + i, th) for h in range(Hq)])
            bk.append([rotate(kk[g * dh:(g + 1) * dh], P + i, th) for g in range(Hkv)])
            bv.append([vv[g * dh:(g + 1) * dh] for g in range(Hkv)])
        keys = ck + bk
        vals = cv + bv
        w_o = _rows(W["w_o"][l])
        new_hs = []
        for i in range(k):
            att: List[float] = []
            for h in range(Hq):
                g = (h * Hkv) // Hq
                sc = [sum(a * b for a, b in zip(bq[i][h], keys[j][g])) / math.sqrt(dh)
                      if visible[i][j] else -math.inf for j in range(n)]
                mx = max(sc)
                ex = [math.exp(s - mx) if s != -math.inf else 0.0 for s in sc]
                tot = sum(ex)
                o = [0.0] * dh
                for j in range(n):
                    if ex[j]:
                        wgt = ex[j] / tot
                        for t in range(dh):
                            o[t] += wgt * vals[j][g][t]
                att.extend(o)
            hi = [a + b for a, b in zip(hs[i], matvec(w_o, att))]
            y = rmsnorm(hi, _vec(W["mlp_norm"][l]), eps)
            gu = matvec(_rows(W["w_gate_up"][l]), y)
            act = [swish(gu[j]) * gu[F + j] for j in range(F)]
            hi = [a + b for a, b in zip(hi, matvec(_rows(W["w_down"][l]), act))]
            new_hs.append(hi)
        hs = new_hs
    lm = _rows(W["lm_head"])
    return [matvec(lm, rmsnorm(hs[i], _vec(W["final_norm"]), eps)) for i in range(k)]


def first_mismatch(draft: Sequence[int], target: Sequence[int], k: int) -> int:
    """Accepted length as the index of the first disagreeing draft (k if none)."""
    return next((i for i in range(k) if int(draft[i]) != int(target[i])), k)
