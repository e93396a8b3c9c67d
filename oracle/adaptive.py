"""Acceptance-driven runtime block size: the plain definition of the controller.

TEST INFRASTRUCTURE ONLY (same rules as dflash_oracle: only the tests, the smoke
check and the bench's CPU baseline use it; the HIP library never does).

The hotdry blog (section on acceptance-rate prediction and dynamic fallback)
describes the mechanism: while the acceptance measured at run time stays below the
scenario's threshold, the system shrinks the block step by step (its example: from
8 to 4) or turns speculative decoding off for a while, and keeps the largest block
where acceptance is high.  Its reference thresholds on the mean accepted length at
block 8: code >= 6.0 keeps the largest block, math >= 5.0 is watched, agent >= 4.0
needs adjustment, open chat < 4.0 should degrade.

This implementation's reading of that description (the pages fix no formula):
  * rungs of the block length: full = k, half = k // 2 (absent when it is 0), off = 0;
  * per sequence an exponential moving average m of the accepted length expressed at
    the full block: after a round that drafted k_b > 0 tokens and accepted a of them,
    tau = 1 + a * (k / k_b) and m <- m + alpha * (tau - m);
  * full: m < theta_down -> one rung down (half; off if there is no half rung);
    half: m < theta_off -> off; m >= theta_up -> full;
    off:  lasts `cooldown` rounds; then half (full if there is no half rung) with
          m = theta_down;
  * the average is kept in float32 with every operation rounded on its own (no fused
    multiply-add), because the rung decisions are integers taken from it and both
    implementations must take them from the same numbers.
Defaults: alpha = 0.25, theta_down = 4.0 (agent), theta_off = 2.0, theta_up = 6.0
(code), cooldown = 16 rounds.  Pinned by tests/test_adaptive_pins.py (closed-form
trajectories of the average, rung sequences, cool-down length); not parity-unpinned.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

f32 = np.float32


@dataclass(frozen=True)
class AdaptParams:
    alpha: float = 0.25
    theta_down: float = 4.0
    theta_off: float = 2.0
    theta_up: float = 6.0
    cooldown: int = 16


def rungs(k: int):
    """(full, half) block lengths; half is None when the ladder has no middle rung."""
    half = k // 2
    return k, (half if 0 < half < k else None)


def ema_update(m, a: int, kb: int, k: int, alpha: float):
    """m + alpha * (tau - m), tau = 1 + a * (k / kb), each operation rounded to float32."""
    scale = f32(k) / f32(kb)
    tau = f32(1.0) + f32(a) * scale
    return f32(f32(m) + f32(f32(alpha) * f32(tau - f32(m))))


def adapt(params: AdaptParams, k: int, block_len, ema, off_left, accept_len):
    """One controller round for every sequence; returns new (block_len, ema, off_left)
    arrays (int64, float32, int64).  accept_len is ignored where block_len is 0."""
    full, half = rungs(k)
    kb = np.array(block_len, dtype=np.int64)
    m = np.array(ema, dtype=np.float32)
    off = np.array(off_left, dtype=np.int64)
    a = np.asarray(accept_len, dtype=np.int64)
    for b in range(kb.shape[0]):
        if kb[b] == 0:
            off[b] -= 1
            if off[b] <= 0:
                kb[b] = half if half is not None else full
                m[b] = f32(params.theta_down)
                off[b] = 0
            continue
        m[b] = ema_update(m[b], int(a[b]), int(kb[b]), k, params.alpha)
        if kb[b] == full:
            if m[b] < f32(params.theta_down):
                if half is not None:
                    kb[b] = half
                else:
                    kb[b], off[b] = 0, params.cooldown
        else:
            if m[b] < f32(params.theta_off):
                kb[b], off[b] = 0, params.cooldown
            elif m[b] >= f32(params.theta_up):
                kb[b] = full
    return kb, m, off
