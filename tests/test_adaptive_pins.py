"""Pins of the runtime block-size controller (oracle/adaptive.py, CPU only).

The rung decisions are compared against closed forms of the moving average
m_n = tau + (m_0 - tau) (1 - alpha)^n under constant acceptance (evaluated in
float64, independently of the controller's float32 arithmetic; every crossing used
is checked to sit well away from a round boundary), plus the cool-down length and
the ladder without a middle rung.
"""
import math

import numpy as np
import pytest

from oracle import adaptive as ad
from oracle.adaptive import AdaptParams

P = AdaptParams()


def crossing(m0, tau, alpha, thr, below=True):
    """First n >= 1 with m_n < thr (below) or m_n >= thr, m_n in closed form."""
    x = math.log((thr - tau) / (m0 - tau)) / math.log(1 - alpha)
    assert abs(x - round(x)) > 1e-3, "crossing too close to a round boundary for this pin"
    return math.floor(x) + 1


def run(k, kb0, m0, accepts, params=P):
    kb, m, off = np.array([kb0]), np.array([m0], np.float32), np.array([0])
    hist = []
    for a in accepts:
        kb, m, off = ad.adapt(params, k, kb, m, off, [a])
        hist.append((int(kb[0]), float(m[0]), int(off[0])))
    return hist


def first_round(hist, pred):
    return next(i + 1 for i, h in enumerate(hist) if pred(h))


def test_full_block_steps_down_when_the_average_crosses_theta_down():
    k, a = 8, 2                                   # tau = 3 at the full block
    hist = run(k, 8, 6.0, [a] * 12)
    n = crossing(6.0, 1 + a, P.alpha, P.theta_down)
    assert first_round(hist, lambda h: h[0] == 4) == n
    assert all(h[0] == 8 for h in hist[:n - 1])


def test_half_block_normalises_to_the_full_block_and_steps_back_up():
    k = 8
    # at the half rung, accepting every draft means tau = 1 + 4 * (8 / 4) = 9
    hist = run(k, 4, 4.0, [4] * 12)
    n = crossing(4.0, 9.0, P.alpha, P.theta_up, below=False)
    assert first_round(hist, lambda h: h[0] == 8) == n


def test_half_block_turns_speculation_off_and_cooldown_is_exact():
    k = 8
    hist = run(k, 4, 4.0, [0] * 40)
    n = crossing(4.0, 1.0, P.alpha, P.theta_off)
    assert first_round(hist, lambda h: h[0] == 0) == n
    # off for exactly `cooldown` rounds (accept lengths of those rounds are ignored),
    # then the half rung with the average reset to theta_down
    first_off = [h[0] for h in hist[n - 1:n - 1 + P.cooldown + 1]]
    assert first_off == [0] * P.cooldown + [4]
    assert hist[n - 1 + P.cooldown][1] == np.float32(P.theta_down)


def test_off_rounds_ignore_accept_lengths():
    def off_run(acc):
        kb, m, off = np.array([0]), np.array([3.0], np.float32), np.array([6])
        out = []
        for _ in range(5):
            kb, m, off = ad.adapt(P, 8, kb, m, off, [acc])
            out.append((int(kb[0]), float(m[0]), int(off[0])))
        return out
    assert off_run(8) == off_run(0)
    assert [h[0] for h in off_run(8)] == [0] * 5


def test_cooldown_then_reset_value():
    params = AdaptParams(cooldown=3)
    kb, m, off = np.array([0]), np.array([1.0], np.float32), np.array([3])
    seen = []
    for _ in range(3):
        kb, m, off = ad.adapt(params, 8, kb, m, off, [7])
        seen.append((int(kb[0]), float(m[0]), int(off[0])))
    assert seen[0][0] == 0 and seen[1][0] == 0
    assert seen[2] == (4, 4.0, 0)


def test_ladder_without_a_middle_rung():
    assert ad.rungs(1) == (1, None) and ad.rungs(8) == (8, 4) and ad.rungs(3) == (3, 1) and ad.rungs(2) == (2, 1)
    hist = run(1, 1, 6.0, [0] * 20)               # tau = 1: full -> off directly
    n = crossing(6.0, 1.0, P.alpha, P.theta_down)
    assert first_round(hist, lambda h: h[0] == 0) == n
    back = hist[n - 1 + P.cooldown]
    assert back[0] == 1                           # back to the full rung


def test_rungs_stay_on_the_ladder_for_random_trajectories():
    rng = np.random.default_rng(9)
    for k in (1, 2, 3, 8, 10, 16):
        full, half = ad.rungs(k)
        allowed = {0, full} | ({half} if half else set())
        kb = np.full(32, k)
        m = np.full(32, 6.0, np.float32)
        off = np.zeros(32, np.int64)
        for _ in range(200):
            acc = np.array([rng.integers(0, max(int(x), 0) + 1) for x in kb])
            kb, m, off = ad.adapt(P, k, kb, m, off, acc)
            assert set(kb.tolist()) <= allowed
            assert np.all((off >= 0) & (off <= P.cooldown))
            assert np.all((off > 0) == (kb == 0))


def test_average_is_float32_with_unfused_operations():
    # 1 + 3 * (8 / 3): the quotient and the product are rounded separately
    m = ad.ema_update(np.float32(5.0), 3, 3, 8, 0.25)
    q = np.float32(8.0) / np.float32(3.0)
    tau = np.float32(1.0) + np.float32(3.0) * q
    assert m == np.float32(np.float32(5.0) + np.float32(np.float32(0.25) * np.float32(tau - np.float32(5.0))))
    assert isinstance(m, np.float32)
