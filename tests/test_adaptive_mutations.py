"""Plant plausible mistakes into the block-size controller and the ragged block
handling of the oracle (CPU only) and check that their pins reject each one."""
import numpy as np
import pytest

from oracle import adaptive as ad
from oracle import dflash_oracle as orc
from tests import test_adaptive_pins as apins
from tests import test_ragged_pins as rpins

_ema, _adapt, _lengths = ad.ema_update, ad.adapt, orc.block_lengths


def battery() -> bool:
    tests = [apins.test_full_block_steps_down_when_the_average_crosses_theta_down,
             apins.test_half_block_normalises_to_the_full_block_and_steps_back_up,
             apins.test_half_block_turns_speculation_off_and_cooldown_is_exact,
             apins.test_cooldown_then_reset_value,
             apins.test_ladder_without_a_middle_rung,
             apins.test_average_is_float32_with_unfused_operations,
             lambda: rpins.test_ragged_rows_equal_a_block_of_that_length([2, 3]),
             lambda: rpins.test_ragged_verify_every_pattern(3)]
    try:
        for t in tests:
            t()
        return True
    except (AssertionError, ValueError, IndexError, StopIteration):
        return False


def _ema_unnormalised(m, a, kb, k, alpha):
    return _ema(m, a, kb, kb, alpha)


def _ema_weight_swapped(m, a, kb, k, alpha):
    return _ema(m, a, kb, k, 1.0 - alpha)


def _ema_fused(m, a, kb, k, alpha):
    tau = 1.0 + a * (k / kb)
    return np.float32(np.float64(m) + alpha * (tau - np.float64(m)) + 1e-6)


def _adapt_long_cooldown(params, k, block_len, ema, off_left, accept_len):
    kb, m, off = _adapt(params, k, block_len, ema, off_left, accept_len)
    starting = (np.asarray(block_len) > 0) & (kb == 0)
    off = np.where(starting, off + 1, off)
    return kb, m, off


def _adapt_no_reset(params, k, block_len, ema, off_left, accept_len):
    kb0 = np.asarray(block_len)
    kb, m, off = _adapt(params, k, block_len, ema, off_left, accept_len)
    back = (kb0 == 0) & (kb > 0)
    return kb, np.where(back, np.asarray(ema, np.float32), m), off


def _lengths_ignored(dims, batch, block_len=None):
    return _lengths(dims, batch, None)


MUTATIONS = {
    "tau_not_normalised": (ad, "ema_update", _ema_unnormalised),
    "ema_weight_swapped": (ad, "ema_update", _ema_weight_swapped),
    "ema_higher_precision": (ad, "ema_update", _ema_fused),
    "cooldown_one_round_long": (ad, "adapt", _adapt_long_cooldown),
    "no_reset_after_cooldown": (ad, "adapt", _adapt_no_reset),
    "block_length_ignored": (orc, "block_lengths", _lengths_ignored),
}


def test_battery_passes_unmutated():
    assert battery()


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    mod, attr, fn = MUTATIONS[name]
    monkeypatch.setattr(mod, attr, fn)
    assert not battery(), f"mutation {name} slipped through the pins"
