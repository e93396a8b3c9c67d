"""Plant plausible mistakes into the sampled-verification oracle (CPU only) and
check that its pins reject every one: the T -> 0 limit, the closed-form
acceptance rate and residual law, and losslessness on the tiny model."""
import numpy as np
import pytest

from oracle import sampling as sp
from tests import test_sampling_pins as pins

_accept, _resid, _gumbel, _lsm, _u32 = sp.accept_score, sp.residual_scores, sp.gumbel, sp.log_softmax, sp.u32_of


def battery() -> bool:
    try:
        return (pins.greedy_limit_ok() and min(pins.gumbel_law_pvalues(3000)) > pins.P_MIN
                and pins.acceptance_checks(n=2500)
                and pins.lossless_pvalue(2500) > pins.P_MIN)
    except (ValueError, IndexError, FloatingPointError):
        return False


def _accept_inverted(lp_x, lq_x, u):
    return _accept(lq_x, lp_x, u)


def _accept_no_draft(lp_x, lq_x, u):
    return lp_x - np.log(u)


def _resid_swapped(lp_row, lq_row):
    return _resid(lq_row, lp_row)


def _resid_target_only(lp_row, lq_row):
    return np.asarray(lp_row, dtype=np.float64)


def _gumbel_negated(h):
    return -_gumbel(h)


def _lsm_no_temperature(z, temperature):
    return _lsm(z, 1.0)


MUTATIONS = {
    "accept_ratio_inverted": ("accept_score", _accept_inverted),
    "accept_ignores_draft_probability": ("accept_score", _accept_no_draft),
    "residual_q_minus_p": ("residual_scores", _resid_swapped),
    "residual_is_target": ("residual_scores", _resid_target_only),
    "gumbel_sign_flipped": ("gumbel", _gumbel_negated),
    "temperature_dropped": ("log_softmax", _lsm_no_temperature),
}


def test_battery_passes_unmutated():
    assert battery()


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(sp, attr, fn)
    assert not battery(), f"mutation {name} slipped through the pins"


def test_half_order_mutation_is_caught(monkeypatch):
    def swapped(block, e):
        return _u32(block, np.asarray(e) ^ 1)
    monkeypatch.setattr(sp, "u32_of", swapped)
    with pytest.raises(AssertionError):
        pins.test_u32_order_matches_numpy_32bit_stream()
