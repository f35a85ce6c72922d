"""Planted mistakes in the attention-backward oracle must each fail at least one pin.

attention_bwd_oracle.c carries BWD_PLANT_* switches; each build below turns
one on and runs the pins of test_bwd_oracle_pins.py against it.
"""
import numpy as np
import pytest

import oracle
import test_bwd_oracle_pins as pins

MUTANTS = ["NO_D", "NO_SCALE_DK", "DV_USES_DS", "TOP_LEFT"]


def _pin_calls():
    return [
        ("finite_diff", pins.test_matches_finite_differences_of_the_forward, (True, 5, 7)),
        ("torch", pins.test_matches_torch_float64_autograd, (1, 2, 33, 47, 16, True)),
        ("equal_v", pins.test_equal_value_rows_give_no_query_or_key_gradient, ()),
        ("q_zero", pins.test_zero_query_gives_prefix_mean_weights, (True, 6, 9)),
        ("single_key", pins.test_single_key_has_no_softmax_gradient, ()),
        ("no_keys", pins.test_rows_without_keys_contribute_nothing, ()),
    ]


@pytest.mark.parametrize("mutant", MUTANTS)
def test_planted_mistake_is_caught(mutant, tmp_path):
    path = oracle.build(force=True, out=str(tmp_path / f"liboracle_bwd_{mutant}.so"),
                        defines=[f"BWD_PLANT_{mutant}"])
    bad = oracle.load(path)
    saved = oracle._lib
    caught = []
    try:
        oracle._lib = bad
        for name, fn, args in _pin_calls():
            try:
                with np.errstate(all="ignore"):
                    fn(*args)
            except (AssertionError, ValueError, FloatingPointError):
                caught.append(name)
    finally:
        oracle._lib = saved
    assert caught, f"no pin caught planted mistake {mutant}"


def test_unplanted_build_passes_every_pin():
    for name, fn, args in _pin_calls():
        fn(*args)
