"""The oracle against its pins (CPU), and each planted oracle mistake against the same pins."""
import pytest

import oracle
import oracle_pins as pins

MUTANTS = {
    1: "0-based layer in lambda_init",
    2: "causal mask drops the diagonal",
    3: "score scale uses the full head width",
    4: "score scale dropped",
    5: "keys of the two maps swapped",
    6: "difference taken with the wrong sign",
    7: "eps added outside the root",
    8: "output scaled by lambda_init instead of 1 - lambda_init",
    9: "mean square over the wrong channel count",
    10: "masked keys kept in the softmax denominator",
}


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    assert oracle._load().oracle_mutant() == 0
    fails = pin()
    assert not fails, f"{pin.__name__}: {fails}"


@pytest.mark.parametrize("mutant", sorted(MUTANTS), ids=lambda k: f"mutant{k}")
def test_planted_mistake_is_caught(mutant):
    oracle.build(mutant)
    assert oracle._load(mutant).oracle_mutant() == mutant
    caught = {p.__name__: p(mutant) for p in pins.ALL_PINS}
    caught = {k: v for k, v in caught.items() if v}
    assert caught, f"mutant {mutant} ({MUTANTS[mutant]}) passes every pin"
