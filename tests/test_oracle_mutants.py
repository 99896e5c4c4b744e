"""Plausible mistakes planted in the oracle (on the CPU) must fail a pin.

Each mutant is oracle.c compiled with -DORACLE_MUTANT=n:
  1 sign of the correction flipped        2 covariance transposed
  3 uncentred second moment               4 n/(n-1) factor
  5 probe scaled by the softmax scale     6 scale dropped from logits
  7 uniform weights in the covariance     8 causal diagonal excluded
 10 query used in place of the probe
Backward (oracle_bwd_f64):
 11 b r_j term dropped from dL/dp        12 sign of dL/dr flipped
 13 softmax scale dropped from dk        14 value weights (1 + r_j - rbar)
 15 rbar b dropped from sum_l p dL/dp     16 values used in place of keys in dq
Exact local-linear probe (oracle_lla_probe_f64):
 17 ridge term dropped                    18 right-hand side q - kbar
 19 uncentred key covariance
"""

import tempfile

import pytest

import oracle
import oracle_pins

MUTANTS = [1, 2, 3, 4, 5, 6, 7, 8, 10, 11, 12, 13, 14, 15, 16, 17, 18, 19]


@pytest.fixture(scope="module")
def mutant_dir():
    with tempfile.TemporaryDirectory(prefix="oracle_mut_") as d:
        yield d


@pytest.mark.parametrize("mutant", MUTANTS)
def test_mutant_is_caught(mutant, mutant_dir):
    orc = oracle.Oracle(oracle.load_mutant(mutant, mutant_dir))
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"mutant {mutant} passed every pin"
