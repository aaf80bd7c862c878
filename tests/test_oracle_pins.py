"""The CPU oracle against brute force, a library routine, closed forms and
invariants.  CPU only."""
import pytest

import oracle
from tests import pins
from workloads import WORKLOADS


@pytest.mark.parametrize("check", pins.FAST_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(oracle)


def test_brute_whole_tiny_mha():
    """All of the tiny MHA workload (B=1, H=2, N=M=128, d=64) by brute force."""
    pins.check_brute_workload(oracle, WORKLOADS["tiny_mha_fp16_d64"])


def test_brute_whole_small_decode():
    """All of the small decode workload (B=1, H=8, M=512, d=128) by brute force,
    partials and merged result."""
    pins.check_brute_workload(oracle, WORKLOADS["small_decode_fp16_d128"])
