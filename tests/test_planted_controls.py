"""Planted controls: each mutant of a NumPy re-implementation carries one
plausible mistake (an off-by-one causal bound, a dropped local block, a broken
head map, a missing softmax scale, mean instead of max pooling, ties to the
higher index, the shared-index-key misuse, local block counted outside top_k).
Every mutant must turn at least one pin red; the unmutated implementation must
pass them all, which shows the pins accept a correct second implementation."""
import pytest

import pins
from oracle_mutants import MUTATIONS, Impl


def test_unmutated_passes_every_pin():
    impl = Impl(None)
    for check in pins.ALL_CHECKS:
        check(impl)


@pytest.mark.parametrize("mutation", MUTATIONS)
def test_mutant_goes_red(mutation):
    impl = Impl(mutation)
    failed = []
    for check in pins.ALL_CHECKS:
        try:
            check(impl)
        except AssertionError:
            failed.append(check.__name__)
    assert failed, f"no pin caught the planted mistake {mutation!r}"
