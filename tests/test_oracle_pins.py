"""The CPU oracle against values fixed by the pages and by mathematics (no GPU)."""
import pytest

import oracle
from oracle_checks import CHECKS


@pytest.fixture(scope="module")
def lib():
    oracle.build(force=False)
    return oracle._load()


@pytest.mark.parametrize("check", CHECKS, ids=[c.__name__ for c in CHECKS])
def test_oracle(lib, check):
    check(lib)
