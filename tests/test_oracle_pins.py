"""The oracle against its pins (CPU only).  See tests/oracle_pins.py for what each pins."""
import pytest

import oracle
from tests import oracle_pins as P

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def test_slot_formula_page_example():
    P.check_slot_formula_page_example()


def test_worked_batch_layout():
    P.check_worked_batch_layout()


@pytest.mark.parametrize("check", P.ALL_CHECKS, ids=lambda f: f.__name__[len("check_"):])
def test_oracle_pin(check):
    check(oracle)


def test_chunking_invariance():
    P.check_chunking_invariance(oracle, long_prompt=True)
