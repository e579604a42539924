"""The CPU oracle against its pins (brute force, library SDPA, closed forms,
invariances, printed facts).  See ``oracle_checks.py`` for what each pin is."""
import pytest

import oracle
import oracle_checks


@pytest.fixture(scope="module")
def lib():
    return oracle.load_library(oracle.build())


@pytest.mark.parametrize("check", oracle_checks.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check, lib):
    check(lib)


def test_bad_block_id_is_rejected(lib):
    c = oracle_checks.Case(3, B=2, ctx=[5, 9])
    c.tables[1, 0] = c.num_blocks          # outside the pool
    with pytest.raises(ValueError):
        c.decode(lib)


def test_context_longer_than_table_is_rejected(lib):
    c = oracle_checks.Case(4, B=2, ctx=[5, 9])
    c.ctx[0] = c.max_blocks * c.bs + 1
    with pytest.raises(ValueError):
        c.decode(lib)


def test_append_slot_outside_pool_is_rejected(lib):
    k, v, slots, kc, vc, _ = oracle_checks._append_case(5)
    slots[0] = kc.shape[0] * kc.shape[2]
    with pytest.raises(ValueError):
        oracle.append(k, v, slots, kc, vc, lib=lib)
