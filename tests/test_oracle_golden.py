"""The oracle reproduces the hand-worked examples (tests/golden)."""

import numpy as np
import pytest

from tests import golden_cases

CASES = golden_cases.load()


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_worked_example(orc, case):
    name, row, k, p, draws, ren_want = case
    for u, tok_want in draws:
        tok, ren, _ = orc.sample_row(row, k, p, u)
        assert tok == tok_want, (name, u)
        np.testing.assert_allclose(ren, np.array(ren_want, np.float32), rtol=2**-23, atol=0)
