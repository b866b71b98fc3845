"""Pin of the oracle's embedding step against the real value of the table
entry (BitExact LLM blog, "Three execution paths": the embedding enters the
integer residual by one rounding to its fixed-point grid).

A table entry E with row mantissa m_v stands for the real number
E * m_v * 2^-w_k (the dyadic weight scale of the pages' DetLLM blog,
"DetLLM"). The residual stream holds integers in units of 2^-f_res, so the
embedded value must be that real number to within half a unit, with exact
halves rounded up (the one rounding rule). Exact rationals, no float."""
from fractions import Fraction

import numpy as np
import pytest

import detint_synth as S
import oracle as O


@pytest.mark.parametrize("name", ["tiny", "tiny_wide"])
def test_embedding_is_the_real_value_on_the_residual_grid(name):
    m = S.make_model(name, seed=3)
    sh = m.shape
    om = O.OracleModel(m, slots=1)
    ids = np.array([0, 1, 7, sh.vocab - 1, 500, 500], np.int32)
    h = om.embed(ids)
    unit = Fraction(1, 2 ** sh.f_res)
    for r, t in enumerate(ids):
        for i in range(0, sh.hidden, 7):
            real = Fraction(int(m.emb[t, i]) * int(m.emb_m[t]), 2 ** sh.w_k)
            got = h[r, i] * unit
            err = got - real
            assert -unit / 2 < err <= unit / 2, (name, int(t), i)
    # equal ids give equal rows; both the 8-bit and 16-bit tables are used
    assert np.array_equal(h[4], h[5])
    assert m.emb.dtype == (np.int16 if sh.wide else np.int8)


def test_embedding_halves_round_up_and_scale_by_the_mantissa():
    """Hand-built one-row tables where the real values sit exactly on half
    units and on whole units of the residual grid."""
    m = S.make_model("tiny", seed=4)
    sh = m.shape
    shift = sh.w_k - sh.f_res
    m.emb = m.emb.copy()
    m.emb_m = m.emb_m.copy()
    # row 0: mantissa 2^shift: the real value is E exactly (E units of 2^-f_res)
    m.emb_m[0] = 1 << 14
    m.emb[0, :4] = [1, -1, 127, -127]
    # row 1: mantissa 3 * 2^13, so E * m_v / 2^shift = 1.5 E
    m.emb_m[1] = 3 << 13
    m.emb[1, :4] = [1, -1, 3, -3]
    om = O.OracleModel(m, slots=1)
    h = om.embed(np.array([0, 1], np.int32))
    scale0 = Fraction(1 << 14, 2 ** shift)
    assert list(h[0, :4]) == [int(e * scale0) for e in (1, -1, 127, -127)]
    # with shift = 14 the real values are 1.5, -1.5, 4.5 and -4.5 units:
    # exact halves, which the rule rounds up (towards +infinity)
    assert shift == 14
    assert list(h[1, :4]) == [2, -1, 5, -4]
