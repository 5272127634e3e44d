"""Pin the structured-input closed forms (tests/_props.py) to the oracle on
small inputs, so the full-size GPU checks built on them are trustworthy."""
import random

import numpy as np
import pytest

from flexible_mask_attention_amd import workloads as wl
from oracle import ffa_oracle as orc
from tests import _props


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_structured_closed_forms_equal_oracle(seed):
    rng = random.Random(seed)
    Tq, Tk, Hq, Hkv, d = 150, 170, 4, 2, 16
    sl = wl.random_slices(rng, Tq, Tk, 5)
    sl.append((0, 0, 0, 0, 0))
    inp = _props.structured_inputs(Tq, Tk, Hq, Hkv, d, seed)
    st = _props.Structured(inp, sl, Tq, Tk)
    o_ref, l_ref = orc.forward(inp["q"], inp["k"], inp["v"], sl)
    dq_ref, dk_ref, dv_ref = orc.backward(inp["q"], inp["k"], inp["v"], inp["do"], sl)
    for h in range(Hq):
        O, L = st.rows(h)
        np.testing.assert_allclose(O, o_ref[:, h], rtol=1e-10, atol=1e-12)
        assert np.array_equal(np.isneginf(L), np.isneginf(l_ref[h]))
        fin = np.isfinite(l_ref[h])
        np.testing.assert_allclose(L[fin], l_ref[h][fin], rtol=1e-12, atol=1e-12)
    keys = np.array(sorted(rng.sample(range(Tk), 60)))
    for g in range(Hkv):
        dK, dV = st.keys(g, keys)
        np.testing.assert_allclose(dK, dk_ref[keys, g], rtol=1e-9, atol=1e-10)
        np.testing.assert_allclose(dV, dv_ref[keys, g], rtol=1e-10, atol=1e-12)
    assert np.abs(dq_ref).max() < 1e-10


def test_structured_values_exact_in_bf16():
    inp = _props.structured_inputs(10, 300, 2, 2, 32, 3)
    v = inp["v"].double()
    prod = inp["f"].double() * inp["u"].double()
    assert (v == prod).all()          # f_j * u is exact in bf16
    assert (inp["k"] == inp["kappa"]).all()
