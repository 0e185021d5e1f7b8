"""Property-based pin of the oracle (CPU only): on random tiny shapes drawn by
hypothesis, both tracks of the oracle equal the 50-digit decimal brute force
bit for bit (the same fact as the fixed-shape brute-force pin, over many more
shapes, seeds, skipped-slot patterns and weight biases)."""
import numpy as np
import pytest

hypothesis = pytest.importorskip("hypothesis")
from hypothesis import given, settings  # noqa: E402
from hypothesis import strategies as st  # noqa: E402

import oracle.boundary as ob  # noqa: E402
from brute_decimal import brute_case  # noqa: E402
from oracle_pins import _as_lists  # noqa: E402
from workloads import make_case  # noqa: E402


@st.composite
def tiny_cases(draw):
    T = draw(st.integers(1, 3))
    H = 8 * draw(st.integers(1, 3))
    K = draw(st.integers(0, 3))
    R = draw(st.integers(1 if K == 0 else 0, 3))
    shared = K > 0 and draw(st.booleans())
    gate = shared and draw(st.booleans())
    wb = draw(st.sampled_from([0.0, 0.5, 1.0]))
    seed = draw(st.integers(0, 10**6))
    c = make_case(T, H, R, seed=seed, K=K, num_experts=max(K, 4), shared=shared, gate=gate,
                  weight_bias=wb, gamma_dist="normal01" if wb else "uniform")
    if K:
        c.idx = c.idx.copy()
        n = c.expert_out.shape[0]
        for _ in range(draw(st.integers(0, 2))):
            t = draw(st.integers(0, T - 1))
            k = draw(st.integers(0, K - 1))
            c.idx[t, k] = draw(st.sampled_from([-1, n, n + 7, -(2**31)]))
    return c


@settings(max_examples=200, deadline=None, derandomize=True)
@given(tiny_cases())
def test_oracle_equals_decimal_brute_force(c):
    out = ob.evaluate(c.partials, c.residual, c.gamma, c.weight_bias, c.eps,
                      expert_out=c.expert_out, idx=c.idx, weights=c.weights,
                      shared=c.shared, gate=c.gate)
    bn, br, bc = brute_case([_as_lists(p) for p in c.partials], _as_lists(c.residual),
                            _as_lists(c.gamma), c.weight_bias, c.eps,
                            expert_out=_as_lists(c.expert_out), idx=_as_lists(c.idx),
                            weights=_as_lists(c.weights), shared=_as_lists(c.shared),
                            gate=_as_lists(c.gate))
    for name, got, want in (("normed", out["normed"], bn), ("residual", out["residual"], br),
                            ("residual_contract", out["residual_contract"], bc)):
        assert np.array_equal(got, np.array(want, dtype=np.uint16)), name
