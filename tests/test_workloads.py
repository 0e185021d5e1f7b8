"""Sanity of the seeded input generators (CPU only)."""
import numpy as np
import pytest

from workloads import CONFIGS, bf16_bits_to_f32, case_for_config, make_case


@pytest.mark.parametrize("T,K,E", [(16, 8, 256), (7, 10, 512), (1, 8, 256), (33, 3, 8)])
def test_routing_invariants(T, K, E):
    c = make_case(T, 64, 2, K=K, num_experts=E, shared=True, seed=3)
    # weights: positive, sum to one per token (fp32 rounding)
    assert c.weights.dtype == np.float32 and c.weights.shape == (T, K)
    assert np.all(c.weights > 0)
    assert np.allclose(c.weights.astype(np.float64).sum(axis=1), 1.0, atol=1e-6)
    # descending (top-k order), distinct expert ids per token
    assert np.all(np.diff(c.weights, axis=1) <= 0)
    ids = c.meta["expert_ids"]
    assert all(len(set(r)) == K for r in ids.tolist())
    assert ids.min() >= 0 and ids.max() < E
    # idx is a permutation of 0..T*K-1, grouped by expert id
    assert np.array_equal(np.sort(c.idx.reshape(-1)), np.arange(T * K))
    e_of_row = np.empty(T * K, np.int64)
    e_of_row[c.idx.reshape(-1)] = ids.reshape(-1)
    assert np.all(np.diff(e_of_row) >= 0), "expanded rows not grouped by expert"
    assert c.expert_out.shape == (T * K, 64)


def test_seeded_and_distributions():
    a = case_for_config("reduce_r2_t1", 1)
    b = case_for_config("reduce_r2_t1", 1)
    assert np.array_equal(a.partials[0], b.partials[0]) and np.array_equal(a.gamma, b.gamma)
    c = make_case(64, 7168, 2, seed=0)
    p = bf16_bits_to_f32(c.partials[0]).astype(np.float64)
    assert abs(p.std() - 0.5) < 0.01 and abs(p.mean()) < 0.01
    g = bf16_bits_to_f32(c.gamma)
    assert g.min() >= 0.5 and g.max() <= 1.5
    gated = case_for_config("gated_h8192_top10", 4)
    g = bf16_bits_to_f32(gated.gamma).astype(np.float64)
    assert abs(g.std() - 0.1) < 0.01 and gated.weight_bias == 1.0 and gated.gate is not None
    assert gated.K == 10 and gated.num_experts == 512


def test_configs_cover_pages_shapes():
    assert CONFIGS["reduce_r2_t1"]["H"] == 7168 and CONFIGS["glm_h6144_top8"]["H"] == 6144 and CONFIGS["gated_h8192_top10"]["H"] == 8192
    assert CONFIGS["headline"]["T"][-1] == 8192
