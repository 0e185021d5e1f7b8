"""Host-side checks of the Python binding that run before any device work (CPU)."""
import os

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "reduce_moe_finalize_amd", "libfused_boundary.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")


def _bf16(*shape):
    return torch.zeros(*shape, dtype=torch.bfloat16)


@pytest.mark.parametrize("residual", [None, "not a tensor"])
def test_missing_residual_raises_before_any_launch(residual):
    """A residual is required (PR #37104, Changes: fail loudly without one):
    both entry points raise ValueError before touching a device."""
    import reduce_moe_finalize_amd as fb

    T, H = 4, 64
    with pytest.raises(ValueError, match="residual"):
        fb.fused_reduce_rmsnorm([_bf16(T, H)], residual, _bf16(H))
    with pytest.raises(ValueError, match="residual"):
        fb.fused_moe_finalize_rmsnorm([_bf16(T, H)], _bf16(T * 2, H),
                                      torch.zeros(T, 2, dtype=torch.int32),
                                      torch.zeros(T, 2, dtype=torch.float32), residual, _bf16(H))


def test_host_tensors_are_refused():
    """There is no CPU path: host tensors are rejected, not computed."""
    import reduce_moe_finalize_amd as fb

    with pytest.raises(ValueError, match="no CPU path"):
        fb.fused_reduce_rmsnorm([_bf16(2, 64)], _bf16(2, 64), _bf16(64))


def test_partial_count_is_checked():
    import reduce_moe_finalize_amd as fb

    with pytest.raises(ValueError):
        fb.fused_reduce_rmsnorm([], _bf16(2, 64), _bf16(64))
    with pytest.raises(ValueError):
        fb.fused_reduce_rmsnorm([_bf16(2, 64)] * 17, _bf16(2, 64), _bf16(64))


def test_bandwidth_probe_refuses_host_tensors_and_empty_calls():
    import reduce_moe_finalize_amd as fb

    with pytest.raises(ValueError, match="GPU"):
        fb.bandwidth_probe([_bf16(2, 64)])
    with pytest.raises(ValueError, match="nothing"):
        fb.bandwidth_probe([])
