"""The pins have teeth: each plausible mistake planted in the oracle (on the CPU)
fails at least one pin.  The real oracle is untouched; every mutant is applied
with ``monkeypatch`` for the duration of one test."""
import numpy as np
import pytest

import oracle.boundary as real
import oracle_pins

_orig_acc64 = real.accumulate_f64
_orig_acc32 = real.accumulate_f32
_orig_norm = real.rms_norm_f64
_orig_round = real.f64_to_bf16


def _norm_eps_outside(x, gamma, wb, eps):
    ms = np.sum(x * x, axis=-1, keepdims=True) / x.shape[-1]
    return x / (np.sqrt(ms) + float(np.float32(eps))) * (real.bf16_to_f64(gamma) + float(np.float32(wb)))


def _norm_h_minus_1(x, gamma, wb, eps):
    ms = np.sum(x * x, axis=-1, keepdims=True) / (x.shape[-1] - 1)
    return x / np.sqrt(ms + float(np.float32(eps))) * (real.bf16_to_f64(gamma) + float(np.float32(wb)))


def _norm_no_bias(x, gamma, wb, eps):
    return _orig_norm(x, gamma, 0.0, eps)


def _norm_eps_on_sum(x, gamma, wb, eps):
    ss = np.sum(x * x, axis=-1, keepdims=True)
    return x / np.sqrt((ss + float(np.float32(eps))) / x.shape[-1]) * (real.bf16_to_f64(gamma) + float(np.float32(wb)))


def _round_via_f32(x):
    return _orig_round(np.asarray(x, np.float64).astype(np.float32).astype(np.float64))


def _round_truncate(x):
    x = np.asarray(x, np.float64).astype(np.float32)
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _wrap_both(fn):
    """Apply the same argument edit to both accumulation tracks."""
    def a64(partials, residual, **kw):
        p, r, kw2 = fn(list(partials), residual, dict(kw))
        return _orig_acc64(p, r, **kw2)

    def a32(partials, residual, **kw):
        p, r, kw2 = fn(list(partials), residual, dict(kw))
        return _orig_acc32(p, r, **kw2)
    return a64, a32


def _drop_shared(p, r, kw):
    kw["shared"] = None
    return p, r, kw


def _shared_twice(p, r, kw):
    if kw.get("shared") is not None and kw.get("gate") is None:
        p = p + [kw["shared"]]
    elif kw.get("shared") is not None:
        kw["gate"] = np.asarray(kw["gate"]) + np.float32(0.7)
    return p, r, kw


def _expert_sign(p, r, kw):
    if kw.get("weights") is not None:
        kw["weights"] = -np.asarray(kw["weights"])
    return p, r, kw


def _weights_reversed(p, r, kw):
    if kw.get("weights") is not None:
        kw["weights"] = np.ascontiguousarray(np.asarray(kw["weights"])[:, ::-1])
    return p, r, kw


def _drop_last_partial(p, r, kw):
    return p[:-1], r, kw


def _drop_residual(p, r, kw):
    return p, np.zeros_like(np.asarray(r)), kw


def _gate_ignored(p, r, kw):
    kw["gate"] = None
    return p, r, kw


def _negative_index_wraps(p, r, kw):
    if kw.get("idx") is not None:
        N = kw["expert_out"].shape[0]
        idx = np.asarray(kw["idx"]).copy()
        idx[idx < 0] += N  # python-style wrap instead of skipping
        kw["idx"] = idx
    return p, r, kw


def _acc32_fused(partials, residual, expert_out=None, idx=None, weights=None, shared=None, gate=None):
    # products kept exact (fused multiply-add) instead of rounded to fp32
    X = real.bf16_to_f64(residual)
    a = np.zeros(X.shape, np.float32)
    for P in partials:
        a = a + real.bf16_to_f64(P).astype(np.float32)
    if idx is not None:
        N = expert_out.shape[0]
        for k in range(idx.shape[1]):
            for t in range(idx.shape[0]):
                j = int(idx[t, k])
                if 0 <= j < N:
                    a[t] = (a[t].astype(np.float64) + float(weights[t, k]) * real.bf16_to_f64(expert_out[j])).astype(np.float32)
    if shared is not None:
        s = real.shared_scale(gate, X.shape[0]).astype(np.float64)
        a = (a.astype(np.float64) + s[:, None] * real.bf16_to_f64(shared)).astype(np.float32)
    return a + X.astype(np.float32)


def _scale_wrong_sign(gate_logits, T):
    if gate_logits is None:
        return np.ones(T, np.float32)
    g = np.asarray(gate_logits, np.float32).astype(np.float64)
    return (1.0 / (1.0 + np.exp(g))).astype(np.float32)


def _split_without_rounding(partials, residual, gamma, weight_bias=0.0, eps=1e-6, **kw):
    out = real.evaluate(partials, residual, gamma, weight_bias, eps, **kw)
    out["sum"] = real.f64_to_bf16(real.accumulate_f64(partials, np.zeros_like(residual), **kw))
    return out


def _evaluate_chunk_routing_slip(partials, residual, gamma, weight_bias=0.0, eps=1e-6,
                                 expert_out=None, idx=None, weights=None, shared=None, gate=None,
                                 chunk_rows=256, keep_unrounded=False):
    """The row-chunk loop with a slicing slip: every chunk takes the routing
    (indices, weights) of the first rows instead of its own."""
    residual = np.asarray(residual)
    T, H = residual.shape
    out = {k: np.empty((T, H), np.uint16) for k in ("normed", "residual", "residual_contract")}
    for r0 in range(0, T, chunk_rows):
        sl = slice(r0, min(T, r0 + chunk_rows))
        n = sl.stop - sl.start
        kw = dict(partials=[np.asarray(P)[sl] for P in partials], residual=residual[sl],
                  expert_out=expert_out, idx=None if idx is None else np.asarray(idx)[:n],
                  weights=None if weights is None else np.asarray(weights)[:n],
                  shared=None if shared is None else np.asarray(shared)[sl],
                  gate=None if gate is None else np.asarray(gate)[sl])
        x = real.accumulate_f64(**kw)
        out["normed"][sl] = real.f64_to_bf16(real.rms_norm_f64(x, gamma, weight_bias, eps))
        out["residual"][sl] = real.f64_to_bf16(x)
        out["residual_contract"][sl] = real.f64_to_bf16(real.accumulate_f32(**kw).astype(np.float64))
    return out


MUTANTS = {
    "chunk_loop_reuses_first_rows_routing": {"evaluate": _evaluate_chunk_routing_slip},
    "split_skips_intermediate_rounding": {"split_evaluate": _split_without_rounding},
    "eps_outside_root": {"rms_norm_f64": _norm_eps_outside},
    "mean_over_H_minus_1": {"rms_norm_f64": _norm_h_minus_1},
    "weight_bias_ignored": {"rms_norm_f64": _norm_no_bias},
    "eps_added_to_sum": {"rms_norm_f64": _norm_eps_on_sum},
    "double_rounding_via_f32": {"f64_to_bf16": _round_via_f32},
    "truncating_round": {"f64_to_bf16": _round_truncate},
    "track_b_fused_products": {"accumulate_f32": _acc32_fused},
    "gate_sign_flipped": {"shared_scale": _scale_wrong_sign},
}
for _name, _fn in {
    "shared_dropped": _drop_shared,
    "shared_added_twice": _shared_twice,
    "expert_sign_flipped": _expert_sign,
    "weights_paired_with_wrong_slot": _weights_reversed,
    "last_partial_dropped": _drop_last_partial,
    "residual_dropped": _drop_residual,
    "gate_ignored": _gate_ignored,
    "negative_index_wraps": _negative_index_wraps,
}.items():
    a64, a32 = _wrap_both(_fn)
    MUTANTS[_name] = {"accumulate_f64": a64, "accumulate_f32": a32}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    for attr, fn in MUTANTS[name].items():
        monkeypatch.setattr(real, attr, fn)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(real)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"mutant {name} passed every pin"
