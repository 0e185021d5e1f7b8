"""Pins for the CPU oracle: checks against facts fixed outside the oracle itself.

Each ``pin_*`` function takes the oracle module (``oracle.boundary`` or a copy of
it with a planted mistake) and raises ``AssertionError`` when the oracle
disagrees with the fact it checks.  ``test_oracle_pins.py`` runs them on the real
oracle; ``test_oracle_mutants.py`` shows that every planted mistake fails at
least one of them.

What pins what:
  * bf16 rounding: hand-derived tie, double-rounding, subnormal and overflow
    cases, and torch's float32 -> bfloat16 conversion;
  * the formula: constant rows normalise to gamma, the eps pin, the exact
    scale identity, the zero row, torch's float64 ``rms_norm`` for R=1 with a
    zero residual, the gate at logit 0, hand cases in ``tests/golden``;
  * the whole call, both tracks: a 50-digit decimal brute force on tiny shapes;
  * the finalize bookkeeping: permutation of expert rows, skipped slots,
    K=1/w=1 as an extra partial, shared expert added once.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

from brute_decimal import brute_case, brute_split
from workloads import bf16_bits_to_f32 as bf16_f32
from workloads import f32_to_bf16_bits, make_case

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits(v):
    return f32_to_bf16_bits(np.asarray(v, dtype=np.float32))


def _const(T, H, v):
    return np.full((T, H), _bits(v), dtype=np.uint16)


# ---------------------------------------------------------------- bf16 rounding
def pin_bf16_hand_cases(ob):
    cases = [
        (1.0, 0x3F80),
        (1.0 + 2.0**-8, 0x3F80),  # tie -> even (mantissa 0)
        (1.0 + 3 * 2.0**-8, 0x3F82),  # tie -> even (mantissa 2)
        (1.0 + 2.0**-8 + 2.0**-30, 0x3F81),  # above the tie: direct rounding goes up
        (-(1.0 + 2.0**-8 + 2.0**-30), 0xBF81),
        (-0.0, 0x8000),
        (0.0, 0x0000),
        (2.0**-133, 0x0001),  # smallest subnormal
        (2.0**-134, 0x0000),  # tie between 0 and 2**-133 -> even
        (3 * 2.0**-134, 0x0002),  # tie -> even
        ((2 - 2.0**-7) * 2.0**127, 0x7F7F),  # largest finite
        ((2 - 2.0**-8) * 2.0**127, 0x7F80),  # tie above the largest finite -> inf
        (-(2 - 2.0**-8) * 2.0**127, 0xFF80),
        (float("inf"), 0x7F80),
    ]
    got = ob.f64_to_bf16(np.array([c[0] for c in cases]))
    for (v, want), g in zip(cases, got):
        assert int(g) == want, f"bf16({v!r}) -> {int(g):#06x}, want {want:#06x}"
    assert int(ob.f64_to_bf16(np.array([float("nan")]))[0]) & 0x7FFF > 0x7F80


def pin_bf16_vs_torch(ob):
    import torch

    rng = np.random.Generator(np.random.PCG64(7))
    u = rng.integers(0, 2**32, 200000, dtype=np.uint64).astype(np.uint32)
    # force many exact ties: clear the low 15 bits and set bit 15
    u[::3] = (u[::3] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    f = u.view(np.float32)
    f = f[np.isfinite(f)]
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = ob.f64_to_bf16(f.astype(np.float64))
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} mismatches vs torch, first {f[bad[0]]!r}"


# ------------------------------------------------------------ formula pins
def pin_constant_row_is_gamma(ob):
    """x = 1 everywhere (built from every kind of term) -> normed == gamma bitwise."""
    T, H = 3, 64
    rng = np.random.Generator(np.random.PCG64(1))
    gamma = _bits(rng.uniform(0.5, 1.5, H))
    partials = [_const(T, H, 0.25), _const(T, H, 0.125)]
    expert_out = np.stack([_bits(np.full(H, 0.5)), _bits(np.full(H, 0.25)), _bits(np.full(H, 7.0))])
    idx = np.array([[0, 1], [1, 0], [0, 1]], dtype=np.int32)
    weights = np.array([[0.5, 0.5], [0.5, 0.5], [0.5, 0.5]], dtype=np.float32)  # 0.375 per row
    shared = _const(T, H, 0.25)
    residual = _const(T, H, -0.0)  # contributes nothing
    # 0.25 + 0.125 + 0.375 + 0.25 = 1.0
    out = ob.evaluate([p for p in partials], residual, gamma, 0.0, 1e-6, expert_out=expert_out,
                      idx=idx, weights=weights, shared=shared, gate=None, keep_unrounded=True)
    assert np.all(out["x"] == 1.0), "constant row does not sum to 1"
    assert np.array_equal(out["normed"], np.broadcast_to(gamma, (T, H))), "normed != gamma"
    assert np.all(out["residual"] == 0x3F80) and np.all(out["residual_contract"] == 0x3F80)


def pin_constant_row_negative_and_bias(ob):
    """x = -c constant: y = -(gamma + wb) / sqrt(1 + eps/c^2) (unrounded)."""
    T, H = 2, 16
    rng = np.random.Generator(np.random.PCG64(2))
    gamma = _bits(rng.normal(0, 0.1, H))
    c = -3.0
    wb, eps = 1.0, 1e-6
    out = ob.evaluate([_const(T, H, c)], _const(T, H, 0.0), gamma, wb, eps, keep_unrounded=True)
    g = gamma.astype(np.uint32) << 16
    g = g.view(np.float32).astype(np.float64)
    e32 = float(np.float32(eps))
    want = -(g + 1.0) / math.sqrt(1.0 + e32 / (c * c))
    assert np.allclose(out["y"][0], want, rtol=1e-14, atol=0), "negative constant row / weight_bias"


def pin_zero_row(ob):
    T, H = 2, 32
    gamma = _bits(np.linspace(0.5, 1.5, H))
    out = ob.evaluate([_const(T, H, 0.0), _const(T, H, -0.0)], _const(T, H, -0.0), gamma, 0.0, 1e-6)
    assert np.all(out["normed"] == 0x0000)
    assert np.all(out["residual"] == 0x0000) and np.all(out["residual_contract"] == 0x0000)


def pin_eps_inside_root_over_mean(ob):
    """c^2 ~ eps: y = gamma * c / sqrt(c^2 + eps)  (about 0.707 gamma)."""
    T, H = 1, 8
    gamma = _bits(np.full(H, 1.0))
    cb = _bits(1e-3)
    c = float(bf16_f32(cb).reshape(-1)[0])
    eps = float(np.float32(1e-6))
    out = ob.evaluate([np.full((T, H), cb, np.uint16)], _const(T, H, 0.0), gamma, 0.0, 1e-6,
                      keep_unrounded=True)
    want = c / math.sqrt(c * c + eps)
    assert abs(out["y"][0, 0] - want) <= 1e-14 * want, (out["y"][0, 0], want)


def pin_scale_identity(ob):
    """y(2^k x) = y(x) * sqrt(ms + eps) / sqrt(ms + eps / 4^k), exactly in real arithmetic."""
    T, H = 4, 128
    c = make_case(T, H, 2, seed=3)
    base = ob.evaluate(c.partials, c.residual, c.gamma, 0.0, 1e-6, keep_unrounded=True)
    k = 3
    sc = [(_scale_bits(p, k)) for p in c.partials]
    scaled = ob.evaluate(sc, _scale_bits(c.residual, k), c.gamma, 0.0, 1e-6, keep_unrounded=True)
    x = base["x"]
    ms = np.mean(x * x, axis=1, keepdims=True)
    e = float(np.float32(1e-6))
    want = base["y"] * np.sqrt(ms + e) / np.sqrt(ms + e / 4.0**k)
    assert np.allclose(scaled["y"], want, rtol=1e-13, atol=0)
    assert np.array_equal(scaled["x"], x * 2.0**k)


def _scale_bits(bits, k):
    """Multiply bf16 values by 2**k by adding k to the exponent field (normal values)."""
    b = bits.astype(np.int32)
    e = (b >> 7) & 0xFF
    nz = e != 0
    b = np.where(nz, b + (k << 7), b)
    return b.astype(np.uint16)


def pin_torch_rms_norm(ob):
    """R=1, zero residual, no finalize == torch.nn.functional.rms_norm in float64."""
    import torch

    T, H = 5, 256
    c = make_case(T, H, 1, seed=4, partial_std=1.0)
    for wb in (0.0, 1.0):
        out = ob.evaluate(c.partials, _const(T, H, 0.0), c.gamma, wb, 1e-6, keep_unrounded=True)
        P = torch.from_numpy((c.partials[0].astype(np.uint32) << 16).view(np.float32)).double()
        g = torch.from_numpy((c.gamma.astype(np.uint32) << 16).view(np.float32)).double() + wb
        ref = torch.nn.functional.rms_norm(P, (H,), g, float(np.float32(1e-6))).numpy()
        assert np.allclose(out["y"], ref, rtol=1e-12, atol=0), f"rms_norm mismatch wb={wb}"
        assert np.array_equal(out["normed"], ob.f64_to_bf16(ref)), "rounded rms_norm differs"


def pin_gate_logit_zero(ob):
    s = ob.shared_scale(np.array([0.0, 40.0, -200.0], dtype=np.float32), 3)
    assert s.dtype == np.float32
    assert s[0] == np.float32(0.5) and s[1] == np.float32(1.0) and s[2] == np.float32(0.0)
    assert np.all(ob.shared_scale(None, 4) == 1.0)
    # sigmoid(1) rounded once to fp32 (value from the closed form 1/(1+e^-1))
    assert ob.shared_scale(np.array([1.0], np.float32), 1)[0] == np.float32(1.0 / (1.0 + math.exp(-1.0)))


def pin_golden_hand_cases(ob):
    """Hand-derived cases in tests/golden/hand_cases.json (derivations in the file)."""
    with open(os.path.join(GOLDEN, "hand_cases.json")) as f:
        spec = json.load(f)
    for case in spec["cases"]:
        H = case["H"]
        to_b = lambda rows: _bits(np.array(rows, dtype=np.float64))  # noqa: E731
        partials = [to_b(p) for p in case["partials"]]
        kw = {}
        if "expert_out" in case:
            kw = dict(expert_out=to_b(case["expert_out"]), idx=np.array(case["idx"], np.int32),
                      weights=np.array(case["weights"], np.float32))
        if "shared" in case:
            kw["shared"] = to_b(case["shared"])
            kw["gate"] = None if case.get("gate") is None else np.array(case["gate"], np.float32)
        out = ob.evaluate(partials, to_b(case["residual"]), _bits(np.array(case["gamma"])),
                          case["weight_bias"], case["eps"], **kw)
        assert np.array_equal(out["residual_contract"], to_b(case["expect_residual"])), case["name"]
        want = to_b(case["expect_normed"])
        assert np.array_equal(out["normed"], want), (case["name"], out["normed"], want)
        assert H == len(case["gamma"])


# ------------------------------------------------------------ brute force
def _as_lists(a):
    return None if a is None else np.asarray(a).tolist()


BRUTE_SHAPES = [
    # T, H, R, K, shared, gate, wb
    (1, 8, 1, 0, False, False, 0.0),
    (2, 16, 3, 0, False, False, 0.0),
    (3, 8, 0, 3, True, True, 1.0),
    (2, 64, 2, 2, True, False, 0.0),
    (3, 16, 3, 3, True, True, 0.5),
    (2, 8, 2, 1, False, False, 0.0),
]


def brute_inputs(T, H, R, K, shared, gate, wb, seed):
    c = make_case(T, H, R, seed=seed, K=K, num_experts=max(K, 4), shared=shared, gate=gate,
                  weight_bias=wb, gamma_dist="normal01" if wb else "uniform")
    if K:
        c.idx = c.idx.copy()
        c.idx[0, 0] = -1  # a skipped slot
        if T > 1:
            c.idx[-1, -1] = c.expert_out.shape[0] + 5  # out of range -> skipped
    return c


def pin_brute_force(ob, shapes=BRUTE_SHAPES, seed0=100, **chunking):
    for i, (T, H, R, K, sh, gt, wb) in enumerate(shapes):
        c = brute_inputs(T, H, R, K, sh, gt, wb, seed=seed0 + i)
        out = ob.evaluate(c.partials, c.residual, c.gamma, c.weight_bias, c.eps,
                          expert_out=c.expert_out, idx=c.idx, weights=c.weights,
                          shared=c.shared, gate=c.gate, **chunking)
        bn, br, bc = brute_case([_as_lists(p) for p in c.partials], _as_lists(c.residual),
                                _as_lists(c.gamma), c.weight_bias, c.eps,
                                expert_out=_as_lists(c.expert_out), idx=_as_lists(c.idx),
                                weights=_as_lists(c.weights), shared=_as_lists(c.shared),
                                gate=_as_lists(c.gate))
        for name, got, want in (("normed", out["normed"], bn), ("residual", out["residual"], br),
                                ("residual_contract", out["residual_contract"], bc)):
            want = np.array(want, dtype=np.uint16)
            assert np.array_equal(got, want), f"brute shape {i} {name}: {np.argwhere(got != want)[:4]}"


# ------------------------------------------------------------ finalize bookkeeping
def pin_permutation_invariance(ob):
    c = make_case(6, 32, 2, seed=5, K=4, num_experts=16, shared=True, gate=True)
    base = ob.evaluate(c.partials, c.residual, c.gamma, 0.0, 1e-6, expert_out=c.expert_out,
                       idx=c.idx, weights=c.weights, shared=c.shared, gate=c.gate)
    N = c.expert_out.shape[0]
    perm = np.random.Generator(np.random.PCG64(9)).permutation(N)  # new row i holds old perm[i]
    inv = np.empty(N, np.int64)
    inv[perm] = np.arange(N)
    out = ob.evaluate(c.partials, c.residual, c.gamma, 0.0, 1e-6, expert_out=c.expert_out[perm],
                      idx=inv[c.idx].astype(np.int32), weights=c.weights, shared=c.shared,
                      gate=c.gate)
    for k in ("normed", "residual", "residual_contract"):
        assert np.array_equal(out[k], base[k]), k


def pin_slot_order_and_weight_pairing(ob):
    """Each weight scales its own slot's row: swapping only the weights changes x."""
    T, H = 2, 8
    E = np.stack([_bits(np.full(H, 1.0)), _bits(np.full(H, 2.0))])
    idx = np.array([[0, 1], [1, 0]], np.int32)
    w = np.array([[0.25, 0.5], [0.25, 0.5]], np.float32)
    out = ob.evaluate([], _const(T, H, 0.0), _bits(np.ones(H)), 0.0, 1e-6, expert_out=E, idx=idx,
                      weights=w, keep_unrounded=True)
    # row 0: 0.25*1 + 0.5*2 = 1.25 ; row 1: 0.25*2 + 0.5*1 = 1.0
    assert np.all(out["x"][0] == 1.25) and np.all(out["x"][1] == 1.0)


def pin_skipped_slots(ob):
    c = make_case(4, 16, 2, seed=6, K=3, num_experts=8)
    red = ob.evaluate(c.partials, c.residual, c.gamma, 0.0, 1e-6)
    N = c.expert_out.shape[0]
    for idx in (np.full_like(c.idx, -1), np.full_like(c.idx, N), np.full_like(c.idx, 2**31 - 1)):
        out = ob.evaluate(c.partials, c.residual, c.gamma, 0.0, 1e-6, expert_out=c.expert_out,
                          idx=idx, weights=c.weights)
        for k in ("normed", "residual", "residual_contract"):
            assert np.array_equal(out[k], red[k]), k
    zero_w = ob.evaluate(c.partials, c.residual, c.gamma, 0.0, 1e-6, expert_out=c.expert_out,
                         idx=c.idx, weights=np.zeros_like(c.weights))
    for k in ("normed", "residual", "residual_contract"):
        assert np.array_equal(zero_w[k], red[k]), k


def pin_k1_unit_weight_is_a_partial(ob):
    c = make_case(5, 24, 2, seed=8, K=1, num_experts=4)
    rows = c.expert_out[c.idx[:, 0]]
    fin = ob.evaluate(c.partials, c.residual, c.gamma, 0.0, 1e-6, expert_out=c.expert_out,
                      idx=c.idx, weights=np.ones_like(c.weights))
    red = ob.evaluate(c.partials + [rows], c.residual, c.gamma, 0.0, 1e-6)
    for k in ("normed", "residual", "residual_contract"):
        assert np.array_equal(fin[k], red[k]), k


def pin_shared_added_once(ob):
    c = make_case(3, 16, 2, seed=10, shared=True)
    fin = ob.evaluate(c.partials, c.residual, c.gamma, 0.0, 1e-6, shared=c.shared,
                      keep_unrounded=True)
    red = ob.evaluate(c.partials + [c.shared], c.residual, c.gamma, 0.0, 1e-6, keep_unrounded=True)
    assert np.array_equal(fin["x"], red["x"])
    assert np.array_equal(fin["residual_contract"], red["residual_contract"])
    # gate logit 0 == ungated with S halved (halving a bf16 value is exact)
    half = _scale_bits(c.shared, -1)
    g0 = ob.evaluate(c.partials, c.residual, c.gamma, 0.0, 1e-6, shared=c.shared,
                     gate=np.zeros(3, np.float32))
    h = ob.evaluate(c.partials, c.residual, c.gamma, 0.0, 1e-6, shared=half)
    for k in ("normed", "residual", "residual_contract"):
        assert np.array_equal(g0[k], h[k]), k


def pin_signed_zero(ob):
    T, H = 1, 8
    nz = _const(T, H, -0.0)
    out = ob.evaluate([nz, nz], nz, _bits(np.ones(H)), 0.0, 1e-6, expert_out=np.stack([nz[0]]),
                      idx=np.array([[0]], np.int32), weights=np.array([[1.0]], np.float32),
                      shared=nz, gate=None)
    assert np.all(out["residual"] == 0x0000) and np.all(out["residual_contract"] == 0x0000)


def pin_track_b_is_float32_ops(ob):
    """A case where the fp32 rounding of w*E matters: the contract track must round
    the product before adding it to the running sum (no fused multiply-add)."""
    T, H = 1, 8
    # w = 1 + 2^-23 (fp32), E = 1 + 2^-7 (bf16): w*E = 1 + 2^-7 + 2^-23 + 2^-30 and
    # fl32(w*E) = 1 + 2^-7 + 2^-23 (2^-30 is below half an ulp).  A partial of
    # -(1 + 2^-7) already in the sum cancels the leading part: the fp32 chain gives
    # 2^-23, the exact (or fused) sum gives 2^-23 + 2^-30.
    w = np.array([[1.0 + 2.0**-23]], np.float32)
    E = _bits(np.full((1, H), 1.0 + 2.0**-7))
    part = _bits(np.full((T, H), -(1.0 + 2.0**-7)))
    zero = _const(T, H, 0.0)
    idx = np.array([[0]], np.int32)
    out = ob.evaluate([part], zero, _bits(np.ones(H)), 0.0, 1e-6, expert_out=E, idx=idx,
                      weights=w, keep_unrounded=True)
    assert np.all(out["x"] == 2.0**-23 + 2.0**-30)
    assert np.all(ob.accumulate_f32([part], zero, expert_out=E, idx=idx, weights=w)
                  == np.float32(2.0**-23))
    assert np.all(out["residual_contract"] == 0x3400)  # bf16(2^-23)
    assert np.all(out["residual"] == 0x3401)  # bf16(2^-23 * (1 + 2^-7))


def pin_split_brute_force(ob, shapes=BRUTE_SHAPES[1:5], seed0=200, **chunking):
    """The split flow against the decimal brute force (stage 1 rounding included)."""
    for i, (T, H, R, K, sh, gt, wb) in enumerate(shapes):
        c = brute_inputs(T, H, R, K, sh, gt, wb, seed=seed0 + i)
        out = ob.split_evaluate(c.partials, c.residual, c.gamma, c.weight_bias, c.eps,
                                expert_out=c.expert_out, idx=c.idx, weights=c.weights,
                                shared=c.shared, gate=c.gate, **chunking)
        by, bn, br, bc = brute_split([_as_lists(p) for p in c.partials], _as_lists(c.residual),
                                     _as_lists(c.gamma), c.weight_bias, c.eps,
                                     expert_out=_as_lists(c.expert_out), idx=_as_lists(c.idx),
                                     weights=_as_lists(c.weights), shared=_as_lists(c.shared),
                                     gate=_as_lists(c.gate))
        for name, got, want in (("sum", out["sum"], by), ("normed", out["normed"], bn),
                                ("residual", out["residual"], br),
                                ("residual_contract", out["residual_contract"], bc)):
            want = np.array(want, dtype=np.uint16)
            assert np.array_equal(got, want), f"split brute shape {i} {name}"


def pin_split_intermediate_rounding(ob):
    """Stage 1 rounds to bf16: 1 + 2^-8 (a tie) becomes 1.0, so adding a residual
    of 2^-8 gives 1.0 again, where the fused sum gives 1 + 2^-7 exactly."""
    T, H = 1, 8
    parts = [_const(T, H, 1.0), _const(T, H, 2.0**-8)]
    resid = _const(T, H, 2.0**-8)
    gamma = _bits(np.ones(H))
    split = ob.split_evaluate(parts, resid, gamma, 0.0, 1e-6)
    fused = ob.evaluate(parts, resid, gamma, 0.0, 1e-6)
    assert np.all(split["sum"] == 0x3F80)
    assert np.all(split["residual_contract"] == 0x3F80) and np.all(split["residual"] == 0x3F80)
    assert np.all(fused["residual_contract"] == 0x3F81)


def pin_split_equals_fused_when_exact(ob):
    """When the stage-1 sum is exactly representable in bf16 the two flows agree."""
    with open(os.path.join(GOLDEN, "hand_cases.json")) as f:
        spec = json.load(f)
    case = spec["cases"][0]
    to_b = lambda rows: _bits(np.array(rows, dtype=np.float64))  # noqa: E731
    parts = [to_b(p) for p in case["partials"]]
    args = (to_b(case["residual"]), _bits(np.array(case["gamma"])), case["weight_bias"], case["eps"])
    split = ob.split_evaluate(parts, *args)
    fused = ob.evaluate(parts, *args)
    for k in ("normed", "residual", "residual_contract"):
        assert np.array_equal(split[k], fused[k]), k


# Shapes of 3 to 5 rows: with two rows per chunk, the oracle's row-chunk loop
# runs several passes and ends on a partial chunk (one row).
CHUNKED_SHAPES = [
    (3, 8, 0, 3, True, True, 1.0),
    (3, 16, 3, 3, True, True, 0.5),
    (5, 16, 2, 2, True, False, 0.0),
]


def pin_brute_force_across_row_chunks(ob):
    """Both tracks and the split flow, brute-forced, with the oracle evaluating
    rows two at a time: a slicing slip in its row-chunk loop (a row dropped,
    repeated or paired with another row's routing) fails here."""
    pin_brute_force(ob, shapes=CHUNKED_SHAPES, seed0=300, chunk_rows=2)
    pin_split_brute_force(ob, shapes=CHUNKED_SHAPES, seed0=400, chunk_rows=2)


ALL_PINS = [
    pin_bf16_hand_cases,
    pin_bf16_vs_torch,
    pin_constant_row_is_gamma,
    pin_constant_row_negative_and_bias,
    pin_zero_row,
    pin_eps_inside_root_over_mean,
    pin_scale_identity,
    pin_torch_rms_norm,
    pin_gate_logit_zero,
    pin_golden_hand_cases,
    pin_brute_force,
    pin_permutation_invariance,
    pin_slot_order_and_weight_pairing,
    pin_skipped_slots,
    pin_k1_unit_weight_is_a_partial,
    pin_shared_added_once,
    pin_signed_zero,
    pin_track_b_is_float32_ops,
    pin_split_brute_force,
    pin_split_intermediate_rounding,
    pin_split_equals_fused_when_exact,
    pin_brute_force_across_row_chunks,
]
