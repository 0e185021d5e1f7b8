"""Scalar brute force of the boundary in 50-digit decimal arithmetic.

Test-only.  Written independently of ``oracle.boundary`` (plain Python loops over
``decimal.Decimal``, its own binary rounding), so agreement pins the vectorised
oracle rather than restating it.  Usable on tiny shapes only.
"""
from __future__ import annotations

import decimal
import math
import struct
from decimal import Decimal

CTX = decimal.Context(prec=50, rounding=decimal.ROUND_HALF_EVEN)


def bf16_bits_to_decimal(b: int) -> Decimal:
    f = struct.unpack("<f", struct.pack("<I", (int(b) & 0xFFFF) << 16))[0]
    return Decimal(f)  # exact: Decimal(float) holds the binary value exactly


def f32_to_decimal(v: float) -> Decimal:
    f = struct.unpack("<f", struct.pack("<f", float(v)))[0]
    return Decimal(f)


def round_binary(d: Decimal, sig_bits: int, min_exp: int) -> Decimal:
    """Round ``d`` to the nearest binary float with ``sig_bits`` significant bits
    (ties to even); ``min_exp`` is the exponent of the smallest normal.
    Overflow is not handled (tiny cases never reach it)."""
    if d == 0:
        return d
    a = abs(d)
    # exponent e with 2**(e-1) <= a < 2**e, found from the float estimate then fixed exactly
    e = math.frexp(float(a))[1]
    while CTX.power(Decimal(2), e - 1) > a:
        e -= 1
    while CTX.power(Decimal(2), e) <= a:
        e += 1
    q_exp = max(e - sig_bits, min_exp - (sig_bits - 1))
    quantum = CTX.power(Decimal(2), q_exp)
    n = CTX.divide(a, quantum).quantize(Decimal(1), rounding=decimal.ROUND_HALF_EVEN, context=CTX)
    r = CTX.multiply(n, quantum)
    return r if d > 0 else -r


def decimal_to_bf16_bits(d: Decimal) -> int:
    r = round_binary(d, 8, -126)
    f = float(r)  # exact: r has 8 significant bits
    if f == 0.0 and d < 0:
        f = -0.0
    return struct.unpack("<I", struct.pack("<f", f))[0] >> 16


def to_f32(d: Decimal) -> Decimal:
    return round_binary(d, 24, -126)


def sigmoid_f32(g: float) -> Decimal:
    x = f32_to_decimal(g)
    s = CTX.divide(Decimal(1), CTX.add(Decimal(1), CTX.exp(-x)))
    return to_f32(s)


def brute_split(partials, residual, gamma, weight_bias, eps, expert_out=None, idx=None,
                weights=None, shared=None, gate=None):
    """The split flow: stage 1 = bf16 of the float32-op sum without the residual;
    stage 2 = brute_case of that single tensor and the residual.
    Returns (sum_bits, normed_bits, residual_bits, residual_contract_bits)."""
    T = len(residual)
    H = len(residual[0])
    y = []
    for t in range(T):
        row = []
        for h in range(H):
            a = Decimal(0)
            for P in partials:
                a = to_f32(CTX.add(a, bf16_bits_to_decimal(P[t][h])))
            if idx is not None:
                N = len(expert_out)
                for k in range(len(idx[t])):
                    j = int(idx[t][k])
                    if 0 <= j < N:
                        p = to_f32(CTX.multiply(f32_to_decimal(weights[t][k]),
                                                bf16_bits_to_decimal(expert_out[j][h])))
                        a = to_f32(CTX.add(a, p))
            if shared is not None:
                s = Decimal(1) if gate is None else sigmoid_f32(gate[t])
                a = to_f32(CTX.add(a, to_f32(CTX.multiply(s, bf16_bits_to_decimal(shared[t][h])))))
            row.append(decimal_to_bf16_bits(a))
        y.append(row)
    n, r, c = brute_case([y], residual, gamma, weight_bias, eps)
    return y, n, r, c


def brute_case(partials, residual, gamma, weight_bias, eps, expert_out=None, idx=None,
               weights=None, shared=None, gate=None):
    """Returns (normed_bits, residual_bits, residual_contract_bits) as lists of lists."""
    T = len(residual)
    H = len(residual[0])
    wb = f32_to_decimal(weight_bias)
    ep = f32_to_decimal(eps)
    normed, resid, contract = [], [], []
    for t in range(T):
        # exact sum and the float32-op sum, element by element
        xs = []
        fs = []
        for h in range(H):
            x = Decimal(0)
            a = Decimal(0)
            for P in partials:
                v = bf16_bits_to_decimal(P[t][h])
                x = CTX.add(x, v)
                a = to_f32(CTX.add(a, v))
            if idx is not None:
                N = len(expert_out)
                for k in range(len(idx[t])):
                    j = int(idx[t][k])
                    if 0 <= j < N:
                        w = f32_to_decimal(weights[t][k])
                        e = bf16_bits_to_decimal(expert_out[j][h])
                        x = CTX.add(x, CTX.multiply(w, e))
                        a = to_f32(CTX.add(a, to_f32(CTX.multiply(w, e))))
            if shared is not None:
                s = Decimal(1) if gate is None else sigmoid_f32(gate[t])
                v = bf16_bits_to_decimal(shared[t][h])
                x = CTX.add(x, CTX.multiply(s, v))
                a = to_f32(CTX.add(a, to_f32(CTX.multiply(s, v))))
            v = bf16_bits_to_decimal(residual[t][h])
            x = CTX.add(x, v)
            a = to_f32(CTX.add(a, v))
            xs.append(x)
            fs.append(a)
        ss = Decimal(0)
        for x in xs:
            ss = CTX.add(ss, CTX.multiply(x, x))
        ms = CTX.divide(ss, Decimal(H))
        inv = CTX.divide(Decimal(1), CTX.sqrt(CTX.add(ms, ep)))
        row_n, row_r, row_c = [], [], []
        for h in range(H):
            g = CTX.add(bf16_bits_to_decimal(gamma[h]), wb)
            y = CTX.multiply(CTX.multiply(xs[h], inv), g)
            row_n.append(decimal_to_bf16_bits(y))
            row_r.append(decimal_to_bf16_bits(xs[h]))
            row_c.append(decimal_to_bf16_bits(fs[h]))
        normed.append(row_n)
        resid.append(row_r)
        contract.append(row_c)
    return normed, resid, contract
