"""Exact-rational brute force used to pin the oracle on tiny problems.

Written independently of ``oracle/``: every element is decoded from its bit
fields (no lookup tables), every product and sum is an exact ``Fraction``, and
the final rounding to bf16 is done on the exact rational by integer arithmetic.
Only small shapes are practical (pure-Python loops).
"""

from __future__ import annotations

from fractions import Fraction


def e2m1(code: int) -> Fraction:
    """FP4 E2M1 from its fields: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0."""
    s = -1 if code & 0b1000 else 1
    e = (code >> 1) & 0b11
    m = code & 1
    if e == 0:
        mag = Fraction(m, 2)                       # subnormal: 0.m * 2**(1-1)
    else:
        mag = Fraction(2) ** (e - 1) * (1 + Fraction(m, 2))
    return s * mag


def fp6(code: int, ebits: int) -> Fraction:
    """FP6 from its fields: sign bit 5, then `ebits` exponent bits (bias 2**(ebits-1) - 1) and
    5 - ebits mantissa bits; exponent 0 is subnormal (OCP MX v1.0: E2M3 has ebits 2, E3M2 3)."""
    mbits = 5 - ebits
    s = -1 if code & 0b100000 else 1
    e = (code >> mbits) & ((1 << ebits) - 1)
    m = code & ((1 << mbits) - 1)
    bias = (1 << (ebits - 1)) - 1
    if e == 0:
        mag = Fraction(m, 1 << mbits) * Fraction(2) ** (1 - bias)
    else:
        mag = Fraction(2) ** (e - bias) * (1 + Fraction(m, 1 << mbits))
    return s * mag


def fp6_code(packed_row, k: int) -> int:
    """Code k of a row of packed FP6 bytes, read bit by bit: bit b of the row's stream is bit
    b % 8 of byte b // 8, and code k is bits 6k .. 6k+5 (lowest first)."""
    v = 0
    for i in range(6):
        b = 6 * k + i
        v |= ((int(packed_row[b // 8]) >> (b % 8)) & 1) << i
    return v


def e8m0(byte: int) -> Fraction:
    if byte == 255:
        raise ValueError("NaN scale")
    return Fraction(2) ** (byte - 127)


def e4m3fn(byte: int) -> Fraction:
    s = -1 if byte & 0x80 else 1
    e = (byte >> 3) & 0xF
    m = byte & 0x7
    if e == 15 and m == 7:
        raise ValueError("NaN")
    if e == 0:
        mag = Fraction(m, 8) * Fraction(2) ** -6
    else:
        mag = Fraction(2) ** (e - 7) * (1 + Fraction(m, 8))
    return s * mag


def bf16(bits: int) -> Fraction:
    s = -1 if bits & 0x8000 else 1
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    if e == 0xFF:
        raise ValueError("inf/NaN")
    if e == 0:
        mag = Fraction(m) * Fraction(2) ** -133
    else:
        mag = Fraction(2) ** (e - 127) * (1 + Fraction(m, 128))
    return s * mag


def _floor_log2(x: Fraction) -> int:
    """floor(log2 x) for x > 0, exactly."""
    e = x.numerator.bit_length() - x.denominator.bit_length()
    while Fraction(2) ** e > x:
        e -= 1
    while Fraction(2) ** (e + 1) <= x:
        e += 1
    return e


def round_bf16(x: Fraction) -> int:
    """Nearest bf16 to the exact rational x, ties to an even mantissa; returns the bit pattern."""
    if x == 0:
        return 0
    sign = 0x8000 if x < 0 else 0
    a = abs(x)
    e = max(_floor_log2(a), -126)
    quantum = Fraction(2) ** (e - 7)
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = fl * quantum
    if v >= Fraction(2) ** 128:
        return sign | 0x7F80
    if v < Fraction(2) ** -126:
        return sign | int(v / Fraction(2) ** -133)
    ev = _floor_log2(v)
    mant = (v / Fraction(2) ** ev - 1) * 128
    assert mant.denominator == 1
    return sign | ((ev + 127) << 7) | int(mant)


def gemm(dtype: str, A, B, SA, SB, bias, M: int, N: int, K: int):
    """C[m][n] bits for D = sigma * sum_k a*b + bias[n], all exact."""
    if dtype.startswith("mxfp6"):
        return gemm_mx(dtype, dtype, A, B, SA, SB, bias, M, N, K)

    def a_val(m, k):
        if dtype == "mxfp4":
            byte = int(A[m][k // 2])
            code = (byte >> 4) if (k & 1) else (byte & 0xF)
            return e2m1(code) * e8m0(int(SA[m][k // 32]))
        if dtype == "mxfp8":
            return e4m3fn(int(A[m][k])) * e8m0(int(SA[m][k // 32]))
        if dtype == "bf16":
            return bf16(int(A[m][k]))
        return e4m3fn(int(A[m][k]))

    def b_val(n, k):
        if dtype == "mxfp4":
            byte = int(B[n][k // 2])
            code = (byte >> 4) if (k & 1) else (byte & 0xF)
            return e2m1(code) * e8m0(int(SB[n][k // 32]))
        if dtype == "mxfp8":
            return e4m3fn(int(B[n][k])) * e8m0(int(SB[n][k // 32]))
        if dtype == "bf16":
            return bf16(int(B[n][k]))
        return e4m3fn(int(B[n][k]))

    sigma = Fraction(1)
    if dtype == "fp8":
        sigma = Fraction(float(SA)) * Fraction(float(SB))
    out = [[0] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            s = sum((a_val(m, k) * b_val(n, k) for k in range(K)), Fraction(0))
            d = sigma * s
            if bias is not None:
                d += bf16(int(bias[n]))
            out[m][n] = round_bf16(d)
    return out


def bf16_backward(dC, A, B, M: int, N: int, K: int):
    """Bits of dA = dC B, dB = dC^T A and dbias = column sums of dC, all exact then rounded once."""
    g = [[bf16(int(dC[m][n])) for n in range(N)] for m in range(M)]
    a = [[bf16(int(A[m][k])) for k in range(K)] for m in range(M)]
    b = [[bf16(int(B[n][k])) for k in range(K)] for n in range(N)]
    dA = [[round_bf16(sum((g[m][n] * b[n][k] for n in range(N)), Fraction(0))) for k in range(K)] for m in range(M)]
    dB = [[round_bf16(sum((g[m][n] * a[m][k] for m in range(M)), Fraction(0))) for k in range(K)] for n in range(N)]
    db = [round_bf16(sum((g[m][n] for m in range(M)), Fraction(0))) for n in range(N)]
    return dA, dB, db


def gemm_mx(a_fmt: str, b_fmt: str, A, B, SA, SB, bias, M: int, N: int, K: int):
    """C bits for operands of MX formats a_fmt / b_fmt ("mxfp4", "mxfp6_e2m3", "mxfp6_e3m2",
    "mxfp8"), all exact."""
    def val(fmt, X, S, r, k):
        return _operand_value(fmt, X, S, r, k)

    out = [[0] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            d = sum((val(a_fmt, A, SA, m, k) * val(b_fmt, B, SB, n, k) for k in range(K)), Fraction(0))
            if bias is not None:
                d += bf16(int(bias[n]))
            out[m][n] = round_bf16(d)
    return out


# ---------------------------------------------------------------- the tolerance arithmetic

def _operand_value(dtype: str, X, S, r: int, k: int) -> Fraction:
    """Element (r, k) of an operand of `dtype`, decoded from its bit fields."""
    if dtype in ("mxfp6_e2m3", "mxfp6_e3m2"):
        return fp6(fp6_code(X[r], k), 2 if dtype.endswith("e2m3") else 3) * e8m0(int(S[r][k // 32]))
    if dtype == "mxfp4":
        byte = int(X[r][k // 2])
        code = (byte >> 4) if (k & 1) else (byte & 0xF)
        return e2m1(code) * e8m0(int(S[r][k // 32]))
    if dtype == "mxfp8":
        return e4m3fn(int(X[r][k])) * e8m0(int(S[r][k // 32]))
    if dtype == "bf16":
        return bf16(int(X[r][k]))
    return e4m3fn(int(X[r][k]))


def abs_sums(dtype: str, A, B, SA, SB, M: int, N: int, K: int):
    """Exact S[m][n] = |sigma| * sum_k |a(m,k) * b(n,k)| (sigma = SA * SB for fp8, else 1),
    and the exact D[m][n] = sigma * sum_k a(m,k) * b(n,k) (no bias), as Fractions."""
    sigma = Fraction(float(SA)) * Fraction(float(SB)) if dtype == "fp8" else Fraction(1)
    S = [[Fraction(0)] * N for _ in range(M)]
    D = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        a = [_operand_value(dtype, A, SA, m, k) for k in range(K)]
        for n in range(N):
            b = [_operand_value(dtype, B, SB, n, k) for k in range(K)]
            S[m][n] = abs(sigma) * sum((abs(x * y) for x, y in zip(a, b)), Fraction(0))
            D[m][n] = sigma * sum((x * y for x, y in zip(a, b)), Fraction(0))
    return S, D


def mixed_abs_sums(a_fmt: str, b_fmt: str, A, B, SA, SB, M: int, N: int, K: int):
    """Exact sum_k |a(m,k) * b(n,k)| for block-scaled operands of formats a_fmt / b_fmt."""
    return [[sum((abs(_operand_value(a_fmt, A, SA, m, k) * _operand_value(b_fmt, B, SB, n, k)) for k in range(K)),
                 Fraction(0)) for n in range(N)] for m in range(M)]


def backward_abs_sums(dC, A, B, M: int, N: int, K: int):
    """Exact error-bound sums of the bf16 backward: sum_n |dC[m][n] B[n][k]|,
    sum_m |dC[m][n] A[m][k]| and sum_m |dC[m][n]|."""
    g = [[bf16(int(dC[m][n])) for n in range(N)] for m in range(M)]
    a = [[bf16(int(A[m][k])) for k in range(K)] for m in range(M)]
    b = [[bf16(int(B[n][k])) for k in range(K)] for n in range(N)]
    sA = [[sum((abs(g[m][n] * b[n][k]) for n in range(N)), Fraction(0)) for k in range(K)] for m in range(M)]
    sB = [[sum((abs(g[m][n] * a[m][k]) for m in range(M)), Fraction(0)) for k in range(K)] for n in range(N)]
    sb = [sum((abs(g[m][n]) for m in range(M)), Fraction(0)) for n in range(N)]
    return sA, sB, sb


def ulp_bf16(x: Fraction) -> Fraction:
    """Spacing of the bf16 grid at |x|, from the format: 8 significant bits, so
    2**(e - 7) for 2**e <= |x| < 2**(e+1) with e >= -126; the subnormal spacing
    2**-133 below 2**-126 (and at 0)."""
    a = abs(Fraction(x))
    if a < Fraction(2) ** -126:
        return Fraction(2) ** -133
    return Fraction(2) ** (_floor_log2(a) - 7)


def accept(c_bits: int, ref_bits: int, D: Fraction, S: Fraction) -> bool:
    """The parity bar, exactly: bits equal (either zero matches either zero), or
    |c - D| <= 2**-7 * S + ulp_bf16(max(|D|, |c|))."""
    if c_bits == ref_bits or ((c_bits | ref_bits) & 0x7FFF) == 0:
        return True
    c = bf16(c_bits)
    return abs(c - D) <= S / 128 + ulp_bf16(max(abs(D), abs(c)))
