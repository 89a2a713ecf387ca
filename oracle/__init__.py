"""CPU oracle for the Stream-K GEMM path.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The product path (the HIP library and its
Python binding in ``persistent_gemm_amd``) never calls it, and this module
imports nothing from the product: the two share no code.  Inputs reach both
sides as plain host bytes made by ``persistent_gemm_amd.inputs`` (a seeded
generator that holds none of the arithmetic below).

What the path computes, written out plainly (fp64 throughout):

    D[m][n] = sigma * sum_{k=0}^{K-1} a(m,k) * b(n,k) + beta[n]
    C[m][n] = RNE_bf16(D[m][n])

Stream-K only changes *who* performs which MAC iterations of this sum and in
which order the fp32 partial tiles are added; the value it aims at is this
one.  Sources:

* The contraction itself, with FP4 (MX) operands and a Stream-K split of the
  K-loop: "Stream-k mxfp4 kernel" (ROCm/tritonBLAS pull request 74), the
  author's description and the Copilot pull request overview.
* bf16 / fp8 ``matmul`` and ``addmm`` checked against ``torch.mm`` /
  ``torch.addmm`` (so alpha = beta = 1): "Fix StreamK Kernel Bias #67",
  the review comments on the two correctness tests.
* The bias runs along N (one value per output column), is broadcast over the
  M rows, and is added once, after the partial tiles of a split tile have been
  aggregated; in the quantized mode it is turned into fp32 before the add:
  "Fix StreamK Kernel Bias #67", Motivation and Technical Details.
* MXFP8 (E4M3 elements with the same E8M0 block scales) is the block-scaled
  form of the quantized mode of "Fix StreamK Kernel Bias #67", Technical
  Details; it is the MXFP4 contraction with 8-bit elements.  MXFP6 (E2M3 or
  E3M2 elements, the same scales) is the same contraction with 6-bit elements,
  and the mixed forms decode each operand by its own format.
* The bf16 backward of addmm (the gradients of A, B and the bias that the
  Stream-K matmul / addmm tests take and compare with torch's): "Fix StreamK
  Kernel Bias #67", review comments on the two Stream-K tests.
* Element encodings are not on those pages.  E2M1 (FP4), E2M3 and E3M2 (FP6)
  and E8M0 (the shared block scale, one per 32 consecutive K elements) follow
  the OCP Microscaling Formats (MX) v1.0 specification; E4M3FN follows the OCP 8-bit Floating Point
  (OFP8) specification; bf16 is the top half of an IEEE binary32.

Readings where the pages are silent: the bf16 output is rounded once, to
nearest-even, straight from the fp64 value (never through fp32, which would
double-round); for fp8 the per-tensor scale is applied before the bias is
added; the two FP4 codes of a byte hold the even K index in the low nibble;
FP6 codes are packed four to three bytes as a little-endian bit stream (code
k at bits 6k .. 6k+5 of the row's stream).

Every function here is pinned by ``tests/test_oracle_pins.py`` against
something other than itself (torch's own format conversions, closed forms,
hand-worked sums, an exact-rational brute force and invariants).
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "E2M1_VALUES",
    "decode_e2m1",
    "decode_e8m0",
    "decode_e4m3fn",
    "decode_bf16",
    "unpack_fp4",
    "mxfp4_operand",
    "mxfp8_operand",
    "rne_bf16_from_double",
    "bf16_to_double",
    "operands",
    "gemm",
    "gemm_elements",
    "abs_product_sums",
    "accept",
    "bf16_backward",
    "gemm_mx",
    "abs_product_sums_mx",
    "decode_e2m3",
    "decode_e3m2",
    "unpack_fp6",
    "mxfp6_operand",
]

# OCP MX v1.0, FP4 (E2M1): code bits are sign | exponent(2, bias 1) | mantissa(1).
# Listed by code 0..15.
E2M1_VALUES = np.array(
    [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
     -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0],
    dtype=np.float64,
)


def decode_e2m1(codes: np.ndarray) -> np.ndarray:
    """FP4 codes (uint8 in 0..15) -> fp64 values, by table lookup."""
    codes = np.asarray(codes, dtype=np.uint8)
    if codes.size and int(codes.max()) > 15:
        raise ValueError("E2M1 codes are 4-bit")
    return E2M1_VALUES[codes]


def _decode_fp6(codes: np.ndarray, ebits: int, mbits: int) -> np.ndarray:
    """6-bit sign | exponent(ebits) | mantissa(mbits) codes -> fp64 (OCP MX v1.0 FP6: no
    infinities or NaNs; bias 2**(ebits-1) - 1; exponent 0 is subnormal)."""
    codes = np.asarray(codes, dtype=np.uint8)
    if codes.size and int(codes.max()) > 63:
        raise ValueError("FP6 codes are 6-bit")
    c = codes.astype(np.int64)
    bias = (1 << (ebits - 1)) - 1
    sign = np.where(c & 0x20, -1.0, 1.0)
    e = (c >> mbits) & ((1 << ebits) - 1)
    m = (c & ((1 << mbits) - 1)).astype(np.float64) / (1 << mbits)
    mag = np.where(e == 0, np.ldexp(m, 1 - bias), np.ldexp(1.0 + m, (e - bias).astype(np.int32)))
    return sign * mag


def decode_e2m3(codes: np.ndarray) -> np.ndarray:
    """FP6 E2M3 codes (0..63) -> fp64: sign bit 5, exponent bits 4:3 (bias 1), mantissa bits 2:0."""
    return _decode_fp6(codes, 2, 3)


def decode_e3m2(codes: np.ndarray) -> np.ndarray:
    """FP6 E3M2 codes (0..63) -> fp64: sign bit 5, exponent bits 4:2 (bias 3), mantissa bits 1:0."""
    return _decode_fp6(codes, 3, 2)


def decode_e8m0(e: np.ndarray) -> np.ndarray:
    """E8M0 scale bytes -> 2**(e - 127); 0xFF is NaN (OCP MX v1.0)."""
    e = np.asarray(e, dtype=np.int64)
    v = np.ldexp(np.ones(e.shape, dtype=np.float64), (e - 127).astype(np.int32))
    return np.where(e == 255, np.nan, v)


def decode_e4m3fn(b: np.ndarray) -> np.ndarray:
    """OCP E4M3FN bytes -> fp64.  Exponent bias 7, no infinities, S.1111.111 is NaN."""
    b = np.asarray(b, dtype=np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    exp = (b >> 3) & 0xF
    man = (b & 0x7).astype(np.float64)
    normal = np.ldexp(1.0 + man / 8.0, (exp - 7).astype(np.int32))
    subnormal = np.ldexp(man / 8.0, -6)
    mag = np.where(exp == 0, subnormal, normal)
    mag = np.where((exp == 15) & ((b & 0x7) == 7), np.nan, mag)
    return sign * mag


def decode_bf16(u: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp64 (bf16 is the upper half of binary32)."""
    u = np.ascontiguousarray(np.asarray(u, dtype=np.uint16))
    return (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


bf16_to_double = decode_bf16


def unpack_fp4(packed: np.ndarray, K: int) -> np.ndarray:
    """uint8[rows][K/2] -> codes uint8[rows][K]; element 2j is the low nibble of byte j."""
    packed = np.asarray(packed, dtype=np.uint8)
    rows = packed.shape[0]
    if packed.shape[1] != K // 2:
        raise ValueError("packed FP4 rows must hold K/2 bytes")
    codes = np.empty((rows, K), dtype=np.uint8)
    codes[:, 0::2] = packed & 0x0F
    codes[:, 1::2] = packed >> 4
    return codes


def unpack_fp6(packed: np.ndarray, K: int) -> np.ndarray:
    """uint8[rows][3K/4] -> codes uint8[rows][K]: each 3 bytes b0 b1 b2 hold four codes as the
    24-bit little-endian word w = b0 | b1 << 8 | b2 << 16, code 4j+i = (w >> 6i) & 63."""
    packed = np.asarray(packed, dtype=np.uint8)
    if K % 4 or packed.shape[1] != 3 * K // 4:
        raise ValueError("packed FP6 rows must hold 3K/4 bytes")
    b = packed.reshape(packed.shape[0], K // 4, 3).astype(np.uint32)
    w = b[:, :, 0] | (b[:, :, 1] << 8) | (b[:, :, 2] << 16)
    codes = np.empty((packed.shape[0], K // 4, 4), dtype=np.uint8)
    for i in range(4):
        codes[:, :, i] = (w >> (6 * i)) & 63
    return codes.reshape(packed.shape[0], K)


def _apply_block_scales(vals: np.ndarray, scales: np.ndarray, K: int) -> np.ndarray:
    """value(r, k) = element(r, k) * 2**(scale[r][k // 32] - 127): one E8M0 scale per 32 consecutive K."""
    if K % 32:
        raise ValueError("MX formats need K to be a multiple of the 32-element scale block")
    sc = decode_e8m0(np.asarray(scales, dtype=np.uint8))
    if sc.shape != (vals.shape[0], K // 32):
        raise ValueError("MX scales must be [rows][K/32]")
    return vals * np.repeat(sc, 32, axis=1)


def mxfp4_operand(packed: np.ndarray, scales: np.ndarray, K: int) -> np.ndarray:
    """Decode an MXFP4 operand: value(r, k) = E2M1(code(r, k)) * 2**(scale[r][k // 32] - 127)."""
    if K % 32:
        raise ValueError("MXFP4 needs K to be a multiple of the 32-element scale block")
    return _apply_block_scales(decode_e2m1(unpack_fp4(packed, K)), scales, K)


def mxfp8_operand(elems: np.ndarray, scales: np.ndarray, K: int) -> np.ndarray:
    """Decode an MXFP8 operand (OCP MX v1.0, E4M3 elements):
    value(r, k) = E4M3FN(byte(r, k)) * 2**(scale[r][k // 32] - 127)."""
    elems = np.asarray(elems, dtype=np.uint8)
    if elems.shape[1] != K:
        raise ValueError("MXFP8 rows must hold K bytes")
    return _apply_block_scales(decode_e4m3fn(elems), scales, K)


def mxfp6_operand(packed: np.ndarray, scales: np.ndarray, K: int, fmt: str = "e2m3") -> np.ndarray:
    """Decode an MXFP6 operand: value(r, k) = FP6(code(r, k)) * 2**(scale[r][k // 32] - 127),
    with FP6 = E2M3 (fmt "e2m3") or E3M2 (fmt "e3m2")."""
    dec = {"e2m3": decode_e2m3, "e3m2": decode_e3m2}[fmt]
    return _apply_block_scales(dec(unpack_fp6(packed, K)), scales, K)


def rne_bf16_from_double(d: np.ndarray) -> np.ndarray:
    """Round fp64 values once to the nearest bf16 (ties to even); return uint16 bit patterns.

    quantum = 2**(max(floor(log2|d|), -126) - 7) is the bf16 spacing at |d| (the
    subnormal spacing 2**-133 below 2**-126); rint() rounds half to even.
    Results of magnitude >= 2**128 become +-inf; NaN becomes 0x7FC0.
    """
    d = np.asarray(d, dtype=np.float64)
    out_shape = d.shape
    d = d.reshape(-1)
    res = np.zeros(d.shape, dtype=np.float64)
    finite = np.isfinite(d)
    nz = finite & (d != 0.0)
    _, ex = np.frexp(d[nz])                     # d = f * 2**ex, 0.5 <= |f| < 1
    e = ex.astype(np.int64) - 1                 # floor(log2 |d|)
    q = np.ldexp(1.0, (np.maximum(e, -126) - 7).astype(np.int32))
    r = np.rint(d[nz] / q) * q
    r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, r), r)
    res[nz] = r
    res[finite & (d == 0.0)] = d[finite & (d == 0.0)]      # keeps the sign of zero
    res[np.isinf(d)] = d[np.isinf(d)]
    bits = (res.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    bits[np.isnan(d)] = 0x7FC0
    return bits.reshape(out_shape)


def operands(dtype: str, A, B, SA=None, SB=None, K: int | None = None):
    """Decoded fp64 operands (a[M][K], b[N][K]) and sigma for one of the three input types.

    dtype "mxfp4": A, B are uint8[rows][K/2] packed E2M1, SA, SB uint8[rows][K/32] E8M0.
    dtype "bf16":  A, B are uint16[rows][K] bf16 bit patterns; sigma = 1.
    dtype "fp8":   A, B are uint8[rows][K] E4M3FN; SA, SB are the per-tensor fp32
                   scale factors (Python floats), sigma = SA * SB.
    dtype "mxfp8": A, B are uint8[rows][K] E4M3FN, SA, SB uint8[rows][K/32] E8M0; sigma = 1.
    dtype "mxfp6_e2m3" / "mxfp6_e3m2": A, B are uint8[rows][3K/4] packed FP6, SA, SB uint8[rows][K/32]
    E8M0; sigma = 1.
    """
    if dtype == "mxfp4":
        if K is None:
            K = 2 * np.asarray(A).shape[1]
        return mxfp4_operand(A, SA, K), mxfp4_operand(B, SB, K), 1.0
    if dtype == "mxfp8":
        if K is None:
            K = np.asarray(A).shape[1]
        return mxfp8_operand(A, SA, K), mxfp8_operand(B, SB, K), 1.0
    if dtype in ("mxfp6_e2m3", "mxfp6_e3m2"):
        if K is None:
            K = 4 * np.asarray(A).shape[1] // 3
        f = dtype[-4:]
        return mxfp6_operand(A, SA, K, f), mxfp6_operand(B, SB, K, f), 1.0
    if dtype == "bf16":
        return decode_bf16(A), decode_bf16(B), 1.0
    if dtype == "fp8":
        sa = 1.0 if SA is None else float(np.float32(SA))
        sb = 1.0 if SB is None else float(np.float32(SB))
        return decode_e4m3fn(A), decode_e4m3fn(B), sa * sb
    raise ValueError(f"unknown dtype {dtype!r}")


def _beta(bias, N: int) -> np.ndarray:
    if bias is None:
        return np.zeros(N, dtype=np.float64)
    beta = decode_bf16(bias).reshape(-1)
    if beta.shape[0] != N:
        raise ValueError("bias must hold N values")
    return beta


def gemm(dtype: str, A, B, SA=None, SB=None, bias=None, K: int | None = None):
    """Whole-output oracle.  Returns (C uint16[M][N] bf16 bits, D float64[M][N]).

    The K-sum is one fp64 matrix product of the decoded operands (a library
    primitive); for MXFP4 inputs every product and partial sum is exact in fp64.
    """
    a, b, sigma = operands(dtype, A, B, SA, SB, K)
    D = sigma * (a @ b.T) + _beta(bias, b.shape[0])[None, :]
    return rne_bf16_from_double(D), D


def gemm_elements(dtype: str, A, B, rows, cols, SA=None, SB=None, bias=None, K: int | None = None):
    """Oracle for sampled outputs (m, n) = (rows[i], cols[i]), one dot product each.

    Returns (C uint16[count], D float64[count], S float64[count]) where S is the
    error-bound sum |sigma| * sum_k |a(m,k) b(n,k)|.
    """
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    ur, ri = np.unique(rows, return_inverse=True)
    uc, ci = np.unique(cols, return_inverse=True)
    if dtype in ("mxfp4", "mxfp8", "mxfp6_e2m3", "mxfp6_e3m2"):
        a, b, sigma = operands(dtype, np.asarray(A)[ur], np.asarray(B)[uc], np.asarray(SA)[ur],
                               np.asarray(SB)[uc], K)
    else:
        a, b, sigma = operands(dtype, np.asarray(A)[ur], np.asarray(B)[uc], SA, SB, K)
    full_n = np.asarray(B).shape[0]
    beta = _beta(bias, full_n)[cols]
    dots = np.einsum("ik,ik->i", a[ri], b[ci])
    D = sigma * dots + beta
    S = abs(sigma) * np.einsum("ik,ik->i", np.abs(a[ri]), np.abs(b[ci]))
    return rne_bf16_from_double(D), D, S


def abs_product_sums(dtype: str, A, B, SA=None, SB=None, K: int | None = None) -> np.ndarray:
    """S[m][n] = |sigma| * sum_k |a(m,k) * b(n,k)|, the scale of the error bound."""
    a, b, sigma = operands(dtype, A, B, SA, SB, K)
    return abs(sigma) * (np.abs(a) @ np.abs(b).T)


def _ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 at |x|: 2**(floor(log2|x|) - 7), and 2**-133 below 2**-126."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    safe = np.where(x > 0, x, 1.0)
    _, ex = np.frexp(safe)
    e = np.maximum(ex.astype(np.int64) - 1, -126)
    return np.where(x >= 2.0 ** -126, np.ldexp(1.0, (e - 7).astype(np.int32)), 2.0 ** -133)


def accept(C_test: np.ndarray, C_ref: np.ndarray, D: np.ndarray, S: np.ndarray | None) -> np.ndarray:
    """Elementwise acceptance of a bf16 result against the oracle.

    An element passes when its bits equal the oracle's (+0 and -0 count as
    equal, any NaN matches NaN), or when |C_test - D| <= 2**-7 * S + ulp_bf16(max(|D|, |C_test|)).
    S=None means bit equality only.  Returns a boolean array (True = pass).
    """
    C_test = np.asarray(C_test, dtype=np.uint16)
    C_ref = np.asarray(C_ref, dtype=np.uint16)
    same = (C_test == C_ref) | (((C_test | C_ref) & 0x7FFF) == 0)
    t = decode_bf16(C_test)
    r = decode_bf16(C_ref)
    same |= np.isnan(t) & np.isnan(r)
    if S is None:
        return same
    D = np.asarray(D, dtype=np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        err = np.abs(t - D)
        bound = np.ldexp(np.asarray(S, dtype=np.float64), -7) + _ulp_bf16(np.maximum(np.abs(D), np.abs(t)))
        ok = np.isfinite(err) & (err <= bound)
    return same | ok


def bf16_backward(dC, A, B):
    """Gradients of C = A . B^T + bias for bf16 operands, given dC = dL/dC.

    dC uint16[M][N], A uint16[M][K], B uint16[N][K] (bf16 bit patterns; A or B
    may be None when its gradient partner is not wanted).  Returns a dict of
    (bits, exact value, error-bound sum) triples:

        dA[m][k] = sum_n dC[m][n] * B[n][k]     (needs B)
        dB[n][k] = sum_m dC[m][n] * A[m][k]     (needs A)
        dbias[n] = sum_m dC[m][n]

    each value in fp64 (two library matrix products and one sum) and rounded
    once to bf16; the error-bound sums are the same sums of absolute values.
    """
    g = decode_bf16(dC)
    out = {}
    if B is not None:
        b = decode_bf16(B)
        D = g @ b
        out["dA"] = (rne_bf16_from_double(D), D, np.abs(g) @ np.abs(b))
    if A is not None:
        a = decode_bf16(A)
        D = g.T @ a
        out["dB"] = (rne_bf16_from_double(D), D, np.abs(g).T @ np.abs(a))
    D = g.sum(axis=0)
    out["dbias"] = (rne_bf16_from_double(D), D, np.abs(g).sum(axis=0))
    return out


def _mx_decode(fmt: str, X, S, K: int) -> np.ndarray:
    if fmt == "mxfp4":
        return mxfp4_operand(X, S, K)
    if fmt == "mxfp8":
        return mxfp8_operand(X, S, K)
    if fmt in ("mxfp6_e2m3", "mxfp6_e3m2"):
        return mxfp6_operand(X, S, K, fmt[-4:])
    raise ValueError(f"not an MX format: {fmt!r}")


def _mx_k(a_fmt: str, A, K):
    if K is not None:
        return K
    cols = np.asarray(A).shape[1]
    if a_fmt == "mxfp4":
        return 2 * cols
    if a_fmt.startswith("mxfp6"):
        return 4 * cols // 3
    return cols


def gemm_mx(a_fmt: str, b_fmt: str, A, B, SA, SB, bias=None, K: int | None = None):
    """Block-scaled operands of any MX element format ("mxfp4", "mxfp6_e2m3", "mxfp6_e3m2" or
    "mxfp8" each):
    the same plain contraction as gemm(), each operand decoded by its own format.
    Returns (C uint16[M][N] bf16 bits, D float64[M][N])."""
    K = _mx_k(a_fmt, A, K)
    a = _mx_decode(a_fmt, A, SA, K)
    b = _mx_decode(b_fmt, B, SB, K)
    D = a @ b.T + _beta(bias, b.shape[0])[None, :]
    return rne_bf16_from_double(D), D


def abs_product_sums_mx(a_fmt: str, b_fmt: str, A, B, SA, SB, K: int | None = None) -> np.ndarray:
    """S[m][n] = sum_k |a(m,k) * b(n,k)| for operands of formats a_fmt / b_fmt (sigma = 1)."""
    K = _mx_k(a_fmt, A, K)
    return np.abs(_mx_decode(a_fmt, A, SA, K)) @ np.abs(_mx_decode(b_fmt, B, SB, K)).T
