"""Pins for the CPU oracle: each checks it against something other than itself.

* decoders against torch's own CPU format conversions (E4M3FN, E8M0, bf16);
* E2M1 against its OCP bit-field definition;
* bf16 rounding against torch's fp32->bf16 conversion, and against hand-built
  doubles where rounding through fp32 first would give the wrong answer;
* whole GEMMs against an exact-rational brute force (tests/bruteforce.py),
  hand-worked sums (MXFP4 and MXFP8, tests/golden/), identity operands, the bias-broadcast property, integer
  matrix products and algebraic invariants.

``test_planted_mistakes_are_caught`` plants plausible mistakes in the oracle
(on the CPU) and checks that at least one pin fails for each.
"""

from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import bruteforce as bf
import oracle
from persistent_gemm_amd.inputs import backward_inputs, integer_inputs, make_inputs, mixed_inputs, pack_fp6

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _pack(codes: np.ndarray) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def _f32_to_bf16_torch(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


# ---------------------------------------------------------------- decoders

def pin_e4m3fn_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().double().numpy()
    got = oracle.decode_e4m3fn(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(got[ok]))


def pin_e8m0_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).float().double().numpy()
    got = oracle.decode_e8m0(codes)
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(ref[:255], got[:255])


def pin_bf16_decode_vs_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = oracle.decode_bf16(bits)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])


def pin_e2m1_bitfields():
    for code in range(16):
        assert float(bf.e2m1(code)) == oracle.decode_e2m1(np.array([code]))[0]
        assert np.signbit(oracle.decode_e2m1(np.array([code]))[0]) == bool(code & 8)


# ---------------------------------------------------------------- rounding

def pin_rne_vs_torch_on_floats():
    rng = np.random.default_rng(7)
    raw = rng.integers(0, 2**32, size=400_000, dtype=np.uint64).astype(np.uint32)
    ties = (raw & 0xFFFF0000) | 0x8000            # exactly on a bf16 midpoint
    near = (raw & 0xFFFF0000) | rng.choice(np.array([0x7FFF, 0x8001, 0x0001, 0xFFFF], np.uint32), raw.size)
    for pat in (raw, ties, near):
        f = pat.view(np.float32)
        f = f[np.isfinite(f)]
        assert np.array_equal(oracle.rne_bf16_from_double(f.astype(np.float64)), _f32_to_bf16_torch(f))


def pin_rne_from_double_not_via_float():
    # mid1 = 1 + 2**-8 lies halfway between bf16 1.0 (0x3F80) and 1 + 2**-7 (0x3F81).
    mid1 = 1.0 + 2.0 ** -8
    # mid2 = 1 + 3 * 2**-8 lies halfway between 0x3F81 and 0x3F82.
    mid2 = 1.0 + 3 * 2.0 ** -8
    cases = {
        mid1: 0x3F80,                    # tie -> even
        mid1 + 2.0 ** -40: 0x3F81,       # float32(x) == mid1 would tie to 0x3F80: wrong
        mid1 - 2.0 ** -40: 0x3F80,
        mid2: 0x3F82,                    # tie -> even mantissa (2)
        mid2 - 2.0 ** -40: 0x3F81,       # float32(x) == mid2 would give 0x3F82: wrong
        -(mid1 + 2.0 ** -40): 0xBF81,
        257.0: 0x4380, 259.0: 0x4382, 258.0: 0x4381,
    }
    pairs = list(cases.items()) + [(0.0, 0x0000), (-0.0, 0x8000)]   # +-0 collide as dict keys
    x = np.array([p[0] for p in pairs], dtype=np.float64)
    want = np.array([p[1] for p in pairs], dtype=np.uint16)
    assert np.array_equal(oracle.rne_bf16_from_double(x), want)


def pin_rne_overflow_subnormal_nan():
    max_bf16 = (2.0 - 2.0 ** -7) * 2.0 ** 127          # 0x7F7F
    half_ulp = 2.0 ** (127 - 8)
    cases = {
        max_bf16: 0x7F7F,
        max_bf16 + half_ulp * 0.999: 0x7F7F,
        max_bf16 + half_ulp: 0x7F80,                       # tie, odd mantissa -> rounds up -> inf
        2.0 ** 128: 0x7F80, -(2.0 ** 129): 0xFF80, float("inf"): 0x7F80,
        2.0 ** -133: 0x0001,                               # smallest subnormal
        1.5 * 2.0 ** -133: 0x0002,                         # tie -> even
        2.0 ** -134: 0x0000,                               # tie between 0 and 2**-133 -> even (0)
        2.0 ** -134 + 2.0 ** -160: 0x0001,
        -(2.0 ** -134 + 2.0 ** -160): 0x8001,
        2.0 ** -126: 0x0080,                               # smallest normal
        2.0 ** -126 - 2.0 ** -134: 0x0080,                 # tie between 0x7F and 0x80 -> even (0x80)
        1e-300: 0x0000,
    }
    x = np.array(list(cases.keys()), dtype=np.float64)
    want = np.array(list(cases.values()), dtype=np.uint16)
    assert np.array_equal(oracle.rne_bf16_from_double(x), want)
    assert oracle.rne_bf16_from_double(np.array([np.nan]))[0] == 0x7FC0


def pin_rne_vs_rational():
    rng = np.random.default_rng(11)
    x = rng.standard_normal(3000) * np.ldexp(1.0, rng.integers(-140, 120, 3000))
    got = oracle.rne_bf16_from_double(x)
    from fractions import Fraction
    want = np.array([bf.round_bf16(Fraction(float(v))) for v in x], dtype=np.uint16)
    assert np.array_equal(got, want)


# ---------------------------------------------------------------- whole GEMMs

def _bruteforce_case(dtype, M, N, K, bias, seed):
    if dtype == "fp8":
        x = make_inputs(dtype, M, N, K, bias=bias, seed=seed, fp8_scales=(0.5, 3.0))
    else:
        x = make_inputs(dtype, M, N, K, bias=bias, seed=seed)
    C, _ = oracle.gemm(dtype, x["A"], x["B"], x["SA"], x["SB"], x["bias"], K=K)
    want = np.array(bf.gemm(dtype, x["A"], x["B"], x["SA"], x["SB"], x["bias"], M, N, K), dtype=np.uint16)
    assert np.array_equal(C, want), (dtype, M, N, K, bias, seed)
    rows = np.repeat(np.arange(M), N)
    cols = np.tile(np.arange(N), M)
    Ce, _, _ = oracle.gemm_elements(dtype, x["A"], x["B"], rows, cols, x["SA"], x["SB"], x["bias"], K=K)
    assert np.array_equal(Ce.reshape(M, N), want)


def pin_bruteforce_mxfp4():
    for seed, (M, N, K) in enumerate([(1, 1, 32), (2, 3, 64), (3, 2, 96), (4, 4, 64)]):
        for bias in (False, True):
            _bruteforce_case("mxfp4", M, N, K, bias, 100 + seed)


def pin_bruteforce_bf16():
    for seed, (M, N, K) in enumerate([(1, 1, 8), (2, 3, 16), (3, 4, 40)]):
        for bias in (False, True):
            _bruteforce_case("bf16", M, N, K, bias, 200 + seed)


def pin_bruteforce_fp8():
    for seed, (M, N, K) in enumerate([(1, 2, 16), (3, 3, 32), (4, 2, 48)]):
        for bias in (False, True):
            _bruteforce_case("fp8", M, N, K, bias, 300 + seed)


def pin_bruteforce_mxfp8():
    for seed, (M, N, K) in enumerate([(1, 1, 32), (2, 3, 64), (3, 2, 96)]):
        for bias in (False, True):
            _bruteforce_case("mxfp8", M, N, K, bias, 400 + seed)


def _one_by_one(a_codes, b_codes, sa=127, sb=127, bias=None):
    """MXFP4 with M = N = 1, K = 32 from explicit codes."""
    A = _pack(np.array([a_codes], dtype=np.uint8))
    B = _pack(np.array([b_codes], dtype=np.uint8))
    SA = np.array([[sa]], dtype=np.uint8)
    SB = np.array([[sb]], dtype=np.uint8)
    bb = None if bias is None else _f32_to_bf16_torch(np.array([bias], np.float32))
    C, D = oracle.gemm("mxfp4", A, B, SA, SB, bb, K=32)
    return int(C[0, 0]), float(D[0, 0])


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _runs(spec):
    """'2*3,10*1' -> [2, 2, 2, 10] (E2M1 codes for k = 0, 1, ...)."""
    out = []
    for part in spec.split(","):
        code, count = part.split("*")
        out += [int(code)] * int(count)
    return out


def golden_handworked():
    """Cases of tests/golden/mxfp4_1x1x32_handworked.txt (worked by hand from the formats)."""
    cases = []
    with open(os.path.join(GOLDEN, "mxfp4_1x1x32_handworked.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, a, b, sa, sb, bias, total, bits = line.split()
            cases.append((name, _runs(a), _runs(b), int(sa), int(sb), None if bias == "none" else float(bias),
                          float(total), int(bits, 16)))
    return cases


def pin_handworked_mxfp4():
    cases = golden_handworked()
    assert len(cases) == 8
    for name, a, b, sa, sb, bias, total, bits in cases:
        assert len(a) == 32 and len(b) == 32, name
        got = _one_by_one(a, b, sa=sa, sb=sb, bias=bias)
        assert got == (bits, total), f"{name}: oracle gives {got}, worked by hand {(bits, total)}"
    # the scale of k in [32, 64) is the second scale byte (K = 64, outside the 1x1x32 file)
    one = 0x2
    A = _pack(np.array([[0] * 32 + [one] * 32], np.uint8))
    B = _pack(np.array([[0] * 32 + [one] * 32], np.uint8))
    C, D = oracle.gemm("mxfp4", A, B, np.array([[120, 128]], np.uint8), np.array([[127, 127]], np.uint8), None, K=64)
    assert D[0, 0] == 64.0 and C[0, 0] == 0x4280


def _hex_runs(spec):
    """'58*1,38*2' -> [0x58, 0x38, 0x38] (E4M3FN bytes for k = 0, 1, ...)."""
    out = []
    for part in spec.split(","):
        byte, count = part.split("*")
        out += [int(byte, 16)] * int(count)
    return out


def golden_handworked_mxfp8():
    """Cases of tests/golden/mxfp8_1x1x64_handworked.txt (worked by hand from the formats)."""
    cases = []
    with open(os.path.join(GOLDEN, "mxfp8_1x1x64_handworked.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, a, b, sa, sb, bias, total, bits = line.split()
            cases.append((name, _hex_runs(a), _hex_runs(b), [int(v) for v in sa.split(",")],
                          [int(v) for v in sb.split(",")], None if bias == "none" else float(bias),
                          float(total), int(bits, 16)))
    return cases


def pin_handworked_mxfp8():
    cases = golden_handworked_mxfp8()
    assert len(cases) == 8
    for name, a, b, sa, sb, bias, total, bits in cases:
        assert len(a) == 64 and len(b) == 64, name
        bb = None if bias is None else _f32_to_bf16_torch(np.array([bias], np.float32))
        C, D = oracle.gemm("mxfp8", np.array([a], np.uint8), np.array([b], np.uint8), np.array([sa], np.uint8),
                           np.array([sb], np.uint8), bb, K=64)
        got = (int(C[0, 0]), float(D[0, 0]))
        assert got == (bits, total), f"{name}: oracle gives {got}, worked by hand {(bits, total)}"


def pin_identity():
    # MXFP4: A = I (code 1.0, scale 2**0) -> C[m][n] = b(n, m) exactly.
    K = 64
    x = make_inputs("mxfp4", 8, 24, K, bias=False, seed=5)
    codes = np.zeros((K, K), np.uint8)
    np.fill_diagonal(codes, 0x2)
    A = _pack(codes)
    SA = np.full((K, K // 32), 127, np.uint8)
    C, _ = oracle.gemm("mxfp4", A, x["B"], SA, x["SB"], None, K=K)
    bvals = np.array([[float(bf.e2m1((int(x["B"][n][k // 2]) >> (4 * (k & 1))) & 0xF) * bf.e8m0(int(x["SB"][n][k // 32])))
                       for k in range(K)] for n in range(24)], dtype=np.float32)
    assert np.array_equal(C, _f32_to_bf16_torch(bvals.T))
    # bf16: A = I -> C = B^T, bit for bit.
    y = make_inputs("bf16", 4, 20, 32, bias=False, seed=6)
    A = np.zeros((32, 32), np.uint16)
    np.fill_diagonal(A, 0x3F80)
    C, _ = oracle.gemm("bf16", A, y["B"], None, None, None)
    assert np.array_equal(C, y["B"].T)
    # fp8: A = I (0x38 = 1.0) -> C = bf16(e4m3 value of B)^T.
    z = make_inputs("fp8", 4, 20, 32, bias=False, seed=7)
    A = np.zeros((32, 32), np.uint8)
    np.fill_diagonal(A, 0x38)
    C, _ = oracle.gemm("fp8", A, z["B"], 1.0, 1.0, None)
    bv = torch.from_numpy(z["B"]).view(torch.float8_e4m3fn).float().numpy()
    assert np.array_equal(C, _f32_to_bf16_torch(bv.T))


def pin_bias_broadcast():
    for dtype in ("mxfp4", "bf16", "fp8"):
        x = make_inputs(dtype, 6, 40, 64, bias=True, seed=8)
        A0 = np.zeros_like(x["A"])
        C, _ = oracle.gemm(dtype, A0, x["B"], x["SA"], x["SB"], x["bias"], K=64)
        assert np.array_equal(C, np.broadcast_to(x["bias"], C.shape))
    for dtype in ("bf16", "fp8"):
        y = integer_inputs(dtype, 5, 12, 16, bias=True, seed=9, lo=-3, hi=3)
        Cb, Db = oracle.gemm(dtype, y["A"], y["B"], y["SA"], y["SB"], y["bias"])
        Cn, Dn = oracle.gemm(dtype, y["A"], y["B"], y["SA"], y["SB"], None)
        diff = oracle.decode_bf16(Cb) - oracle.decode_bf16(Cn)
        bias = oracle.decode_bf16(y["bias"])
        assert np.array_equal(diff, np.broadcast_to(bias, diff.shape))
        assert np.array_equal(Db - Dn, np.broadcast_to(bias, Db.shape))


def _mx_int(packed, scales, K):
    """MXFP4 values times 2**3, as exact integers (scales restricted to >= 125)."""
    out = np.zeros((packed.shape[0], K), np.int64)
    for r in range(packed.shape[0]):
        for k in range(K):
            code = (int(packed[r][k // 2]) >> (4 * (k & 1))) & 0xF
            v = bf.e2m1(code) * bf.e8m0(int(scales[r][k // 32])) * 8
            assert v.denominator == 1
            out[r, k] = int(v)
    return out


def pin_integer_matmul():
    # MXFP4: 8 * a and 8 * b are integers, so 64 * D is an int64 matrix product.
    x = make_inputs("mxfp4", 9, 7, 160, bias=False, seed=10)
    _, D = oracle.gemm("mxfp4", x["A"], x["B"], x["SA"], x["SB"], None, K=160)
    ref = _mx_int(x["A"], x["SA"], 160) @ _mx_int(x["B"], x["SB"], 160).T
    assert np.array_equal(D * 64, ref.astype(np.float64))
    # bf16 / fp8 small integers: D equals the int64 product plus the bias; C is torch's rounding of it.
    for dtype in ("bf16", "fp8"):
        y = integer_inputs(dtype, 11, 13, 64, bias=True, seed=12)
        C, D = oracle.gemm(dtype, y["A"], y["B"], y["SA"], y["SB"], y["bias"])
        if dtype == "bf16":
            ai = torch.from_numpy(y["A"].view(np.int16)).view(torch.bfloat16).long().numpy()
            bi = torch.from_numpy(y["B"].view(np.int16)).view(torch.bfloat16).long().numpy()
        else:
            ai = torch.from_numpy(y["A"]).view(torch.float8_e4m3fn).float().long().numpy()
            bi = torch.from_numpy(y["B"]).view(torch.float8_e4m3fn).float().long().numpy()
        bias = torch.from_numpy(y["bias"].view(np.int16)).view(torch.bfloat16).long().numpy()
        ref = ai @ bi.T + bias[None, :]
        assert np.array_equal(D, ref.astype(np.float64))
        assert np.array_equal(C, _f32_to_bf16_torch(ref.astype(np.float32)))


def pin_invariants_mxfp4():
    K = 128
    x = make_inputs("mxfp4", 6, 5, K, bias=False, seed=13)
    C, D = oracle.gemm("mxfp4", x["A"], x["B"], x["SA"], x["SB"], None, K=K)
    # one more in every A scale byte doubles the result exactly
    C2, D2 = oracle.gemm("mxfp4", x["A"], x["B"], x["SA"] + 1, x["SB"], None, K=K)
    assert np.array_equal(D2, 2 * D)
    # permuting whole 32-wide K blocks (data and scales together) changes nothing
    perm = np.array([2, 0, 3, 1])
    Ab = x["A"].reshape(6, 4, 16)[:, perm].reshape(6, 64)
    Bb = x["B"].reshape(5, 4, 16)[:, perm].reshape(5, 64)
    C3, D3 = oracle.gemm("mxfp4", Ab, Bb, x["SA"][:, perm], x["SB"][:, perm], None, K=K)
    assert np.array_equal(D3, D) and np.array_equal(C3, C)
    # swapping the operands transposes the result
    C4, _ = oracle.gemm("mxfp4", x["B"], x["A"], x["SB"], x["SA"], None, K=K)
    assert np.array_equal(C4, C.T)
    # permuting rows of A permutes rows of C
    rp = np.array([3, 1, 5, 0, 2, 4])
    C5, _ = oracle.gemm("mxfp4", x["A"][rp], x["B"], x["SA"][rp], x["SB"], None, K=K)
    assert np.array_equal(C5, C[rp])
    # shifting only the first K block's scale changes the value by exactly that block's part
    SA6 = x["SA"].copy()
    SA6[:, 0] += 1
    _, D6 = oracle.gemm("mxfp4", x["A"], x["B"], SA6, x["SB"], None, K=K)
    Afirst = x["A"].copy()
    Afirst[:, 16:] = 0
    _, Dfirst = oracle.gemm("mxfp4", Afirst, x["B"], x["SA"], x["SB"], None, K=K)
    assert np.array_equal(D6 - D, Dfirst)


def pin_invariants_mxfp8():
    K = 128
    x = make_inputs("mxfp8", 5, 7, K, bias=True, seed=15)
    C, D = oracle.gemm("mxfp8", x["A"], x["B"], x["SA"], x["SB"], None, K=K)
    # one more in every B scale byte doubles the result exactly
    _, D2 = oracle.gemm("mxfp8", x["A"], x["B"], x["SA"], x["SB"] + 1, None, K=K)
    assert np.array_equal(D2, 2 * D)
    # unit block scales reduce MXFP8 to fp8 with per-tensor scales of 1
    ones_a = np.full_like(x["SA"], 127)
    ones_b = np.full_like(x["SB"], 127)
    C3, D3 = oracle.gemm("mxfp8", x["A"], x["B"], ones_a, ones_b, x["bias"], K=K)
    C4, D4 = oracle.gemm("fp8", x["A"], x["B"], 1.0, 1.0, x["bias"], K=K)
    assert np.array_equal(C3, C4) and np.array_equal(D3, D4)
    # a block's scale multiplies exactly that block's 32 K elements
    SB5 = x["SB"].copy()
    SB5[:, 2] += 2
    _, D5 = oracle.gemm("mxfp8", x["A"], x["B"], x["SA"], SB5, None, K=K)
    Bblk = x["B"].copy()
    Bblk[:, :64] = 0
    Bblk[:, 96:] = 0
    _, Dblk = oracle.gemm("mxfp8", x["A"], Bblk, x["SA"], x["SB"], None, K=K)
    assert np.array_equal(D5 - D, 3 * Dblk)
    # swapping the operands transposes the result
    C6, _ = oracle.gemm("mxfp8", x["B"], x["A"], x["SB"], x["SA"], None, K=K)
    assert np.array_equal(C6, C.T)


def pin_bruteforce_bf16_backward():
    for seed, (M, N, K) in enumerate([(1, 1, 1), (2, 3, 4), (3, 3, 3), (4, 2, 5)]):
        x = backward_inputs(M, N, K, seed=500 + seed)
        o = oracle.bf16_backward(x["dC"], x["A"], x["B"])
        dA, dB, db = bf.bf16_backward(x["dC"], x["A"], x["B"], M, N, K)
        assert np.array_equal(o["dA"][0], np.array(dA, np.uint16)), (M, N, K)
        assert np.array_equal(o["dB"][0], np.array(dB, np.uint16)), (M, N, K)
        assert np.array_equal(o["dbias"][0], np.array(db, np.uint16)), (M, N, K)


def pin_bf16_backward_vs_autograd():
    """torch's own autograd of addmm (fp64, on the CPU) gives the same gradients:
    bit for bit on integer inputs, to fp64 rounding on random ones."""
    for integer, (M, N, K) in [(True, (6, 5, 7)), (True, (8, 8, 8)), (False, (9, 4, 6))]:
        x = backward_inputs(M, N, K, seed=600 + M, integer=integer)
        a = torch.from_numpy(oracle.decode_bf16(x["A"])).requires_grad_()
        b = torch.from_numpy(oracle.decode_bf16(x["B"])).requires_grad_()
        bias = torch.zeros(N, dtype=torch.float64, requires_grad=True)
        g = torch.from_numpy(oracle.decode_bf16(x["dC"]))
        torch.addmm(bias, a, b.t()).backward(g)
        o = oracle.bf16_backward(x["dC"], x["A"], x["B"])
        for name, ref in (("dA", a.grad), ("dB", b.grad), ("dbias", bias.grad)):
            got = o[name][1]
            if integer:
                assert np.array_equal(got, ref.numpy()), name
            else:
                assert np.allclose(got, ref.numpy(), rtol=1e-12, atol=1e-12), name


def pin_bf16_backward_identities():
    x = backward_inputs(8, 8, 8, seed=700, integer=True)
    o = oracle.bf16_backward(x["dC"], x["A"], x["B"])
    g, a, b = (oracle.decode_bf16(x[k]) for k in ("dC", "A", "B"))
    # adjoint identity: <dC, A B^T> = <dA, A> = <dB, B> (exact on integers)
    lhs = float((g * (a @ b.T)).sum())
    assert lhs == float((o["dA"][1] * a).sum()) == float((o["dB"][1] * b).sum())
    # B = I gives dA = dC; A = I gives dB = dC^T; dbias is the column sum
    eye = np.eye(8, dtype=np.float32).view(np.uint32) >> 16
    eye = eye.astype(np.uint16)
    assert np.array_equal(oracle.bf16_backward(x["dC"], None, eye)["dA"][0], x["dC"])
    assert np.array_equal(oracle.bf16_backward(x["dC"], eye, None)["dB"][0], x["dC"].T)
    ones = np.full((8, 1), 0x3F80, np.uint16)                       # bf16 1.0
    assert np.array_equal(oracle.bf16_backward(x["dC"], ones, None)["dB"][0][:, 0], o["dbias"][0])


def pin_bruteforce_mixed_mx():
    for a_fmt, b_fmt in (("mxfp4", "mxfp8"), ("mxfp8", "mxfp4")):
        for seed, (M, N, K) in enumerate([(1, 1, 32), (2, 3, 64), (3, 2, 32)]):
            for bias in (False, True):
                x = mixed_inputs(a_fmt, b_fmt, M, N, K, bias=bias, seed=800 + seed)
                C, _ = oracle.gemm_mx(a_fmt, b_fmt, x["A"], x["B"], x["SA"], x["SB"], x["bias"], K=K)
                want = bf.gemm_mx(a_fmt, b_fmt, x["A"], x["B"], x["SA"], x["SB"], x["bias"], M, N, K)
                assert np.array_equal(C, np.array(want, np.uint16)), (a_fmt, b_fmt, M, N, K, bias)


def pin_mixed_mx_reduces_to_mxfp4():
    """B given as torch's own E4M3 encodings of E2M1 values: the mixed product equals
    the MXFP4 product of the same codes, and equal formats reduce to gemm()."""
    M, N, K = 5, 6, 96
    x = make_inputs("mxfp4", M, N, K, bias=True, seed=16)
    C4, D4 = oracle.gemm("mxfp4", x["A"], x["B"], x["SA"], x["SB"], x["bias"], K=K)
    bvals = oracle.decode_e2m1(oracle.unpack_fp4(x["B"], K))
    B8 = torch.from_numpy(bvals).float().to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    Cm, Dm = oracle.gemm_mx("mxfp4", "mxfp8", x["A"], B8, x["SA"], x["SB"], x["bias"], K=K)
    assert np.array_equal(Cm, C4) and np.array_equal(Dm, D4)
    avals = oracle.decode_e2m1(oracle.unpack_fp4(x["A"], K))
    A8 = torch.from_numpy(avals).float().to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    Cr, _ = oracle.gemm_mx("mxfp8", "mxfp4", A8, x["B"], x["SA"], x["SB"], x["bias"], K=K)
    assert np.array_equal(Cr, C4)
    Ce, _ = oracle.gemm_mx("mxfp4", "mxfp4", x["A"], x["B"], x["SA"], x["SB"], x["bias"], K=K)
    assert np.array_equal(Ce, C4)


def pin_accept():
    x = make_inputs("bf16", 16, 24, 256, bias=True, seed=14)
    C, D = oracle.gemm("bf16", x["A"], x["B"], None, None, x["bias"])
    S = oracle.abs_product_sums("bf16", x["A"], x["B"])
    assert oracle.accept(C, C, D, S).all()
    assert oracle.accept(C, C, D, None).all()
    # one bf16 ulp away: inside the bound, not bit-equal
    C1 = C.copy()
    C1[0, 0] ^= 1
    assert oracle.accept(C1, C, D, S).all()
    assert not oracle.accept(C1, C, D, None)[0, 0]
    # far away: rejected
    Cbad = C.copy()
    Cbad[3, 4] = oracle.rne_bf16_from_double(np.array([D[3, 4] + 2 * S[3, 4] + 1.0]))[0]
    assert not oracle.accept(Cbad, C, D, S)[3, 4]
    # +0 and -0 count as equal
    z = np.array([0x0000], np.uint16)
    assert oracle.accept(np.array([0x8000], np.uint16), z, np.zeros(1), None).all()


# ---------------------------------------------------------------- MXFP6

def pin_fp6_bitfields():
    """E2M3 and E3M2 on all 64 codes against the field-by-field definition (and the sign of zero)."""
    codes = np.arange(64, dtype=np.uint8)
    for dec, eb in ((oracle.decode_e2m3, 2), (oracle.decode_e3m2, 3)):
        got = dec(codes)
        want = np.array([float(bf.fp6(c, eb)) for c in range(64)])
        assert np.array_equal(got, want)
        assert np.array_equal(np.signbit(got), codes >= 32)
    # the format's extremes: largest finite and smallest subnormal
    assert oracle.decode_e2m3(np.array([0x1F, 0x01]))[0] == 7.5 and oracle.decode_e2m3(np.array([0x01]))[0] == 0.125
    assert oracle.decode_e3m2(np.array([0x1F]))[0] == 28.0 and oracle.decode_e3m2(np.array([0x01]))[0] == 0.0625


def pin_fp6_bit_order():
    """Four codes in three bytes, the lowest bits first: worked by hand, then bit by bit."""
    # bytes c1 20 08 -> word 0x0820C1 -> codes 0x01, 0x03, 0x02, 0x02
    assert np.array_equal(oracle.unpack_fp6(np.array([[0xC1, 0x20, 0x08]], np.uint8), 4), [[1, 3, 2, 2]])
    rng = np.random.default_rng(23)
    codes = rng.integers(0, 64, (3, 96)).astype(np.uint8)
    packed = pack_fp6(codes)
    got = oracle.unpack_fp6(packed, 96)
    assert np.array_equal(got, [[bf.fp6_code(packed[r], k) for k in range(96)] for r in range(3)])
    assert np.array_equal(got, codes)


def golden_handworked_mxfp6():
    cases = []
    with open(os.path.join(GOLDEN, "mxfp6_1x1x64_handworked.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, fmt, a, b, sa, sb, bias, total, bits = line.split()
            cases.append((name, fmt, _hex_runs(a), _hex_runs(b), [int(v) for v in sa.split(",")],
                          [int(v) for v in sb.split(",")], None if bias == "none" else float(bias),
                          float(total), int(bits, 16)))
    return cases


def pin_handworked_mxfp6():
    cases = golden_handworked_mxfp6()
    assert len(cases) == 11
    for name, fmt, a, b, sa, sb, bias, total, bits in cases:
        assert len(a) == 64 and len(b) == 64, name
        bb = None if bias is None else _f32_to_bf16_torch(np.array([bias], np.float32))
        C, D = oracle.gemm("mxfp6_" + fmt, pack_fp6(np.array([a], np.uint8)), pack_fp6(np.array([b], np.uint8)),
                           np.array([sa], np.uint8), np.array([sb], np.uint8), bb, K=64)
        got = (int(C[0, 0]), float(D[0, 0]))
        assert got == (bits, total), f"{name}: oracle gives {got}, worked by hand {(bits, total)}"


def pin_bruteforce_mxfp6():
    for dtype in ("mxfp6_e2m3", "mxfp6_e3m2"):
        for seed, (M, N, K) in enumerate([(1, 1, 32), (2, 3, 64), (3, 2, 96)]):
            for bias in (False, True):
                _bruteforce_case(dtype, M, N, K, bias, 950 + seed)


def pin_mxfp6_reduces_to_mxfp8():
    """Every E2M3 and E3M2 value is an E4M3FN value: with B's elements re-encoded as torch's own
    E4M3FN bytes of the same values, the MXFP6 result equals the MXFP8 oracle's, bit for bit."""
    for dtype, dec in (("mxfp6_e2m3", oracle.decode_e2m3), ("mxfp6_e3m2", oracle.decode_e3m2)):
        M, N, K = 4, 5, 96
        x = make_inputs(dtype, M, N, K, bias=True, seed=960)
        C6, D6 = oracle.gemm(dtype, x["A"], x["B"], x["SA"], x["SB"], x["bias"], K=K)
        e4 = lambda X: torch.from_numpy(dec(oracle.unpack_fp6(X, K))).float().to(torch.float8_e4m3fn).view(
            torch.uint8).numpy()
        C8, D8 = oracle.gemm("mxfp8", e4(x["A"]), e4(x["B"]), x["SA"], x["SB"], x["bias"], K=K)
        assert np.array_equal(C6, C8) and np.array_equal(D6, D8), dtype
        Cm, _ = oracle.gemm_mx(dtype, "mxfp8", x["A"], e4(x["B"]), x["SA"], x["SB"], x["bias"], K=K)
        assert np.array_equal(Cm, C6), dtype


def pin_invariants_mxfp6():
    for dtype in ("mxfp6_e2m3", "mxfp6_e3m2"):
        K = 128
        x = make_inputs(dtype, 5, 6, K, bias=False, seed=970)
        C, D = oracle.gemm(dtype, x["A"], x["B"], x["SA"], x["SB"], None, K=K)
        _, D2 = oracle.gemm(dtype, x["A"], x["B"], x["SA"] + 1, x["SB"], None, K=K)
        assert np.array_equal(D2, 2 * D)
        # permuting whole 32-wide blocks (24 bytes each) with their scales changes nothing
        perm = np.array([3, 1, 0, 2])
        Ab = x["A"].reshape(5, 4, 24)[:, perm].reshape(5, 96)
        Bb = x["B"].reshape(6, 4, 24)[:, perm].reshape(6, 96)
        _, D3 = oracle.gemm(dtype, Ab, Bb, x["SA"][:, perm], x["SB"][:, perm], None, K=K)
        assert np.array_equal(D3, D)
        C4, _ = oracle.gemm(dtype, x["B"], x["A"], x["SB"], x["SA"], None, K=K)
        assert np.array_equal(C4, C.T)


# ---------------------------------------------------------------- the tolerance arithmetic
#
# The parity bar for inexact results is |C - D| <= 2**-7 * S + ulp_bf16(max(|D|, |C|)) with
# S = |sigma| * sum_k |a b|.  Every bounded GPU result rests on S, the ulp and accept(); each is
# pinned here to an exact-rational computation written from the definitions (tests/bruteforce.py).

def _exact_float(x) -> float:
    """A Fraction that must be exactly representable in fp64, as that float."""
    f = float(x)
    assert bf.Fraction(f) == x, f"{x} is not exact in fp64"
    return f


def pin_abs_sums_vs_rational():
    """abs_product_sums and the S and D of gemm_elements equal the exact sums (every product
    and partial sum of these tiny cases is exact in fp64, so any summation order gives them)."""
    cases = [("mxfp4", 3, 4, 96), ("bf16", 4, 3, 40), ("fp8", 3, 5, 48), ("mxfp8", 2, 4, 64)]
    for i, (dtype, M, N, K) in enumerate(cases):
        kw = {"fp8_scales": (0.5, 3.0)} if dtype == "fp8" else {}     # sigma = 1.5
        x = make_inputs(dtype, M, N, K, bias=True, seed=900 + i, **kw)
        S, D = bf.abs_sums(dtype, x["A"], x["B"], x["SA"], x["SB"], M, N, K)
        Sx = np.array([[_exact_float(v) for v in row] for row in S])
        Dx = np.array([[_exact_float(v) for v in row] for row in D])
        got = oracle.abs_product_sums(dtype, x["A"], x["B"], x["SA"], x["SB"], K=K)
        assert np.array_equal(got, Sx), dtype
        rows = np.repeat(np.arange(M), N)
        cols = np.tile(np.arange(N), M)
        _, De, Se = oracle.gemm_elements(dtype, x["A"], x["B"], rows, cols, x["SA"], x["SB"], None, K=K)
        assert np.array_equal(Se.reshape(M, N), Sx), dtype
        assert np.array_equal(De.reshape(M, N), Dx), dtype
        # with the bias, D moves by exactly bias[n] and S does not move
        _, Db, Sb = oracle.gemm_elements(dtype, x["A"], x["B"], rows, cols, x["SA"], x["SB"], x["bias"], K=K)
        assert np.array_equal(Sb.reshape(M, N), Sx), dtype
        assert np.array_equal(Db.reshape(M, N) - Dx, np.broadcast_to(oracle.decode_bf16(x["bias"]), (M, N)))


def pin_mixed_abs_sums_vs_rational():
    for a_fmt, b_fmt in (("mxfp4", "mxfp8"), ("mxfp8", "mxfp4")):
        M, N, K = 3, 2, 64
        x = mixed_inputs(a_fmt, b_fmt, M, N, K, bias=False, seed=910)
        want = bf.mixed_abs_sums(a_fmt, b_fmt, x["A"], x["B"], x["SA"], x["SB"], M, N, K)
        got = oracle.abs_product_sums_mx(a_fmt, b_fmt, x["A"], x["B"], x["SA"], x["SB"], K=K)
        assert np.array_equal(got, np.array([[_exact_float(v) for v in r] for r in want])), (a_fmt, b_fmt)


def pin_backward_abs_sums_vs_rational():
    for seed, (M, N, K) in enumerate([(2, 3, 4), (4, 2, 5)]):
        x = backward_inputs(M, N, K, seed=920 + seed)
        o = oracle.bf16_backward(x["dC"], x["A"], x["B"])
        sA, sB, sb = bf.backward_abs_sums(x["dC"], x["A"], x["B"], M, N, K)
        assert np.array_equal(o["dA"][2], np.array([[_exact_float(v) for v in r] for r in sA]))
        assert np.array_equal(o["dB"][2], np.array([[_exact_float(v) for v in r] for r in sB]))
        assert np.array_equal(o["dbias"][2], np.array([_exact_float(v) for v in sb]))


def pin_ulp_bf16():
    """The bf16 spacing: hand-picked values, the gap to the next bf16 read off the bit
    patterns of every positive finite bf16 (below the largest), and the exact-rational
    definition on random doubles (including values between bf16 grid points)."""
    hand = {1.0: 2.0 ** -7, 1.99: 2.0 ** -7, 2.0: 2.0 ** -6, -1.5: 2.0 ** -7, 3 * 2.0 ** 100: 2.0 ** 94,
            2.0 ** -126: 2.0 ** -133, 2.0 ** -130: 2.0 ** -133, 0.0: 2.0 ** -133, 255.9: 1.0, 256.0: 2.0}
    x = np.array(list(hand.keys()))
    assert np.array_equal(oracle._ulp_bf16(x), np.array(list(hand.values())))
    bits = np.arange(1, 0x7F7F, dtype=np.uint16)              # +denormals .. below the largest finite
    v = oracle.decode_bf16(bits)
    gap = oracle.decode_bf16(bits + np.uint16(1)) - v
    assert np.array_equal(oracle._ulp_bf16(v), gap)
    rng = np.random.default_rng(17)
    r = rng.standard_normal(2000) * np.ldexp(1.0, rng.integers(-140, 120, 2000))
    want = np.array([float(bf.ulp_bf16(bf.Fraction(float(t)))) for t in r])
    assert np.array_equal(oracle._ulp_bf16(r), want)


def pin_accept_exact():
    """accept() against the exact-rational bar on results placed at, just inside and just
    outside the bound (values chosen so every fp64 step of accept() is exact)."""
    # by hand: D = 100, S = 128 -> 2**-7 S = 1; the bf16 spacing at 100 is 0.5, so the bound is 1.5
    D = np.array([100.0] * 6)
    S = np.array([128.0] * 6)
    c = np.array([101.5, 102.0, 98.5, 98.0, 100.5, 100.0])
    want = np.array([True, False, True, False, True, True])
    cb = oracle.rne_bf16_from_double(c)
    ref = oracle.rne_bf16_from_double(D)
    assert np.array_equal(oracle.accept(cb, ref, D, S), want)
    # random: D with 20-bit mantissas, S with 12, results at the bf16 points around D +- the bound
    rng = np.random.default_rng(19)
    cases = []
    for _ in range(400):
        d = float(rng.integers(-2**20, 2**20)) * 2.0 ** int(rng.integers(-30, -10))
        sv = float(rng.integers(0, 2**12)) * 2.0 ** int(rng.integers(-16, -4))
        bound = sv / 128 + float(bf.ulp_bf16(bf.Fraction(abs(d))))
        for t in (-1.0, 1.0):
            target = d + t * bound
            below = int(oracle.rne_bf16_from_double(np.array([target]))[0])
            for bits in {below, below + 1, below - 1} - {-1}:
                if (bits & 0x7FFF) < 0x7F80:
                    cases.append((bits, d, sv))
    cb = np.array([c[0] for c in cases], np.uint16)
    Dv = np.array([c[1] for c in cases])
    Sv = np.array([c[2] for c in cases])
    ref = oracle.rne_bf16_from_double(Dv)
    got = oracle.accept(cb, ref, Dv, Sv)
    want = np.array([bf.accept(int(b), int(r), bf.Fraction(d), bf.Fraction(sv))
                     for b, r, d, sv in zip(cb, ref, Dv, Sv)])
    assert got.sum() > 100 and (~got).sum() > 100          # both sides of the bar are exercised
    assert np.array_equal(got, want)


PINS = [
    pin_e4m3fn_vs_torch, pin_e8m0_vs_torch, pin_bf16_decode_vs_torch, pin_e2m1_bitfields,
    pin_rne_vs_torch_on_floats, pin_rne_from_double_not_via_float, pin_rne_overflow_subnormal_nan,
    pin_rne_vs_rational, pin_bruteforce_mxfp4, pin_bruteforce_bf16, pin_bruteforce_fp8,
    pin_bruteforce_mxfp8, pin_handworked_mxfp4, pin_handworked_mxfp8, pin_identity, pin_bias_broadcast,
    pin_integer_matmul, pin_invariants_mxfp4, pin_invariants_mxfp8, pin_accept,
    pin_bruteforce_bf16_backward, pin_bf16_backward_vs_autograd, pin_bf16_backward_identities,
    pin_bruteforce_mixed_mx, pin_mixed_mx_reduces_to_mxfp4,
    pin_abs_sums_vs_rational, pin_mixed_abs_sums_vs_rational, pin_backward_abs_sums_vs_rational,
    pin_ulp_bf16, pin_accept_exact,
    pin_fp6_bitfields, pin_fp6_bit_order, pin_handworked_mxfp6, pin_bruteforce_mxfp6, pin_mxfp6_reduces_to_mxfp8,
    pin_invariants_mxfp6,
]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


# ---------------------------------------------------------------- planted mistakes

def _mut_e2m1_entry(mp):
    t = oracle.E2M1_VALUES.copy()
    t[5] = 2.5
    mp.setattr(oracle, "E2M1_VALUES", t)


def _mut_nibble_order(mp):
    # A consistent nibble swap in both operands permutes K inside one scale block
    # and cannot change C; the plausible mistake is a swap in one operand only.
    real = oracle.operands

    def ops(dtype, A, B, SA=None, SB=None, K=None):
        if dtype == "mxfp4":
            A = np.asarray(A, np.uint8)
            A = ((A >> 4) | (A << 4)).astype(np.uint8)
        return real(dtype, A, B, SA, SB, K)
    mp.setattr(oracle, "operands", ops)


def _mut_scale_block(mp):
    real = oracle.decode_e8m0

    def shifted(e):
        e = np.asarray(e)
        return real(np.roll(e, 1, axis=-1) if e.ndim == 2 else e)
    mp.setattr(oracle, "decode_e8m0", shifted)


def _mut_drop_bias(mp):
    mp.setattr(oracle, "_beta", lambda bias, N: np.zeros(N))


def _mut_double_bias(mp):
    real = oracle._beta
    mp.setattr(oracle, "_beta", lambda bias, N: 2 * real(bias, N))


def _mut_round_via_float(mp):
    real = oracle.rne_bf16_from_double
    mp.setattr(oracle, "rne_bf16_from_double",
               lambda d: real(np.asarray(d, dtype=np.float64).astype(np.float32).astype(np.float64)))


def _mut_round_truncate(mp):
    def trunc(d):
        d = np.asarray(d, dtype=np.float64)
        return (d.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    mp.setattr(oracle, "rne_bf16_from_double", trunc)


def _mut_e4m3_bias(mp):
    real = oracle.decode_e4m3fn
    mp.setattr(oracle, "decode_e4m3fn", lambda b: real(b) * 0.5)


def _mut_fp8_sigma(mp):
    real = oracle.operands

    def ops(dtype, A, B, SA=None, SB=None, K=None):
        a, b, s = real(dtype, A, B, SA, SB, K)
        return a, b, 1.0
    mp.setattr(oracle, "operands", ops)


def _mut_transpose_b(mp):
    real = oracle.operands

    def ops(dtype, A, B, SA=None, SB=None, K=None):
        a, b, s = real(dtype, A, B, SA, SB, K)
        if b.shape[0] == b.shape[1]:
            b = b.T.copy()
        else:
            b = b[::-1].copy()
        return a, b, s
    mp.setattr(oracle, "operands", ops)


def _mut_bf16_decode(mp):
    real = oracle.decode_bf16
    mp.setattr(oracle, "decode_bf16", lambda u: real(np.asarray(u, np.uint16) ^ np.uint16(1)))


def _mut_mxfp8_no_scales(mp):
    mp.setattr(oracle, "mxfp8_operand", lambda elems, scales, K: oracle.decode_e4m3fn(elems))


def _mut_mxfp8_scale_per_16(mp):
    # each E8M0 byte applied to 16 elements (and the row's second half given the first half's scales)
    def op(elems, scales, K):
        sc = oracle.decode_e8m0(np.asarray(scales, np.uint8))
        rep = np.repeat(sc, 16, axis=1)
        return oracle.decode_e4m3fn(elems) * np.concatenate([rep, rep], axis=1)[:, :K]
    mp.setattr(oracle, "mxfp8_operand", op)


def _mut_backward_transposed_b(mp):
    # dA taken with B transposed (only shape-consistent when N == K)
    real = oracle.bf16_backward

    def bwd(dC, A, B):
        out = real(dC, A, B)
        if B is not None and np.asarray(B).shape[0] == np.asarray(B).shape[1]:
            g, b = oracle.decode_bf16(dC), oracle.decode_bf16(B)
            D = g @ b.T
            out["dA"] = (oracle.rne_bf16_from_double(D), D, out["dA"][2])
        return out
    mp.setattr(oracle, "bf16_backward", bwd)


def _mut_backward_dbias_rows(mp):
    real = oracle.bf16_backward

    def bwd(dC, A, B):
        out = real(dC, A, B)
        g = oracle.decode_bf16(dC)
        if g.shape[0] == g.shape[1]:
            D = g.sum(axis=1)
            out["dbias"] = (oracle.rne_bf16_from_double(D), D, out["dbias"][2])
        return out
    mp.setattr(oracle, "bf16_backward", bwd)


def _mut_mixed_b_scales_ignored(mp):
    real = oracle.gemm_mx

    def gm(a_fmt, b_fmt, A, B, SA, SB, bias=None, K=None):
        if a_fmt != b_fmt:
            SB = np.full_like(np.asarray(SB), 127)
        return real(a_fmt, b_fmt, A, B, SA, SB, bias, K)
    mp.setattr(oracle, "gemm_mx", gm)


def _mut_abs_sums_one_sided(mp):
    # |a| @ b^T: the absolute value taken on one operand only
    def S(dtype, A, B, SA=None, SB=None, K=None):
        a, b, sigma = oracle.operands(dtype, A, B, SA, SB, K)
        return abs(sigma) * (np.abs(a) @ b.T)
    mp.setattr(oracle, "abs_product_sums", S)


def _mut_abs_sums_outer(mp):
    # (sum_k |a|)(sum_k |b|): an outer product of row sums instead of sum_k |a b|
    def S(dtype, A, B, SA=None, SB=None, K=None):
        a, b, sigma = oracle.operands(dtype, A, B, SA, SB, K)
        return abs(sigma) * np.outer(np.abs(a).sum(axis=1), np.abs(b).sum(axis=1))
    mp.setattr(oracle, "abs_product_sums", S)


def _mut_abs_sums_no_sigma(mp):
    def S(dtype, A, B, SA=None, SB=None, K=None):
        a, b, sigma = oracle.operands(dtype, A, B, SA, SB, K)
        return np.abs(a) @ np.abs(b).T
    mp.setattr(oracle, "abs_product_sums", S)


def _mut_elements_S_one_sided(mp):
    real = oracle.gemm_elements

    def ge(dtype, A, B, rows, cols, SA=None, SB=None, bias=None, K=None):
        C, D, S = real(dtype, A, B, rows, cols, SA, SB, bias, K)
        a, b, sigma = oracle.operands(dtype, A, B, SA, SB, K)
        S = abs(sigma) * np.einsum("ik,ik->i", np.abs(a[np.asarray(rows)]), b[np.asarray(cols)])
        return C, D, S
    mp.setattr(oracle, "gemm_elements", ge)


def _mut_backward_S_one_sided(mp):
    real = oracle.bf16_backward

    def bwd(dC, A, B):
        out = real(dC, A, B)
        if B is not None:
            g, b = oracle.decode_bf16(dC), oracle.decode_bf16(B)
            out["dA"] = (out["dA"][0], out["dA"][1], np.abs(g) @ b)
        return out
    mp.setattr(oracle, "bf16_backward", bwd)


def _mut_mixed_S_one_sided(mp):
    def S(a_fmt, b_fmt, A, B, SA, SB, K=None):
        K = oracle._mx_k(a_fmt, A, K)
        return np.abs(oracle._mx_decode(a_fmt, A, SA, K)) @ oracle._mx_decode(b_fmt, B, SB, K).T
    mp.setattr(oracle, "abs_product_sums_mx", S)


def _mut_ulp_half(mp):
    real = oracle._ulp_bf16
    mp.setattr(oracle, "_ulp_bf16", lambda x: real(x) / 2)


def _mut_bound_without_ulp(mp):
    mp.setattr(oracle, "_ulp_bf16", lambda x: np.zeros(np.shape(x)))


def _mut_fp6_formats_swapped(mp):
    # E2M3 codes decoded as E3M2 (and the other way round)
    a, b = oracle.decode_e2m3, oracle.decode_e3m2
    mp.setattr(oracle, "decode_e2m3", b)
    mp.setattr(oracle, "decode_e3m2", a)


def _mut_fp6_big_endian(mp):
    # the three bytes of a group read as a big-endian word
    def unpack(packed, K):
        p = np.asarray(packed, dtype=np.uint8).reshape(np.asarray(packed).shape[0], -1, 3)[:, :, ::-1]
        return _real_unpack_fp6(np.ascontiguousarray(p).reshape(p.shape[0], -1), K)
    mp.setattr(oracle, "unpack_fp6", unpack)


def _mut_fp6_subnormal_scale(mp):
    # subnormals without the 2^(1 - bias) factor
    def dec(codes, ebits, mbits):
        c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
        bias = (1 << (ebits - 1)) - 1
        sign = np.where(c & 0x20, -1.0, 1.0)
        e = (c >> mbits) & ((1 << ebits) - 1)
        m = (c & ((1 << mbits) - 1)).astype(np.float64) / (1 << mbits)
        return sign * np.where(e == 0, m, np.ldexp(1.0 + m, (e - bias).astype(np.int32)))
    mp.setattr(oracle, "_decode_fp6", dec)


_real_unpack_fp6 = oracle.unpack_fp6


MUTATIONS = [
    _mut_e2m1_entry, _mut_nibble_order, _mut_scale_block, _mut_drop_bias, _mut_double_bias,
    _mut_round_via_float, _mut_round_truncate, _mut_e4m3_bias, _mut_fp8_sigma, _mut_transpose_b,
    _mut_bf16_decode, _mut_mxfp8_no_scales, _mut_mxfp8_scale_per_16, _mut_backward_transposed_b,
    _mut_backward_dbias_rows, _mut_mixed_b_scales_ignored,
    _mut_abs_sums_one_sided, _mut_abs_sums_outer, _mut_abs_sums_no_sigma, _mut_elements_S_one_sided,
    _mut_backward_S_one_sided, _mut_mixed_S_one_sided, _mut_ulp_half, _mut_bound_without_ulp,
    _mut_fp6_formats_swapped, _mut_fp6_big_endian, _mut_fp6_subnormal_scale,
]


@pytest.mark.parametrize("mutation", MUTATIONS, ids=[m.__name__ for m in MUTATIONS])
def test_planted_mistakes_are_caught(mutation, monkeypatch):
    mutation(monkeypatch)
    caught = []
    for pin in PINS:
        try:
            pin()
        except Exception:
            caught.append(pin.__name__)
    assert caught, f"no pin caught {mutation.__name__}"
