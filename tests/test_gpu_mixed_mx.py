"""GPU parity of products of block-scaled operands of different widths (one
MXFP4, one MXFP8) through sk_gemm_mx against the CPU oracle: bit for bit when
the MXFP8 operand holds small integers (every sum exact), within |err| <=
2**-7 * sum|a*b| + one bf16 ulp on random E4M3 inputs, with bit-identical
repeats; equal formats (MXFP4, MXFP6, MXFP8) give the same bits as the
dtype's own kernels."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import persistent_gemm_amd as pg
from persistent_gemm_amd.inputs import mixed_inputs

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gpu_util import assert_bitexact, assert_within_bound, say


def _dev(x):
    d = {}
    for op, fmt in (("A", x["a_fmt"]), ("B", x["b_fmt"])):
        t = torch.from_numpy(np.ascontiguousarray(x[op])).cuda()
        d[op] = t if fmt == "mxfp4" else t.view(torch.float8_e4m3fn)
    for k in ("SA", "SB"):
        d[k] = torch.from_numpy(np.ascontiguousarray(x[k])).cuda()
    b = x["bias"]
    d["bias"] = None if b is None else torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda()
    return d


def _run(x, d, **kw):
    c = pg.gemm_mx(x["a_fmt"], x["b_fmt"], d["A"], d["B"], d["SA"], d["SB"], d["bias"], **kw)
    pg.check()
    return c.view(torch.int16).cpu().numpy().view(np.uint16)


FMTS = [("mxfp4", "mxfp8"), ("mxfp8", "mxfp4")]


@pytest.mark.parametrize("a_fmt,b_fmt", FMTS)
@pytest.mark.parametrize("M,N,K", [(1, 8, 32), (100, 72, 96), (300, 200, 512), (257, 520, 1056)])
def test_mixed_exact(a_fmt, b_fmt, M, N, K):
    x = mixed_inputs(a_fmt, b_fmt, M, N, K, bias=True, seed=M + N + K, integer_fp8=True)
    C, _ = oracle.gemm_mx(a_fmt, b_fmt, x["A"], x["B"], x["SA"], x["SB"], x["bias"], K=K)
    d = _dev(x)
    for cap in (0, 5):
        say(f"mixed {a_fmt} x {b_fmt} {M}x{N}x{K} cap {cap}")
        assert_bitexact(_run(x, d, grid_cap=cap), C, f"{a_fmt} x {b_fmt} {M}x{N}x{K} cap {cap}")


@pytest.mark.parametrize("a_fmt,b_fmt", FMTS)
def test_mixed_random_within_bound_and_repeatable(a_fmt, b_fmt):
    M, N, K = 513, 388, 1056
    x = mixed_inputs(a_fmt, b_fmt, M, N, K, bias=True, seed=31)
    C, D = oracle.gemm_mx(a_fmt, b_fmt, x["A"], x["B"], x["SA"], x["SB"], x["bias"], K=K)
    S = oracle.abs_product_sums_mx(a_fmt, b_fmt, x["A"], x["B"], x["SA"], x["SB"], K=K)
    d = _dev(x)
    say(f"mixed {a_fmt} x {b_fmt} random {M}x{N}x{K}")
    first = _run(x, d)
    assert_within_bound(first, C, D, S, f"{a_fmt} x {b_fmt}")
    assert np.array_equal(_run(x, d), first)


def test_equal_mxfp6_formats_match_gemm_ex():
    from persistent_gemm_amd.inputs import exact_inputs
    from gpu_util import assert_exact_inputs, device_inputs, oracle_full, run
    for fmt in ("mxfp6_e2m3", "mxfp6_e3m2"):
        x = exact_inputs(fmt, 130, 72, 160, bias=True, seed=33)
        assert_exact_inputs(x)
        d = device_inputs(x)
        say(f"gemm_mx {fmt} x {fmt}")
        got = pg.gemm_mx(fmt, fmt, d["A"], d["B"], d["SA"], d["SB"], d["bias"])
        pg.check()
        got = got.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, run(d))
        C, _ = oracle_full(x)
        assert_bitexact(got, C, f"{fmt} x {fmt}")


def test_equal_formats_match_their_entry_points():
    for fmt in ("mxfp4", "mxfp8"):
        x = mixed_inputs(fmt, fmt, 130, 72, 160, bias=True, seed=32, integer_fp8=True)
        d = _dev(x)
        say(f"gemm_mx {fmt} x {fmt}")
        got = _run(x, d)
        fn = pg.gemm_mxfp4 if fmt == "mxfp4" else pg.gemm_mxfp8
        own = fn(d["A"], d["B"], d["SA"], d["SB"], d["bias"])
        pg.check()
        assert np.array_equal(got, own.view(torch.int16).cpu().numpy().view(np.uint16))
        C, _ = oracle.gemm_mx(fmt, fmt, x["A"], x["B"], x["SA"], x["SB"], x["bias"], K=160)
        assert_bitexact(got, C, f"{fmt} x {fmt}")
