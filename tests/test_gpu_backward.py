"""GPU parity of the bf16 backward (dA = dC B, dB = dC^T A, dbias = column sums
of dC) through the C ABI against the CPU oracle: bit for bit on integer inputs
(every sum exact, so any order and split gives the one rounding of the exact
value), within |err| <= 2**-7 * sum|terms| + one bf16 ulp on random inputs,
with bit-identical repeats."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import persistent_gemm_amd as pg
from persistent_gemm_amd.inputs import WORKLOADS, backward_inputs

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gpu_util import assert_bitexact, assert_within_bound, say


def _dev(x):
    return {k: torch.from_numpy(np.ascontiguousarray(x[k]).view(np.int16)).view(torch.bfloat16).cuda()
            for k in ("dC", "A", "B")}


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _run(d, **kw):
    out = pg.gemm_bf16_backward(d["dC"], d["A"], d["B"], **kw)
    pg.check()
    return [None if t is None else _bits(t) for t in out]


@pytest.mark.parametrize("M,N,K", [(8, 8, 8), (136, 72, 200), (264, 520, 328), (1024, 512, 768), (16, 4096, 1024)])
def test_backward_integer_inputs_exact(M, N, K):
    x = backward_inputs(M, N, K, seed=M + 3 * N + 7 * K, integer=True)
    o = oracle.bf16_backward(x["dC"], x["A"], x["B"])
    d = _dev(x)
    for cap in (0, 7):
        say(f"bf16 backward integers {M}x{N}x{K} cap {cap}")
        dA, dB, db = _run(d, grid_cap=cap)
        assert_bitexact(dA, o["dA"][0], f"dA {M}x{N}x{K}")
        assert_bitexact(dB, o["dB"][0], f"dB {M}x{N}x{K}")
        assert_bitexact(db[None, :], o["dbias"][0][None, :], f"dbias {M}x{N}x{K}")


def test_backward_partial_outputs():
    x = backward_inputs(72, 40, 56, seed=11, integer=True)
    o = oracle.bf16_backward(x["dC"], x["A"], x["B"])
    d = _dev(x)
    say("bf16 backward dA only, dB only, dbias only")
    dA, dB, db = _run(d, need_dB=False, need_dbias=False)
    assert dB is None and db is None
    assert_bitexact(dA, o["dA"][0], "dA only")
    dA, dB, db = pg.gemm_bf16_backward(d["dC"], d["A"], None, need_dA=False, need_dbias=False)
    pg.check()
    assert dA is None and db is None
    assert_bitexact(_bits(dB), o["dB"][0], "dB only")
    _, _, db = pg.gemm_bf16_backward(d["dC"], d["A"], None, need_dA=False, need_dB=False)
    pg.check()
    assert_bitexact(_bits(db)[None, :], o["dbias"][0][None, :], "dbias only")


def test_backward_random_within_bound_and_repeatable():
    M, N, K = 520, 392, 1064
    x = backward_inputs(M, N, K, seed=12)
    o = oracle.bf16_backward(x["dC"], x["A"], x["B"])
    d = _dev(x)
    say(f"bf16 backward random {M}x{N}x{K}")
    first = _run(d)
    for name, got in zip(("dA", "dB", "dbias"), first):
        bits, D, S = o[name]
        if name == "dbias":
            got, bits, D, S = got[None, :], bits[None, :], D[None, :], S[None, :]
        assert_within_bound(got, bits, D, S, name)
    again = _run(d)
    for a, b in zip(first, again):
        assert np.array_equal(a, b)


def test_backward_full_size():
    """The whole 4096^3 backward (dA, dB, dbias) against the oracle under the bound, and a repeat."""
    w = WORKLOADS["bf16_addmm_backward_4096"]
    x = backward_inputs(w.M, w.N, w.K, seed=w.seed)
    o = oracle.bf16_backward(x["dC"], x["A"], x["B"])
    d = _dev(x)
    say("bf16 backward 4096^3")
    first = _run(d)
    for name, got in zip(("dA", "dB", "dbias"), first):
        bits, D, S = o[name]
        if name == "dbias":
            got, bits, D, S = got[None, :], bits[None, :], D[None, :], S[None, :]
        assert_within_bound(got, bits, D, S, f"4096^3 {name}")
    say("bf16 backward 4096^3, repeat")
    for a, b in zip(first, _run(d)):
        assert np.array_equal(a, b)


def test_backward_argument_errors():
    x = backward_inputs(16, 16, 16, seed=13, integer=True)
    d = _dev(x)
    lib = pg.load()
    s = torch.cuda.current_stream().cuda_stream
    out = torch.empty(16 * 16, dtype=torch.bfloat16, device="cuda")
    p = lambda t: t.data_ptr()
    # M not a multiple of 8
    assert lib.sk_gemm_bf16_backward(p(d["dC"]), p(d["A"]), p(d["B"]), p(out), None, None, 12, 16, 16, 0, s) == 2
    # nothing asked for; dA without B
    assert lib.sk_gemm_bf16_backward(p(d["dC"]), p(d["A"]), p(d["B"]), None, None, None, 16, 16, 16, 0, s) == 1
    assert lib.sk_gemm_bf16_backward(p(d["dC"]), p(d["A"]), None, p(out), None, None, 16, 16, 16, 0, s) == 1
    # an output over an input
    assert lib.sk_gemm_bf16_backward(p(d["dC"]), p(d["A"]), p(d["B"]), p(d["A"]), None, None, 16, 16, 16, 0, s) == 1
