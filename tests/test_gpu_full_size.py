"""GPU parity at the workloads' full sizes.

Each workload is first run through the plain entry point (policy AUTO: the
tuned kernel and policy, which is exactly the launch bench.py times) and the
whole output is compared with the oracle; then other tiles and policies of
interest are checked against the oracle or against that first result."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import persistent_gemm_amd as pg
from persistent_gemm_amd.inputs import WORKLOADS, make_inputs, mixed_inputs

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gpu_util import abs_sums, assert_bitexact, assert_within_bound, device_inputs, oracle_full, run, say


def _wl(name):
    w = WORKLOADS[name]
    return w, make_inputs(w.dtype, w.M, w.N, w.K, bias=w.bias, seed=w.seed)


# The kernels the tuned table picks for the timed workloads (variant indices as in
# sk_variant_info); the tests assert them so that a retuned table cannot leave
# the timed kernel unchecked.
BENCHED = {"mxfp4_addmm_8192": 23, "bf16_addmm_4096": 25, "mxfp4_gemm_16x8192x8192": 53}


def _auto_plan(w):
    p = pg.plan(w.dtype, w.M, w.N, w.K, grid_cap=w.grid_cap, policy=pg.AUTO)
    assert p.variant == BENCHED[w.name], f"{w.name}: AUTO now picks kernel {p.variant}; update BENCHED"
    return p


def _plain(w, d, bias=True):
    """The plain entry point (AUTO), as bench.py calls it; C as uint16 bits."""
    b = d["bias"] if bias else None
    if w.dtype == "mxfp4":
        out = pg.gemm_mxfp4(d["A"], d["B"], d["SA"], d["SB"], b, grid_cap=w.grid_cap)
    else:
        out = pg.gemm_bf16(d["A"], d["B"], b, grid_cap=w.grid_cap)
    pg.check()
    return out.view(torch.int16).cpu().numpy().view(np.uint16)


def test_skinny_mxfp4_16x8192x8192_bitexact():
    w, x = _wl("mxfp4_gemm_16x8192x8192")
    d = device_inputs(x)
    C, _ = oracle_full(x)
    p = _auto_plan(w)
    say(f"skinny 16x8192x8192, plain entry point (kernel {p.variant}, grid {p.grid}, sk_tiles {p.sk_tiles})")
    assert_bitexact(_plain(w, d), C, "AUTO")
    for tile, policy, g in [(None, pg.HYBRID, 0), ((16, 128), pg.HYBRID, 0), ((16, 256), pg.PURE_SK, 100),
                            ((16, 256), pg.PURE_DP, 0), ((64, 64), pg.HYBRID, 0)]:
        say(f"skinny 16x8192x8192 tile {tile} policy {policy} grid {g}")
        assert_bitexact(run(d, tile=tile, policy=policy, grid_cap=g), C, f"{tile} {policy} {g}")
    # the 16 x 128 kernel with 128-byte k-steps, each tile split four ways (the
    # Stream-K fixup at this shape), and the k-split kernel split by MAC
    # iteration too (its waves' sums added before a partial tile is published)
    for variant, policy, g in [(28, pg.HYBRID, 0), (p.variant, pg.PURE_SK, 100), (p.variant, pg.HYBRID, 200)]:
        say(f"skinny 16x8192x8192 kernel {variant} policy {policy} grid {g}")
        assert_bitexact(run(d, variant=variant, policy=policy, grid_cap=g), C, f"kernel {variant} {policy} {g}")


def test_large_mxfp4_addmm_8192_bitexact():
    """The whole 8192^3 output of the timed launch, bit for bit (the oracle takes seconds)."""
    w, x = _wl("mxfp4_addmm_8192")
    d = device_inputs(x)
    p = _auto_plan(w)
    say(f"8192^3 mxfp4 addmm, plain entry point (kernel {p.variant}, grid {p.grid}, policy {p.policy})")
    got = _plain(w, d)
    say("8192^3 oracle")
    C, _ = oracle_full(x)
    assert_bitexact(got, C, "8192^3 AUTO")
    say("8192^3 repeat")
    assert np.array_equal(_plain(w, d), got)
    # other kernels and partitions: every fp32 partial sum is exact, so the same bits
    for tile, policy, g in [(None, pg.HYBRID, 0), ((128, 128), pg.HYBRID, 0), ((256, 256), pg.PURE_SK, 0),
                            ((256, 256), pg.HYBRID, 200)]:
        say(f"8192^3 tile {tile} policy {policy} grid {g}")
        again = run(d, tile=tile, policy=policy, grid_cap=g)
        assert np.array_equal(again, got), f"{tile} {policy} {g} differs from the oracle"


@pytest.fixture(scope="module")
def bf16_4096():
    w, x = _wl("bf16_addmm_4096")
    C, D = oracle_full(x)
    S = oracle.abs_product_sums("bf16", x["A"], x["B"])
    return w, x, device_inputs(x), C, D, S


def test_bf16_addmm_4096_timed_launch_within_bound(bf16_4096):
    w, x, d, C, D, S = bf16_4096
    p = _auto_plan(w)
    say(f"bf16 4096^3 addmm, plain entry point (kernel {p.variant}, grid {p.grid})")
    first = _plain(w, d)
    assert_within_bound(first, C, D, S, "AUTO")
    assert np.array_equal(_plain(w, d), first)


@pytest.mark.parametrize("tile", [None, (128, 192), (128, 128)])
def test_bf16_addmm_4096_within_bound(bf16_4096, tile):
    w, x, d, C, D, S = bf16_4096
    say(f"bf16 4096^3 addmm tile {tile}")
    first = run(d, tile=tile)
    assert_within_bound(first, C, D, S, f"tile {tile}")
    assert np.array_equal(run(d, tile=tile), first)


def test_fp8_4096_cap_sweep_within_bound():
    w, x = _wl("fp8_gemm_4096_capsweep")
    d = device_inputs(x)
    C, D = oracle_full(x)
    S = oracle.abs_product_sums("fp8", x["A"], x["B"], x["SA"], x["SB"])
    results = {}
    for cap in w.caps:
        say(f"fp8 4096^3 cap {cap}")
        got = run(d, grid_cap=cap)
        assert_within_bound(got, C, D, S, f"cap {cap}")
        results[cap] = got
    # every cap divides the 256 tiles: the same whole-tile partition, the same bits
    for cap in w.caps:
        assert np.array_equal(results[cap], results[256])


def test_mxfp8_addmm_8192_sampled_within_bound():
    w, x = _wl("mxfp8_addmm_8192")
    d = device_inputs(x)
    say("8192^3 mxfp8 addmm, default plan")
    got = run(d)
    rng = np.random.default_rng(1)
    # a 64 x 64 block across a tile corner, the last row and column, and random samples
    rows = np.concatenate([np.repeat(np.arange(224, 288), 64), np.full(64, 8191), np.arange(8128, 8192),
                           rng.integers(0, 8192, 20000)])
    cols = np.concatenate([np.tile(np.arange(224, 288), 64), np.arange(8128, 8192), np.full(64, 8191),
                           rng.integers(0, 8192, 20000)])
    Cs, Ds, Ss = oracle.gemm_elements("mxfp8", x["A"], x["B"], rows, cols, x["SA"], x["SB"], x["bias"], K=w.K)
    ok = oracle.accept(got[rows, cols], Cs, Ds, Ss)
    assert ok.all(), f"{(~ok).sum()} of {ok.size} sampled elements outside the bound"
    say("8192^3 mxfp8 addmm, repeat")
    assert np.array_equal(run(d), got)


@pytest.mark.parametrize("name", ["mxfp6_e2m3_addmm_8192", "mxfp6_e3m2_addmm_8192", "mxfp4_mxfp8_addmm_8192"])
def test_other_mx_addmm_8192_within_bound(name):
    """MXFP6 (both element types) and mixed MXFP4 x MXFP8 at 8192^3, the plain launch (AUTO):
    the whole output within the bound, then a bit-identical repeat.  Random codes over the
    whole range and scales 2**-2 .. 2**2 make the sums inexact in fp32, hence the bound."""
    w = WORKLOADS[name]
    if w.dtype == "mxfp4_mxfp8":
        x = mixed_inputs("mxfp4", "mxfp8", w.M, w.N, w.K, bias=w.bias, seed=w.seed)
    else:
        x = make_inputs(w.dtype, w.M, w.N, w.K, bias=w.bias, seed=w.seed)
    d = device_inputs(x)
    p = pg.plan(w.dtype, w.M, w.N, w.K, policy=pg.AUTO)
    say(f"8192^3 {w.dtype} addmm, AUTO (kernel {p.variant}, grid {p.grid}, policy {p.policy})")
    got = run(d, policy=pg.AUTO)
    say(f"8192^3 {w.dtype} oracle")
    C, D = oracle_full(x)
    S = abs_sums(x)
    assert_within_bound(got, C, D, S, f"{name} AUTO")
    say(f"8192^3 {w.dtype} repeat")
    assert np.array_equal(run(d, policy=pg.AUTO), got)
