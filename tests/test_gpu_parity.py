"""GPU parity: the HIP path through the C ABI against the CPU oracle.

MXFP4 inputs make every fp32 partial sum exact (products are multiples of
2**-6 below 576, sums stay far below 2**18), so MXFP4 results must match the
oracle bit for bit at every grid size, policy and tile.  bf16 / fp8 / MXFP8
inputs with small integer values are exact too, and so are the MXFP6 and
mixed MXFP4 x MXFP8 inputs of inputs.exact_inputs (elements on a coarse grid,
checked against their sums); random bf16 / fp8 / MXFP8 / MXFP6 inputs are
held to |err| <= 2**-7 * sum|a*b| + one bf16 ulp, and must repeat bit for bit.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import persistent_gemm_amd as pg
from persistent_gemm_amd.inputs import WORKLOADS, exact_inputs, integer_inputs, make_inputs

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gpu_util import (abs_sums, assert_bitexact, assert_exact_inputs, assert_within_bound, device_inputs,
                          oracle_full, run, say)


def _wl(name, bias=None):
    w = WORKLOADS[name]
    return make_inputs(w.dtype, w.M, w.N, w.K, bias=w.bias if bias is None else bias, seed=w.seed)


# ---------------------------------------------------------------- the small MXFP4 addmm (grid of 5)

@pytest.fixture(scope="module")
def small():
    x = _wl("mxfp4_addmm_256x256x512_g5")
    C, D = oracle_full(x)
    return x, device_inputs(x), C


@pytest.mark.parametrize("policy", [pg.HYBRID, pg.PURE_SK, pg.PURE_DP])
def test_small_mxfp4_addmm_grid5(small, policy):
    x, d, C = small
    say(f"small mxfp4 addmm 256x256x512 tile 64x64 grid 5 policy {policy}")
    got = run(d, grid_cap=5, tile=(64, 64), policy=policy)
    assert_bitexact(got, C, f"policy {policy}")


def test_small_mxfp4_grid_sweep(small):
    x, d, C = small
    for policy in (pg.HYBRID, pg.PURE_SK, pg.PURE_DP):
        for g in (1, 2, 3, 4, 5, 7, 8, 16, 31, 64, 128, 255, 256):
            say(f"grid sweep policy {policy} grid {g}")
            got = run(d, grid_cap=g, tile=(64, 64), policy=policy)
            assert_bitexact(got, C, f"policy {policy} grid {g}")


def test_small_mxfp4_other_tiles(small):
    x, d, C = small
    for tile in [(16, 256), (16, 128), (128, 128), (256, 256), None]:
        for g in (3, 5, 256):
            say(f"tile {tile} grid {g}")
            got = run(d, grid_cap=g, tile=tile, policy=pg.PURE_SK)
            assert_bitexact(got, C, f"tile {tile} grid {g}")


# ---------------------------------------------------------------- ragged shapes and edges

RAGGED = [(1, 1, 32), (100, 72, 96), (33, 300, 1056), (257, 129, 544), (16, 520, 4096), (515, 260, 288)]


@pytest.mark.parametrize("M,N,K", RAGGED)
def test_mxfp4_ragged(M, N, K):
    x = make_inputs("mxfp4", M, N, K, bias=True, seed=M * 7 + N * 3 + K)
    d = device_inputs(x)
    C, _ = oracle_full(x)
    Cn, _ = oracle_full(x, bias=False)
    for tile in [None, (64, 64), (16, 256), (128, 128), (256, 256)]:
        for policy, g in [(pg.HYBRID, 0), (pg.PURE_SK, 7), (pg.PURE_DP, 3), (pg.PURE_SK, 256)]:
            say(f"mxfp4 {M}x{N}x{K} tile {tile} policy {policy} grid {g}")
            assert_bitexact(run(d, grid_cap=g, tile=tile, policy=policy), C, f"{M}x{N}x{K} {tile} {policy} {g}")
        assert_bitexact(run(d, bias=False, tile=tile, policy=pg.PURE_SK, grid_cap=5), Cn, f"no bias {tile}")


@pytest.mark.parametrize("dtype,M,N,K", [
    (dt, M, N, K) for dt in ("bf16", "fp8") for M, N, K in [(1, 8, 16), (100, 72, 96), (300, 200, 512), (64, 384, 1040)]
] + [("mxfp8", M, N, K) for M, N, K in [(1, 8, 32), (100, 72, 96), (300, 200, 512), (64, 384, 1056)]])
def test_integer_inputs_exact(dtype, M, N, K):
    x = integer_inputs(dtype, M, N, K, bias=True, seed=M + N + K)
    d = device_inputs(x)
    C, _ = oracle_full(x)
    tiles = [None, (64, 64), (128, 128), (256, 256)] + ([(128, 192)] if dtype == "bf16" else [(16, 256)])
    for tile in tiles:
        for policy, g in [(pg.HYBRID, 0), (pg.PURE_SK, 5), (pg.PURE_DP, 2)]:
            say(f"{dtype} integers {M}x{N}x{K} tile {tile} policy {policy} grid {g}")
            assert_bitexact(run(d, grid_cap=g, tile=tile, policy=policy), C, f"{dtype} {tile} {policy} {g}")


@pytest.mark.parametrize("dtype", ["mxfp6_e2m3", "mxfp6_e3m2", "mxfp4_mxfp8", "mxfp8_mxfp4"])
@pytest.mark.parametrize("M,N,K", [(1, 8, 32), (100, 72, 96), (300, 200, 512), (64, 384, 1056)])
def test_exact_mx_inputs(dtype, M, N, K):
    """MXFP6 and mixed MXFP4 x MXFP8 on exact inputs: every tile shape, three policies."""
    x = exact_inputs(dtype, M, N, K, bias=True, seed=M + N + K)
    assert_exact_inputs(x)
    d = device_inputs(x)
    C, _ = oracle_full(x)
    for tile in [None, (64, 64), (128, 128), (256, 256), (16, 256)]:
        for policy, g in [(pg.HYBRID, 0), (pg.PURE_SK, 5), (pg.PURE_DP, 2)]:
            say(f"{dtype} exact {M}x{N}x{K} tile {tile} policy {policy} grid {g}")
            assert_bitexact(run(d, grid_cap=g, tile=tile, policy=policy), C, f"{dtype} {tile} {policy} {g}")


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "mxfp8", "mxfp6_e2m3", "mxfp6_e3m2"])
def test_random_within_bound_and_repeatable(dtype):
    M, N, K = 513, 388, 1056
    kw = {"fp8_scales": (0.5, 3.0)} if dtype == "fp8" else {}
    x = make_inputs(dtype, M, N, K, bias=True, seed=77, **kw)
    d = device_inputs(x)
    C, D = oracle_full(x)
    S = abs_sums(x)
    for tile in [None, (64, 64), (128, 128), (256, 256)]:
        for policy, g in [(pg.HYBRID, 0), (pg.PURE_SK, 9)]:
            say(f"{dtype} random {M}x{N}x{K} tile {tile} policy {policy} grid {g}")
            first = run(d, grid_cap=g, tile=tile, policy=policy)
            assert_within_bound(first, C, D, S, f"{dtype} {tile} {policy}")
            for _ in range(2):
                assert np.array_equal(run(d, grid_cap=g, tile=tile, policy=policy), first)


# ---------------------------------------------------------------- every compiled kernel

_DTYPES = {0: "mxfp4", 1: "bf16", 2: "fp8", 3: "mxfp8", 4: "mxfp6_e2m3", 5: "mxfp6_e3m2", 6: "mxfp4_mxfp8",
           7: "mxfp8_mxfp4"}
_MX = ["mxfp4", "mxfp8", "mxfp6_e2m3", "mxfp6_e3m2", "mxfp4_mxfp8", "mxfp8_mxfp4"]


def _num_variants():
    try:
        return len(pg.variants())
    except Exception:  # library not built: the load error surfaces in every other test
        return 1


@pytest.mark.parametrize("index", range(_num_variants()))
def test_every_variant_exact(index):
    """Each compiled kernel, chosen by index, on exact inputs spanning several
    tiles with ragged M, N and K tails, under all three policies.  N is once a
    multiple of 8 (whole 16-byte output pieces) and once not (element
    stores) and once a multiple of 4 but not of 8 (8-byte runs, or the staged
    path's ragged last chunk); K is once whole k-steps and once a ragged last
    k-step (for the MX types, one whose scale block is only partly inside K)."""
    v = pg.variants()[index]
    dtype, bm, bn = _DTYPES[v["dtype"]], v["tile_m"], v["tile_n"]
    M = 2 * bm + 7
    ragged_k = {"bf16": 200, "fp8": 208, "mxfp4": 448}.get(dtype, 224)   # the ABI needs K % 8, % 16, % 32
    whole_k = 512 if dtype == "mxfp4" else 256
    shapes = [(2 * bn + 16, whole_k), (bn + 13, ragged_k), (bn + 12, whole_k)]
    if v["direct_only"]:
        # whole k-steps only (each of k_slices k-slices); K of one k-step and of three
        shapes = [(2 * bn + 16, v["tile_k"]), (bn + 13, 3 * v["tile_k"]), (bn + 12, v["tile_k"])]
    for N, K in shapes:
        x = exact_inputs(dtype, M, N, K, bias=True, seed=3000 + index)
        assert_exact_inputs(x)
        d = device_inputs(x)
        C, _ = oracle_full(x)
        for policy, g in [(pg.HYBRID, 0), (pg.PURE_SK, 7), (pg.PURE_DP, 3)]:
            say(f"variant {index} ({dtype} {bm}x{bn}, {v['threads']} threads) {M}x{N}x{K} policy {policy} grid {g}")
            got = run(d, grid_cap=g, policy=policy, variant=index)
            assert_bitexact(got, C, f"variant {index} {M}x{N}x{K} policy {policy} grid {g}")


@pytest.mark.parametrize("dtype", _MX)
def test_direct_scale_reads(dtype):
    """MX kernels of up to 128-row tiles read the scales straight from the caller's
    [rows][K/32] arrays when K is a whole number of k-steps and the arrays are
    4-byte aligned, and otherwise (or under DEBUG_RELAYOUT) re-lay them first.
    Every such kernel, all three policies, both paths, against the oracle;
    then scale arrays starting 4 bytes (still direct) and 1 byte (re-laid)
    into their allocation."""
    for index, v in enumerate(pg.variants()):
        if _DTYPES[v["dtype"]] != dtype or v["tile_m"] > 128:
            continue
        M, N, K = 2 * v["tile_m"] + 3, 2 * v["tile_n"] + 8, 1024
        x = exact_inputs(dtype, M, N, K, bias=True, seed=3500 + index)
        assert_exact_inputs(x)
        d = device_inputs(x)
        C, _ = oracle_full(x)
        # a direct-only kernel has no re-laid path: asked for one, it is refused
        flag_set = (0,) if v["direct_only"] else (0, pg.DEBUG_RELAYOUT)
        for policy, g in [(pg.HYBRID, 0), (pg.PURE_SK, 7), (pg.PURE_DP, 3)]:
            for flags in flag_set:
                say(f"variant {index} ({dtype} {v['tile_m']}x{v['tile_n']}) {M}x{N}x{K} policy {policy} flags {flags}")
                got = run(d, grid_cap=g, policy=policy, variant=index, debug_flags=flags)
                assert_bitexact(got, C, f"variant {index} policy {policy} flags {flags}")
        for shift in (4, 1):
            e = dict(d)
            for k in ("SA", "SB"):
                t = d[k]
                buf = torch.zeros(t.numel() + 16, dtype=torch.uint8, device=t.device)
                buf[shift:shift + t.numel()] = t.reshape(-1)
                e[k] = buf[shift:shift + t.numel()].view(t.shape)
            say(f"variant {index} scale arrays at offset {shift}")
            if v["direct_only"]:
                # (16-byte scale loads: offsets 4 and 1 are refused, below)
                continue
            got = run(e, grid_cap=0, policy=pg.HYBRID, variant=index)
            assert_bitexact(got, C, f"variant {index} scales at offset {shift}")
        if v["direct_only"]:
            for why, kw, shift in [("relayout flag", {"debug_flags": pg.DEBUG_RELAYOUT}, 0),
                                   ("scales 4 bytes off 16", {}, 4), ("scales 1 byte off", {}, 1)]:
                e = dict(d)
                if shift:
                    for k in ("SA", "SB"):
                        buf = torch.zeros(d[k].numel() + 32, dtype=torch.uint8, device=d[k].device)
                        e[k] = buf[shift:shift + d[k].numel()].view(d[k].shape)
                say(f"variant {index}: refused with {why}")
                with pytest.raises(pg.SkError) as ei:
                    run(e, grid_cap=0, policy=pg.HYBRID, variant=index, **kw)
                assert ei.value.name == "SK_ERR_UNSUPPORTED"


def _midpoint_inputs(M, N, K):
    """MXFP4 operands whose exact products sum to +-257 (seven 6*6, one 2*2, one
    1*1) or, where A's scale is 2^3, to +-2056: both lie exactly on a bf16
    rounding boundary.  The bias of column n is one of +-2^-20, +-2^-16
    (which the fp32 sum swallows or ties on, leaving it on the boundary), 0,
    -0, 1 and 2^-32, so the correct bf16 depends on the bias's sign even
    where the fp32 sum does not show it."""
    row = np.zeros(K, np.uint8)
    row[:7], row[7], row[8] = 7, 4, 2
    a = np.tile(row, (M, 1))
    a[1::2] |= 8                                   # odd rows negative
    b = np.tile(row, (N, 1))
    pack = lambda c: (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)
    sa = np.full((M, K // 32), 127, np.uint8)
    sa[2::4] = 130
    sb = np.full((N, K // 32), 127, np.uint8)
    pattern = np.array([0x3580, 0xB580, 0x3780, 0xB780, 0x0000, 0x8000, 0x3F80, 0x2F80], np.uint16)
    bias = pattern[np.arange(N) % len(pattern)]
    return {"dtype": "mxfp4", "M": M, "N": N, "K": K, "A": pack(a), "B": pack(b), "SA": sa, "SB": sb,
            "bias": bias}


def test_bias_add_on_bf16_rounding_boundaries():
    """The epilogue rounds acc + bias once: sums whose fp32 value sits exactly on
    a bf16 rounding boundary must still round by the exact sum's side of it,
    on whole and on split tiles, in the 256x256, 64x64 and 16-row kernels."""
    x = _midpoint_inputs(69, 131, 256)
    C, _ = oracle_full(x)
    # the pins of this test: 257 + 2^-20 rounds up to 258, 257 - 2^-20 down to 256, 257 to 256 (even)
    assert C[0, 0] == 0x4381 and C[0, 1] == 0x4380 and C[0, 4] == 0x4380
    d = device_inputs(x)
    for kw in [dict(policy=pg.AUTO), dict(tile=(256, 256), policy=pg.HYBRID),
               dict(tile=(64, 64), policy=pg.PURE_SK, grid_cap=7), dict(tile=(64, 64), policy=pg.PURE_DP),
               dict(tile=(16, 128), policy=pg.PURE_SK, grid_cap=11)]:
        say(f"midpoint sums {kw}")
        assert_bitexact(run(d, **kw), C, f"midpoint sums {kw}")


# ---------------------------------------------------------------- fixup protocol

def test_bias_added_exactly_once_on_split_tiles():
    # A = 0 and a bias of 1024: a missing or doubled bias on a split tile shows as 0 or 2048.
    x = make_inputs("mxfp4", 192, 256, 1024, bias=False, seed=5)
    x["A"] = np.zeros_like(x["A"])
    x["bias"] = np.full(256, 0x4480, np.uint16)            # bf16 1024.0
    d = device_inputs(x)
    for g in (2, 3, 7, 13, 64):
        say(f"bias once grid {g}")
        got = run(d, grid_cap=g, tile=(64, 64), policy=pg.PURE_SK)
        assert (got == 0x4480).all()
    y = make_inputs("mxfp4", 192, 256, 1024, bias=True, seed=6)
    C, _ = oracle_full(y)
    dy = device_inputs(y)
    for g in (2, 3, 7, 13, 64):
        assert_bitexact(run(dy, grid_cap=g, tile=(64, 64), policy=pg.PURE_SK), C, f"grid {g}")


def test_poisoned_scratch_and_stale_flags(small):
    x, d, C = small
    p = pg.plan("mxfp4", 256, 256, 512, grid_cap=7, tile=(64, 64), policy=pg.PURE_SK)
    for _ in range(3):
        say("poison then run")
        pg.poison_workspace(p.scratch_bytes)
        assert_bitexact(run(d, grid_cap=7, tile=(64, 64), policy=pg.PURE_SK), C, "after poison")


def test_delayed_publication_keeps_bits(small):
    x, d, C = small
    for seed in (1, 2, 3, 99):
        say(f"delay seed {seed}")
        got = run(d, grid_cap=7, tile=(64, 64), policy=pg.PURE_SK, debug_flags=pg.DEBUG_DELAY, delay_seed=seed)
        assert_bitexact(got, C, f"delay seed {seed}")
    y = make_inputs("bf16", 300, 260, 2048, bias=True, seed=8)
    dy = device_inputs(y)
    ref = run(dy, grid_cap=11, tile=(64, 64), policy=pg.PURE_SK)
    for seed in (4, 5):
        got = run(dy, grid_cap=11, tile=(64, 64), policy=pg.PURE_SK, debug_flags=pg.DEBUG_DELAY, delay_seed=seed)
        assert np.array_equal(got, ref)


def test_timeout_is_reported_and_recovers(small):
    x, d, C = small
    p = pg.plan("mxfp4", 256, 256, 512, grid_cap=5, tile=(64, 64), policy=pg.PURE_SK)
    # find a workgroup that publishes a partial
    w = next(w for w in range(p.grid) if any(m == 1 for (_, _, _, m, _) in pg.plan_wg_work(p, w)))
    say(f"drop signal of workgroup {w}, 1 ms spin limit")
    pg.gemm_ex("mxfp4", d["A"], d["B"], d["SA"], d["SB"], d["bias"], grid_cap=5, tile=(64, 64),
               policy=pg.PURE_SK, debug_flags=pg.DEBUG_DROP_SIGNAL, drop_signal_wg=w, spin_limit_ticks=100_000)
    with pytest.raises(pg.SkError) as e:
        pg.check()
    assert e.value.name == "SK_ERR_TIMEOUT"
    pg.check()                                   # cleared
    assert_bitexact(run(d, grid_cap=5, tile=(64, 64), policy=pg.PURE_SK), C, "after timeout")


def test_two_streams_keep_separate_scratch():
    xs = [make_inputs("mxfp4", 256, 320, 1024, bias=True, seed=s) for s in (11, 12)]
    ds = [device_inputs(x) for x in xs]
    Cs = [oracle_full(x)[0] for x in xs]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for rep in range(3):
        for d, s in zip(ds, streams):
            with torch.cuda.stream(s):
                outs.append(pg.gemm_ex("mxfp4", d["A"], d["B"], d["SA"], d["SB"], d["bias"], grid_cap=9,
                                       tile=(64, 64), policy=pg.PURE_SK, stream=s))
    for s in streams:
        pg.check(s)
    torch.cuda.synchronize()
    for i, out in enumerate(outs):
        got = out.view(torch.int16).cpu().numpy().view(np.uint16)
        assert_bitexact(got, Cs[i % 2], f"stream result {i}")


# ---------------------------------------------------------------- entry points

def test_entry_points_agree(small):
    x, d, C = small
    say("entry points")
    c1 = pg.gemm_mxfp4(d["A"], d["B"], d["SA"], d["SB"], d["bias"], grid_cap=5)
    c2 = pg.addmm("mxfp4", d["bias"], d["A"], d["B"], d["SA"], d["SB"], grid_cap=5)
    pg.check()
    for c in (c1, c2):
        assert_bitexact(c.view(torch.int16).cpu().numpy().view(np.uint16), C, "entry point")
    y = integer_inputs("bf16", 130, 70, 136, bias=True, seed=3)
    dy = device_inputs(y)
    Cy, _ = oracle_full(y)
    for c in (pg.gemm_bf16(dy["A"], dy["B"], dy["bias"]), pg.addmm("bf16", dy["bias"], dy["A"], dy["B"])):
        pg.check()
        assert_bitexact(c.view(torch.int16).cpu().numpy().view(np.uint16), Cy, "bf16 entry point")
    z = integer_inputs("fp8", 130, 70, 144, bias=True, seed=4)
    dz = device_inputs(z)
    Cz, _ = oracle_full(z)
    for c in (pg.gemm_fp8(dz["A"], dz["B"], dz["SA"], dz["SB"], dz["bias"]),
              pg.addmm("fp8", dz["bias"], dz["A"], dz["B"], dz["SA"], dz["SB"])):
        pg.check()
        assert_bitexact(c.view(torch.int16).cpu().numpy().view(np.uint16), Cz, "fp8 entry point")
    u = integer_inputs("mxfp8", 130, 70, 160, bias=True, seed=5)
    du = device_inputs(u)
    Cu, _ = oracle_full(u)
    for c in (pg.gemm_mxfp8(du["A"], du["B"], du["SA"], du["SB"], du["bias"]),
              pg.addmm("mxfp8", du["bias"], du["A"], du["B"], du["SA"], du["SB"])):
        pg.check()
        assert_bitexact(c.view(torch.int16).cpu().numpy().view(np.uint16), Cu, "mxfp8 entry point")


def test_errors_are_status_codes(small):
    x, d, C = small
    out = torch.empty(256 * 256 + 1, dtype=torch.int16, device="cuda")
    lib = pg.load()
    s = torch.cuda.current_stream().cuda_stream
    # C one element into an allocation: not 16-byte aligned
    st = lib.sk_gemm_mxfp4(d["A"].data_ptr(), d["B"].data_ptr(), d["SA"].data_ptr(), d["SB"].data_ptr(),
                           None, out.data_ptr() + 2, 256, 256, 512, 0, s)
    assert st == 2
    st = lib.sk_gemm_mxfp4(d["A"].data_ptr(), d["B"].data_ptr(), None, d["SB"].data_ptr(),
                           None, out.data_ptr(), 256, 256, 512, 0, s)
    assert st == 1
    st = lib.sk_gemm_mxfp4(d["A"].data_ptr(), d["B"].data_ptr(), d["SA"].data_ptr(), d["SB"].data_ptr(),
                           None, d["A"].data_ptr(), 256, 256, 512, 0, s)
    assert st == 1
    pg.check()


def test_graph_capture_is_refused(small):
    """A stream that is being captured into a HIP graph is refused with
    SK_ERR_UNSUPPORTED before anything is enqueued (the fixup's epoch is a kernel
    argument, so a replay would reuse it); after the capture the same call runs
    normally."""
    x, d, C = small
    lib = pg.load()
    out = torch.full((256, 256), 7.0, dtype=torch.bfloat16, device="cuda")
    side = torch.zeros(16, device="cuda")
    p = lambda t: t.data_ptr()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    got = []
    say("capture: sk_gemm_mxfp4, sk_gemm_mx and sk_check on a capturing stream")
    with torch.cuda.graph(graph):
        s = torch.cuda.current_stream().cuda_stream
        got.append(lib.sk_gemm_mxfp4(p(d["A"]), p(d["B"]), p(d["SA"]), p(d["SB"]), p(d["bias"]), p(out),
                                     256, 256, 512, 5, s))
        got.append(lib.sk_gemm_mx(0, 0, p(d["A"]), p(d["B"]), p(d["SA"]), p(d["SB"]), p(d["bias"]), p(out),
                                  256, 256, 512, 5, s))
        got.append(lib.sk_check(s))
        side.add_(1.0)
    assert got == [3, 3, 3], got
    for i in range(3):
        graph.replay()
        torch.cuda.synchronize()
        assert float(side[0]) == i + 1.0
        assert bool((out == 7.0).all()), "a refused call wrote C"
    say("after capture: the same call, eager")
    pg.gemm_mxfp4(d["A"], d["B"], d["SA"], d["SB"], d["bias"], out, grid_cap=5)
    pg.check()
    assert_bitexact(out.view(torch.int16).cpu().numpy().view(np.uint16), C, "after capture")


def test_phase_trace_is_ordered_and_changes_nothing(small):
    """A traced call gives the same bits; every workgroup's stamps are in phase order and its
    recorded item count is the length of its work list from the host planner."""
    x, d, C = small
    for policy, g in [(pg.PURE_SK, 5), (pg.HYBRID, 7), (pg.PURE_DP, 3)]:
        p = pg.plan("mxfp4", 256, 256, 512, grid_cap=g, tile=(64, 64), policy=policy)
        buf = torch.zeros(32 * p.grid, dtype=torch.int64, device="cuda")
        say(f"traced call policy {policy} grid {g}")
        got = run(d, grid_cap=g, tile=(64, 64), policy=policy, trace=buf)
        assert_bitexact(got, C, f"traced policy {policy}")
        t = buf.cpu().numpy().reshape(p.grid, 32)
        for w in range(p.grid):
            items = pg.plan_wg_work(p, w)
            assert t[w, 30] == len(items), (w, t[w, 30], len(items))
            seq = [t[w, 0], t[w, 29], t[w, 28], t[w, 27]]
            for j in range(min(len(items), 6)):
                seq += [t[w, 1 + 4 * j + i] for i in range(4)]
            seq.append(t[w, 31])
            assert all(a <= b for a, b in zip(seq, seq[1:])), (w, seq)
        s = pg.phase_summary(buf.cpu().numpy(), p.grid)
        assert s["span_us"] > 0 and len(s["items"]) == int(t[:, 30].max())


# ---------------------------------------------------------------- CU-partitioned streams

def _device_cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def test_cu_masked_stream_sizes_the_grid():
    """On a stream held to 48 CUs the grid is 48 workgroups: 256 tiles of 64x64
    then leave 16 over, so the plan has a Stream-K head of 64 tiles."""
    x = make_inputs("mxfp4", 1024, 1024, 2048, bias=True, seed=21)
    d = device_inputs(x)
    C, _ = oracle_full(x)
    out = torch.empty((1024, 1024), dtype=torch.bfloat16, device="cuda")   # allocated on torch's own stream
    torch.cuda.synchronize()
    s = pg.cu_masked_stream(range(48))
    try:
        assert pg.stream_cu_count(s) == 48
        p = pg.plan("mxfp4", 1024, 1024, 2048, tile=(64, 64), num_cus=pg.stream_cu_count(s))
        assert p.grid == 48 and p.sk_tiles == 64
        with torch.cuda.stream(s):
            for cap in (0, 100, 20):
                say(f"mxfp4 1024x1024x2048 tile 64x64 on a 48-CU stream, cap {cap}")
                assert_bitexact(run(d, tile=(64, 64), grid_cap=cap, C=out), C, f"48-CU stream cap {cap}")
    finally:
        pg.destroy_stream(s)
    assert pg.stream_cu_count(torch.cuda.current_stream()) == _device_cus()


def test_co_scheduled_gemm_beside_other_work():
    """The GEMM on one half of the CUs while a memory-bound elementwise loop
    runs on the other half: every result still equals the oracle's."""
    n = _device_cus()
    x = make_inputs("mxfp4", 2048, 2048, 4096, bias=True, seed=22)
    d = device_inputs(x)
    C, _ = oracle_full(x)
    s1 = pg.cu_masked_stream(range(n // 2))
    s2 = pg.cu_masked_stream(range(n // 2, n))
    try:
        # every tensor is allocated on torch's own stream, before the masked streams are used
        src = torch.ones(64 << 20, device="cuda")
        dst = torch.empty_like(src)
        outs = [torch.empty((2048, 2048), dtype=torch.bfloat16, device="cuda") for _ in range(4)]
        torch.cuda.synchronize()
        with torch.cuda.stream(s2):
            for _ in range(20):
                torch.add(src, 1.0, out=dst)
        with torch.cuda.stream(s1):
            for i, o in enumerate(outs):
                say(f"co-scheduled mxfp4 2048x2048x4096 call {i}")
                pg.gemm_ex("mxfp4", d["A"], d["B"], d["SA"], d["SB"], d["bias"], o)
            pg.check()
        s2.synchronize()
        for o in outs:
            assert_bitexact(o.view(torch.int16).cpu().numpy().view(np.uint16), C, "co-scheduled")
        assert float(dst[0]) == 2.0
    finally:
        pg.destroy_stream(s1)
        pg.destroy_stream(s2)


def test_fixup_many_splits_repeated_calls_exact():
    """Regression test for the publish ordering (every wave's partial stores
    complete before the flag is written): back-to-back calls whose tiles are
    all split between several workgroups, each checked bit for bit."""
    cases = [("mxfp4", 16, 8192, 4096, (16, 128)), ("mxfp4", 256, 768, 2048, (64, 64)),
             ("mxfp8", 128, 1024, 2048, (64, 64))]
    for dtype, M, N, K, tile in cases:
        x = (make_inputs(dtype, M, N, K, bias=True, seed=M + K) if dtype == "mxfp4"
             else integer_inputs(dtype, M, N, K, bias=True, seed=M + K))
        d = device_inputs(x)
        C, _ = oracle_full(x)
        outs = [torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for _ in range(24)]
        say(f"repeated split calls {dtype} {M}x{N}x{K} tile {tile}")
        for i, o in enumerate(outs):
            pg.gemm_ex(dtype, d["A"], d["B"], d["SA"], d["SB"], d["bias"], o, policy=pg.PURE_SK,
                       grid_cap=(256, 200, 97)[i % 3], tile=tile)
        pg.check()
        for o in outs:
            assert_bitexact(o.view(torch.int16).cpu().numpy().view(np.uint16), C, f"{dtype} {M}x{N}x{K} {tile}")
