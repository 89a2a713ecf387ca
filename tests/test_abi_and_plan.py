"""Host-side tests of the C ABI (no GPU): exported symbols, argument checks,
and the Stream-K planner / work lists that the kernel walks."""

from __future__ import annotations

import ctypes
import itertools
import os
import re

import pytest

import persistent_gemm_amd as pg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "sk_gemm.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sk_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = pg.load()
    names = _declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), n


def test_variants_table():
    v = pg.variants()
    shapes = {(x["dtype"], x["tile_m"], x["tile_n"]) for x in v}
    for need in [(pg.MXFP4, 256, 256), (pg.MXFP4, 64, 64), (pg.MXFP4, 16, 256), (pg.BF16, 256, 256),
                 (pg.BF16, 128, 192), (pg.FP8, 256, 256), (pg.MXFP8, 256, 256), (pg.MXFP8, 16, 256)]:
        assert need in shapes
    for x in v:
        assert x["threads"] in (64, 128, 256, 512) and 0 < x["lds_bytes"] <= 160 * 1024


# ---------------------------------------------------------------- argument checks (host only)

def _args(**kw):
    a = pg._Args()
    a.dtype, a.policy = pg.MXFP4, pg.HYBRID
    a.A, a.B, a.A_scale, a.B_scale, a.C = 0x10000, 0x20000, 0x30000, 0x40000, 0x50000
    a.M, a.N, a.K = 64, 64, 128
    a.drop_signal_wg = -1
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,status", [
    (dict(A=None), 1), (dict(B=None), 1), (dict(C=None), 1), (dict(A_scale=None), 1),
    (dict(M=0), 1), (dict(N=-3), 1), (dict(K=0), 1), (dict(K=(1 << 21) + 32), 1), (dict(M=1 << 31), 1),
    (dict(dtype=8), 1), (dict(policy=9), 1),
    (dict(K=48), 2), (dict(A=0x10008), 2), (dict(C=0x50002), 2), (dict(bias=0x60001), 2),
    (dict(C=0x10000 + 64), 1),                        # C overlaps A
    (dict(dtype=pg.BF16, K=12, A_scale=None, B_scale=None), 2),
    (dict(dtype=pg.BF16), 1),                         # bf16 takes no scales
    (dict(dtype=pg.FP8, K=24), 2),
    (dict(dtype=pg.FP8, A_scale=0x30002), 2),
    (dict(dtype=pg.MXFP8, A_scale=None), 1),          # MXFP8 needs its block scales
    (dict(dtype=pg.MXFP8, B_scale=None), 1),
    (dict(dtype=pg.MXFP8, K=80), 2),                  # K must be whole 32-element scale blocks
    (dict(dtype=pg.MXFP8, C=0x30000 + 16), 1),        # C overlaps A's scales ([M][K/32] bytes)
    (dict(dtype=pg.MXFP6_E2M3, K=48), 2),
    (dict(dtype=pg.MXFP6_E3M2, A_scale=None), 1),
    (dict(dtype=pg.MXFP6_E2M3, C=0x20000 + 4096 + 16), 1),   # B spans 64 rows * 96 bytes
    (dict(dtype=pg.MXFP4_MXFP8, C=0x20000 + 6144 + 16), 1),  # B is MXFP8: 64 rows * 128 bytes
    (dict(dtype=pg.MXFP8_MXFP4, C=0x10000 + 4096 + 16), 1),  # A is MXFP8
    (dict(dtype=pg.MXFP8_MXFP4, K=80), 2),
])
def test_argument_checks(kw, status):
    a = _args(**kw)
    assert pg.load().sk_gemm_ex(ctypes.byref(a)) == status


def test_gemm_mx_format_pairs():
    """Formats that are not MX are rejected; an MXFP6 operand with one of another format has
    no compiled kernel.  Both are decided before anything touches a device."""
    lib = pg.load()
    call = lambda fa, fb: lib.sk_gemm_mx(fa, fb, 0x10000, 0x20000, 0x30000, 0x40000, None, 0x50000, 64, 64, 128,
                                         0, None)
    assert call(pg.BF16, pg.MXFP4) == 1
    assert call(pg.MXFP4, pg.FP8) == 1
    assert call(pg.MXFP4_MXFP8, pg.MXFP4_MXFP8) == 1
    assert call(pg.MXFP6_E2M3, pg.MXFP4) == 3
    assert call(pg.MXFP6_E2M3, pg.MXFP6_E3M2) == 3
    assert call(pg.MXFP8, pg.MXFP6_E3M2) == 3


def test_addmm_requires_bias():
    lib = pg.load()
    assert lib.sk_addmm(0, None, 0x10000, 0x20000, 0x30000, 0x40000, 0x50000, 64, 64, 128, 0, None) == 1


def test_status_strings():
    lib = pg.load()
    for s in range(8):
        assert lib.sk_status_string(s)
    assert b"scratch" in lib.sk_status_string(7)
    assert lib.sk_check  # exported


# ---------------------------------------------------------------- planner

def test_plan_worked_mxfp4_64x64_grid5():
    # 256 x 256 x 512 MXFP4 on 64 x 64 tiles with 128 K per iteration and 5 workgroups.
    p = pg.plan("mxfp4", 256, 256, 512, grid_cap=5, tile=(64, 64), num_cus=256)
    assert (p.tiles, p.iters_per_tile, p.grid) == (16, 4, 5)
    assert (p.sk_tiles, p.sk_iters, p.iters_per_wg, p.iters_extra) == (6, 24, 4, 4)
    assert [pg.plan_wg_range(p, w) for w in range(5)] == [(0, 5), (5, 10), (10, 15), (15, 20), (20, 24)]
    # tiles 1, 2, 3 are split; the holder of the last iteration finishes each one
    assert pg.plan_wg_work(p, 1) == [(2, 0, 2, 1, -1), (1, 1, 4, 2, 0), (7, 0, 4, 0, -1), (12, 0, 4, 0, -1)]
    ps = pg.plan("mxfp4", 256, 256, 512, grid_cap=5, tile=(64, 64), num_cus=256, policy=pg.PURE_SK)
    assert [pg.plan_wg_range(ps, w) for w in range(5)] == [(0, 13), (13, 26), (26, 39), (39, 52), (52, 64)]


def test_plan_worked_large():
    # 4096^3 bf16 on 256 x 256 tiles: 256 tiles on 256 CUs -> no Stream-K head.
    p = pg.plan("bf16", 4096, 4096, 4096, num_cus=256)
    assert (p.tile_m, p.tile_n, p.tiles, p.grid, p.sk_tiles) == (256, 256, 256, 256, 0)
    # 128 x 192 tiles: 32 x 22 = 704 tiles -> head of 192 + 256 tiles, tail of 256 (one round).
    p = pg.plan("bf16", 4096, 4096, 4096, tile=(128, 192), num_cus=256)
    assert (p.tiles, p.sk_tiles, p.tiles - p.sk_tiles) == (704, 448, 256)
    # 8192^3 MXFP4: 1024 tiles, four data-parallel rounds, no head.
    p = pg.plan("mxfp4", 8192, 8192, 8192, num_cus=256)
    assert (p.tiles, p.iters_per_tile, p.sk_tiles, p.grid) == (1024, 8192 // p.tile_k, 0, 256)
    # skinny 16 x 8192 x 8192 MXFP4: 32 tiles of 16 x 256, all Stream-K, 8 workgroups per tile.
    p = pg.plan("mxfp4", 16, 8192, 8192, num_cus=256)
    I = 8192 // p.tile_k
    assert (p.tile_m, p.tile_n, p.tiles, p.sk_tiles, p.grid, p.iters_per_wg, p.iters_extra) == \
        (16, 256, 32, 32, 256, 32 * I // 256, 0)
    # the cap clamps to the CU count
    assert pg.plan("fp8", 4096, 4096, 4096, grid_cap=300, num_cus=256).grid == 256
    assert pg.plan("fp8", 4096, 4096, 4096, grid_cap=32, num_cus=256).grid == 32


def _check_plan(p, cap):
    T, I, G = p.tiles, p.iters_per_tile, p.grid
    assert 1 <= G <= cap
    work = [pg.plan_wg_work(p, w) for w in range(G)]
    covered = {}
    finished = {}
    contrib_of = {}
    for w, items in enumerate(work):
        modes = [m for (_, _, _, m, _) in items]
        assert modes.count(1) <= 1 and (1 not in modes or modes[0] == 1)
        assert modes.count(2) <= 1
        for (t, k0, k1, m, first) in items:
            assert 0 <= t < T and 0 <= k0 < k1 <= I
            for k in range(k0, k1):
                assert (t, k) not in covered, (t, k)
                covered[(t, k)] = w
            if m == 1:
                contrib_of[w] = (t, k0, k1)
            else:
                assert t not in finished
                finished[t] = (w, k0, m, first)
    assert len(covered) == T * I
    assert sorted(finished) == list(range(T))
    for t, (w, k0, m, first) in finished.items():
        if m == 0:
            assert k0 == 0
            continue
        assert 0 <= first < w and k0 > 0
        expect = 0
        for v in range(first, w):                # contributors, in K order
            ct, c0, c1 = contrib_of[v]
            assert ct == t and c0 == expect
            expect = c1
        assert expect == k0
    return work


def _dispatch_completes(work, slots):
    """Resident-slot model: workgroups start in id order when a slot is free and run their items
    in order; an owner item waits until all its contributors have published."""
    G = len(work)
    published = set()
    pos = [0] * G
    running, next_wg, done = [], 0, 0
    while done < G:
        while len(running) < slots and next_wg < G:
            running.append(next_wg)
            next_wg += 1
        progressed = False
        for w in list(running):
            items = work[w]
            while pos[w] < len(items):
                t, k0, k1, m, first = items[pos[w]]
                if m == 2 and not all(v in published for v in range(first, w)):
                    break
                if m == 1:
                    published.add(w)
                pos[w] += 1
                progressed = True
            if pos[w] == len(items):
                running.remove(w)
                done += 1
                progressed = True
        if not progressed:
            return False
    return True


def test_plan_invariants_exhaustive():
    n = 0
    for tm, tn, I, cap, pol in itertools.product(range(1, 5), range(1, 4), range(1, 6), [1, 2, 3, 5, 7, 11, 16],
                                                 [pg.HYBRID, pg.PURE_SK, pg.PURE_DP]):
        p = pg.plan("mxfp4", 64 * tm, 64 * tn, 128 * I, grid_cap=cap, policy=pol, tile=(64, 64), num_cus=256)
        work = _check_plan(p, cap)
        for slots in (1, 2, max(1, p.grid // 2), p.grid):
            assert _dispatch_completes(work, slots), (tm, tn, I, cap, pol, slots)
        n += 1
    assert n > 1000


def test_plan_ragged_and_hybrid_shapes():
    for (M, N, K, cap) in [(100, 72, 96, 5), (300, 130, 1000 // 32 * 32, 17), (16, 8192, 8192, 256),
                           (4096, 4096, 4096, 256), (8192, 8192, 8192, 256), (1000, 3000, 2048, 256)]:
        for pol in (pg.HYBRID, pg.PURE_SK, pg.PURE_DP):
            p = pg.plan("mxfp4", M, N, K, grid_cap=cap, policy=pol, num_cus=256)
            assert p.tiles_m == -(-M // p.tile_m) and p.iters_per_tile == -(-K // p.tile_k)
            if p.tiles * p.iters_per_tile <= 20000:
                _check_plan(p, cap)


def test_stream_entry_points_check_arguments():
    lib = pg.load()
    one = (ctypes.c_uint32 * 1)(1)
    out = ctypes.c_void_p()
    assert lib.sk_stream_create_cu_masked(None, 1, ctypes.byref(out)) == 1
    assert lib.sk_stream_create_cu_masked(one, 0, ctypes.byref(out)) == 1
    assert lib.sk_stream_create_cu_masked(one, 65, ctypes.byref(out)) == 1
    assert lib.sk_stream_create_cu_masked(one, 1, None) == 1
    assert lib.sk_stream_destroy(None) == 1
    assert lib.sk_stream_cu_count(None, None) == 1


def test_auto_policy_takes_the_measured_choice():
    """AUTO plans take (kernel, policy) from the compiled table of measured
    choices at the nearest swept shape; a fixed tile or kernel runs HYBRID."""
    import re
    table = open(os.path.join(ROOT, "persistent_gemm_amd", "csrc", "sk_tuning_table.inc")).read()
    rows = [tuple(int(v) for v in m.groups()) for m in re.finditer(
        r"\{(\d+), (\d+), (\d+), (\d+), (\d+), (\d+), (\d+), (\d+), (\d+)\}", table)]
    vs = pg.variants()
    assert rows, "the table holds measured entries"
    for dtype, M, N, K, vi, pol, bm, bn, threads in rows:
        v = vs[vi]
        assert (v["dtype"], v["tile_m"], v["tile_n"], v["threads"]) == (dtype, bm, bn, threads)
        p = pg.plan(dtype, M, N, K, policy=pg.AUTO, num_cus=256)
        assert (p.variant, p.policy) == (vi, pol), (dtype, M, N, K)
        # a shape a little off the grid takes the same entry (for a direct-only
        # kernel, K whole k-steps; one that is not falls back to the choice by shape)
        dk = v["tile_k"] if v["direct_only"] else 32
        q = pg.plan(dtype, M + 8, N - 8, K + dk, policy=pg.AUTO, num_cus=256)
        assert (q.variant, q.policy) == (vi, pol), (dtype, M, N, K)
        if v["direct_only"]:
            q = pg.plan(dtype, M, N, K + 32, policy=pg.AUTO, num_cus=256)
            assert not vs[q.variant]["direct_only"] and q.policy == pg.HYBRID, (dtype, M, N, K)
    p = pg.plan(pg.MXFP4, 8192, 8192, 8192, policy=pg.AUTO, tile=(128, 128), num_cus=256)
    assert (p.tile_m, p.tile_n, p.policy) == (128, 128, pg.HYBRID)


def test_direct_only_kernels_need_whole_k_steps():
    """A k-split kernel reads only the caller's scales: it plans where K is a
    whole number of its k-steps and is refused elsewhere; a choice by tile
    shape never lands on it."""
    vs = pg.variants()
    split = [i for i, v in enumerate(vs) if v["direct_only"]]
    assert split, "k-split kernels are compiled"
    for i in split:
        v = vs[i]
        assert v["k_slices"] > 1 and v["dtype"] == pg.MXFP4
        p = pg.plan(pg.MXFP4, 16, 8192, 4 * v["tile_k"], variant=i, num_cus=256)
        assert (p.variant, p.tile_k, p.iters_per_tile) == (i, v["tile_k"], 4)
        for K in (4 * v["tile_k"] + 32, v["tile_k"] // 2):
            with pytest.raises(pg.SkError) as e:
                pg.plan(pg.MXFP4, 16, 8192, K, variant=i, num_cus=256)
            assert e.value.name == "SK_ERR_UNSUPPORTED"
        tile = (v["tile_m"], v["tile_n"])
        if any((x["dtype"], x["tile_m"], x["tile_n"]) == (pg.MXFP4, *tile) and not x["direct_only"] for x in vs):
            p = pg.plan(pg.MXFP4, 16, 8192, 8192, tile=tile, num_cus=256)
            assert not vs[p.variant]["direct_only"]
        else:
            with pytest.raises(pg.SkError):
                pg.plan(pg.MXFP4, 16, 8192, 8192, tile=tile, num_cus=256)


def test_auto_choice_cache_keeps_answers_apart():
    """The AUTO lookup remembers its last answer per host thread: interleaved
    shapes and dtypes, and several threads at once, must still each get the
    entry their own shape selects (the answers of a first, serial pass)."""
    from concurrent.futures import ThreadPoolExecutor
    queries = [(d, M, N, K) for d in (pg.MXFP4, pg.BF16, pg.FP8, pg.MXFP8)
               for (M, N, K) in ((16, 8192, 8192), (8192, 8192, 8192), (1024, 4096, 1024), (16, 1024, 1024))]

    def answer(q):
        p = pg.plan(q[0], q[1], q[2], q[3], policy=pg.AUTO, num_cus=256)
        return p.variant, p.policy, p.grid

    want = {q: answer(q) for q in queries}
    for q in reversed(queries):            # interleaved, each differing from the one before
        assert answer(q) == want[q], q
    for q in queries:                      # the same query twice in a row
        assert answer(q) == answer(q) == want[q], q
    with ThreadPoolExecutor(max_workers=4) as ex:
        got = list(ex.map(answer, queries * 8))
    assert got == [want[q] for q in queries * 8]


def test_probe_library_exports_its_probes():
    """libskprobe.so (bench.py --ceiling) is built beside the GEMM library and exports its probes."""
    import os
    path = os.path.join(os.path.dirname(pg.library_path()), "libskprobe.so")
    lib = ctypes.CDLL(path)
    assert hasattr(lib, "skp_mfma_rate") and hasattr(lib, "skp_mfma_dma") and hasattr(lib, "skp_stream")
