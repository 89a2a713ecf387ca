"""sk_gemm_mxfp4_noalloc: the MXFP4 entry point whose scratch is the library's fixed
device array.  Its results must equal sk_gemm_mxfp4's (and the oracle's, bit for
bit: MXFP4 sums are exact) on calls in a row of decreasing size, which reuse the
array that the previous call left behind; a call whose scratch would not fit is
refused before anything is enqueued."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import persistent_gemm_amd as pg
from persistent_gemm_amd.inputs import make_inputs

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from gpu_util import assert_bitexact, device_inputs, say

# largest first: 256x256 tiles whose tuned plan needs 64 MiB of partial tiles (so the
# call runs data-parallel) with re-laid scales in the array; then 128x128 and 64x64
# tiles with a Stream-K head, whose partial tiles (16 and 4 MiB) live in the array;
# then two skinny calls on the k-split kernel, data-parallel and with every tile
# split four ways (its waves' sums added before a partial is published)
SHAPES = [(3072, 3072, 2048), (1024, 1024, 4096), (512, 512, 2048), (1024, 1024, 4096), (16, 4096, 8192),
          (16, 2048, 8192)]


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def test_noalloc_matches_the_allocating_entry_point():
    for i, (M, N, K) in enumerate(SHAPES):
        x = make_inputs("mxfp4", M, N, K, bias=True, seed=4100 + i)
        d = device_inputs(x)
        C, _ = oracle.gemm("mxfp4", x["A"], x["B"], x["SA"], x["SB"], x["bias"], K=K)
        out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        ref = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        say(f"noalloc call {i}: mxfp4 {M}x{N}x{K}")
        pg.gemm_mxfp4_noalloc(d["A"], d["B"], d["SA"], d["SB"], d["bias"], out)
        pg.check()
        say(f"allocating call {i}: mxfp4 {M}x{N}x{K}")
        pg.gemm_mxfp4(d["A"], d["B"], d["SA"], d["SB"], d["bias"], ref)
        pg.check()
        got = _bits(out)
        assert np.array_equal(got, _bits(ref)), f"call {i}: noalloc differs from sk_gemm_mxfp4"
        assert_bitexact(got, C, f"noalloc call {i} {M}x{N}x{K}")


def test_noalloc_refuses_scratch_beyond_its_buffer():
    # 8192 x 8192 with K = 69632 on 256x256 tiles: 34 MiB of re-laid scales > 32 MiB
    M = N = 8192
    K = 69632
    A = torch.zeros((M, K // 2), dtype=torch.uint8, device="cuda")
    B = torch.zeros((N, K // 2), dtype=torch.uint8, device="cuda")
    SA = torch.full((M, K // 32), 127, dtype=torch.uint8, device="cuda")
    SB = torch.full((N, K // 32), 127, dtype=torch.uint8, device="cuda")
    C = torch.full((M, N), 3.0, dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    lib = pg.load()
    s = torch.cuda.current_stream().cuda_stream
    say("noalloc call beyond the fixed buffer: mxfp4 8192x8192x69632")
    st = lib.sk_gemm_mxfp4_noalloc(A.data_ptr(), B.data_ptr(), SA.data_ptr(), SB.data_ptr(), None, C.data_ptr(),
                                   M, N, K, 0, s)
    assert st == 7, st
    assert lib.sk_status_string(st) and b"scratch" in lib.sk_status_string(st)
    pg.check()
    assert bool((C == 3.0).all()), "a refused call wrote C"
    # a following call that fits still runs
    x = make_inputs("mxfp4", 512, 512, 2048, bias=False, seed=4200)
    d = device_inputs(x)
    want, _ = oracle.gemm("mxfp4", x["A"], x["B"], x["SA"], x["SB"], None, K=2048)
    say("noalloc call after the refusal: mxfp4 512x512x2048")
    out = pg.gemm_mxfp4_noalloc(d["A"], d["B"], d["SA"], d["SB"])
    pg.check()
    assert_bitexact(_bits(out), want, "after refusal")
