"""Helpers shared by the GPU tests: move seeded host inputs to the device, run the
library through its binding, and compare with the oracle."""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import persistent_gemm_amd as pg


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def device_inputs(x: dict) -> dict:
    """Host arrays from persistent_gemm_amd.inputs -> device tensors for the binding."""
    d = {"dtype": x["dtype"], "M": x["M"], "N": x["N"], "K": x["K"]}
    dt = x["dtype"]
    if dt == "mxfp4":
        for k in ("A", "B", "SA", "SB"):
            d[k] = torch.from_numpy(np.ascontiguousarray(x[k])).cuda()
    elif dt == "mxfp8":
        for k in ("A", "B"):
            d[k] = torch.from_numpy(np.ascontiguousarray(x[k])).view(torch.float8_e4m3fn).cuda()
        for k in ("SA", "SB"):
            d[k] = torch.from_numpy(np.ascontiguousarray(x[k])).cuda()
    elif dt == "bf16":
        for k in ("A", "B"):
            d[k] = torch.from_numpy(np.ascontiguousarray(x[k]).view(np.int16)).view(torch.bfloat16).cuda()
        d["SA"] = d["SB"] = None
    else:
        for k in ("A", "B"):
            d[k] = torch.from_numpy(np.ascontiguousarray(x[k])).view(torch.float8_e4m3fn).cuda()
        d["SA"] = torch.tensor([x["SA"]], dtype=torch.float32).cuda()
        d["SB"] = torch.tensor([x["SB"]], dtype=torch.float32).cuda()
    b = x.get("bias")
    d["bias"] = None if b is None else torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).cuda()
    return d


def run(d: dict, *, bias=True, C=None, **kw) -> np.ndarray:
    """One call through sk_gemm_ex; returns C as uint16 bf16 bits (host)."""
    out = pg.gemm_ex(d["dtype"], d["A"], d["B"], d["SA"], d["SB"], d["bias"] if bias else None, C, **kw)
    pg.check()
    return out.view(torch.int16).cpu().numpy().view(np.uint16)


def oracle_full(x: dict, bias=True):
    C, D = oracle.gemm(x["dtype"], x["A"], x["B"], x["SA"], x["SB"], x["bias"] if bias else None, K=x["K"])
    return C, D


def assert_bitexact(got: np.ndarray, want: np.ndarray, what: str):
    ok = oracle.accept(got, want, None, None)
    if not ok.all():
        bad = np.argwhere(~ok)
        i, j = bad[0]
        raise AssertionError(f"{what}: {len(bad)} of {ok.size} elements differ; first at ({i},{j}): "
                             f"got 0x{int(got[i, j]):04x} want 0x{int(want[i, j]):04x}")


def assert_within_bound(got: np.ndarray, want: np.ndarray, D: np.ndarray, S: np.ndarray, what: str):
    ok = oracle.accept(got, want, D, S)
    if not ok.all():
        bad = np.argwhere(~ok)
        i, j = bad[0]
        g = oracle.decode_bf16(got[i, j])
        raise AssertionError(f"{what}: {len(bad)} of {ok.size} elements outside the bound; first at ({i},{j}): "
                             f"got {g} want {D[i, j]} (S={S[i, j]})")
