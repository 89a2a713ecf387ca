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


# element format of A and of B per dtype
_FORMATS = {"mxfp4_mxfp8": ("mxfp4", "mxfp8"), "mxfp8_mxfp4": ("mxfp8", "mxfp4")}


def formats(dtype: str):
    return _FORMATS.get(dtype, (dtype, dtype))


def device_inputs(x: dict) -> dict:
    """Host arrays from persistent_gemm_amd.inputs -> device tensors for the binding."""
    d = {"dtype": x["dtype"], "M": x["M"], "N": x["N"], "K": x["K"]}
    for op, fmt in zip(("A", "B"), formats(x["dtype"])):
        t = np.ascontiguousarray(x[op])
        if fmt == "bf16":
            d[op] = torch.from_numpy(t.view(np.int16)).view(torch.bfloat16).cuda()
        elif fmt in ("mxfp8", "fp8"):
            d[op] = torch.from_numpy(t).view(torch.float8_e4m3fn).cuda()
        else:  # packed E2M1 or FP6 bytes
            d[op] = torch.from_numpy(t).cuda()
    if x["dtype"] == "bf16":
        d["SA"] = d["SB"] = None
    elif x["dtype"] == "fp8":
        d["SA"] = torch.tensor([x["SA"]], dtype=torch.float32).cuda()
        d["SB"] = torch.tensor([x["SB"]], dtype=torch.float32).cuda()
    else:
        for k in ("SA", "SB"):
            d[k] = torch.from_numpy(np.ascontiguousarray(x[k])).cuda()
    b = x.get("bias")
    d["bias"] = None if b is None else torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).cuda()
    return d


def run(d: dict, *, bias=True, C=None, **kw) -> np.ndarray:
    """One call through sk_gemm_ex; returns C as uint16 bf16 bits (host)."""
    out = pg.gemm_ex(d["dtype"], d["A"], d["B"], d["SA"], d["SB"], d["bias"] if bias else None, C, **kw)
    pg.check()
    return out.view(torch.int16).cpu().numpy().view(np.uint16)


def oracle_full(x: dict, bias=True):
    fa, fb = formats(x["dtype"])
    b = x["bias"] if bias else None
    if fa != fb:
        return oracle.gemm_mx(fa, fb, x["A"], x["B"], x["SA"], x["SB"], b, K=x["K"])
    return oracle.gemm(x["dtype"], x["A"], x["B"], x["SA"], x["SB"], b, K=x["K"])


def abs_sums(x: dict):
    """The oracle's S = |sigma| * sum_k |a*b| for the inputs x."""
    fa, fb = formats(x["dtype"])
    if fa != fb:
        return oracle.abs_product_sums_mx(fa, fb, x["A"], x["B"], x["SA"], x["SB"], K=x["K"])
    return oracle.abs_product_sums(x["dtype"], x["A"], x["B"], x["SA"], x["SB"], K=x["K"])


def assert_exact_inputs(x: dict):
    """The precondition of inputs.exact_inputs: every partial sum representable in fp32."""
    S = abs_sums(x)
    assert S.max() < x["exact_below"], f"inputs not exact: max S {S.max()} >= {x['exact_below']}"


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
