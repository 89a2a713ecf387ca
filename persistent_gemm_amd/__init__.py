"""persistent_gemm_amd: a Stream-K GEMM for MI355X (gfx950) behind a small C ABI.

This module is a thin ctypes binding over ``libskgemm.so`` (built from
``persistent_gemm_amd/csrc`` by ``persistent_gemm_amd/build.py``): it checks
tensor shapes and dtypes, passes device pointers and the current HIP stream,
and turns status codes into exceptions.  Every step of the GEMM runs in the
library's HIP kernels; there is no fallback.  PyTorch supplies device memory
and streams only.

Entry points mirror ``include/sk_gemm.h``:
``gemm_mxfp4``, ``gemm_mxfp8``, ``gemm_bf16``, ``gemm_fp8``, ``addmm`` and ``gemm_ex`` (policy,
tile and test hooks), plus ``plan``, ``plan_wg_range``, ``check``,
``release_workspace``, ``poison_workspace``, ``variants`` and the CU-masked
streams ``cu_masked_stream`` / ``destroy_stream`` / ``stream_cu_count``.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

__all__ = [
    "SkError", "MXFP4", "BF16", "FP8", "MXFP8", "MXFP6_E2M3", "MXFP6_E3M2", "MXFP4_MXFP8", "MXFP8_MXFP4", "HYBRID", "PURE_SK", "PURE_DP", "AUTO", "DEBUG_DELAY", "DEBUG_DROP_SIGNAL", "DEBUG_RELAYOUT",
    "library_path", "load", "gemm_mxfp4", "gemm_mxfp4_noalloc", "gemm_mxfp8", "gemm_bf16", "gemm_bf16_backward", "gemm_mx", "gemm_fp8", "addmm", "gemm_ex", "plan", "plan_wg_range",
    "plan_wg_work", "check", "release_workspace", "poison_workspace", "variants", "Plan",
    "cu_masked_stream", "destroy_stream", "stream_cu_count", "phase_summary",
]

MXFP4, BF16, FP8, MXFP8 = 0, 1, 2, 3
MXFP6_E2M3, MXFP6_E3M2, MXFP4_MXFP8, MXFP8_MXFP4 = 4, 5, 6, 7
HYBRID, PURE_SK, PURE_DP, AUTO = 0, 1, 2, 3
DEBUG_DELAY, DEBUG_DROP_SIGNAL, DEBUG_RELAYOUT = 1, 2, 4

_STATUS = {0: "SK_OK", 1: "SK_ERR_ARG", 2: "SK_ERR_ALIGN", 3: "SK_ERR_UNSUPPORTED", 4: "SK_ERR_HIP",
           5: "SK_ERR_NOMEM", 6: "SK_ERR_TIMEOUT", 7: "SK_ERR_SCRATCH"}
_DTYPES = {"mxfp4": MXFP4, "bf16": BF16, "fp8": FP8, "mxfp8": MXFP8, "mxfp6_e2m3": MXFP6_E2M3,
           "mxfp6_e3m2": MXFP6_E3M2, "mxfp4_mxfp8": MXFP4_MXFP8, "mxfp8_mxfp4": MXFP8_MXFP4}
# element format of A and of B for each block-scaled dtype
_MX_FORMATS = {MXFP4: (MXFP4, MXFP4), MXFP8: (MXFP8, MXFP8), MXFP6_E2M3: (MXFP6_E2M3, MXFP6_E2M3),
               MXFP6_E3M2: (MXFP6_E3M2, MXFP6_E3M2), MXFP4_MXFP8: (MXFP4, MXFP8), MXFP8_MXFP4: (MXFP8, MXFP4)}


class SkError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        self.name = _STATUS.get(status, str(status))
        super().__init__(f"{where}: {self.name}")


class _Args(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32), ("policy", ctypes.c_int32),
        ("A", ctypes.c_void_p), ("B", ctypes.c_void_p),
        ("A_scale", ctypes.c_void_p), ("B_scale", ctypes.c_void_p),
        ("bias", ctypes.c_void_p), ("C", ctypes.c_void_p),
        ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
        ("grid_cap", ctypes.c_int32), ("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32),
        ("stream", ctypes.c_void_p),
        ("debug_flags", ctypes.c_uint32), ("delay_seed", ctypes.c_uint32),
        ("drop_signal_wg", ctypes.c_int32), ("variant", ctypes.c_int32),
        ("spin_limit_ticks", ctypes.c_uint64),
        ("trace", ctypes.c_void_p),
    ]


class _PlanQuery(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32), ("policy", ctypes.c_int32),
        ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
        ("grid_cap", ctypes.c_int32), ("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32),
        ("num_cus", ctypes.c_int32), ("variant", ctypes.c_int32),
    ]


class _PlanInfo(ctypes.Structure):
    _fields_ = [
        ("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32), ("tile_k", ctypes.c_int32),
        ("tiles_m", ctypes.c_int32), ("tiles_n", ctypes.c_int32),
        ("tiles", ctypes.c_int64), ("iters_per_tile", ctypes.c_int32), ("grid", ctypes.c_int32),
        ("policy", ctypes.c_int32), ("variant", ctypes.c_int32),
        ("sk_tiles", ctypes.c_int64), ("sk_iters", ctypes.c_int64),
        ("iters_per_wg", ctypes.c_int64), ("iters_extra", ctypes.c_int64),
        ("scratch_bytes", ctypes.c_int64), ("threads", ctypes.c_int32), ("lds_bytes", ctypes.c_int32),
    ]


class _WorkItem(ctypes.Structure):
    _fields_ = [("tile", ctypes.c_int64), ("k0", ctypes.c_int32), ("k1", ctypes.c_int32),
                ("mode", ctypes.c_int32), ("first", ctypes.c_int32)]


@dataclass(frozen=True)
class Plan:
    tile_m: int
    tile_n: int
    tile_k: int
    tiles_m: int
    tiles_n: int
    tiles: int
    iters_per_tile: int
    grid: int
    policy: int
    variant: int
    sk_tiles: int
    sk_iters: int
    iters_per_wg: int
    iters_extra: int
    scratch_bytes: int
    threads: int
    lds_bytes: int
    _raw: object = None


_LIB = None


def library_path() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "libskgemm.so")


def load():
    """Load libskgemm.so (raises if it has not been built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python persistent_gemm_amd/build.py`")
    lib = ctypes.CDLL(path)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.sk_gemm_mxfp4.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, vp]
    lib.sk_gemm_mxfp4_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, vp]
    lib.sk_gemm_mxfp8.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, vp]
    lib.sk_gemm_bf16.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, vp]
    lib.sk_gemm_fp8.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, vp]
    lib.sk_gemm_bf16_backward.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, vp]
    lib.sk_gemm_mx.argtypes = [i32, i32, vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, vp]
    lib.sk_addmm.argtypes = [i32, vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, vp]
    lib.sk_gemm_ex.argtypes = [ctypes.POINTER(_Args)]
    lib.sk_plan.argtypes = [ctypes.POINTER(_PlanQuery), ctypes.POINTER(_PlanInfo)]
    lib.sk_plan_wg_range.argtypes = [ctypes.POINTER(_PlanInfo), ctypes.c_int32,
                                     ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)]
    lib.sk_plan_wg_work.argtypes = [ctypes.POINTER(_PlanInfo), ctypes.c_int32, ctypes.POINTER(_WorkItem),
                                    ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)]
    lib.sk_check.argtypes = [vp]
    lib.sk_release_workspace.argtypes = []
    lib.sk_release_workspace.restype = None
    lib.sk_debug_poison_workspace.argtypes = [vp, i64]
    lib.sk_num_variants.argtypes = []
    lib.sk_variant_info.argtypes = [ctypes.c_int32] + [ctypes.POINTER(ctypes.c_int32)] * 6
    lib.sk_variant_k_split.argtypes = [ctypes.c_int32] + [ctypes.POINTER(ctypes.c_int32)] * 2
    lib.sk_stream_create_cu_masked.argtypes = [ctypes.POINTER(ctypes.c_uint32), ctypes.c_int32,
                                               ctypes.POINTER(ctypes.c_void_p)]
    lib.sk_stream_destroy.argtypes = [vp]
    lib.sk_stream_cu_count.argtypes = [vp, ctypes.POINTER(ctypes.c_int32)]
    lib.sk_status_string.argtypes = [ctypes.c_int]
    lib.sk_status_string.restype = ctypes.c_char_p
    for name in ("sk_gemm_mxfp4", "sk_gemm_mxfp4_noalloc", "sk_gemm_mxfp8", "sk_gemm_bf16", "sk_gemm_bf16_backward", "sk_gemm_mx", "sk_gemm_fp8", "sk_addmm", "sk_gemm_ex", "sk_plan",
                 "sk_plan_wg_range", "sk_plan_wg_work", "sk_check", "sk_debug_poison_workspace", "sk_variant_info",
                 "sk_variant_k_split", "sk_stream_create_cu_masked", "sk_stream_destroy", "sk_stream_cu_count"):
        getattr(lib, name).restype = ctypes.c_int
    lib.sk_num_variants.restype = ctypes.c_int32
    _LIB = lib
    return lib


def _ok(status: int, where: str):
    if status != 0:
        raise SkError(status, where)


# ---------------------------------------------------------------- tensor marshalling

def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(t, stream):
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    torch = _torch()
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None and t.device.type == "cuda":
        return raw(t.device.index if t.device.index is not None else torch.cuda.current_device())
    return torch.cuda.current_stream(t.device).cuda_stream


def _need(t, name, dtypes, shape, device):
    """Raises unless t is a contiguous tensor of one of `dtypes`, of `shape`, on `device`."""
    try:
        ok = t.device == device and t.dtype in dtypes and t.shape == shape and t.is_contiguous()
    except AttributeError:
        raise TypeError(f"{name} must be a tensor") from None
    if ok:
        return
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    raise ValueError(f"{name} must be contiguous")


def _out(C, M, N, device):
    torch = _torch()
    if C is None:
        return torch.empty((M, N), dtype=torch.bfloat16, device=device)
    _need(C, "C", (torch.bfloat16, torch.int16, torch.uint16), (M, N), device)
    return C


def _mx_k(fmt, cols):
    """K of a row of `cols` bytes of MX element format fmt (E2M1 4 bits, FP6 6, E4M3 8)."""
    if fmt == MXFP4:
        return 2 * cols
    if fmt in (MXFP6_E2M3, MXFP6_E3M2):
        if cols % 3:
            raise ValueError("an MXFP6 row holds 3K/4 bytes")
        return 4 * cols // 3
    return cols


def _mx_operand(t, nm, fmt, rows, K, dev):
    torch = _torch()
    if fmt == MXFP4:
        _need(t, nm, (torch.uint8,), (rows, K // 2), dev)
    elif fmt in (MXFP6_E2M3, MXFP6_E3M2):
        _need(t, nm, (torch.uint8,), (rows, 3 * K // 4), dev)
    else:
        _need(t, nm, (torch.float8_e4m3fn, torch.uint8), (rows, K), dev)


def _marshal(dtype, A, B, A_scale, B_scale, bias, C):
    """Checks tensors for one dtype; returns (M, N, K, C)."""
    torch = _torch()
    dev = A.device
    if dtype in _MX_FORMATS:
        fa, fb = _MX_FORMATS[dtype]
        M, N = A.shape[0], B.shape[0]
        K = _mx_k(fa, A.shape[1])
        _mx_operand(A, "A", fa, M, K, dev)
        _mx_operand(B, "B", fb, N, K, dev)
        _need(A_scale, "A_scale", (torch.uint8,), (M, K // 32), dev)
        _need(B_scale, "B_scale", (torch.uint8,), (N, K // 32), dev)
    elif dtype == BF16:
        M, K = A.shape
        N = B.shape[0]
        _need(A, "A", (torch.bfloat16, torch.int16, torch.uint16), (M, K), dev)
        _need(B, "B", (torch.bfloat16, torch.int16, torch.uint16), (N, K), dev)
        if A_scale is not None or B_scale is not None:
            raise ValueError("bf16 takes no scales")
    elif dtype == FP8:
        M, K = A.shape
        N = B.shape[0]
        _need(A, "A", (torch.float8_e4m3fn, torch.uint8), (M, K), dev)
        _need(B, "B", (torch.float8_e4m3fn, torch.uint8), (N, K), dev)
        for s, nm in ((A_scale, "A_scale"), (B_scale, "B_scale")):
            if s is not None:
                _need(s, nm, (torch.float32,), tuple(s.shape), dev)
                if s.numel() != 1:
                    raise ValueError(f"{nm} must hold one fp32 value")
    else:
        raise ValueError(f"unknown dtype {dtype}")
    if bias is not None:
        _need(bias, "bias", (torch.bfloat16, torch.int16, torch.uint16), (N,), dev)
    C = _out(C, M, N, dev)
    return M, N, K, C


def _dt(dtype):
    return _DTYPES[dtype] if isinstance(dtype, str) else int(dtype)


def gemm_mxfp4(A, B, A_scale, B_scale, bias=None, C=None, grid_cap=0, stream=None):
    """C = A . B^T (+ bias) for packed MXFP4 operands; returns C (bf16 [M, N])."""
    M, N, K, C = _marshal(MXFP4, A, B, A_scale, B_scale, bias, C)
    _ok(load().sk_gemm_mxfp4(_ptr(A), _ptr(B), _ptr(A_scale), _ptr(B_scale), _ptr(bias), _ptr(C), M, N, K,
                             int(grid_cap), _stream(A, stream)), "sk_gemm_mxfp4")
    return C


def gemm_mxfp4_noalloc(A, B, A_scale, B_scale, bias=None, C=None, grid_cap=0, stream=None):
    """gemm_mxfp4 with the library's fixed device scratch (no device allocation by the
    library; pass C to avoid the binding's own torch.empty).  Returns C."""
    M, N, K, C = _marshal(MXFP4, A, B, A_scale, B_scale, bias, C)
    _ok(load().sk_gemm_mxfp4_noalloc(_ptr(A), _ptr(B), _ptr(A_scale), _ptr(B_scale), _ptr(bias), _ptr(C), M, N, K,
                                     int(grid_cap), _stream(A, stream)), "sk_gemm_mxfp4_noalloc")
    return C


def gemm_mxfp8(A, B, A_scale, B_scale, bias=None, C=None, grid_cap=0, stream=None):
    """C = A . B^T (+ bias) for MXFP8 operands (E4M3 elements, E8M0 scales per 32 K); returns C."""
    M, N, K, C = _marshal(MXFP8, A, B, A_scale, B_scale, bias, C)
    _ok(load().sk_gemm_mxfp8(_ptr(A), _ptr(B), _ptr(A_scale), _ptr(B_scale), _ptr(bias), _ptr(C), M, N, K,
                             int(grid_cap), _stream(A, stream)), "sk_gemm_mxfp8")
    return C


def gemm_bf16(A, B, bias=None, C=None, grid_cap=0, stream=None):
    M, N, K, C = _marshal(BF16, A, B, None, None, bias, C)
    _ok(load().sk_gemm_bf16(_ptr(A), _ptr(B), _ptr(bias), _ptr(C), M, N, K, int(grid_cap), _stream(A, stream)),
        "sk_gemm_bf16")
    return C


def gemm_mx(a_fmt, b_fmt, A, B, A_scale, B_scale, bias=None, C=None, grid_cap=0, stream=None):
    """C = A . B^T (+ bias) for block-scaled operands: a_fmt, b_fmt in ("mxfp4", "mxfp6_e2m3",
    "mxfp6_e3m2", "mxfp8").

    An MXFP4 operand is uint8 [rows, K/2] (packed E2M1), an MXFP6 one uint8 [rows, 3K/4] (packed
    6-bit codes), an MXFP8 one E4M3 [rows, K]; scales uint8 [rows, K/32]."""
    torch = _torch()
    fa, fb = _dt(a_fmt), _dt(b_fmt)
    fmts = (MXFP4, MXFP8, MXFP6_E2M3, MXFP6_E3M2)
    if fa not in fmts or fb not in fmts:
        raise ValueError("gemm_mx takes mxfp4, mxfp6_e2m3, mxfp6_e3m2 or mxfp8 operands")
    dev = A.device
    M = A.shape[0]
    N = B.shape[0]
    K = _mx_k(fa, A.shape[1])
    _mx_operand(A, "A", fa, M, K, dev)
    _mx_operand(B, "B", fb, N, K, dev)
    _need(A_scale, "A_scale", (torch.uint8,), (M, K // 32), dev)
    _need(B_scale, "B_scale", (torch.uint8,), (N, K // 32), dev)
    if bias is not None:
        _need(bias, "bias", (torch.bfloat16, torch.int16, torch.uint16), (N,), dev)
    C = _out(C, M, N, dev)
    _ok(load().sk_gemm_mx(fa, fb, _ptr(A), _ptr(B), _ptr(A_scale), _ptr(B_scale), _ptr(bias), _ptr(C), M, N, K,
                          int(grid_cap), _stream(A, stream)), "sk_gemm_mx")
    return C


def gemm_bf16_backward(dC, A=None, B=None, *, need_dA=True, need_dB=True, need_dbias=True, grid_cap=0,
                       stream=None):
    """Gradients of C = A . B^T + bias for bf16: returns (dA, dB, dbias), None where not asked for.

    dC is bf16 [M, N]; A [M, K] is needed for dB and B [N, K] for dA."""
    torch = _torch()
    M, N = dC.shape
    dev = dC.device
    _need(dC, "dC", (torch.bfloat16, torch.int16, torch.uint16), (M, N), dev)
    ref = A if A is not None else B
    if ref is None:
        raise ValueError("A or B is needed")
    K = ref.shape[1]
    if need_dB:
        _need(A, "A", (torch.bfloat16, torch.int16, torch.uint16), (M, K), dev)
    if need_dA:
        _need(B, "B", (torch.bfloat16, torch.int16, torch.uint16), (N, K), dev)
    dA = torch.empty((M, K), dtype=torch.bfloat16, device=dev) if need_dA else None
    dB = torch.empty((N, K), dtype=torch.bfloat16, device=dev) if need_dB else None
    db = torch.empty((N,), dtype=torch.bfloat16, device=dev) if need_dbias else None
    _ok(load().sk_gemm_bf16_backward(_ptr(dC), _ptr(A), _ptr(B), _ptr(dA), _ptr(dB), _ptr(db), M, N, K,
                                     int(grid_cap), _stream(dC, stream)), "sk_gemm_bf16_backward")
    return dA, dB, db


def gemm_fp8(A, B, A_scale=None, B_scale=None, bias=None, C=None, grid_cap=0, stream=None):
    M, N, K, C = _marshal(FP8, A, B, A_scale, B_scale, bias, C)
    _ok(load().sk_gemm_fp8(_ptr(A), _ptr(B), _ptr(A_scale), _ptr(B_scale), _ptr(bias), _ptr(C), M, N, K,
                           int(grid_cap), _stream(A, stream)), "sk_gemm_fp8")
    return C


def addmm(dtype, bias, A, B, A_scale=None, B_scale=None, C=None, grid_cap=0, stream=None):
    """addmm(bias, A, B): the dtype's GEMM with a required bias (alpha = beta = 1)."""
    d = _dt(dtype)
    M, N, K, C = _marshal(d, A, B, A_scale, B_scale, bias, C)
    _ok(load().sk_addmm(d, _ptr(bias), _ptr(A), _ptr(B), _ptr(A_scale), _ptr(B_scale), _ptr(C), M, N, K,
                        int(grid_cap), _stream(A, stream)), "sk_addmm")
    return C


def gemm_ex(dtype, A, B, A_scale=None, B_scale=None, bias=None, C=None, *, grid_cap=0, policy=HYBRID,
            tile=None, stream=None, debug_flags=0, delay_seed=0, drop_signal_wg=-1, spin_limit_ticks=0,
            variant=None, trace=None):
    """The same kernels with an explicit policy / tile and the test hooks of sk_gemm_ex.

    trace: None, or a device int64 tensor of at least 32 * grid elements that receives the
    launch's phase trace (see sk_gemm_args.trace; phase_summary turns it into durations)."""
    d = _dt(dtype)
    M, N, K, C = _marshal(d, A, B, A_scale, B_scale, bias, C)
    a = _Args()
    a.dtype, a.policy = d, int(policy)
    a.A, a.B, a.A_scale, a.B_scale = _ptr(A), _ptr(B), _ptr(A_scale), _ptr(B_scale)
    a.bias, a.C = _ptr(bias), _ptr(C)
    a.M, a.N, a.K = M, N, K
    a.grid_cap = int(grid_cap)
    a.tile_m, a.tile_n = (0, 0) if tile is None else (int(tile[0]), int(tile[1]))
    a.stream = _stream(A, stream)
    a.debug_flags, a.delay_seed = int(debug_flags), int(delay_seed)
    a.drop_signal_wg, a.spin_limit_ticks = int(drop_signal_wg), int(spin_limit_ticks)
    a.variant = 0 if variant is None else int(variant) + 1
    if trace is not None:
        p = plan(d, M, N, K, grid_cap=grid_cap, policy=policy, tile=tile, variant=variant,
                 num_cus=stream_cu_count(a.stream))
        if trace.device != A.device or trace.dtype.itemsize != 8 or trace.numel() < 32 * p.grid or \
                not trace.is_contiguous():
            raise ValueError(f"trace must be a contiguous 8-byte tensor of at least {32 * p.grid} elements on "
                             f"{A.device}")
        a.trace = trace.data_ptr()
    _ok(load().sk_gemm_ex(ctypes.byref(a)), "sk_gemm_ex")
    return C


def phase_summary(words, grid: int, plan: "Plan | None" = None) -> dict:
    """Phase durations (microseconds) from a launch's trace words (host int array of 32 * grid):
    min / median / max over the workgroups of each phase, relative to the earliest entry.
    Given the launch's plan, each item's phases are also split by the item's role
    (whole tile, contributor, owner) from the host's copy of the work lists."""
    import numpy as np
    t = np.asarray(words, dtype=np.int64).reshape(-1, 32)[:grid]
    t0 = t[:, 0].min()
    us = lambda v: (np.asarray(v, dtype=np.float64)) / 100.0
    f = lambda a: [round(float(np.min(a)), 2), round(float(np.median(a)), 2), round(float(np.max(a)), 2)]
    out = {"workgroups": int(grid), "span_us": round(float(us(t[:, 31].max() - t0)), 2),
           "entry_us": f(us(t[:, 0] - t0)), "exit_us": f(us(t[:, 31] - t0)),
           "prologue_args_us": f(us(t[:, 29] - t[:, 0])), "prologue_issue_us": f(us(t[:, 28] - t[:, 29])),
           "prologue_land_us": f(us(t[:, 27] - t[:, 28])), "items": []}
    n = t[:, 30]
    roles = None
    if plan is not None:
        names = {0: "whole", 1: "contributor", 2: "owner"}
        lists = [plan_wg_work(plan, w) for w in range(grid)]
        roles = [[names[x[3]] for x in lst] for lst in lists]
    for j in range(min(int(n.max()), 6)):
        has = n > j
        st, ke, fx, en = (t[has, 1 + 4 * j + i] for i in range(4))
        item = {"item": j, "workgroups": int(has.sum()), "start_us": f(us(st - t0)),
                "ksteps_us": f(us(ke - st)), "publish_or_wait_us": f(us(fx - ke)),
                "epilogue_us": f(us(en - fx)), "end_us": f(us(en - t0))}
        if roles is not None:
            idx = np.nonzero(has)[0]
            by = {}
            for w in idx:
                if j < len(roles[w]):
                    by.setdefault(roles[w][j], []).append(w)
            item["by_role"] = {}
            for role, ws in by.items():
                r = t[ws]
                st2, ke2, fx2, en2 = (r[:, 1 + 4 * j + i] for i in range(4))
                item["by_role"][role] = {"workgroups": len(ws), "ksteps_end_us": f(us(ke2 - t0)),
                                         "publish_or_wait_us": f(us(fx2 - ke2)), "epilogue_us": f(us(en2 - fx2)),
                                         "end_us": f(us(en2 - t0))}
        out["items"].append(item)
    return out


def plan(dtype, M, N, K, *, grid_cap=0, policy=HYBRID, tile=None, num_cus=0, variant=None) -> Plan:
    """The partition a call would use (host-only; num_cus=0 asks the current device)."""
    q = _PlanQuery()
    q.dtype, q.policy = _dt(dtype), int(policy)
    q.M, q.N, q.K = int(M), int(N), int(K)
    q.grid_cap = int(grid_cap)
    q.tile_m, q.tile_n = (0, 0) if tile is None else (int(tile[0]), int(tile[1]))
    q.num_cus = int(num_cus)
    q.variant = 0 if variant is None else int(variant) + 1
    info = _PlanInfo()
    _ok(load().sk_plan(ctypes.byref(q), ctypes.byref(info)), "sk_plan")
    vals = {f: getattr(info, f) for f, _ in _PlanInfo._fields_}
    return Plan(**vals, _raw=info)


def plan_wg_range(p: Plan, wg: int):
    b, e = ctypes.c_int64(), ctypes.c_int64()
    _ok(load().sk_plan_wg_range(ctypes.byref(p._raw), int(wg), ctypes.byref(b), ctypes.byref(e)),
        "sk_plan_wg_range")
    return b.value, e.value


def plan_wg_work(p: Plan, wg: int):
    """Ordered work list of workgroup wg: tuples (tile, k0, k1, mode, first); mode 0 whole, 1 contributor, 2 owner."""
    lib = load()
    n = ctypes.c_int32()
    _ok(lib.sk_plan_wg_work(ctypes.byref(p._raw), int(wg), None, 0, ctypes.byref(n)), "sk_plan_wg_work")
    buf = (_WorkItem * max(n.value, 1))()
    _ok(lib.sk_plan_wg_work(ctypes.byref(p._raw), int(wg), buf, n.value, ctypes.byref(n)), "sk_plan_wg_work")
    return [(x.tile, x.k0, x.k1, x.mode, x.first) for x in buf[:n.value]]


def check(stream=None):
    """Waits for the stream; raises SkError(SK_ERR_TIMEOUT) if a workgroup gave up waiting."""
    if stream is None:
        torch = _torch()
        stream = torch.cuda.current_stream().cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    _ok(load().sk_check(stream), "sk_check")


def release_workspace():
    load().sk_release_workspace()


def poison_workspace(scratch_bytes: int, stream=None):
    if stream is None:
        torch = _torch()
        stream = torch.cuda.current_stream().cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    _ok(load().sk_debug_poison_workspace(stream, int(scratch_bytes)), "sk_debug_poison_workspace")


def variants():
    """Compiled kernel shapes: list of dicts (dtype, tile_m, tile_n, tile_k, threads,
    lds_bytes, k_slices, direct_only)."""
    lib = load()
    out = []
    for i in range(lib.sk_num_variants()):
        v = [ctypes.c_int32() for _ in range(8)]
        _ok(lib.sk_variant_info(i, *[ctypes.byref(x) for x in v[:6]]), "sk_variant_info")
        _ok(lib.sk_variant_k_split(i, *[ctypes.byref(x) for x in v[6:]]), "sk_variant_k_split")
        out.append(dict(zip(("dtype", "tile_m", "tile_n", "tile_k", "threads", "lds_bytes", "k_slices", "direct_only"),
                            [x.value for x in v])))
    return out


# ---------------------------------------------------------------- CU-partitioned streams

def cu_masked_stream(cus, device=None):
    """A stream whose kernels run only on the compute units listed in `cus`
    (indices 0 .. CU count - 1), as a torch ExternalStream; the library's
    calls on it size their grid to those units.  Release with destroy_stream."""
    torch = _torch()
    cus = sorted(set(int(c) for c in cus))
    if not cus or cus[0] < 0:
        raise ValueError("cus must list compute unit indices >= 0")
    words = cus[-1] // 32 + 1
    mask = (ctypes.c_uint32 * words)()
    for c in cus:
        mask[c // 32] |= 1 << (c % 32)
    h = ctypes.c_void_p()
    _ok(load().sk_stream_create_cu_masked(mask, words, ctypes.byref(h)), "sk_stream_create_cu_masked")
    return torch.cuda.ExternalStream(h.value, device=device)


def destroy_stream(stream):
    """Waits for a stream made by cu_masked_stream, frees the library's scratch for it and destroys it."""
    _ok(load().sk_stream_destroy(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)),
        "sk_stream_destroy")


def stream_cu_count(stream=None) -> int:
    """Compute units kernels on `stream` may use (torch's current stream if None)."""
    if stream is None:
        torch = _torch()
        stream = torch.cuda.current_stream().cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    n = ctypes.c_int32()
    _ok(load().sk_stream_cu_count(stream, ctypes.byref(n)), "sk_stream_cu_count")
    return n.value
