"""Measures the fastest (kernel, policy) per problem shape and writes the table
the library's SK_POLICY_AUTO reads (the best-config search of "SM-constraint-GEMM
by triton persistent kernel", description, checklist).

    python -m persistent_gemm_amd.tune [--dtypes mxfp4,bf16,fp8,mxfp8] [--reps 5]

For every dtype and every shape of a fixed log-spaced grid, each compiled kernel
of that dtype runs under each policy (HYBRID, PURE_SK, PURE_DP) on the whole
device, once per distinct plan (kernel, grid, Stream-K tiles); the median of
`reps` timed calls (HIP events on the launch stream, after warm-up calls)
ranks them.  The (up to four) challengers within RUNOFF of the fastest are
timed again together with the untuned choice, alternating, four rounds each;
the fastest of them by median is kept only if it is more than MARGIN faster
than the untuned choice (large shapes vary by several percent from run to
run, so a single timing does not separate close kernels).  Writes

* persistent_gemm_amd/csrc/sk_tuning_table.inc: the table compiled into the
  library (rebuild afterwards), one entry per shape with the kernel's tile and
  thread count, so an entry stops applying if the kernel list changes;
* profiles/tuning_table.md: per shape, the time of the untuned choice (HYBRID
  with the kernel chosen by shape), of the tuned one, and the ratio.

Inputs are seeded random operands of the right encoding (the values do not
change the timing); results are not checked here, since every kernel and policy
is covered by the parity tests.
"""

from __future__ import annotations

import argparse
import datetime
import itertools
import os
import sys

import numpy as np
import torch

import persistent_gemm_amd as pg

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
TABLE = os.path.join(HERE, "csrc", "sk_tuning_table.inc")
SUMMARY = os.path.join(ROOT, "profiles", "tuning_table.md")

DTYPE_CODE = {"mxfp4": pg.MXFP4, "bf16": pg.BF16, "fp8": pg.FP8, "mxfp8": pg.MXFP8, "mxfp6_e2m3": pg.MXFP6_E2M3,
              "mxfp6_e3m2": pg.MXFP6_E3M2, "mxfp4_mxfp8": pg.MXFP4_MXFP8, "mxfp8_mxfp4": pg.MXFP8_MXFP4}
# element format of A and of B
FORMATS = {"mxfp4_mxfp8": ("mxfp4", "mxfp8"), "mxfp8_mxfp4": ("mxfp8", "mxfp4")}
POLICIES = {"hybrid": pg.HYBRID, "sk": pg.PURE_SK, "dp": pg.PURE_DP}
MARGIN = 0.03
RUNOFF = 0.08
MS = (16, 128, 1024, 4096, 8192)
NS = (1024, 4096, 8192)
KS = (1024, 4096, 8192)


def _buffers(dtype: str, rows: int, K: int, g: torch.Generator):
    """Operand bytes and scales for `rows` rows of K elements, on the device."""
    if dtype == "mxfp4":
        x = torch.randint(0, 256, (rows, K // 2), generator=g, dtype=torch.uint8)
        s = torch.full((rows, K // 32), 127, dtype=torch.uint8)
        return x.cuda(), s.cuda()
    if dtype.startswith("mxfp6"):
        x = torch.randint(0, 256, (rows, 3 * K // 4), generator=g, dtype=torch.uint8)
        s = torch.full((rows, K // 32), 127, dtype=torch.uint8)
        return x.cuda(), s.cuda()
    if dtype == "mxfp8":
        x = torch.randn(rows, K, generator=g).to(torch.float8_e4m3fn)
        s = torch.full((rows, K // 32), 127, dtype=torch.uint8)
        return x.cuda(), s.cuda()
    if dtype == "fp8":
        return torch.randn(rows, K, generator=g).to(torch.float8_e4m3fn).cuda(), None
    return torch.randn(rows, K, generator=g).to(torch.bfloat16).cuda(), None


def _time(fn, reps: int) -> float:
    for _ in range(2):
        fn()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in ev]))


def sweep(dtype: str, reps: int):
    """Rows (M, N, K, untuned (variant, policy, ms), best (variant, policy, ms))."""
    code = DTYPE_CODE[dtype]
    kernels = [i for i, v in enumerate(pg.variants()) if v["dtype"] == code]
    g = torch.Generator().manual_seed(2024)
    Kmax, Mmax, Nmax = max(KS), max(MS), max(NS)
    fa, fb = FORMATS.get(dtype, (dtype, dtype))
    A, SA = _buffers(fa, Mmax, Kmax, g)
    B, SB = _buffers(fb, Nmax, Kmax, g)
    C = torch.empty(Mmax * Nmax, dtype=torch.bfloat16, device="cuda")
    rows = []
    for M, N, K in itertools.product(MS, NS, KS):
        row = {"mxfp4": K // 2, "mxfp6_e2m3": 3 * K // 4, "mxfp6_e3m2": 3 * K // 4}
        ka, kb = row.get(fa, K), row.get(fb, K)
        a = A.view(-1)[: M * ka].view(M, ka)
        b = B.view(-1)[: N * kb].view(N, kb)
        sa = None if SA is None else SA.view(-1)[: M * (K // 32)].view(M, K // 32)
        sb = None if SB is None else SB.view(-1)[: N * (K // 32)].view(N, K // 32)
        c = C[: M * N].view(M, N)

        def run(variant, policy):
            return lambda: pg.gemm_ex(dtype, a, b, sa, sb, None, c, policy=policy, variant=variant)

        base = pg.plan(dtype, M, N, K, policy=pg.HYBRID)
        t_base = _time(run(None, pg.HYBRID), reps)
        cands = []
        seen = {(base.variant, base.grid, base.sk_tiles)}
        for vi in kernels:
            for pname, pol in POLICIES.items():
                p = pg.plan(dtype, M, N, K, policy=pol, variant=vi)
                if (vi, p.grid, p.sk_tiles) in seen:
                    continue
                seen.add((vi, p.grid, p.sk_tiles))
                cands.append((_time(run(vi, pol), reps), vi, pname))
        cands.sort()
        best = (base.variant, "hybrid", t_base)
        # every challenger within RUNOFF of the fastest first timing, if any
        # beats the untuned choice, is timed again, alternating with it
        finalists = [c for c in cands if c[0] < t_base and c[0] <= (1.0 + RUNOFF) * cands[0][0]][:4]
        if finalists:
            tb, tn = [], {c[1:]: [] for c in finalists}
            for _ in range(4):
                tb.append(_time(run(None, pg.HYBRID), reps))
                for _t, vi, pname in finalists:
                    tn[(vi, pname)].append(_time(run(vi, POLICIES[pname]), reps))
            t_base = float(np.median(tb))
            (vi, pname), ts = min(tn.items(), key=lambda kv: float(np.median(kv[1])))
            t_new = float(np.median(ts))
            best = (vi, pname, t_new) if t_new < (1.0 - MARGIN) * t_base else (base.variant, "hybrid", t_base)
        pg.check()
        rows.append((M, N, K, (base.variant, "hybrid", t_base), best))
        print(f"{dtype} {M}x{N}x{K}: untuned kernel {base.variant} {t_base:.4f} ms, "
              f"best kernel {best[0]} {best[1]} {best[2]:.4f} ms ({t_base / best[2]:.2f}x)", flush=True)
    return rows


def _kept(table: str, summary: str, swept) -> tuple:
    """Entries (table lines) and summary rows of the dtypes not swept now, from the current files."""
    names = {v: k for k, v in DTYPE_CODE.items()}
    lines, rows = [], []
    if os.path.exists(table):
        for line in open(table):
            t = line.strip()
            if t.startswith("{") and "//" in t:
                code = int(t[1:].split(",")[0])
                if code in names and names[code] not in swept:
                    lines.append("    " + t)
    if os.path.exists(summary):
        for line in open(summary):
            cells = [c.strip() for c in line.strip().strip("|").split("|")]
            if line.startswith("| ") and cells and cells[0] in DTYPE_CODE and cells[0] not in swept:
                rows.append(line.rstrip("\n"))
    return lines, rows


def write(results: dict, table: str, summary: str, keep_others: bool = True) -> None:
    vs = pg.variants()
    # entries of the other dtypes come from the table in the tree (the outputs may be elsewhere)
    kept_lines, kept_rows = _kept(TABLE, SUMMARY, set(results)) if keep_others else ([], [])
    stamp = datetime.date.today().isoformat()
    lines = ["// Measured (kernel, policy) choices for SK_POLICY_AUTO.  Written by",
             f"// persistent_gemm_amd/tune.py ({stamp}, one MI355X): the fastest kernel and policy",
             "// at each swept shape, by the median of HIP-event timed calls.",
             "// Fields: dtype, M, N, K, kernel index, policy, tile_m, tile_n, threads.",
             "static const TuneEntry kTuneTable[] = {"]
    for dtype, rows in results.items():
        for M, N, K, _, (vi, pname, _t) in rows:
            v = vs[vi]
            lines.append(f"    {{{DTYPE_CODE[dtype]}, {M}, {N}, {K}, {vi}, {POLICIES[pname]}, "
                         f"{v['tile_m']}, {v['tile_n']}, {v['threads']}}},  // {dtype}")
    lines += kept_lines
    lines.append("    {-1, 1, 1, 1, 0, 0, 0, 0, 0},  // end marker (never matches a dtype)")
    lines.append("};")
    with open(table, "w") as f:
        f.write("\n".join(lines) + "\n")
    md = ["# Tuning table: untuned vs measured-best kernel and policy per shape", "",
          f"Command (repository root, one MI355X, {stamp}):", "",
          "```", "python -m persistent_gemm_amd.tune --dtypes " + ",".join(results), "```", "",
          "Rows of dtypes not named in the command are kept from the previous sweep.", "",
          "Untuned: HYBRID with the kernel chosen by problem shape.  Best: the fastest kernel and policy",
          "(HYBRID, PURE_SK, PURE_DP) over every compiled kernel of the dtype.  Median of timed calls",
          "(HIP events on the launch stream), whole device.", "",
          "| dtype | M | N | K | untuned kernel | untuned ms | best kernel | best policy | best ms | speedup |",
          "|---|---|---|---|---|---|---|---|---|---|"]
    for dtype, rows in results.items():
        for M, N, K, (bv, _bp, bt), (vi, pname, t) in rows:
            v = vs[vi]
            md.append(f"| {dtype} | {M} | {N} | {K} | {bv} | {bt:.4f} | {vi} ({v['tile_m']}x{v['tile_n']}, "
                      f"{v['threads']} threads) | {pname} | {t:.4f} | {bt / t:.2f} |")
    md += kept_rows
    with open(summary, "w") as f:
        f.write("\n".join(md) + "\n")


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--dtypes", default="mxfp4,bf16,fp8,mxfp8")
    ap.add_argument("--reps", type=int, default=5)
    ap.add_argument("--table-out", default=TABLE)
    ap.add_argument("--summary-out", default=SUMMARY)
    ap.add_argument("--replace-all", action="store_true",
                    help="drop the entries of dtypes not swept (default: keep them)")
    args = ap.parse_args()
    torch.cuda.set_device(0)
    results = {d: sweep(d, args.reps) for d in args.dtypes.split(",")}
    write(results, args.table_out, args.summary_out, keep_others=not args.replace_all)
    print(f"wrote {args.table_out} and {args.summary_out}; rebuild the library to use the table", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
