#!/usr/bin/env python3
"""Throughput of the exact-attention hot path on one MI355X.

One step = one pass over every kernel of the path on synthetic bf16 inputs already in HBM:
  * causal forward + backward at B=2, H=16, N=8192, d=128 (fa_fwd, then the backward's three
    phases: D preprocess, dK/dV, dQ), and
  * one split-KV decode step at B=8, H=32, KV length 65536, d=128 (fa_decode).
`value` is the attention TFLOP/s of the causal forward + backward (algorithmic FLOPs:
4 B H N^2 d, halved for the causal mask, times 3.5 for forward plus 2.5x backward), from the HIP
events around those kernels; `ms_per_step` is the wall time of the whole step including the decode.
The decode is reported in GB/s of K and V read. Every kernel's own rate and roofline fraction is
listed, and `roofline` repeats the entry of the step's kernel that takes the most time. Further
entries are timed apart from the step: the decode with grouped query heads over a paged and
over a contiguous cache, a
causal forward + backward over a batch of eight sequences of different lengths (TFLOP/s of the
valid rows and keys only), the same batch with 4 K/V heads and dropout as well, the forward + backward workload with dropout on P, with an additive
bias, with d_v = 64 and with 4 K/V heads (grouped query heads), and the FP8 forward with
incoherent processing (against the dense fp8 peak), and the forward alone on the other shapes
(B1 H1 N256 d64; B4 H16 N2048 d128 with and without the causal mask; causal B1 H32 N32768 d128
and B1 H64 N32768 d64). Last, a plain 8192^3 bf16 GEMM on random data (the vendor library) gives the rate the
matrix cores sustain on such data; every bf16 MFMA entry also carries its fraction of that rate.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from exact_attention_fa_amd import inputs, metrics  # noqa: E402

FB = dict(B=2, H=16, N=8192, d=128, causal=True, seed=3)         # forward + backward workload
DEC = dict(B=8, H=32, Nk=65536, d=128, seed=5)                  # decode workload
# forward on the other shapes: (entry, B, H, N, d, causal, launches per timed block)
SHAPES = [("fwd_b1h1n256d64", 1, 1, 256, 64, False, 200),
          ("fwd_b4h16n2048", 4, 16, 2048, 128, False, 50),
          ("fwd_b4h16n2048_causal", 4, 16, 2048, 128, True, 50),
          ("fwd_b1h32n32768", 1, 32, 32768, 128, True, 4),
          ("fwd_b1h64n32768_d64", 1, 64, 32768, 64, True, 4)]
PAGED = dict(H_kv=8, block_size=16, seed=9)  # paged GQA decode: the decode workload's first 8
                                             # K/V heads as a shuffled block cache, 4 q heads each
VARLEN = dict(B=8, H=16, N=8192, d=128, n_min=1024, causal=True, seed=21)  # variable lengths,
                                             # uniform on [n_min, N], padded to N
DROPOUT = dict(p=0.1, seed=0x5EED, offset=0)  # dropout on P over the forward+backward workload
EXT = dict(H_kv=4, p=0.1, seed=0xE47, offset=0)  # the variable-length batch with grouped K/V
                                                # heads and dropout together
FP8 = dict(incoherent=True, seed=0xF8)          # FP8 forward over the forward workload
BIAS = dict(seed=0xB1A5)  # additive bias [1, H, N, N] (shared by the batch), 2 N(0, 1) in bf16
GQA = dict(H_kv=4)  # grouped query heads: the forward+backward workload with 4 K/V heads
GEMM = dict(n=8192, seed=0x6E, reps=10)  # plain bf16 GEMM on random data: the sustained MFMA rate
# matrix-core calibration loop: 2 workgroups of 4 waves per CU, 8 independent 32x32x16 bf16
# accumulators per wave on random operands; iters per launch (about 30 ms)
CALIB = dict(blocks=512, iters=100000, iters_fp8=50000, seed=0xCA1)


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---- profiles: which kernels each bench entry launches, in the order the bench runs them ------
# A kernel instance is named as "name<template arguments>"; rocprofv3 reports some names mangled
# and some demangled, and _matches accepts either form. Entry kinds: "step" entries run
# warmup + steps times, "other" entries max(warmup, 3) + steps times, "shape" entries
# max(warmup, 3) + max(1, steps // 4) * reps times. A kernel shared by several entries has its
# calls split over them in this order.
def _k(name, *args):
    return f"{name}<{', '.join(str(a).lower() for a in args)}>"


def _mangled(key: str) -> str:
    name, args = key[:-1].split("<")
    enc = "".join(f"Lb{int(a == 'true')}E" if a in ("true", "false") else f"Li{a}E"
                  for a in args.split(", "))
    return f"{len(name)}{name}I{enc}E"


def _matches(kernel_name: str, key: str) -> bool:
    return _mangled(key) in kernel_name or f"::{key}(" in kernel_name


def _fwd(d, dv, nw, c, vl, dr, bi):
    return _k("fwd_kernel", d, dv, nw, bool(c), bool(vl), bool(dr), bool(bi))


def _dkdv(d, c, vl, dr, mode, bi, dv):
    return _k("bwd_dkdv_kernel", d, bool(c), bool(vl), bool(dr), mode, bool(bi), dv)


def _dq(d, c, vl, dr, bi, dv):
    return _k("bwd_dq_kernel", d, bool(c), bool(vl), bool(dr), bool(bi), dv)


_DELTA, _DELTA64 = _k("bwd_delta_kernel", 128), _k("bwd_delta_kernel", 64)
_COMBINE = _k("decode_combine_kernel", 128)
PROFILE_ENTRIES = [  # (entry, kind, reps, [kernel patterns])
    ("fwd", "step", 1, [_fwd(128, 128, 8, 1, 0, 0, 0)]),
    ("bwd_preprocess", "step", 1, [_DELTA]),
    ("bwd_dkdv", "step", 1, [_dkdv(128, 1, 0, 0, 0, 0, 128)]),
    ("bwd_dq", "step", 1, [_dq(128, 1, 0, 0, 0, 128)]),
    ("decode", "step", 1, [_k("decode_split_kernel", 128), _COMBINE]),
    ("decode_paged_gqa", "other", 1, [_k("decode_paged_mfma_kernel", 128, True), _COMBINE]),
    ("decode_gqa", "other", 1, [_k("decode_paged_mfma_kernel", 128, False), _COMBINE]),
    ("fwd_varlen", "other", 1, [_fwd(128, 128, 8, 1, 1, 0, 0)]),
    ("bwd_varlen", "other", 1, [_DELTA, _dkdv(128, 1, 1, 0, 0, 0, 128), _dq(128, 1, 1, 0, 0, 128)]),
    ("fwd_varlen_gqa_dropout", "other", 1, [_fwd(128, 128, 8, 1, 1, 1, 0)]),
    ("bwd_varlen_gqa_dropout", "other", 1,
     [_DELTA, _dkdv(128, 1, 1, 1, 1, 0, 128), _dkdv(128, 1, 1, 1, 2, 0, 128),
      _k("bwd_gqa_reduce_kernel", 128), _dq(128, 1, 1, 1, 0, 128)]),
    ("fwd_dropout", "other", 1, [_fwd(128, 128, 8, 1, 0, 1, 0)]),
    ("bwd_dropout", "other", 1,
     [_DELTA, _dkdv(128, 1, 0, 1, 1, 0, 128), _dkdv(128, 1, 0, 1, 2, 0, 128),
      _dq(128, 1, 0, 1, 0, 128)]),
    ("fwd_bias", "other", 1, [_fwd(128, 128, 8, 1, 0, 0, 1)]),
    ("bwd_bias", "other", 1,
     [_DELTA, _dkdv(128, 1, 0, 0, 1, 1, 128), _dkdv(128, 1, 0, 0, 2, 1, 128),
      _dq(128, 1, 0, 0, 1, 128)]),
    ("fwd_dv64", "other", 1, [_fwd(128, 64, 8, 1, 0, 0, 0)]),
    ("bwd_dv64", "other", 1, [_DELTA64, _dkdv(128, 1, 0, 0, 0, 0, 64), _dq(128, 1, 0, 0, 0, 64)]),
    ("fwd_gqa", "other", 1, [_fwd(128, 128, 8, 1, 0, 0, 0)]),
    ("bwd_gqa", "other", 1, [_DELTA, _dkdv(128, 1, 0, 0, 0, 0, 128),
                             _k("bwd_gqa_reduce_kernel", 128), _dq(128, 1, 0, 0, 0, 128)]),
    ("fwd_fp8", "other", 1, [_k("fp8_prep_kernel", 128), _k("fp8_prep_v_kernel", 128),
                             _k("fwd_fp8_kernel", 128, 4, True)]),
    ("fwd_b1h1n256d64", "shape", 200, [_fwd(64, 64, 4, 0, 0, 0, 0)]),
    ("fwd_b4h16n2048", "shape", 50, [_fwd(128, 128, 8, 0, 0, 0, 0)]),
    ("fwd_b4h16n2048_causal", "shape", 50, [_fwd(128, 128, 8, 1, 0, 0, 0)]),
    ("fwd_b1h32n32768", "shape", 4, [_fwd(128, 128, 8, 1, 0, 0, 0)]),
    ("fwd_b1h64n32768_d64", "shape", 4, [_fwd(64, 64, 4, 1, 0, 0, 0)]),
]
# sources each entry's kernels are built from (a change to any of them retires its counters)
_COMMON_SOURCES = ["fa_device.h", "fa_launch.h", "fa_api.cpp"]
KERNEL_SOURCES = {"fwd": ["fa_fwd.hip"], "bwd": ["fa_bwd.hip"], "decode": ["fa_decode.hip"],
                  "fp8": ["fa_fp8.hip"]}


def _family(entry: str) -> str:
    return "fp8" if entry == "fwd_fp8" else entry.split("_")[0]


def _source_hash(family: str) -> str:
    import hashlib
    m = hashlib.sha256()
    for src in KERNEL_SOURCES[family] + _COMMON_SOURCES:
        with open(os.path.join(ROOT, "exact_attention_fa_amd", "csrc", src), "rb") as f:
            m.update(f.read())
    return m.hexdigest()[:16]


def measured_traffic() -> dict:
    """HBM bytes per launch of each bench entry from the committed rocprofv3 counter runs
    (profiles/traffic.json), kept only for entries whose kernel sources are unchanged since."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return {}
    with open(path) as f:
        rec = json.load(f).get("entries", {})
    return {name: e["bytes_per_launch"] for name, e in rec.items()
            if e["source_hash"] == _source_hash(_family(name))}


def _entry_calls(kind: str, reps: int, steps: int, warmup: int) -> tuple[int, int]:
    """(calls, timed calls) of one bench entry's kernels."""
    if kind == "step":
        return warmup + steps, steps
    if kind == "other":
        return max(warmup, 3) + steps, steps
    timed = max(1, steps // 4) * reps
    return max(warmup, 3) + timed, timed


def _read_csv(path: str) -> list:
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _find(run: str, sub: str, suffix: str) -> str:
    for dirpath, _, files in os.walk(os.path.join(run, sub)):
        for fn in files:
            if fn.endswith(suffix):
                return os.path.join(dirpath, fn)
    raise FileNotFoundError(f"no *{suffix} under {os.path.join(run, sub)}")


def _split_calls(names: list, steps: int, warmup: int) -> dict:
    """Dispatch indices of every (entry, pattern) in the bench's order: each pattern's calls
    (in dispatch order) are handed out to the entries that use it, in PROFILE_ENTRIES order."""
    by_pat, out = {}, {}
    for entry, kind, reps, pats in PROFILE_ENTRIES:
        for pat in pats:
            if pat not in by_pat:
                by_pat[pat] = [i for i, n in enumerate(names) if _matches(n, pat)]
    taken = {p: 0 for p in by_pat}
    for entry, kind, reps, pats in PROFILE_ENTRIES:
        calls, timed = _entry_calls(kind, reps, steps, warmup)
        for pat in pats:
            idx = by_pat[pat][taken[pat]:taken[pat] + calls]
            taken[pat] += calls
            out[(entry, pat)] = (idx, timed)
    short = {p: (taken[p], len(by_pat[p])) for p in by_pat if taken[p] != len(by_pat[p])}
    if short:
        raise ValueError(f"calls expected vs found per kernel do not match the bench: {short}")
    return out


def summarize_profiles(run: str, steps: int, warmup: int, pmc_steps: int, pmc_warmup: int,
                       out_dir: str = "") -> None:
    """Write profiles/ summaries from a directory of rocprofv3 results (see the command list in
    the summaries): kernel durations per bench entry, HBM bytes per launch scaled by what the
    same counters read for a plain 1 GiB copy, and profiles/traffic.json for the bench.
    out_dir: where to write them (default: profiles/ of this repository)."""
    out_dir = out_dir or os.path.join(ROOT, "profiles")
    import statistics
    trace = _read_csv(_find(run, "stats", "kernel_trace.csv"))
    trace.sort(key=lambda r: int(r["Dispatch_Id"]))
    names = [r["Kernel_Name"] for r in trace]
    dur = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in trace]
    split = _split_calls(names, steps, warmup)
    cmd_t = ("rocprofv3 --kernel-trace --stats --output-format csv -d <out>/stats -o bench -- "
             f"python3 bench.py --steps {steps} --warmup {warmup} --cpu-heads 0")
    lines = ["# Kernel durations per bench entry: causal attention fwd+bwd B2 H16 N8192 d128, "
             "decode B8 H32 KV65536 d128, and the bench's other entries", "",
             "Command (repository root, one MI355X):", "", "    " + cmd_t, "",
             "Each entry's kernels over its timed launches (the bench's warm-up launches left out), "
             "from `bench_kernel_trace.csv`; a kernel shared by several entries has its calls "
             "handed to them in the order the bench runs them. Summarised by "
             f"`python3 bench.py --summarize-profiles <out> --steps {steps} --warmup {warmup}`.",
             "", "| entry | kernel | timed calls | average (us) | min (us) | max (us) |",
             "|---|---|---|---|---|---|"]
    entry_us = {}
    for entry, kind, reps, pats in PROFILE_ENTRIES:
        tot = 0.0
        for pat in pats:
            idx, timed = split[(entry, pat)]
            t = [dur[i] for i in idx[-timed:]] if idx else []
            if not t:
                continue
            tot += statistics.mean(t)
            lines.append(f"| {entry} | `{pat}` | {len(t)} | {statistics.mean(t):.1f} | "
                         f"{min(t):.1f} | {max(t):.1f} |")
        entry_us[entry] = tot
    lines += ["", "Per launch of each entry (sum over its kernels):", "", "| entry | average (us) |",
              "|---|---|"] + [f"| {e} | {u:.1f} |" for e, u in entry_us.items()]
    with open(os.path.join(out_dir, "kernel_durations_causal_b2h16n8192d128_"
                           "decode_b8h32k65536.md"), "w") as f:
        f.write("\n".join(lines) + "\n")

    # HBM bytes: FETCH_SIZE and WRITE_SIZE (KiB per dispatch), one counter per run
    def counter(sub, cname):
        rows = _read_csv(_find(run, sub, "counter_collection.csv"))
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        return [(r["Kernel_Name"], float(r["Counter_Value"])) for r in rows
                if r["Counter_Name"] == cname]
    copy_f = [v for n, v in counter("FETCH_SIZE_copy", "FETCH_SIZE") if "copyBuffer" in n]
    copy_w = [v for n, v in counter("WRITE_SIZE_copy", "WRITE_SIZE") if "copyBuffer" in n]
    gib_kib = float(1 << 20)
    ff, fw = gib_kib / statistics.median(copy_f), gib_kib / statistics.median(copy_w)
    fetch, write = counter("FETCH_SIZE", "FETCH_SIZE"), counter("WRITE_SIZE", "WRITE_SIZE")
    sf = _split_calls([n for n, _ in fetch], pmc_steps, pmc_warmup)
    sw = _split_calls([n for n, _ in write], pmc_steps, pmc_warmup)
    cmds = [f"rocprofv3 --pmc {c} --output-format csv -d <out>/{c} -o bench -- python3 bench.py "
            f"--steps {pmc_steps} --warmup {pmc_warmup} --cpu-heads 0" for c in ("FETCH_SIZE",
                                                                                 "WRITE_SIZE")]
    cmds += [f"rocprofv3 --pmc {c} --output-format csv -d <out>/{c}_copy -o copy -- python3 "
             f"bench.py --calibrate-copy 1024" for c in ("FETCH_SIZE", "WRITE_SIZE")]
    lines = ["# HBM traffic per launch of each bench entry: causal attention fwd+bwd B2 H16 N8192 "
             "d128, decode B8 H32 KV65536 d128, and the bench's other entries", "",
             "Commands (repository root, one MI355X), one counter per run:", ""]
    lines += ["    " + c for c in cmds]
    lines += ["", f"Calibration: a plain 1 GiB device-to-device copy reads FETCH_SIZE = "
              f"{statistics.median(copy_f):.0f} KiB and WRITE_SIZE = {statistics.median(copy_w):.0f}"
              f" KiB per dispatch for 1048576 KiB moved each way, so the scale factors are "
              f"{ff:.4f} (FETCH_SIZE) and {fw:.4f} (WRITE_SIZE). Each entry's value is the median "
              f"over its launches of the scaled sum over its kernels. Summarised by `python3 "
              f"bench.py --summarize-profiles <out> --pmc-steps {pmc_steps} --pmc-warmup "
              f"{pmc_warmup}`.", "",
              "| entry | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | scaled traffic (MB per launch) |",
              "|---|---|---|---|"]
    entries = {}
    for entry, kind, reps, pats in PROFILE_ENTRIES:
        fk = wk = 0.0
        ok = True
        for pat in pats:
            i_f, _ = sf[(entry, pat)]
            i_w, _ = sw[(entry, pat)]
            if not i_f or not i_w:
                ok = False
                break
            fk += statistics.median(fetch[i][1] for i in i_f)
            wk += statistics.median(write[i][1] for i in i_w)
        if not ok:
            continue
        nbytes = (fk * ff + wk * fw) * 1024
        entries[entry] = {"bytes_per_launch": int(nbytes),
                          "source_hash": _source_hash(_family(entry))}
        lines.append(f"| {entry} | {fk:.0f} | {wk:.0f} | {nbytes / 1e6:.1f} |")
    with open(os.path.join(out_dir, "hbm_traffic_causal_b2h16n8192d128_"
                           "decode_b8h32k65536.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    with open(os.path.join(out_dir, "traffic.json"), "w") as f:
        json.dump({"note": f"(FETCH_SIZE * {ff:.4f} + WRITE_SIZE * {fw:.4f}) KiB per launch, "
                           "from profiles/hbm_traffic_*.md", "entries": entries}, f, indent=1)
        f.write("\n")

    # matrix-core, vector-ALU and LDS counters, all in one run
    sq = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_INSTS_VALU_TRANS_F32",
          "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_WAVES", "GRBM_GUI_ACTIVE"]
    rows = _read_csv(_find(run, "mfma", "counter_collection.csv"))
    per = {}
    for r in rows:
        per.setdefault(int(r["Dispatch_Id"]), [r["Kernel_Name"], {}])[1][r["Counter_Name"]] = \
            float(r["Counter_Value"])
    disp = [per[k] for k in sorted(per)]
    sm = _split_calls([n for n, _ in disp], pmc_steps, pmc_warmup)
    lines = ["# Matrix-core, vector-ALU and LDS counters per bench entry: causal attention fwd+bwd "
             "B2 H16 N8192 d128, decode B8 H32 KV65536 d128, and the bench's other entries", "",
             "Command (repository root, one MI355X):", "",
             f"    rocprofv3 --pmc {' '.join(sq)} --output-format csv -d <out>/mfma -o bench -- "
             f"python3 bench.py --steps {pmc_steps} --warmup {pmc_warmup} --cpu-heads 0", "",
             "Per launch, the mean over the entry's launches. MfmaUtil = SQ_VALU_MFMA_BUSY_CYCLES / "
             "(GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs): the fraction of elapsed cycles the matrix "
             "cores were busy. The clock column is GRBM_GUI_ACTIVE / 8 over the kernel's average "
             "duration in the kernel-trace run: the mean shader clock while it ran (left out under "
             "100 us, where launch gaps dominate the count).", "",
             "| entry | kernel | MFMA instr | VALU instr | VALU per MFMA | transcendental instr | "
             "LDS instr | LDS bank-conflict cycles | MfmaUtil | clock (MHz) |",
             "|---|---|---|---|---|---|---|---|---|---|"]
    for entry, kind, reps, pats in PROFILE_ENTRIES:
        for pat in pats:
            idx, _ = sm[(entry, pat)]
            if not idx:
                continue
            c = {n: statistics.mean(disp[i][1].get(n, 0.0) for i in idx) for n in sq}
            util = c["SQ_VALU_MFMA_BUSY_CYCLES"] / max(c["GRBM_GUI_ACTIVE"] / 8 * 1024, 1.0)
            i_t, timed = split[(entry, pat)]
            us = statistics.mean(dur[i] for i in i_t[-timed:]) if i_t else 0.0
            mhz = f"{c['GRBM_GUI_ACTIVE'] / 8 / us:.0f}" if us >= 100 else "-"
            vpm = (f"{c['SQ_INSTS_VALU'] / c['SQ_INSTS_MFMA']:.1f}" if c["SQ_INSTS_MFMA"]
                   else "-")
            lines.append(f"| {entry} | `{pat}` | {c['SQ_INSTS_MFMA']:.3g} | {c['SQ_INSTS_VALU']:.3g}"
                         f" | {vpm} | {c['SQ_INSTS_VALU_TRANS_F32']:.3g} | {c['SQ_INSTS_LDS']:.3g} | "
                         f"{c['SQ_LDS_BANK_CONFLICT']:.3g} | {util:.2f} | {mhz} |")
    with open(os.path.join(out_dir, "mfma_valu_lds_counters_causal_b2h16n8192d128_"
                           "decode_b8h32k65536.md"), "w") as f:
        f.write("\n".join(lines) + "\n")


def cpu_baseline(heads: int) -> dict:
    """The fp64 oracle (as it stands) on `heads` heads of the forward + backward workload."""
    import oracle
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"] or threadpool_info()
        threads = max((i.get("num_threads", 1) for i in info), default=1)
        if info:
            blas = ", ".join(f"{i.get('internal_api', '?')} {i.get('version', '')} "
                             f"({i.get('num_threads', '?')} threads)".replace("  ", " ")
                             for i in info)
    except Exception:  # threadpoolctl missing: report the visible cores
        threads = os.cpu_count() or 1
    N, d = FB["N"], FB["d"]
    scale = 1.0 / math.sqrt(d)
    f = inputs.bf16_to_f64
    t = 0.0
    for h in range(heads):
        q = f(inputs.slice_bf16(FB["seed"], "q", 0, h, N, d))
        k = f(inputs.slice_bf16(FB["seed"], "k", 0, h, N, d))
        v = f(inputs.slice_bf16(FB["seed"], "v", 0, h, N, d))
        do = f(inputs.slice_bf16(FB["seed"], "do", 0, h, N, d))
        t0 = time.perf_counter()
        oracle.forward_head(q, k, v, scale, True)
        oracle.backward_head(q, k, v, do, scale, True)
        t += time.perf_counter() - t0
    flops = (metrics.attention_flops(1, heads, N, N, d, causal=True)
             + metrics.attention_flops(1, heads, N, N, d, causal=True, backward=True))
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "blas": blas, "host_cpus": os.cpu_count(),
            "sample": f"fp64 numpy oracle, forward + backward of {heads} head(s) (b=0) of the "
                      f"causal B2 H16 N8192 d128 workload, {t:.1f} s; the oracle computes the full "
                      f"unmasked score matrix, the rate uses the same causal-halved formula"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-heads", type=int, default=16,
                    help="heads of the oracle CPU baseline sample (0 = skip)")
    ap.add_argument("--summarize-profiles", default="", metavar="DIR",
                    help="only turn the rocprofv3 results under DIR into the profiles/ summaries "
                         "(no GPU needed); --steps/--warmup are those of the kernel-trace run")
    ap.add_argument("--pmc-steps", type=int, default=2)
    ap.add_argument("--pmc-warmup", type=int, default=1)
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB, three times (the "
                         "reference the HBM byte counters are scaled against), and exit")
    args = ap.parse_args()
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles, args.steps, args.warmup, args.pmc_steps,
                           args.pmc_warmup)
        return 0
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this library has no multi-GPU path "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        return 2

    import torch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy > 0:
        n = args.calibrate_copy << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {n} bytes three times")
        return 0
    from exact_attention_fa_amd import _lib as fa
    fa.load()

    def to_dev(u16):
        import numpy as np
        return torch.from_numpy(u16.view(np.int16)).view(torch.bfloat16).to(dev)

    B, H, N, d, causal = FB["B"], FB["H"], FB["N"], FB["d"], FB["causal"]
    q, k, v = (to_dev(x) for x in inputs.qkv_bf16(FB["seed"], B, H, N, N, d))
    do = to_dev(inputs.tensor_bf16(FB["seed"], "do", B, H, N, d))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa.bwd_workspace_bytes(B, H, N, N, d), dtype=torch.uint8, device=dev)
    log("forward/backward inputs resident")

    DB, DH, DN, Dd = DEC["B"], DEC["H"], DEC["Nk"], DEC["d"]
    dq1 = to_dev(inputs.tensor_bf16(DEC["seed"], "q", DB, DH, 1, Dd))
    dkc = to_dev(inputs.tensor_bf16(DEC["seed"], "k", DB, DH, DN, Dd))
    dvc = to_dev(inputs.tensor_bf16(DEC["seed"], "v", DB, DH, DN, Dd))
    dout_o = torch.empty_like(dq1)
    dout_l = torch.empty((DB, DH, 1), dtype=torch.float32, device=dev)
    splits = fa.decode_num_splits(DB, DH, DN, Dd)
    dws = torch.empty(fa.decode_workspace_bytes(DB, DH, DN, Dd, splits), dtype=torch.uint8,
                      device=dev)
    log(f"decode inputs resident (splits {splits})")

    names = ["fwd", "bwd_preprocess", "bwd_dkdv", "bwd_dq", "decode"]

    def step(ev):
        ev[0].record()
        fa.fwd(q, k, v, causal=causal, out=(o, lse))
        ev[1].record()
        fa.bwd_phase("preprocess", q, k, v, o, lse, do, dq, dk, dv, ws, causal=causal)
        ev[2].record()
        fa.bwd_phase("dkdv", q, k, v, o, lse, do, dq, dk, dv, ws, causal=causal)
        ev[3].record()
        fa.bwd_phase("dq", q, k, v, o, lse, do, dq, dk, dv, ws, causal=causal)
        ev[4].record()
        fa.decode(dq1, dkc, dvc, num_splits=splits, workspace=dws, out=(dout_o, dout_l))
        ev[5].record()

    mk = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(6)]  # noqa: E731
    for _ in range(args.warmup):
        step(mk())
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")

    events = [mk() for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for ev in events:
        step(ev)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / max(args.steps, 1)
    ms = {n: sum(ev[i].elapsed_time(ev[i + 1]) for ev in events) / len(events)
          for i, n in enumerate(names)}
    log("timed steps done: " + ", ".join(f"{n} {ms[n]:.3f} ms" for n in names))

    peak_tf, peak_bw = metrics.MI355X_BF16_DENSE_TFLOPS, metrics.MI355X_HBM_GBPS
    f_fwd = metrics.attention_flops(B, H, N, N, d, causal=causal)
    f_bwd = metrics.attention_flops(B, H, N, N, d, causal=causal, backward=True)
    gemm = f_fwd / 2  # one N x N x d product, causal-halved
    pre_bytes = 2 * B * H * N * d * 2 + B * H * N * 12  # O, dO, LSE read; -D, -LSE/scale written
    dec_bytes = metrics.decode_bytes(DB, DH, DN, Dd)

    def mfma_entry(flops, t_ms, note):
        a = flops / (t_ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": a, "peak": peak_tf, "unit": "TFLOP/s",
                "frac": a / peak_tf, "traffic": None, "ms": t_ms, "work": note}

    def hbm_entry(nbytes, t_ms, note):
        a = nbytes / (t_ms * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": a, "peak": peak_bw, "unit": "GB/s",
                "frac": a / peak_bw, "traffic": None, "ms": t_ms, "work": note}

    kernels = {
        "fwd": mfma_entry(f_fwd, ms["fwd"], "4 B H N^2 d / 2 (QK^T and PV, causal)"),
        "bwd_dkdv": mfma_entry(4 * gemm, ms["bwd_dkdv"], "4 products (S, dP, dV, dK), causal"),
        "bwd_dq": mfma_entry(1 * gemm, ms["bwd_dq"],
                             "1 algorithmic product (dQ); it also re-runs S and dP"),
        "bwd_preprocess": hbm_entry(pre_bytes, ms["bwd_preprocess"], "read O, dO and LSE, write -D and -LSE/scale"),
        "decode": hbm_entry(dec_bytes, ms["decode"],
                            "K and V read once + q, o, lse (split + combine kernels)"),
    }
    kernels["bwd_dq"]["executed_tflops"] = 3 * gemm / (ms["bwd_dq"] * 1e-3) / 1e12
    traffic = measured_traffic()
    for name, nbytes in traffic.items():
        if name in kernels:
            kernels[name]["traffic"] = nbytes
    dominant = max(kernels, key=lambda n: kernels[n]["ms"])
    roof = dict(kernels[dominant])
    roof["kernel"] = dominant

    fb_ms = ms["fwd"] + ms["bwd_preprocess"] + ms["bwd_dkdv"] + ms["bwd_dq"]
    value = (f_fwd + f_bwd) / (fb_ms * 1e-3) / 1e12
    out = {
        "metric": "attention TFLOP/s (causal fwd+bwd, bf16) + decode HBM GB/s",
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded iid N(0,1) rounded to bf16)",
        "config": {"workload": "causal attention forward+backward B=2 H=16 N=8192 d=128, plus one "
                               "split-KV decode step B=8 H=32 KV=65536 d=128",
                   "global_batch": B, "seq_len": N, "heads": H, "head_dim": d,
                   "parallelism": "single-gpu"},
        "fwd_tflops": kernels["fwd"]["achieved"],
        "fwd_frac_peak": kernels["fwd"]["frac"],
        "bwd_tflops": f_bwd / ((ms["bwd_preprocess"] + ms["bwd_dkdv"] + ms["bwd_dq"]) * 1e-3) / 1e12,
        "decode_gbps": kernels["decode"]["achieved"],
        "decode_frac_peak": kernels["decode"]["frac"],
        "decode_splits": splits,
        "kernels": kernels,
        "roofline": roof,
    }
    # ---- paged KV cache with grouped query heads (timed on its own, outside the step)
    Hkv, bs = PAGED["H_kv"], PAGED["block_size"]
    mb = DN // bs
    nblk = DB * mb
    blocks = (dkc[:, :Hkv].reshape(DB, Hkv, mb, bs, Dd).permute(0, 2, 1, 3, 4)
              .reshape(nblk, Hkv, bs, Dd))
    vblocks = (dvc[:, :Hkv].reshape(DB, Hkv, mb, bs, Dd).permute(0, 2, 1, 3, 4)
               .reshape(nblk, Hkv, bs, Dd))
    gen = torch.Generator(device="cpu").manual_seed(PAGED["seed"])
    perm = torch.randperm(nblk, generator=gen).to(dev)
    kcache = torch.empty_like(blocks)
    vcache = torch.empty_like(vblocks)
    kcache[perm] = blocks
    vcache[perm] = vblocks
    del blocks, vblocks
    table = perm.to(torch.int32).reshape(DB, mb).contiguous()
    lens = torch.full((DB,), DN, dtype=torch.int32, device=dev)
    qp = dq1.reshape(DB, DH, Dd)
    po, pl = torch.empty_like(qp), torch.empty((DB, DH), dtype=torch.float32, device=dev)
    psplits = fa.decode_paged_num_splits(DB, DH, Hkv, mb, bs, Dd)
    pws = torch.empty(fa.decode_paged_workspace_bytes(DB, DH, Hkv, mb, bs, Dd, psplits),
                      dtype=torch.uint8, device=dev)
    run_p = lambda: fa.decode_paged(qp, kcache, vcache, table, lens, num_splits=psplits,  # noqa: E731
                                    workspace=pws, out=(po, pl))
    for _ in range(max(args.warmup, 3)):
        run_p()
    torch.cuda.synchronize()
    pev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for a_, b_ in pev:
        a_.record()
        run_p()
        b_.record()
    torch.cuda.synchronize()
    p_ms = sum(a_.elapsed_time(b_) for a_, b_ in pev) / len(pev)
    p_bytes = 2 * DB * Hkv * DN * Dd * 2 + DB * DH * Dd * 2 * 2 + DB * DH * 4 + DB * mb * 4
    log(f"paged GQA decode {p_ms:.3f} ms")
    kernels["decode_paged_gqa"] = hbm_entry(
        p_bytes, p_ms, f"paged K/V cache (B{DB}, {Hkv} K/V heads, {DN} positions, block {bs}) "
                       f"read once for {DH} query heads; q, o, lse, block table; timed apart "
                       f"from the step")
    kernels["decode_paged_gqa"]["splits"] = psplits
    del kcache, vcache

    # ---- the same grouped-query decode over a contiguous cache [B, H_kv, N_k, d]
    kg, vg = dkc[:, :Hkv].contiguous(), dvc[:, :Hkv].contiguous()
    go, gl = torch.empty_like(dq1), torch.empty((DB, DH, 1), dtype=torch.float32, device=dev)
    gsplits = fa.decode_gqa_num_splits(DB, DH, Hkv, DN, Dd)
    gws = torch.empty(fa.decode_gqa_workspace_bytes(DB, DH, Hkv, DN, Dd, gsplits),
                      dtype=torch.uint8, device=dev)
    run_g = lambda: fa.decode_gqa(dq1, kg, vg, num_splits=gsplits, workspace=gws,  # noqa: E731
                                  out=(go, gl))
    for _ in range(max(args.warmup, 3)):
        run_g()
    torch.cuda.synchronize()
    gev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for a_, b_ in gev:
        a_.record()
        run_g()
        b_.record()
    torch.cuda.synchronize()
    g_ms = sum(a_.elapsed_time(b_) for a_, b_ in gev) / len(gev)
    g_bytes = 2 * DB * Hkv * DN * Dd * 2 + DB * DH * Dd * 2 * 2 + DB * DH * 4
    log(f"contiguous GQA decode {g_ms:.3f} ms")
    kernels["decode_gqa"] = hbm_entry(
        g_bytes, g_ms, f"contiguous K/V cache [B{DB}, {Hkv} K/V heads, {DN} positions, d{Dd}] read "
                       f"once for {DH} query heads; q, o, lse; timed apart from the step")
    kernels["decode_gqa"]["splits"] = gsplits
    del kg, vg

    # ---- variable-length batch: causal forward + backward (timed on its own, outside the step)
    VB, VH, VN, Vd = VARLEN["B"], VARLEN["H"], VARLEN["N"], VARLEN["d"]
    vlens_np = inputs.varlen_lengths(VARLEN["seed"], VB, VARLEN["n_min"], VN)
    vlens = torch.as_tensor(vlens_np).to(dev)
    vq, vk, vv, vdo = (to_dev(x) for x in inputs.qkv_bf16(VARLEN["seed"], VB, VH, VN, VN, Vd,
                                                            with_do=True))
    vo = torch.empty_like(vq)
    vlse = torch.empty((VB, VH, VN), dtype=torch.float32, device=dev)
    vgrads = (torch.empty_like(vq), torch.empty_like(vk), torch.empty_like(vv))
    vws = torch.empty(fa.bwd_workspace_bytes(VB, VH, VN, VN, Vd), dtype=torch.uint8, device=dev)
    vc = VARLEN["causal"]
    run_vf = lambda: fa.fwd_varlen(vq, vk, vv, vlens, vlens, causal=vc, out=(vo, vlse))  # noqa: E731
    run_vb = lambda: fa.bwd_varlen(vq, vk, vv, vo, vlse, vdo, vlens, vlens, causal=vc,  # noqa: E731
                                   workspace=vws, out=vgrads)
    for _ in range(max(args.warmup, 3)):
        run_vf()
        run_vb()
    torch.cuda.synchronize()
    vev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for e in vev:
        e[0].record()
        run_vf()
        e[1].record()
        run_vb()
        e[2].record()
    torch.cuda.synchronize()
    vf_ms = sum(e[0].elapsed_time(e[1]) for e in vev) / len(vev)
    vb_ms = sum(e[1].elapsed_time(e[2]) for e in vev) / len(vev)
    vf_flops = sum(metrics.attention_flops(1, VH, int(n), int(n), Vd, causal=vc) for n in vlens_np)
    log(f"varlen fwd {vf_ms:.3f} ms, bwd {vb_ms:.3f} ms (lengths {vlens_np.tolist()})")
    vnote = (f"B{VB} H{VH} d{Vd} causal, lengths {vlens_np.tolist()} padded to {VN}: FLOPs of "
             f"the valid rows and keys only")
    kernels["fwd_varlen"] = mfma_entry(vf_flops, vf_ms, vnote)
    kernels["bwd_varlen"] = mfma_entry(2.5 * vf_flops, vb_ms,
                                       vnote + "; preprocess + dK/dV + dQ, 2.5x the forward")

    # ---- the same batch with grouped K/V heads and dropout too (fa_fwd_ext / fa_bwd_ext): the
    # first EXT["H_kv"] K/V heads shared by all query heads, dropout on P
    eh = EXT["H_kv"]
    ek, ev = vk[:, :eh].contiguous(), vv[:, :eh].contiguous()
    egrads = (torch.empty_like(vq), torch.empty_like(ek), torch.empty_like(ev))
    ews = torch.empty(fa.bwd_ext_workspace_bytes(VB, VH, eh, VN, VN, Vd), dtype=torch.uint8,
                      device=dev)
    ep, es, eo = EXT["p"], EXT["seed"], EXT["offset"]
    run_ef = lambda: fa.fwd_ext(vq, ek, ev, vlens, vlens, ep, es, eo, causal=vc,  # noqa: E731
                                out=(vo, vlse))
    run_eb = lambda: fa.bwd_ext(vq, ek, ev, vo, vlse, vdo, vlens, vlens, ep, es, eo,  # noqa: E731
                                causal=vc, workspace=ews, out=egrads)
    for _ in range(max(args.warmup, 3)):
        run_ef()
        run_eb()
    torch.cuda.synchronize()
    eev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for e in eev:
        e[0].record()
        run_ef()
        e[1].record()
        run_eb()
        e[2].record()
    torch.cuda.synchronize()
    ef_ms = sum(e[0].elapsed_time(e[1]) for e in eev) / len(eev)
    eb_ms = sum(e[1].elapsed_time(e[2]) for e in eev) / len(eev)
    log(f"varlen + GQA + dropout fwd {ef_ms:.3f} ms, bwd {eb_ms:.3f} ms")
    enote = (vnote + f", {eh} K/V heads ({VH // eh} query heads each), dropout p = {ep}")
    kernels["fwd_varlen_gqa_dropout"] = mfma_entry(vf_flops, ef_ms, enote)
    kernels["bwd_varlen_gqa_dropout"] = mfma_entry(
        2.5 * vf_flops, eb_ms, enote + "; preprocess + dK/dV + dQ, 2.5x the forward")
    del vq, vk, vv, vdo, vo, vgrads, vws, ek, ev, egrads, ews

    # ---- dropout on P: the forward + backward workload again (timed on its own, outside the step)
    dp_, dseed, doff = DROPOUT["p"], DROPOUT["seed"], DROPOUT["offset"]
    run_df = lambda: fa.fwd_dropout(q, k, v, dp_, dseed, doff, causal=causal, out=(o, lse))  # noqa: E731
    run_db = lambda: fa.bwd_dropout(q, k, v, o, lse, do, dp_, dseed, doff, causal=causal,  # noqa: E731
                                    workspace=ws, out=(dq, dk, dv))
    for _ in range(max(args.warmup, 3)):
        run_df()
        run_db()
    torch.cuda.synchronize()
    dev_ = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for e in dev_:
        e[0].record()
        run_df()
        e[1].record()
        run_db()
        e[2].record()
    torch.cuda.synchronize()
    df_ms = sum(e[0].elapsed_time(e[1]) for e in dev_) / len(dev_)
    db_ms = sum(e[1].elapsed_time(e[2]) for e in dev_) / len(dev_)
    log(f"dropout fwd {df_ms:.3f} ms, bwd {db_ms:.3f} ms (p = {dp_})")
    dnote = (f"causal B{B} H{H} N{N} d{d}, dropout p = {dp_} (mask regenerated by "
             f"Philox-4x32-10 in every kernel)")
    kernels["fwd_dropout"] = mfma_entry(f_fwd, df_ms, dnote)
    kernels["bwd_dropout"] = mfma_entry(f_bwd, db_ms, dnote + "; preprocess + dK/dV + dQ")

    # ---- additive bias [1, H, N, N] on the forward + backward workload, timed on its own
    gen_b = torch.Generator(device=dev).manual_seed(BIAS["seed"])
    bias_t = (2 * torch.randn((1, H, N, N), generator=gen_b, device=dev)).to(torch.bfloat16)
    run_bf = lambda: fa.fwd_bias(q, k, v, bias_t, causal=causal, out=(o, lse))  # noqa: E731
    run_bb = lambda: fa.bwd_bias(q, k, v, o, lse, do, bias_t, causal=causal,  # noqa: E731
                                 workspace=ws, out=(dq, dk, dv))
    for _ in range(max(args.warmup, 3)):
        run_bf()
        run_bb()
    torch.cuda.synchronize()
    bev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for e in bev:
        e[0].record()
        run_bf()
        e[1].record()
        run_bb()
        e[2].record()
    torch.cuda.synchronize()
    bf_ms = sum(e[0].elapsed_time(e[1]) for e in bev) / len(bev)
    bb_ms = sum(e[1].elapsed_time(e[2]) for e in bev) / len(bev)
    log(f"bias fwd {bf_ms:.3f} ms, bwd {bb_ms:.3f} ms")
    bnote = f"causal B{B} H{H} N{N} d{d} plus a bf16 bias [1, {H}, {N}, {N}] read from HBM"
    kernels["fwd_bias"] = mfma_entry(f_fwd, bf_ms, bnote)
    kernels["bwd_bias"] = mfma_entry(f_bwd, bb_ms, bnote + "; preprocess + dK/dV + dQ")
    del bias_t

    # ---- V with its own head dimension: d = 128, d_v = 64 on the forward + backward workload
    vsmall = v[..., :64].contiguous()
    dosmall = do[..., :64].contiguous()
    o64 = torch.empty((B, H, N, 64), dtype=torch.bfloat16, device=dev)
    dv64 = torch.empty_like(vsmall)
    run_vf2 = lambda: fa.fwd_dv(q, k, vsmall, causal=causal, out=(o64, lse))  # noqa: E731
    run_vb2 = lambda: fa.bwd_dv(q, k, vsmall, o64, lse, dosmall, causal=causal,  # noqa: E731
                                workspace=ws, out=(dq, dk, dv64))
    for _ in range(max(args.warmup, 3)):
        run_vf2()
        run_vb2()
    torch.cuda.synchronize()
    dvev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for e in dvev:
        e[0].record()
        run_vf2()
        e[1].record()
        run_vb2()
        e[2].record()
    torch.cuda.synchronize()
    dvf_ms = sum(e[0].elapsed_time(e[1]) for e in dvev) / len(dvev)
    dvb_ms = sum(e[1].elapsed_time(e[2]) for e in dvev) / len(dvev)
    log(f"d_v = 64 fwd {dvf_ms:.3f} ms, bwd {dvb_ms:.3f} ms")
    # FLOPs: QK^T with d = 128 and PV with d_v = 64 per visible pair; backward 2.5x
    f_dv = metrics.attention_flops(B, H, N, N, (d + 64) // 2, causal=causal)
    dvnote = f"causal B{B} H{H} N{N}, d = {d}, d_v = 64 (2 N^2 (d + d_v) FLOPs, causal-halved)"
    kernels["fwd_dv64"] = mfma_entry(f_dv, dvf_ms, dvnote)
    kernels["bwd_dv64"] = mfma_entry(2.5 * f_dv, dvb_ms, dvnote + "; preprocess + dK/dV + dQ")
    del vsmall, dosmall, o64, dv64

    # ---- grouped query heads: the forward + backward workload with H_kv = 4 (4 query heads per
    # K/V head; K and V are the first 4 heads of the workload's), timed on its own
    Hkv = GQA["H_kv"]
    kg, vg = k[:, :Hkv].contiguous(), v[:, :Hkv].contiguous()
    dkg, dvg = torch.empty_like(kg), torch.empty_like(vg)
    gws = torch.empty(fa.bwd_gqa_workspace_bytes(B, H, Hkv, N, N, d), dtype=torch.uint8,
                      device=dev)
    run_gf = lambda: fa.fwd_gqa(q, kg, vg, causal=causal, out=(o, lse))  # noqa: E731
    run_gb = lambda: fa.bwd_gqa(q, kg, vg, o, lse, do, causal=causal, workspace=gws,  # noqa: E731
                                out=(dq, dkg, dvg))
    for _ in range(max(args.warmup, 3)):
        run_gf()
        run_gb()
    torch.cuda.synchronize()
    gev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for e in gev:
        e[0].record()
        run_gf()
        e[1].record()
        run_gb()
        e[2].record()
    torch.cuda.synchronize()
    gf_ms = sum(e[0].elapsed_time(e[1]) for e in gev) / len(gev)
    gb_ms = sum(e[1].elapsed_time(e[2]) for e in gev) / len(gev)
    log(f"grouped query heads fwd {gf_ms:.3f} ms, bwd {gb_ms:.3f} ms (H_kv = {Hkv})")
    gnote = f"causal B{B} H{H} N{N} d{d} with {Hkv} K/V heads ({H // Hkv} query heads each)"
    kernels["fwd_gqa"] = mfma_entry(f_fwd, gf_ms, gnote)
    kernels["bwd_gqa"] = mfma_entry(f_bwd, gb_ms, gnote + "; preprocess + dK/dV + dQ")
    del kg, vg, dkg, dvg, gws

    # ---- FP8 forward with incoherent processing (rotation + quantization + attention on the
    # codes), the forward workload again, timed on its own
    f8ws = torch.empty(fa.fwd_fp8_workspace_bytes(B, H, N, N, d), dtype=torch.uint8, device=dev)
    run_f8 = lambda: fa.fwd_fp8(q, k, v, causal=causal, incoherent=FP8["incoherent"],  # noqa: E731
                                seed=FP8["seed"], workspace=f8ws, out=(o, lse))
    for _ in range(max(args.warmup, 3)):
        run_f8()
    torch.cuda.synchronize()
    fev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for a_, b_ in fev:
        a_.record()
        run_f8()
        b_.record()
    torch.cuda.synchronize()
    f8_ms = sum(a_.elapsed_time(b_) for a_, b_ in fev) / len(fev)
    log(f"fp8 forward {f8_ms:.3f} ms (rotation + quantization + attention)")
    e8 = mfma_entry(f_fwd, f8_ms, f"causal B{B} H{H} N{N} d{d}: signed Hadamard rotation of Q, K, "
                                  f"E4M3 quantization of Q, K, V and attention on the codes, "
                                  f"against the dense fp8 peak")
    e8["peak"] = metrics.MI355X_FP8_DENSE_TFLOPS
    e8["frac"] = e8["achieved"] / e8["peak"]
    kernels["fwd_fp8"] = e8
    del f8ws

    # ---- the forward on the other shapes of the workload table (iid N(0, 1) bf16 inputs): R
    # back-to-back launches between one event pair, so that launch overhead does not dominate the
    # small ones
    for sname, sB, sH, sN, sd, scausal, reps in SHAPES:
        sq, sk, sv = (torch.randn((sB, sH, sN, sd), device=dev).to(torch.bfloat16) for _ in range(3))
        so = torch.empty_like(sq)
        sl = torch.empty((sB, sH, sN), dtype=torch.float32, device=dev)
        run_s = lambda: fa.fwd(sq, sk, sv, causal=scausal, out=(so, sl))  # noqa: E731
        for _ in range(max(args.warmup, 3)):
            run_s()
        torch.cuda.synchronize()
        sev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(max(1, args.steps // 4))]
        for a_, b_ in sev:
            a_.record()
            for _ in range(reps):
                run_s()
            b_.record()
        torch.cuda.synchronize()
        s_ms = sum(a_.elapsed_time(b_) for a_, b_ in sev) / len(sev) / reps
        log(f"forward {sname} {s_ms:.4f} ms")
        kernels[sname] = mfma_entry(metrics.attention_flops(sB, sH, sN, sN, sd, causal=scausal),
                                    s_ms, f"{'causal' if scausal else 'non-causal'} B{sB} H{sH} "
                                          f"N{sN} d{sd}, average of {reps} back-to-back launches")
        del sq, sk, sv, so, sl

    for name, nbytes in traffic.items():  # the entries timed apart from the step
        if name in kernels and kernels[name]["traffic"] is None:
            kernels[name]["traffic"] = nbytes

    # ---- the vendor GEMM on random bf16 data, for context beside the published-peak fractions:
    # with operands like the attention's the card holds a shader clock well below the 2.4 GHz the
    # published peak assumes, so this is what its matrix cores sustain on such data
    gm = GEMM["n"]
    gen_g = torch.Generator(device=dev).manual_seed(GEMM["seed"])
    ga = torch.randn((gm, gm), generator=gen_g, device=dev).to(torch.bfloat16)
    gb = torch.randn((gm, gm), generator=gen_g, device=dev).to(torch.bfloat16)
    gc = torch.empty((gm, gm), dtype=torch.bfloat16, device=dev)
    for _ in range(3):
        torch.matmul(ga, gb, out=gc)
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record()
    for _ in range(GEMM["reps"]):
        torch.matmul(ga, gb, out=gc)
    g1.record()
    torch.cuda.synchronize()
    g_ms = g0.elapsed_time(g1) / GEMM["reps"]
    g_tf = 2.0 * gm ** 3 / (g_ms * 1e-3) / 1e12
    log(f"bf16 GEMM {gm}^3 on N(0,1) data: {g_ms:.3f} ms, {g_tf:.0f} TFLOP/s")
    out["gemm_bf16_random"] = {
        "what": f"torch.matmul {gm} x {gm} x {gm} bf16 (hipBLASLt), iid N(0,1) operands",
        "tflops": g_tf, "frac_peak": g_tf / peak_tf}
    for e in kernels.values():
        if e["unit"] == "TFLOP/s" and e["peak"] == peak_tf:
            e["frac_of_gemm"] = e["achieved"] / g_tf
    roof["frac_of_gemm"] = kernels[dominant].get("frac_of_gemm")
    del ga, gb, gc

    # ---- the matrix cores' own ceiling on random bf16 operands, and the shader clock meanwhile
    # (libfa_calib.so: a loop of independent 32x32x16 bf16 MFMAs, no memory traffic, timed by
    # events; the clock from each wave's s_memtime against s_memrealtime at 100 MHz)
    import ctypes
    calib = ctypes.CDLL(os.path.join(ROOT, "exact_attention_fa_amd", "libfa_calib.so"))
    calib.fa_calib_mfma_bf16.restype = ctypes.c_int
    calib.fa_calib_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    cb, ci = CALIB["blocks"], CALIB["iters"]
    gen_c = torch.Generator(device=dev).manual_seed(CALIB["seed"])
    c_ops = torch.randn((cb * 256 * 16 * 8,), generator=gen_c, device=dev).to(torch.bfloat16)
    c_clk = torch.zeros((cb * 4, 4), dtype=torch.int64, device=dev)
    c_sink = torch.empty((cb * 256,), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    run_c = lambda: calib.fa_calib_mfma_bf16(c_ops.data_ptr(), cb, ci, c_clk.data_ptr(),  # noqa: E731
                                             c_sink.data_ptr(), stream)
    if run_c() != 0:
        raise RuntimeError("calibration loop failed to launch")
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    run_c()
    c1.record()
    torch.cuda.synchronize()
    c_ms = c0.elapsed_time(c1)
    c_tf = cb * 4 * ci * 8 * 2.0 * 32 * 32 * 16 / (c_ms * 1e-3) / 1e12
    clk = c_clk.cpu().double()
    mhz = float(((clk[:, 1] - clk[:, 0]) / (clk[:, 3] - clk[:, 2]) * 100.0).median())
    log(f"MFMA loop on random bf16: {c_ms:.2f} ms, {c_tf:.0f} TFLOP/s at {mhz:.0f} MHz")
    out["mfma_ceiling_bf16"] = {
        "what": f"{cb} workgroups x 4 waves, each {ci} x 8 independent v_mfma_f32_32x32x16_bf16 "
                "on random bf16 operands (no memory traffic)",
        "tflops": c_tf, "frac_peak": c_tf / peak_tf, "clock_mhz": mhz,
        "peak_at_clock": peak_tf * mhz / 2400.0}
    for e in kernels.values():
        if e["unit"] == "TFLOP/s" and e["peak"] == peak_tf:
            e["frac_of_mfma_ceiling"] = e["achieved"] / c_tf
    roof["frac_of_mfma_ceiling"] = kernels[dominant].get("frac_of_mfma_ceiling")
    out["fwd_frac_of_mfma_ceiling"] = kernels["fwd"]["frac_of_mfma_ceiling"]
    del c_ops
    # the same on random E4M3 codes (never the NaN codes 0x7F, 0xFF): the FP8 forward's ceiling
    calib.fa_calib_mfma_fp8.restype = ctypes.c_int
    calib.fa_calib_mfma_fp8.argtypes = calib.fa_calib_mfma_bf16.argtypes
    ci8 = CALIB["iters_fp8"]
    r8 = torch.randint(0, 254, (cb * 256 * 32 * 16,), generator=gen_c, device=dev,
                       dtype=torch.int32)
    c8_ops = (r8 + (r8 >= 127).to(torch.int32)).to(torch.uint8)
    del r8
    run_c8 = lambda: calib.fa_calib_mfma_fp8(c8_ops.data_ptr(), cb, ci8, c_clk.data_ptr(),  # noqa: E731
                                             c_sink.data_ptr(), stream)
    if run_c8() != 0:
        raise RuntimeError("fp8 calibration loop failed to launch")
    torch.cuda.synchronize()
    c0.record()
    run_c8()
    c1.record()
    torch.cuda.synchronize()
    c8_ms = c0.elapsed_time(c1)
    c8_tf = cb * 4 * ci8 * 8 * 2.0 * 32 * 32 * 64 / (c8_ms * 1e-3) / 1e12
    clk = c_clk.cpu().double()
    mhz8 = float(((clk[:, 1] - clk[:, 0]) / (clk[:, 3] - clk[:, 2]) * 100.0).median())
    log(f"MFMA loop on random E4M3: {c8_ms:.2f} ms, {c8_tf:.0f} TFLOP/s at {mhz8:.0f} MHz")
    peak8 = metrics.MI355X_FP8_DENSE_TFLOPS
    out["mfma_ceiling_fp8"] = {
        "what": f"{cb} workgroups x 4 waves, each {ci8} x 8 independent "
                "v_mfma_scale_f32_32x32x64_f8f6f4 on random E4M3 codes (no memory traffic)",
        "tflops": c8_tf, "frac_peak": c8_tf / peak8, "clock_mhz": mhz8,
        "peak_at_clock": peak8 * mhz8 / 2400.0}
    kernels["fwd_fp8"]["frac_of_mfma_ceiling"] = kernels["fwd_fp8"]["achieved"] / c8_tf
    del c8_ops, c_clk, c_sink

    if args.cpu_heads > 0:
        log(f"oracle CPU baseline on {args.cpu_heads} head(s) ...")
        out["cpu_baseline"] = cpu_baseline(args.cpu_heads)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
