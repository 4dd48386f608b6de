"""The bench's profile summariser (bench.py --summarize-profiles) on synthetic rocprofv3 CSVs laid
out in the order the bench launches its kernels: each entry's durations and HBM bytes come from
that entry's own dispatches, also where several entries launch the same kernel, and a table that
does not match the dispatches raises instead of mislabelling them."""
from __future__ import annotations

import csv
import json
import os

import pytest

import bench


def reported(key: str, i: int) -> str:
    """The name rocprofv3 reports for a kernel instance: mangled or demangled (it does both)."""
    if i % 3 == 0:
        return f"void fa::(anonymous namespace)::{key}(float const*, int)"
    return "_ZN2fa12_GLOBAL__N_1" + bench._mangled(key) + "EvPKDF16bS3_"


def dispatch_order(steps: int, warmup: int) -> list:
    """(entry, kernel pattern) per dispatch, in the bench's order, with unrelated kernels between."""
    out = []
    step = [e for e in bench.PROFILE_ENTRIES if e[1] == "step"]
    for _ in range(warmup + steps):
        for entry, _, _, pats in step:
            out += [(entry, p) for p in pats]
        out.append((None, "elementwise_kernel"))
    for entry, kind, reps, pats in bench.PROFILE_ENTRIES:
        if kind == "step":
            continue
        calls, _ = bench._entry_calls(kind, reps, steps, warmup)
        for _ in range(calls):
            out += [(entry, p) for p in pats]
        out.append((None, "randn_kernel"))
    return out


def write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def entry_value(entry: str) -> int:
    return 1000 + 37 * [e[0] for e in bench.PROFILE_ENTRIES].index(entry)


def make_run(root, steps, warmup, pmc_steps, pmc_warmup):
    trace, t = [], 0
    for i, (entry, pat) in enumerate(dispatch_order(steps, warmup)):
        # every kernel of an entry lasts entry_value(entry) ns; warm-up launches far longer
        du = 5 if entry is None else entry_value(entry)
        trace.append([i + 1, reported(pat, i) if entry else pat, t, t + du])
        t += du + 10
    # warm-up launches: make the first `warmup`-worth of every entry slow, so that counting them
    # would change the averages
    seen = {}
    for row, (entry, pat) in zip(trace, dispatch_order(steps, warmup)):
        if entry is None:
            continue
        kind = next(k for e, k, _, _ in bench.PROFILE_ENTRIES if e == entry)
        n_warm = warmup if kind == "step" else max(warmup, 3)
        seen[(entry, pat)] = seen.get((entry, pat), 0) + 1
        if seen[(entry, pat)] <= n_warm:
            row[3] = row[2] + 10 ** 7
    write_csv(os.path.join(root, "stats", "host", "bench_kernel_trace.csv"),
              ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"], trace)
    pmc = dispatch_order(pmc_steps, pmc_warmup)
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    for c, val in (("FETCH_SIZE", lambda e: entry_value(e)), ("WRITE_SIZE", lambda e: 3)):
        write_csv(os.path.join(root, c, "bench_counter_collection.csv"), hdr,
                  [[i + 1, reported(p, i) if e else p, c, 0 if e is None else val(e)]
                   for i, (e, p) in enumerate(pmc)])
        full = 524288 if c == "FETCH_SIZE" else 1048576
        write_csv(os.path.join(root, c + "_copy", "copy_counter_collection.csv"), hdr,
                  [[i + 1, "__amd_rocclr_copyBuffer", c, full] for i in range(3)])
    sq = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_INSTS_VALU_TRANS_F32",
          "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_WAVES", "GRBM_GUI_ACTIVE"]
    write_csv(os.path.join(root, "mfma", "bench_counter_collection.csv"), hdr,
              [[i + 1, reported(p, i) if e else p, c, 8] for i, (e, p) in enumerate(pmc)
               for c in sq])


def test_summaries_take_each_entrys_own_dispatches(tmp_path):
    run, out = str(tmp_path / "run"), str(tmp_path / "out")
    os.makedirs(out)
    make_run(run, 6, 2, 2, 1)
    bench.summarize_profiles(run, 6, 2, 2, 1, out_dir=out)
    text = open(os.path.join(out, "kernel_durations_causal_b2h16n8192d128_decode_b8h32k65536.md")).read()
    sums = {}
    for line in text.splitlines():
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) == 2 and cells[0] in {e[0] for e in bench.PROFILE_ENTRIES}:
            sums[cells[0]] = float(cells[1])
    for entry, _, _, pats in bench.PROFILE_ENTRIES:
        us = len(pats) * entry_value(entry) / 1e3
        assert abs(sums[entry] - us) <= 0.051, (entry, sums.get(entry), us)
    with open(os.path.join(out, "traffic.json")) as f:
        rec = json.load(f)["entries"]
    assert set(rec) == {e[0] for e in bench.PROFILE_ENTRIES}
    for entry, _, _, pats in bench.PROFILE_ENTRIES:
        # FETCH_SIZE scaled by 2 (the copy reads half its bytes), WRITE_SIZE by 1, in KiB
        want = len(pats) * (2 * entry_value(entry) + 3) * 1024
        assert abs(rec[entry]["bytes_per_launch"] - want) <= 1, entry
        assert rec[entry]["source_hash"] == bench._source_hash(bench._family(entry))
    assert os.path.exists(os.path.join(out, "mfma_valu_lds_counters_causal_b2h16n8192d128_"
                                            "decode_b8h32k65536.md"))


def test_summaries_reject_a_table_that_does_not_match(tmp_path):
    run, out = str(tmp_path / "run"), str(tmp_path / "out")
    os.makedirs(out)
    make_run(run, 6, 2, 2, 1)
    with pytest.raises(ValueError, match="do not match"):
        bench.summarize_profiles(run, 5, 2, 2, 1, out_dir=out)
