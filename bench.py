"""Throughput of causal GQA flash-attention prefill against a cached prefix on
one MI355X.

One step = one attn_prefill call (the whole hot path: Q load, K/V tile
staging, scores, causal mask, online softmax, PV, normalisation, store) over
one chunk whose inputs are already resident in HBM.

Default workload: fp32 chunk C=2048 at prefix P=2048 (4096 cache positions),
32 query heads, 8 KV heads, d=64, q/k/v i.i.d. N(0,1), synthetic and seeded.
Metric: causal attention TFLOP/s = 4*d FLOPs per visible (row, key) pair per
query head, divided by the time per call.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Prints ONE JSON line.  The oracle (CPU, double) is timed on the host cores on
the whole workload as the cpu_baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "causal attn TFLOP/s and % MFMA peak at C=2048,P=2048 (32q/8kv heads, d=64)"
# MI355X dense matrix peaks (TFLOP/s): fp32 MFMA 157.3, bf16 2516.6 (no sparsity).
PEAK_TFLOPS = {"f32": 157.3, "bf16": 2516.6}
HBM_PEAK_GBS = 8000.0

WORKLOADS = {
    # name: (C, P, dtype, seed base, description)
    "c2048_p2048_f32": (2048, 2048, "f32", 200,
                        "fp32 serving chunk C=2048 at P=2048 (4096 KV positions), 32 query heads, 8 KV heads, "
                        "d=64, q/k/v i.i.d. N(0,1)"),
    "c512_p15872_f32": (512, 15872, "f32", 400,
                        "fp32 long cached prefix C=512 at P=15872 (16384 KV positions), last key of KV head 0 "
                        "planted at 4.0"),
    "t2048_p0_f32": (2048, 0, "f32", 300, "fp32 plain causal prompt prefill T=2048, P=0"),
    "t1024_p0_f32": (1024, 0, "f32", 310, "fp32 plain causal prompt prefill T=1024, P=0"),
    "t512_p0_f32": (512, 0, "f32", 320, "fp32 plain causal prompt prefill T=512, P=0"),
    "c4096_p28672_bf16": (4096, 28672, "bf16", 500,
                          "bf16 q/k/v, fp32 accumulation and output, C=4096 at P=28672 (32768 KV positions)"),
    "c1_p16383_f32_splitkv": (1, 16383, "f32", 800,
                              "fp32 decode: one token at P=16383 (16384 KV positions), key range split across "
                              "workgroups and merged; q/k/v i.i.d. N(0,1)"),
    "c1_p131071_f32_splitkv": (1, 131071, "f32", 820,
                               "fp32 decode: one token at P=131071 (131072 KV positions, 512 MiB of K/V, more "
                               "than the 256 MB Infinity Cache holds), split across workgroups"),
    "c1_p32767_bf16_splitkv": (1, 32767, "bf16", 810,
                               "bf16 decode: one token at P=32767 (32768 KV positions), split across workgroups"),
    "c1_p16383_f32_splitkv_paged16": (1, 16383, "f32", 800,
                                      "fp32 decode: one token at P=16383 against a cache in shuffled 16-position "
                                      "pages (block table, 3 spare pages), key range split across workgroups"),
    "c1_p131071_f32_splitkv_paged16": (1, 131071, "f32", 820,
                                       "fp32 decode: one token at P=131071 (512 MiB of K/V) against a cache in "
                                       "shuffled 16-position pages, key range split across workgroups"),
    "c1_p32767_bf16_splitkv_paged16": (1, 32767, "bf16", 810,
                                       "bf16 decode: one token at P=32767 against a cache in shuffled 16-position "
                                       "pages, key range split across workgroups"),
    "c2048_p2048_f32_paged16": (2048, 2048, "f32", 200,
                                "fp32 C=2048 at P=2048 with the cache in shuffled 16-position pages "
                                "(block table, 3 spare pages), q/k/v i.i.d. N(0,1)"),
}
DEFAULT = "c2048_p2048_f32"
KERNEL_NAME = "attn_prefill_kernel"
KERNEL_SRC = os.path.join(ROOT, "chunked_prefill_flash_amd", "csrc", "attn_prefill.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


NOMINAL_MHZ = 2400.0   # the clock the published peaks assume


def clock_from_log(clocks):
    """The clock attn_prefill_clocked logged: each workgroup's shader-clock
    cycles over its 100 MHz ticks, as the median over workgroups and as the
    ratio of the sums (the average over the kernel's busy time); and where a
    workgroup's time goes, from the phase marks (medians over workgroups, each
    phase's cycles over that workgroup's own clock)."""
    import numpy as np
    c = clocks.cpu().numpy().astype(np.float64)
    cyc, tick = c[:, 2] - c[:, 0], c[:, 3] - c[:, 1]
    mhz_wg = cyc / tick * 100.0
    mhz = np.sort(mhz_wg)

    def med_us(a, b, rows=None):
        sel = np.ones(len(c), bool) if rows is None else rows
        if not sel.any():
            return None
        return round(float(np.median((c[sel, b] - c[sel, a]) / mhz_wg[sel])), 2)

    two = c[:, 7] != 0                       # workgroups with a second work item
    phases = {
        "first_item_prologue": med_us(0, 4),   # start until its Q and first K/V tile have landed
        "first_item_key_loop": med_us(4, 5),
        "first_item_epilogue": med_us(5, 6),   # key-split merge, output store, barrier
        "second_item_prologue": med_us(6, 7, two),
        "second_item_rest": med_us(7, 2, two),
        "workgroup": med_us(0, 2),
        "workgroups_with_two_items": int(two.sum()),
        "kernel_span": round(float((c[:, 3].max() - c[:, 1].min()) / 100.0), 2),
        "start_spread": round(float((c[:, 1].max() - c[:, 1].min()) / 100.0), 2),
    }
    return {"median_mhz": round(float(mhz[len(mhz) // 2]), 1), "min_mhz": round(float(mhz[0]), 1),
            "max_mhz": round(float(mhz[-1]), 1), "busy_average_mhz": round(float(cyc.sum() / tick.sum() * 100.0), 1),
            "workgroups": int(len(mhz)), "phases_us": phases,
            "source": "attn_prefill_clocked (the same kernels): each workgroup's shader-clock counter over the fixed "
                      "100 MHz counter from its start to its end, on the middle one of the timed steps (that step "
                      "goes through attn_prefill_clocked, the same kernel logging into a buffer allocated beforehand); "
                      "phases are the medians over workgroups of the spans between its marks"}


def kernel_source_hash() -> str:
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


# ---- rocprofv3 harness ------------------------------------------------------
# The profiles under profiles/ come from these rocprofv3 passes over this
# benchmark (one counter set per run: the hardware cannot collect more at
# once) and from summarize_rocprof() below, which turns their CSV output into
# the summaries and the traffic table.  Neither function touches the GPU.
SQ_SET_1 = ("SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES SQ_WAVES SQ_INSTS_MFMA SQ_INSTS_VALU SQ_INSTS_LDS "
            "SQ_LDS_BANK_CONFLICT SQ_INSTS_VALU_MFMA_MOPS_F32 GRBM_GUI_ACTIVE")
SQ_SET_2 = "SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_ACTIVE_INST_VALU SQ_WAIT_INST_LDS SQ_WAIT_INST_ANY SQ_ACTIVE_INST_LDS GRBM_GUI_ACTIVE"
COPY_MIB = 512   # calibration copy: a plain elementwise op that reads and writes this many MiB


def rocprof_passes(name, outdir):
    """(pass, command) for each rocprofv3 run of workload `name`, writing
    under outdir/<pass>/."""
    bench = os.path.join(ROOT, "bench.py")
    short = ("python %s --workload %s --steps 3 --warmup 1 --warmup-seconds 0 --no-cpu --no-check --no-speedup "
             "--no-clock --calibrate-copy-mib %d" % (bench, name, COPY_MIB))
    passes = [("trace", "timeout -s KILL 300 rocprofv3 --kernel-trace --stats",
               "python %s --workload %s --steps 200 --warmup 20 --no-cpu" % (bench, name)),
              ("fetch", "timeout -s KILL 90 rocprofv3 --pmc FETCH_SIZE", short),
              ("write", "timeout -s KILL 90 rocprofv3 --pmc WRITE_SIZE", short),
              ("sq1", "timeout -s KILL 90 rocprofv3 --pmc " + SQ_SET_1, short),
              ("sq2", "timeout -s KILL 90 rocprofv3 --pmc " + SQ_SET_2, short)]
    return [(p, "cd /tmp && TMPDIR=/tmp %s --output-format csv -d %s -o %s -- %s"
             % (prof, os.path.join(outdir, p), p, prog)) for p, prof, prog in passes]


PRODUCT_KERNELS = ("attn_prefill_kernel", "attn_decode_split_kernel", "attn_merge_splits_kernel")


def _demangled_args(rest):
    """Template arguments of an Itanium-mangled kernel name's suffix, for the
    few forms these kernels use (float, __bf16, ints, bools)."""
    args, i = [], 0
    if not rest.startswith("I"):
        return None
    i = 1
    while i < len(rest) and rest[i] != "E":
        if rest.startswith("DF16b", i):
            args.append("__bf16")
            i += 5
        elif rest[i] == "f":
            args.append("float")
            i += 1
        elif rest.startswith("Lb", i):
            args.append("true" if rest[i + 2] == "1" else "false")
            i += 4
        elif rest.startswith("Li", i):
            j = rest.index("E", i)
            args.append(rest[i + 2:j])
            i = j + 1
        else:
            return None
    return args


def _short_kernel(name):
    if name.startswith("_Z"):
        for k in PRODUCT_KERNELS + ("attn_rowwise_kernel", "naive_scores_kernel", "naive_softmax_kernel",
                                    "naive_pv_kernel"):
            at = name.find(k)
            if at >= 0:
                args = _demangled_args(name[at + len(k):])
                return k + ("<%s>" % ", ".join(args) if args else "")
        return name[:70]
    n = name.replace("(anonymous namespace)::", "").replace("void ", "")
    for k in PRODUCT_KERNELS + ("attn_rowwise_kernel", "naive_scores_kernel", "naive_softmax_kernel",
                                "naive_pv_kernel"):
        if n.startswith(k):
            tmpl = n[len(k):].split("(")[0]
            return k + tmpl
    return n.split("(")[0][:70]


def _read_csv(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _counters(dirpath):
    """{counter: {"product": mean per call over the product kernels (summed
    over the kernels of one call), "copy": mean over the calibration copies,
    "us": mean profiled duration per call}} from one --pmc pass."""
    import glob
    files = glob.glob(os.path.join(dirpath, "*counter_collection.csv"))
    if not files:
        return None
    rows = _read_csv(files[0])
    per = {}   # counter -> kernel -> list of values
    dur = {}
    for r in rows:
        k = _short_kernel(r["Kernel_Name"])
        per.setdefault(r["Counter_Name"], {}).setdefault(k, []).append(float(r["Counter_Value"]))
        dur.setdefault(k, {})[r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    out = {}
    for cname, bykernel in per.items():
        prod = [k for k in bykernel if k.split("<")[0] in PRODUCT_KERNELS]
        value = sum(sum(bykernel[k]) / len(bykernel[k]) for k in prod)
        copies = [v for k, vs in bykernel.items() if "elementwise" in k for v in vs]
        big = [v for v in copies if copies and v >= 0.9 * max(copies)]
        out[cname] = {"product": value, "copy": sum(big) / len(big) if big else None,
                      "kernels": sorted(prod),
                      "us": sum(sum(dur[k].values()) / len(dur[k]) for k in prod)}
    return out


def summarize_rocprof(name, outdir, profiles_dir=None):
    """Write <kernel>_<workload>_kernel_trace.md and _counters.md under
    profiles_dir (default profiles/) from the passes of
    rocprof_passes(name, outdir) that are present, and record the scaled HBM
    bytes per call in its traffic.json."""
    profiles_dir = profiles_dir or os.path.join(ROOT, "profiles")
    traffic_file = os.path.join(profiles_dir, "traffic.json")
    import chunked_prefill_flash_amd as cpf
    C, P, dt, _, desc = WORKLOADS[name]
    decode = "splitkv" in name
    base = "attn_decode" if decode and C == 1 else "attn_prefill"
    src = kernel_source_hash()
    flop = cpf.flops(C, P)
    esz = 4 if dt == "f32" else 2
    alg = C * 32 * 64 * esz + 2 * (P + C) * 8 * 64 * esz + C * 32 * 64 * 4
    if "paged" in name:
        alg += -(-(P + C) // int(name.rsplit("paged", 1)[1])) * 4
    cmds = dict(rocprof_passes(name, outdir))
    written = []
    tdir = os.path.join(outdir, "trace")
    stats = os.path.join(tdir, "trace_kernel_stats.csv")
    if os.path.exists(stats):
        rows = _read_csv(stats)
        md = ["# %s kernel trace: %s" % (base, desc), "",
              "Kernel source sha256[:16]: `%s`. Command:" % src, "", "```", cmds["trace"], "```", "",
              "| Kernel | Calls | Average (us) | Min (us) | Max (us) | Std dev (us) | Share |",
              "|---|---|---|---|---|---|---|"]
        per_call = 0.0
        for r in rows:
            k = _short_kernel(r["Name"])
            md.append("| %s | %s | %.2f | %.2f | %.2f | %.2f | %s%% |" % (
                k, r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3,
                float(r["StdDev"]) / 1e3, r["Percentage"]))
            if k.split("<")[0] in PRODUCT_KERNELS:
                per_call += float(r["AverageNs"]) / 1e3
        md.append("")
        if per_call <= 0:
            md.append("(no product kernel found in this trace)")
        elif decode:
            md.append("Per call (the product kernels' averages summed): %.2f us -> %.1f GB/s over %d algorithmic "
                      "bytes (%.1f%% of 8 TB/s)." % (per_call, alg / per_call / 1e3, alg,
                                                     alg / per_call / 1e3 / HBM_PEAK_GBS * 100))
        else:
            md.append("Per call: %.2f us -> %.1f TFLOP/s over %.4e FLOP (%.1f%% of the %s MFMA peak %.1f TFLOP/s)."
                      % (per_call, flop / per_call / 1e6, flop, flop / per_call / 1e6 / PEAK_TFLOPS[dt] * 100, dt,
                         PEAK_TFLOPS[dt]))
        md.append("")
        path = os.path.join(profiles_dir, "%s_%s_kernel_trace.md" % (base, name))
        open(path, "w").write("\n".join(md))
        written.append(path)
    cnt = {}
    for p in ("fetch", "write", "sq1", "sq2"):
        c = _counters(os.path.join(outdir, p))
        if c:
            cnt.update(c)
    if cnt:
        copy_bytes = COPY_MIB << 20
        md = ["# %s counters: %s" % (base, desc), "",
              "Kernel source sha256[:16]: `%s`. Values are per call (the product kernels of one call summed), "
              "averaged over the profiled calls." % src, "", "Commands (one counter set per run):", "", "```"]
        md += [cmds[p] for p in ("fetch", "write", "sq1", "sq2")]
        md += ["```", "", "The calibration kernel is the benchmark's `--calibrate-copy-mib %d` leg: an elementwise "
               "`torch.mul(src, 1.0, out=dst)` over %d MiB of float32, which reads and writes %d KiB."
               % (COPY_MIB, COPY_MIB, copy_bytes >> 10), "", "| Counter | Value |", "|---|---|"]
        entry = None
        if "FETCH_SIZE" in cnt and "WRITE_SIZE" in cnt and cnt["FETCH_SIZE"]["copy"] and cnt["WRITE_SIZE"]["copy"]:
            f, w = cnt["FETCH_SIZE"], cnt["WRITE_SIZE"]
            fs, ws = copy_bytes / 1024 / f["copy"], copy_bytes / 1024 / w["copy"]
            hbm = f["product"] * 1024 * fs + w["product"] * 1024 * ws
            md += ["| kernels | %s |" % ", ".join(f["kernels"]),
                   "| FETCH_SIZE (KiB per call, raw) | %.1f |" % f["product"],
                   "| WRITE_SIZE (KiB per call, raw) | %.1f |" % w["product"],
                   "| copy FETCH_SIZE (KiB) | %.1f -> fetch scale %.4f |" % (f["copy"], fs),
                   "| copy WRITE_SIZE (KiB) | %.1f -> write scale %.4f |" % (w["copy"], ws),
                   "| HBM-side bytes per call (scaled) | %.2f MiB (algorithmic %.2f MiB, ratio %.3f) |"
                   % (hbm / 2 ** 20, alg / 2 ** 20, hbm / alg)]
            entry = {"kernel_source_sha256_16": src, "bytes_per_launch": int(round(hbm)), "kernels": f["kernels"],
                     "fetch_kib_raw": round(f["product"], 1), "write_kib_raw": round(w["product"], 1),
                     "fetch_scale": round(fs, 4), "write_scale": round(ws, 4), "algorithmic_bytes": alg}
        mops = cnt.get("SQ_INSTS_VALU_MFMA_MOPS_F32" if dt == "f32" else "SQ_INSTS_VALU_MFMA_MOPS_BF16")
        if mops:
            md.append("| MFMA FLOP (SQ_INSTS_VALU_MFMA_MOPS x 512) | %.4e (algorithmic %.4e) |"
                      % (mops["product"] * 512, flop))
        busy = cnt.get("SQ_VALU_MFMA_BUSY_CYCLES")
        if busy and busy["us"] > 0:
            per_simd = busy["product"] / 1024
            cyc = busy["us"] * 1e-6 * NOMINAL_MHZ * 1e6
            md.append("| SQ_VALU_MFMA_BUSY_CYCLES | %.4e (per SIMD %.4e = %.1f%% of %.0f cycles at 2.4 GHz over "
                      "the profiled %.1f us) |" % (busy["product"], per_simd, per_simd / cyc * 100, cyc, busy["us"]))
        for cname in ("SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_WAIT_INST_LDS",
                      "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_ANY", "SQ_BUSY_CYCLES",
                      "GRBM_GUI_ACTIVE", "SQ_WAVES"):
            if cname in cnt:
                md.append("| %s | %.4e |" % (cname, cnt[cname]["product"]))
        if "SQ_INSTS_MFMA" in cnt and "SQ_INSTS_VALU" in cnt and cnt["SQ_INSTS_MFMA"]["product"] > 0:
            mf, va = cnt["SQ_INSTS_MFMA"]["product"], cnt["SQ_INSTS_VALU"]["product"]
            md.append("| non-MFMA VALU instructions per MFMA | %.2f |" % ((va - mf) / mf))
        if "SQ_INSTS_LDS" in cnt and "SQ_LDS_BANK_CONFLICT" in cnt and cnt["SQ_INSTS_LDS"]["product"] > 0:
            md.append("| LDS bank-conflict cycles per LDS instruction | %.3f |"
                      % (cnt["SQ_LDS_BANK_CONFLICT"]["product"] / cnt["SQ_INSTS_LDS"]["product"]))
        md.append("")
        path = os.path.join(profiles_dir, "%s_%s_counters.md" % (base, name))
        open(path, "w").write("\n".join(md))
        written.append(path)
        if entry:
            try:
                table = json.load(open(traffic_file))
            except (OSError, ValueError):
                table = {}
            table[name] = entry
            with open(traffic_file, "w") as fh:
                json.dump(table, fh, indent=1, sort_keys=True)
                fh.write("\n")
            written.append(traffic_file)
    return written


def make_inputs(name):
    import synth
    C, P, dt, seed, _ = WORKLOADS[name]
    if name.startswith("c512_p15872"):
        q, k, v, _ = synth.case_last_key(C, P, seed)
    else:
        q, k, v = synth.case_plain(C, P, seed)
    return q, k, v


def to_device(x, dt, dev):
    import numpy as np
    import torch
    import synth
    if dt == "f32":
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)
    return torch.from_numpy(synth.to_bf16_bits(x).view(np.int16)).view(torch.bfloat16).to(dev)


def traffic_entry(name):
    """HBM bytes per launch from committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    runs, scaled by the copy-kernel calibration; None when missing or taken
    on a different kernel source."""
    try:
        data = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    e = data.get(name)
    if not e or e.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return e.get("bytes_per_launch")


def cpu_baseline(name, q, k, v, P, dt, budget_s=15.0, min_s=10.0):
    """Time the CPU oracle, on all the host threads OpenMP gives it.

    The whole workload is run when a short trial predicts it fits the budget
    (repeated until about min_s seconds of work, within the budget); otherwise
    an evenly spaced sample of rows (all 32 heads each) sized to the budget.  The value counts the
    same 4*d FLOPs per visible pair as the GPU figure, over what was run."""
    import numpy as np
    import oracle
    import synth
    import chunked_prefill_flash_amd as cpf
    if dt == "bf16":
        q, k, v = (synth.bf16_bits_to_f32(synth.to_bf16_bits(x)) for x in (q, k, v))
    C = q.shape[0]
    threads = oracle.max_threads()

    def rows_flop(rows):
        return int(sum(4 * 64 * 32 * (P + int(r) + 1) for r in rows))

    def run_rows(rows):
        rr = np.repeat(np.asarray(rows), 32)
        hh = np.tile(np.arange(32), len(rows))
        t0 = time.perf_counter()
        oracle.attn_rows(q, k, v, P, rr, hh)
        return time.perf_counter() - t0

    trial = np.linspace(0, C - 1, num=min(C, 16)).astype(int)
    rate = rows_flop(trial) / run_rows(trial)            # FLOP/s of the oracle
    full = cpf.flops(C, P)
    if full / rate <= budget_s:
        times = []
        t_all = time.perf_counter()
        while True:
            t0 = time.perf_counter()
            oracle.attn_prefill(q, k, v, P)
            times.append(time.perf_counter() - t0)
            elapsed = time.perf_counter() - t_all
            if elapsed >= min_s or elapsed + times[-1] > budget_s:
                break
        per = float(np.mean(times))
        return {"value": round(full / per / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
                "sample": "whole workload (all %d rows x 32 heads), %d run(s), mean %.3f s per run, double "
                          "sums, OpenMP over (row, head)" % (C, len(times), per)}
    n = int(max(16, min(C, C * budget_s * rate / full)))
    rows = np.linspace(0, C - 1, num=n).astype(int)
    t = run_rows(rows)
    return {"value": round(rows_flop(rows) / t / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "%d evenly spaced rows of %d (all 32 heads each, %.3g GFLOP), %.2f s, double sums, "
                      "OpenMP over (row, head)" % (n, C, rows_flop(rows) / 1e9, t)}


def sampled_parity(got, q, k, v, P, dt):
    """Spot-check the benchmarked output against the oracle on 8 rows (all
    heads).  Returns (all within tolerance, error statistics): max absolute,
    max relative (over |ref| >= 1e-3), RMS, and the largest error as a fraction
    of its element's tolerance."""
    import numpy as np
    import oracle
    import synth
    C = q.shape[0]
    if dt == "bf16":
        q, k, v = (synth.bf16_bits_to_f32(synth.to_bf16_bits(x)) for x in (q, k, v))
    rows = np.array(sorted({r for r in (0, 1, C // 3, C // 2, C - 2, C - 1, 7 % C, (5 * C) // 7) if 0 <= r < C}))
    rr = np.repeat(rows, 32)
    hh = np.tile(np.arange(32), len(rows))
    ref = oracle.attn_rows(q, k, v, P, rr, hh).astype(np.float64)
    g = got[rr, hh].astype(np.float64)
    if dt == "f32":
        tol = 1e-4 + 1e-3 * np.abs(ref)
    else:
        tol = 1e-5 + 2.0 ** -8 * oracle.attn_rows(q, k, np.abs(v), P, rr, hh).astype(np.float64)
    err = np.abs(g - ref)
    big = np.abs(ref) >= 1e-3
    stats = {"sampled_rows": int(len(rows)), "max_abs_err": float(err.max()),
             "max_rel_err": float((err[big] / np.abs(ref[big])).max()) if big.any() else None,
             "rms_err": float(np.sqrt(np.mean(err ** 2))), "worst_err_over_tol": float((err / tol).max())}
    return bool(np.all(err <= tol)), stats


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--warmup-seconds", type=float, default=0.5,
                    help="keep calling for at least this long before timing (lets the GPU clock settle)")
    ap.add_argument("--workload", default=DEFAULT, choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-check", action="store_true", help="skip the sampled parity check")
    ap.add_argument("--no-speedup", action="store_true",
                    help="skip timing the per-row baseline kernel (the pages' starter algorithm)")
    ap.add_argument("--cold", action="store_true",
                    help="also time 20 calls each preceded by a 1 GiB read, so inputs come from HBM "
                         "rather than the 256 MB Infinity Cache")
    ap.add_argument("--no-clock", action="store_true", help="do not sample the shader clock")
    ap.add_argument("--rocprof-commands", metavar="DIR",
                    help="print the rocprofv3 passes for --workload (output under DIR/<pass>) and exit")
    ap.add_argument("--rocprof-summary", metavar="DIR",
                    help="write the profiles/ summaries and traffic entry for --workload from the rocprofv3 "
                         "output under DIR/<pass> and exit (no GPU use)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="after timing, run a plain elementwise copy of this many MiB three times "
                         "(reference kernel of known traffic for HBM byte counters)")
    args = ap.parse_args()

    if args.rocprof_commands:
        for _, cmd in rocprof_passes(args.workload, os.path.abspath(args.rocprof_commands)):
            print(cmd)
        return
    if args.rocprof_summary:
        for path in summarize_rocprof(args.workload, os.path.abspath(args.rocprof_summary)):
            print(path)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs as a single process on one GPU", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import chunked_prefill_flash_amd as cpf

    name = args.workload
    C, P, dt, _, desc = WORKLOADS[name]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    q, k, v = make_inputs(name)
    qd, kd, vd = to_device(q, dt, dev), to_device(k, dt, dev), to_device(v, dt, dev)
    out = torch.empty((C, 32, 64), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    paged = "paged" in name
    if paged:
        import synth
        page = int(name.rsplit("paged", 1)[1])
        kp, vp, table = synth.to_pages(k, v, page, 5600 + page)
        kpd, vpd = to_device(kp, dt, dev), to_device(vp, dt, dev)
        tabd = torch.from_numpy(table).to(dev)

    splitkv = "splitkv" in name
    if splitkv:
        need, _ = cpf.splitkv_workspace(C, P, torch.float32 if dt == "f32" else torch.bfloat16)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)

    def call():
        if splitkv and paged:
            cpf.attn_prefill_paged_splitkv(qd, kpd, vpd, tabd, P, out=out, workspace=ws, stream=stream)
        elif splitkv:
            cpf.attn_prefill_splitkv(qd, kd, vd, out=out, P=P, workspace=ws, stream=stream)
        elif paged:
            cpf.attn_prefill_paged(qd, kpd, vpd, tabd, P, out=out, stream=stream)
        else:
            cpf.attn_prefill(qd, kd, vd, out=out, P=P, stream=stream)

    # the output of a first call is checked against the oracle on the CPU
    # before the warmup, so that the GPU does not sit idle (and its clock drop)
    # between the warmup and the timed steps
    call()
    torch.cuda.synchronize()
    ok, errstats = (True, None) if args.no_check else sampled_parity(out.cpu().numpy(), q, k, v, P, dt)
    if not ok:
        print("bench: sampled parity check FAILED (%s)" % json.dumps(errstats), file=sys.stderr)
        sys.exit(1)
    t_w = time.perf_counter()
    n_w = 0
    while n_w < max(args.warmup, 1) or time.perf_counter() - t_w < args.warmup_seconds:
        call()
        n_w += 1
        if n_w % 10 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()

    # timed region: K steps, synchronised on both sides; HIP events on the
    # stream the kernel is launched on give the per-launch device time.  The
    # middle step (plain caches) goes through attn_prefill_clocked: the same
    # kernel, which then also logs its clock into a buffer allocated before
    # the region, so the clock is the one the timed steps ran at
    logged = not args.no_clock and not paged and not splitkv
    if logged:
        plan_grid = cpf.plan(C, P, torch.float32 if dt == "f32" else torch.bfloat16)["grid"]
        clk_buf = torch.zeros((max(plan_grid, 1), cpf.CLOCK_WORDS), dtype=torch.int64, device=dev)
    mid = args.steps // 2
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        if logged and i == mid:
            cpf.attn_prefill_clocked(qd, kd, vd, out=out, P=P, stream=stream, clocks=clk_buf)
        else:
            call()
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall = t1 - t0
    clock = clock_from_log(clk_buf[:plan_grid]) if logged else None
    kernel_ms = ev0.elapsed_time(ev1) / args.steps
    ms_per_step = wall * 1e3 / args.steps

    # per-launch spread: 20 calls, each between its own pair of events
    pairs = []
    for _ in range(20):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        call()
        b.record(stream)
        pairs.append((a, b))
    torch.cuda.synchronize()
    each = sorted(a.elapsed_time(b) for a, b in pairs)
    launch_ms = {"median": round(each[len(each) // 2], 5), "min": round(each[0], 5), "max": round(each[-1], 5),
                 "n": len(each)}
    cold_ms = None
    if args.cold:
        flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB, four times the MALL
        sink = torch.empty((), dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        pairs = []
        for i in range(20):
            torch.sum(flush, dim=0, out=sink)   # a read: evicts the inputs, leaves no dirty lines
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            call()
            b.record(stream)
            pairs.append((a, b))
        torch.cuda.synchronize()
        each_c = sorted(a.elapsed_time(b) for a, b in pairs)
        cold_ms = {"median": round(each_c[len(each_c) // 2], 5), "min": round(each_c[0], 5),
                   "max": round(each_c[-1], 5), "n": len(each_c),
                   "note": "each call after a 1 GiB device read (inputs not cache-resident)"}
        del flush, sink

    flop = cpf.flops(C, P)
    value = flop / (ms_per_step * 1e-3) / 1e12
    achieved = flop / (kernel_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[dt]
    plan = cpf.plan(C, P, torch.float32 if dt == "f32" else torch.bfloat16, paged=paged)
    if splitkv:
        plan = {"splits": cpf.splitkv_workspace(C, P, torch.float32 if dt == "f32" else torch.bfloat16)[1],
                "kernels": "split attention + merge"}

    result = {
        "metric": METRIC if name == DEFAULT else "causal attn TFLOP/s (%s)" % name,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": n_w,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt,
        "data": "synthetic (seeded N(0,1), inputs resident in HBM)",
        "config": {"workload": desc, "C": C, "P": P, "q_heads": 32, "kv_heads": 8, "head_dim": 64,
                   "flop_per_call": flop, "launch": plan},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": traffic_entry(name),
                     "kernel": KERNEL_NAME, "kernel_ms": round(kernel_ms, 5)},
        "launch_ms": launch_ms,
        "clock": clock,
        "cold_launch_ms": cold_ms,
        "parity": dict({"sampled_rows_ok": ok}, **(errstats or {})),
    }
    if clock:
        # the same fraction against the peak at the clock the chip ran at
        mhz = clock["median_mhz"]
        result["roofline"]["peak_at_clock"] = round(peak * mhz / NOMINAL_MHZ, 2)
        result["roofline"]["frac_at_clock"] = round(achieved / (peak * mhz / NOMINAL_MHZ), 4)
    esz = 4 if dt == "f32" else 2
    alg_bytes = C * 32 * 64 * esz + 2 * (P + C) * 8 * 64 * esz + C * 32 * 64 * 4
    if paged:
        alg_bytes += -(-(P + C) // page) * 4     # the block table
    if splitkv:
        # decode is bandwidth-bound: roofline against HBM on the compulsory bytes
        gbs = alg_bytes / (kernel_ms * 1e-3) / 1e9
        result["roofline"] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                              "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic_entry(name),
                              "kernel": ("attn_decode_split_kernel" if C == 1 and dt == "f32" else
                                         "attn_prefill_kernel (split)") + (" (paged)" if paged else "") +
                                        " + attn_merge_splits_kernel",
                              "kernel_ms": round(kernel_ms, 5), "algorithmic_bytes": alg_bytes}
    if not args.no_speedup and not paged and not splitkv:
        # the per-row starter algorithm on the same inputs, same run: the page's SPEEDUP
        out2 = torch.empty_like(out)
        for _ in range(2):
            cpf.attn_prefill_rowwise(qd, kd, vd, out=out2, P=P, stream=stream)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        n_base = 5
        for _ in range(n_base):
            cpf.attn_prefill_rowwise(qd, kd, vd, out=out2, P=P, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        base_ms = e0.elapsed_time(e1) / n_base
        result["speedup_vs_rowwise"] = {"rowwise_ms": round(base_ms, 4), "tiled_ms": round(kernel_ms, 5),
                                        "speedup": round(base_ms / kernel_ms, 2),
                                        "baseline": "per-row kernel with no tiling: one (row, head) per wave, scores lane per key, "
                                                    "weighted sum lane per dim, every row streams its whole prefix "
                                                    "(the pages' starter)"}
    if not args.no_speedup and P == 0 and dt == "f32" and not paged and not splitkv:
        # the three-kernel pipeline with the full score matrix on the same prompt
        need = cpf.naive_workspace(C)
        ws_n = torch.empty(need, dtype=torch.uint8, device=dev)
        out3 = torch.empty_like(out)
        for _ in range(3):
            cpf.attn_naive(qd, kd, vd, out=out3, workspace=ws_n, stream=stream)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        n_base = 10
        for _ in range(n_base):
            cpf.attn_naive(qd, kd, vd, out=out3, workspace=ws_n, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        naive_ms = e0.elapsed_time(e1) / n_base
        result["vs_naive_pipeline"] = {"naive_ms": round(naive_ms, 4), "fused_ms": round(kernel_ms, 5),
                                       "speedup": round(naive_ms / kernel_ms, 2), "workspace_bytes": need,
                                       "baseline": "scores -> in-place row softmax -> PV, 32 x T x T fp32 "
                                                   "score matrix in HBM between the kernels"}
        del ws_n
    if args.calibrate_copy_mib > 0:
        src = torch.ones(args.calibrate_copy_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)   # reads and writes calibrate_copy_mib MiB each
        torch.cuda.synchronize()
        result["calibration_copy_bytes"] = src.numel() * 4
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(name, q, k, v, P, dt)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
