"""Turn rocprofv3 result databases into the short text summaries kept in profiles/.

Called as ``python bench.py --summarize PROF_DIR``. PROF_DIR holds the
outputs of these commands (run from the repository root, TMPDIR=/tmp), for
each workload <wl>:

  rocprofv3 --kernel-trace --stats -d PROF_DIR/kt_<wl> -o kt -- python3 bench.py [ARGS]
  rocprofv3 --pmc <counters> -d PROF_DIR/pmc_<set>_<wl> -o pmc -- python3 bench.py \
      --workload <wl> --steps 3 --warmup 1 --preload-ms 0 --b2b-ms 0 --no-cpu --no-bf16 \\
      --no-ceiling

where the default workload's trace is of the bench command itself (no
ARGS) and the others use ARGS = --workload <wl> --no-cpu --no-bf16
--no-ceiling; the counter sets are FETCH (FETCH_SIZE), WRITE (WRITE_SIZE),
MFMA (SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_I8 SQ_BUSY_CYCLES
GRBM_GUI_ACTIVE) and VALU (SQ_ACTIVE_INST_VALU SQ_INSTS_VALU
SQ_BUSY_CU_CYCLES GRBM_GUI_ACTIVE); plus, for the calibration, the same
trace and FETCH/WRITE runs of ``python3 bench.py --copy-calib --steps 10``
(tag "copy"). HBM bytes per launch = counter KiB * 1024 * (known copy bytes /
copy counter bytes).
"""
from __future__ import annotations

import collections
import glob
import json
import os
import re
import sqlite3

# The default workload's trace is of the bench command itself (default steps
# and warmup), so its average kernel durations match the bench line.
DEFAULT_WORKLOAD = "up_proj"
KT_CMD = "rocprofv3 --kernel-trace --stats -d {d}/kt_{wl} -o kt -- python3 bench.py"
KT_ARGS = " --workload {wl} --no-cpu --no-bf16 --no-ceiling"
PMC_SETS = {
    "FETCH": "FETCH_SIZE",
    "WRITE": "WRITE_SIZE",
    "MFMA": "SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_I8 SQ_BUSY_CYCLES GRBM_GUI_ACTIVE",
    "VALU": "SQ_ACTIVE_INST_VALU SQ_INSTS_VALU SQ_BUSY_CU_CYCLES GRBM_GUI_ACTIVE",
}
PMC_CMD = ("rocprofv3 --pmc {c} -d {d}/pmc_{s}_{wl} -o pmc -- python3 bench.py --workload {wl} "
           "--steps 3 --warmup 1 --preload-ms 0 --b2b-ms 0 --no-cpu --no-bf16 --no-ceiling")
COPY_KT_CMD = "rocprofv3 --kernel-trace --stats -d {d}/kt_copy -o kt -- python3 bench.py --copy-calib --steps 10"
COPY_PMC_CMD = ("rocprofv3 --pmc {c} -d {d}/pmc_{s}_copy -o pmc -- python3 bench.py --copy-calib "
                "--steps 10")
COPY_BYTES = 1 << 30
N_XCD = 8                      # GRBM counters are summed over the 8 XCDs
N_CU = 256
N_SIMD = 4 * N_CU
INT8_PEAK_OPS = 5.0e15         # dense INT8 MFMA at the rated 2.4 GHz
RATED_GHZ = 2.4

WORKLOAD_SHAPES = {
    "up_proj": "M=28672 N=16384 K=4096 (RMSNorm+quant -> post-scale GEMM)",
    "down_proj": "M=32760 N=5120 K=13824 (quant -> post-scale GEMM)",
    "square": "M=N=K=4096 (quant -> post-scale GEMM)",
    "blockwise_small": "M=1000 N=K=5120 (1x128 quant -> blockwise GEMM)",
    "blockwise_large": "M=32760 N=K=5120 (1x128 quant -> blockwise GEMM)",
    "ln_up_proj": "M=28672 N=16384 K=4096 (LayerNorm+modulation+quant -> post-scale GEMM)",
    "up_proj_gelu": "M=28672 N=16384 K=4096 (RMSNorm+quant -> post-scale GEMM + bias + GELU)",
    "small_m": "M=256 N=5120 K=13824 (quant -> split-K: INT32 partial sums + post-scale pass)",
    "m1000": "M=1000 N=5120 K=5120 (quant -> post-scale GEMM on 128 x 160 tiles)",
    "tiny": "M=64 N=128 K=256",
}


def short_name(kernel: str) -> str:
    if "gemm_i8_t160_blockwise" in kernel:
        return "gemm_blockwise_t160"
    if "gemm_i8_t160_postscale" in kernel:
        m = re.search(r"Epilogue\)(\d)|EpilogueE(\d)", kernel)
        e = (m.group(1) or m.group(2)) if m else "?"
        return {"0": "gemm_postscale_t160", "3": "gemm_postscale_bias_t160",
                "4": "gemm_postscale_gelu_t160", "5": "gemm_postscale_bias_gelu_t160"}.get(e, "gemm_t160")
    if "gemm_i8_blockwise" in kernel:
        return "gemm_blockwise"
    if "gemm_i8_" in kernel:
        m = re.search(r"Epilogue\)(\d)|EpilogueE(\d)", kernel)
        e = (m.group(1) or m.group(2)) if m else "?"
        return {"0": "gemm_postscale", "1": "gemm_i32", "3": "gemm_postscale_bias",
                "4": "gemm_postscale_gelu", "5": "gemm_postscale_bias_gelu"}.get(e, "gemm")
    if "splitk" in kernel and "postscale_kernel" in kernel:
        return "splitk_postscale"
    if "rmsnorm_quant_kernel" in kernel:
        return "rmsnorm_quant"
    if "layernorm_quant" in kernel:
        return "layernorm_quant"
    if "quant_rows_long_kernel" in kernel:
        return "quant_rows_long"
    if "quant_rows_split_kernel" in kernel:
        # quant_rows_split_kernel<vectors per lane, 128-wide groups?, full rows?>:
        # the few-rows form, several waves per row
        m = re.search(r"quant_rows_split_kernel<\d+, (true|false)", kernel)
        return "quant_rows_1x128_split" if m and m.group(1) == "true" else "quant_rows_split"
    if "quant_rows_kernel" in kernel:
        # quant_rows_kernel<vectors per lane, 128-wide groups?, full rows?>
        m = re.search(r"quant_rows_kernel<\d+, (true|false)", kernel)
        return "quant_rows_1x128" if m and m.group(1) == "true" else "quant_rows"
    if "quant_block128" in kernel:
        return "quant_block128"
    if "copyBuffer" in kernel:
        return "hip_copy_buffer"
    if "mainloop<" in kernel:
        # the GEMM main-loop ceiling probe the default bench line also runs
        return "probe_mainloop_norefill" if "mainloop<false>" in kernel else "probe_mainloop"
    if "clock_stamp" in kernel:
        return "probe_clock_stamp"
    if "at::native" in kernel:
        return "torch_" + ("fill" if "FillFunctor" in kernel else "elementwise")
    return kernel.split("(")[0][-40:]


def kernel_stats(db: str):
    con = sqlite3.connect(db)
    rows = con.execute("select name, total_calls, total_duration, average, percentage "
                       "from top_kernels").fetchall()
    return [(short_name(n), n, c, t, a, p) for n, c, t, a, p in rows]


def pmc_values(db: str, counter: str):
    """{(kernel short name, grid size): [value per dispatch]} for one counter."""
    con = sqlite3.connect(db)
    rows = con.execute("select kernel_name, grid_size, value from counters_collection "
                       "where counter_name=?", (counter,)).fetchall()
    out = collections.defaultdict(list)
    for k, g, v in rows:
        out[(short_name(k), g)].append(v)
    return out


def pmc_dispatches(db: str):
    """{dispatch id: (kernel short name, grid size, duration ns, {counter: value})}."""
    con = sqlite3.connect(db)
    rows = con.execute("select dispatch_id, kernel_name, grid_size, duration, counter_name, value "
                       "from counters_collection").fetchall()
    out = {}
    for d, k, g, dur, c, v in rows:
        rec = out.setdefault(d, (short_name(k), g, dur, {}))
        rec[3][c] = rec[3].get(c, 0.0) + v
    return out


def write_kernel_trace(prof_dir, out_dir, wl, path, gemm_hash, quant_hash):
    stats = kernel_stats(path)
    if wl == "copy":
        cmd = COPY_KT_CMD.format(d=prof_dir)
        title = "plain 1 GiB device copy (HBM calibration)"
    else:
        cmd = KT_CMD.format(d=prof_dir, wl=wl)
        if wl != DEFAULT_WORKLOAD:
            cmd += KT_ARGS.format(wl=wl)
        title = WORKLOAD_SHAPES.get(wl, wl)
    lines = [f"# rocprofv3 kernel trace: {wl} -- {title}", "",
             "Command (repository root, TMPDIR=/tmp, one MI355X):", f"    {cmd}", "",
             f"{'kernel':<28} {'calls':>6} {'avg_us':>10} {'total_us':>11} {'pct':>6}"]
    for short, full, c, t, a, p in stats:
        lines.append(f"{short:<28} {c:>6} {a:>10.3f} {t:>11.3f} {p:>6.2f}")
    lines += ["", "Full kernel names:"] + [f"  {s}: {f[:160]}" for s, f, *_ in stats]
    lines += ["", f"GEMM sources hash: {gemm_hash}  quant sources hash: {quant_hash}"]
    with open(os.path.join(out_dir, f"kernels_{wl}.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")


def main(prof_dir: str, out_dir: str, gemm_hash: str, quant_hash: str) -> None:
    os.makedirs(out_dir, exist_ok=True)
    # ---- kernel-trace summaries --------------------------------------------
    for path in sorted(glob.glob(os.path.join(prof_dir, "kt_*", "kt_results.db"))):
        wl = os.path.basename(os.path.dirname(path))[3:]
        write_kernel_trace(prof_dir, out_dir, wl, path, gemm_hash, quant_hash)

    def src_of(k):
        return gemm_hash if k.startswith("gemm") or k.startswith("splitk") else quant_hash

    # ---- HBM traffic from FETCH_SIZE / WRITE_SIZE --------------------------
    calib = {}
    for sname, c in (("FETCH", "FETCH_SIZE"), ("WRITE", "WRITE_SIZE")):
        db = os.path.join(prof_dir, f"pmc_{sname}_copy", "pmc_results.db")
        if os.path.exists(db):
            vals = [v for (k, g), vs in pmc_values(db, c).items() if k == "hip_copy_buffer"
                    and g >= 65536 for v in vs]
            calib[c] = COPY_BYTES / (sum(vals) / len(vals) * 1024.0)
    for path in sorted(glob.glob(os.path.join(prof_dir, "pmc_FETCH_*", "pmc_results.db"))):
        wl = os.path.basename(os.path.dirname(path))[len("pmc_FETCH_"):]
        if wl == "copy" or len(calib) < 2:
            continue
        fetch = pmc_values(path, "FETCH_SIZE")
        wpath = os.path.join(prof_dir, f"pmc_WRITE_{wl}", "pmc_results.db")
        write = pmc_values(wpath, "WRITE_SIZE") if os.path.exists(wpath) else {}
        lines = [f"# HBM traffic per launch: {wl} -- {WORKLOAD_SHAPES.get(wl, wl)}", "",
                 "Commands (repository root, TMPDIR=/tmp, one MI355X):"]
        for sname in ("FETCH", "WRITE"):
            lines.append("    " + PMC_CMD.format(c=PMC_SETS[sname], d=prof_dir, s=sname, wl=wl))
            lines.append("    " + COPY_PMC_CMD.format(c=PMC_SETS[sname], d=prof_dir, s=sname))
        lines += ["", f"Calibration on a 1 GiB copy: FETCH_SIZE x{calib['FETCH_SIZE']:.4f}, "
                      f"WRITE_SIZE x{calib['WRITE_SIZE']:.4f} (true bytes / counter bytes)", "",
                  f"{'kernel':<28} {'launches':>8} {'fetch_MB':>10} {'write_MB':>10} {'total_MB':>10}"]
        for (k, g), vs in sorted(fetch.items()):
            if k == "hip_copy_buffer" or k.startswith(("torch", "__amd", "probe")):
                continue
            fb = sum(vs) / len(vs) * 1024 * calib["FETCH_SIZE"]
            wv = write.get((k, g), [])
            wb = (sum(wv) / len(wv) * 1024 * calib["WRITE_SIZE"]) if wv else float("nan")
            lines.append(f"{k:<28} {len(vs):>8} {fb / 1e6:>10.1f} {wb / 1e6:>10.1f} {(fb + wb) / 1e6:>10.1f}")
            if k.startswith(("gemm", "rmsnorm", "layernorm", "quant", "splitk")) and wv:
                with open(os.path.join(out_dir, f"traffic_{k}_{wl}.json"), "w") as f:
                    json.dump({"kernel": k, "workload": wl, "hbm_bytes_per_launch": round(fb + wb),
                               "fetch_bytes": round(fb), "write_bytes": round(wb),
                               "source_hash": src_of(k), "launches": len(vs)}, f, indent=1)
        with open(os.path.join(out_dir, f"traffic_{wl}.txt"), "w") as f:
            f.write("\n".join(lines) + "\n")

    # ---- MFMA and VALU activity, and the clock -----------------------------
    for path in sorted(glob.glob(os.path.join(prof_dir, "pmc_MFMA_*", "pmc_results.db"))):
        wl = os.path.basename(os.path.dirname(path))[len("pmc_MFMA_"):]
        sets = {"MFMA": pmc_dispatches(path)}
        vpath = os.path.join(prof_dir, f"pmc_VALU_{wl}", "pmc_results.db")
        if os.path.exists(vpath):
            sets["VALU"] = pmc_dispatches(vpath)
        lines = [f"# MFMA / VALU counters per launch: {wl} -- {WORKLOAD_SHAPES.get(wl, wl)}", "",
                 "Commands (repository root, TMPDIR=/tmp, one MI355X):"]
        for sname in sets:
            lines.append("    " + PMC_CMD.format(c=PMC_SETS[sname], d=prof_dir, s=sname, wl=wl))
        lines += ["",
                  "Per launch (averages over the launches of the run; GRBM_GUI_ACTIVE is summed",
                  "over the 8 XCDs, so the clock is GUI_ACTIVE / 8 / duration):",
                  "  clock_GHz        = GRBM_GUI_ACTIVE / 8 / duration",
                  "  mfma_ops         = SQ_INSTS_VALU_MFMA_MOPS_I8 * 512",
                  "  mfma_busy        = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 * 1024 SIMDs)",
                  "                     (the share of the cycles that ran in which the MFMA units were busy)",
                  "  frac_of_peak     = mfma_ops / duration / 5.0e15 (dense INT8 at the rated 2.4 GHz)",
                  "  valu_busy        = 100 * SQ_ACTIVE_INST_VALU / 256 CUs / (GRBM_GUI_ACTIVE / 8)",
                  "                     (rocprofv3's VALUBusy)",
                  "  valu_insts       = SQ_INSTS_VALU (wave instructions issued)",
                  "(GUI_ACTIVE also counts a few us around each dispatch, so the clock of a",
                  "launch of tens of us reads high; for the ~1 ms GEMMs it is within ~1%.)", "",
                  f"{'kernel':<28} {'set':<5} {'n':>3} {'dur_us':>9} {'clk_GHz':>8} {'mfma_busy':>9} "
                  f"{'frac_peak':>9} {'valu_busy%':>10} {'valu_insts':>12}"]
        for sname, disp in sets.items():
            agg = collections.defaultdict(list)
            for d, (k, g, dur, cv) in disp.items():
                if k.startswith(("torch", "__amd", "hip_copy", "probe")):
                    continue
                agg[(k, g)].append((dur, cv))
            for (k, g), recs in sorted(agg.items()):
                n = len(recs)
                dur = sum(r[0] for r in recs) / n                     # ns
                c = {key: sum(r[1].get(key, 0.0) for r in recs) / n for key in recs[0][1]}
                gui = c.get("GRBM_GUI_ACTIVE", 0.0) / N_XCD
                clk = gui / dur if dur > 0 else float("nan")
                row = {"dur_us": dur / 1e3, "clock_ghz": clk}
                if sname == "MFMA":
                    ops = c.get("SQ_INSTS_VALU_MFMA_MOPS_I8", 0.0) * 512
                    busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (gui * N_SIMD) if gui else 0.0
                    frac = ops / (dur * 1e-9) / INT8_PEAK_OPS if dur else 0.0
                    lines.append(f"{k:<28} {sname:<5} {n:>3} {dur / 1e3:>9.1f} {clk:>8.3f} {busy:>9.4f} "
                                 f"{frac:>9.4f} {'':>10} {'':>12}")
                    if ops > 0 and k.startswith("gemm"):
                        with open(os.path.join(out_dir, f"mfma_{k}_{wl}.json"), "w") as f:
                            json.dump({"kernel": k, "workload": wl, "launches": n,
                                       "duration_us": round(dur / 1e3, 2),
                                       "clock_ghz": round(clk, 4),
                                       "mfma_busy_frac": round(busy, 4),
                                       "frac_of_peak_at_clock": round(frac * RATED_GHZ / clk, 4),
                                       "frac_of_peak": round(frac, 4),
                                       "mfma_ops_counted": round(ops),
                                       "source": f"profiles/counters_{wl}.txt",
                                       "source_hash": src_of(k)}, f, indent=1)
                else:
                    valu = 100.0 * c.get("SQ_ACTIVE_INST_VALU", 0.0) / N_CU / gui if gui else 0.0
                    lines.append(f"{k:<28} {sname:<5} {n:>3} {dur / 1e3:>9.1f} {clk:>8.3f} {'':>9} "
                                 f"{'':>9} {valu:>10.1f} {c.get('SQ_INSTS_VALU', 0.0):>12.0f}")
        lines += ["", f"GEMM sources hash: {gemm_hash}  quant sources hash: {quant_hash}"]
        with open(os.path.join(out_dir, f"counters_{wl}.txt"), "w") as f:
            f.write("\n".join(lines) + "\n")
