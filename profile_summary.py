"""Turn rocprofv3 result databases into the short text summaries kept in profiles/.

Called as ``python bench.py --summarize PROF_DIR``. PROF_DIR holds the
outputs of these commands (run from the repository root, TMPDIR=/tmp):

  rocprofv3 --kernel-trace --stats -d PROF_DIR/kt_up_proj -o kt -- python3 bench.py
  rocprofv3 --kernel-trace --stats -d PROF_DIR/kt_<workload> -o kt -- \\
      python3 bench.py --workload <workload> --no-cpu --no-bf16      (other workloads)
  rocprofv3 --kernel-trace --stats -d PROF_DIR/kt_copy -o kt -- python3 bench.py --copy-calib --steps 10
  rocprofv3 --pmc FETCH_SIZE -d PROF_DIR/pmc_FETCH_SIZE_<wl> -o pmc -- \\
      python3 bench.py --workload <workload> --steps 3 --warmup 1 --no-cpu --no-bf16
  rocprofv3 --pmc WRITE_SIZE -d PROF_DIR/pmc_WRITE_SIZE_<wl> -o pmc -- (same)
  rocprofv3 --pmc FETCH_SIZE|WRITE_SIZE -d PROF_DIR/pmc_<C>_copy -o pmc -- \\
      python3 bench.py --copy-calib --steps 3

(<wl> is the workload name, with "_proj" dropped for up and down). HBM bytes
per launch = counter KiB * 1024 * (known copy bytes / copy counter bytes).
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
KT_ARGS = " --workload {wl} --no-cpu --no-bf16"
PMC_CMD = ("rocprofv3 --pmc {c} -d {d}/pmc_{c}_{tag} -o pmc -- python3 bench.py "
           "--workload {wl} --steps 3 --warmup 1 --no-cpu --no-bf16")
COPY_PMC_CMD = "rocprofv3 --pmc {c} -d {d}/pmc_{c}_copy -o pmc -- python3 bench.py --copy-calib --steps 3"
COPY_BYTES = 1 << 30

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
    if "layernorm_quant_kernel" in kernel:
        return "layernorm_quant"
    if "quant_rows_long_kernel" in kernel:
        return "quant_rows_long"
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
    if "at::native" in kernel:
        return "torch_" + ("fill" if "FillFunctor" in kernel else "elementwise")
    return kernel.split("(")[0][-40:]


def kernel_stats(db: str):
    con = sqlite3.connect(db)
    rows = con.execute("select name, total_calls, total_duration, average, percentage "
                       "from top_kernels").fetchall()
    return [(short_name(n), n, c, t, a, p) for n, c, t, a, p in rows]


def pmc_values(db: str, counter: str):
    con = sqlite3.connect(db)
    rows = con.execute("select kernel_name, grid_size, value from counters_collection "
                       "where counter_name=?", (counter,)).fetchall()
    out = collections.defaultdict(list)
    for k, g, v in rows:
        out[(short_name(k), g)].append(v)
    return out


def main(prof_dir: str, out_dir: str, gemm_hash: str, quant_hash: str) -> None:
    os.makedirs(out_dir, exist_ok=True)
    # ---- kernel-trace summaries --------------------------------------------
    for path in sorted(glob.glob(os.path.join(prof_dir, "kt_*", "kt_results.db"))):
        wl = os.path.basename(os.path.dirname(path))[3:]
        stats = kernel_stats(path)
        if wl == "copy":
            cmd = f"rocprofv3 --kernel-trace --stats -d {prof_dir}/kt_copy -o kt -- python3 bench.py --copy-calib --steps 10"
            title = "plain 1 GiB device copy (HBM calibration)"
        else:
            cmd = KT_CMD.format(d=prof_dir, wl=wl)
            if wl != DEFAULT_WORKLOAD:
                cmd += KT_ARGS.format(wl=wl)
            title = WORKLOAD_SHAPES.get(wl, wl)
        lines = [f"# rocprofv3 kernel trace: {wl} -- {title}", "",
                 "Command (repository root, TMPDIR=/tmp, one MI355X):", f"    {cmd}", "",
                 f"{'kernel':<20} {'calls':>6} {'avg_us':>10} {'total_us':>11} {'pct':>6}"]
        for short, full, c, t, a, p in stats:
            lines.append(f"{short:<20} {c:>6} {a:>10.3f} {t:>11.3f} {p:>6.2f}")
        lines += ["", "Full kernel names:"] + [f"  {s}: {f[:160]}" for s, f, *_ in stats]
        lines += ["", f"gemm.hip source hash: {gemm_hash}  quant.hip source hash: {quant_hash}"]
        with open(os.path.join(out_dir, f"kernels_{wl}.txt"), "w") as f:
            f.write("\n".join(lines) + "\n")
    # ---- HBM traffic from FETCH_SIZE / WRITE_SIZE --------------------------
    calib = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        db = os.path.join(prof_dir, f"pmc_{c}_copy", "pmc_results.db")
        if not os.path.exists(db):
            return
        vals = [v for (k, g), vs in pmc_values(db, c).items() if k == "hip_copy_buffer"
                and g >= 65536 for v in vs]
        calib[c] = COPY_BYTES / (sum(vals) / len(vals) * 1024.0)
    for path in sorted(glob.glob(os.path.join(prof_dir, "pmc_FETCH_SIZE_*", "pmc_results.db"))):
        tag = os.path.basename(os.path.dirname(path))[len("pmc_FETCH_SIZE_"):]
        if tag == "copy":
            continue
        wl = tag if tag in WORKLOAD_SHAPES else f"{tag}_proj"
        fetch = pmc_values(path, "FETCH_SIZE")
        wpath = os.path.join(prof_dir, f"pmc_WRITE_SIZE_{tag}", "pmc_results.db")
        write = pmc_values(wpath, "WRITE_SIZE") if os.path.exists(wpath) else {}
        lines = [f"# HBM traffic per launch: {wl} -- {WORKLOAD_SHAPES.get(wl, wl)}", "",
                 "Commands (repository root, TMPDIR=/tmp, one MI355X):"]
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            lines.append("    " + PMC_CMD.format(c=c, d=prof_dir, tag=tag, wl=wl))
            lines.append("    " + COPY_PMC_CMD.format(c=c, d=prof_dir))
        lines += ["", f"Calibration on a 1 GiB copy: FETCH_SIZE x{calib['FETCH_SIZE']:.4f}, "
                      f"WRITE_SIZE x{calib['WRITE_SIZE']:.4f} (true bytes / counter bytes)", "",
                  f"{'kernel':<18} {'launches':>8} {'fetch_MB':>10} {'write_MB':>10} {'total_MB':>10}"]
        for (k, g), vs in sorted(fetch.items()):
            if k == "hip_copy_buffer":
                continue
            fb = sum(vs) / len(vs) * 1024 * calib["FETCH_SIZE"]
            wv = write.get((k, g), [])
            wb = (sum(wv) / len(wv) * 1024 * calib["WRITE_SIZE"]) if wv else float("nan")
            lines.append(f"{k:<18} {len(vs):>8} {fb / 1e6:>10.1f} {wb / 1e6:>10.1f} {(fb + wb) / 1e6:>10.1f}")
            if k.startswith(("gemm", "rmsnorm", "layernorm", "quant")):
                src = gemm_hash if k.startswith("gemm") else quant_hash
                with open(os.path.join(out_dir, f"traffic_{k}_{wl}.json"), "w") as f:
                    json.dump({"kernel": k, "workload": wl, "hbm_bytes_per_launch": round(fb + wb),
                               "fetch_bytes": round(fb), "write_bytes": round(wb),
                               "source_hash": src, "launches": len(vs)}, f, indent=1)
        with open(os.path.join(out_dir, f"traffic_{wl}.txt"), "w") as f:
            f.write("\n".join(lines) + "\n")
