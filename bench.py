"""Benchmark of the W8A8 INT8 Linear hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload up_proj]

One step = one pass of the whole per-call path over one batch of synthetic
activations, with the weights quantised once beforehand (the init-time step,
timed separately and reported, not part of a step):

  up_proj   (default)  RMSNorm+per-token quant [28672 x 4096] ->
                       INT8 GEMM + post-scale vs W [16384 x 4096] -> BF16
  down_proj            per-token quant [32760 x 13824] -> GEMM vs W [5120 x 13824]
  square               per-token quant [4096 x 4096] -> GEMM vs W [4096 x 4096]
  blockwise_small/large  1x128 quant [1000|32760 x 5120] -> blockwise GEMM vs
                       128x128-quantised W [5120 x 5120]
  m1000                per-token quant [1000 x 5120] -> GEMM vs W [5120 x 5120]
  (also ln_up_proj, up_proj_gelu, small_m: see workloads/)

Prints ONE JSON line: whole-step INT8 throughput (TOP/s, 2*M*N*K ops per
step), the per-kernel roofline of the dominant kernel (the GEMM, against the
5.0 POP/s dense INT8 MFMA peak), the quant kernel's HBM bandwidth, and the CPU
oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W8A8 GEMM INT8 TOPS + % INT8 MFMA peak at DiT FFN shapes; quant GB/s"
INT8_PEAK_TOPS = 5000.0        # MI355X dense INT8 MFMA, TOP/s
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
N_ROTATE = 3                   # activation buffers cycled so inputs come from HBM
GEMM_SOURCES = ("gemm.hip", "gemm_pipelined.hip", "gemm_blockwise.hip", "gemm_tile160.hip",
                "splitk.hip", "pipeline.hpp", "device_common.hpp", "launch.hpp")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    # about 0.2 s of untimed steps at the default workload: the engine clock
    # needs ~150 ms of load to ramp before timing is representative
    p.add_argument("--warmup", type=int, default=100)
    p.add_argument("--workload", default="up_proj",
                   help="up_proj (default), down_proj, ln_up_proj, up_proj_gelu, square, m1000, "
                        "blockwise_small, blockwise_large, small_m or tiny (sizes in workloads/)")
    p.add_argument("--preload-ms", type=float, default=250.0,
                   help="untimed load before the timed steps: at least this much wall time "
                        "(and at least --warmup steps)")
    p.add_argument("--b2b-ms", type=float, default=20.0,
                   help="back-to-back launches of each kernel after the timed steps: at least "
                        "this much GPU time (and at least 10 launches)")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--no-bf16", action="store_true", help="skip the torch BF16 Linear yardstick")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--copy-calib", action="store_true",
                   help="only run a plain 1 GiB device-to-device copy (HBM counter calibration)")
    p.add_argument("--no-ceiling", action="store_true",
                   help="skip the main-loop ceiling probe in the bench line's extra fields")
    p.add_argument("--ceiling", action="store_true",
                   help="only time the post-scale GEMM's main loop alone (probe library) on "
                        "constant and on random operands")
    p.add_argument("--summarize", metavar="PROF_DIR",
                   help="summarise rocprofv3 results under PROF_DIR into profiles/ (no GPU)")
    return p.parse_args()


def copy_calibration(steps: int) -> None:
    """A plain copy of known size: its FETCH_SIZE / WRITE_SIZE readings scale
    the counters of the W8A8 kernels, and its time is the achievable HBM rate."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dsts = [torch.empty_like(src) for _ in range(2)]
    for d in dsts:
        d.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        dsts[i % 2].copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "copy_ms": round(ms, 4),
                      "copy_gbs": round(2 * n / (ms * 1e-3) / 1e9, 1)}), flush=True)


def measure_mainloop_ceiling(verbose: bool = False):
    """The post-scale GEMM's inner loop alone (libw8a8_probe.so: the same LDS
    ring, fragment reads and MFMA stream, no epilogue, operands L2-resident),
    timed on constant operands, on uniformly random ones, and on random ones
    without the stage refills. The first is the rate the schedule allows; the
    drop to the second is what the power drawn by random operands costs.
    Returns {case: {...}} or None if the probe library is not built."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "w8a8_int8_quantized_token_amd", "libw8a8_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.w8a8_probe_mainloop_workgroups.restype = ctypes.c_int
    lib.w8a8_probe_mainloop.restype = ctypes.c_int
    lib.w8a8_probe_mainloop.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
                                        ctypes.c_void_p]
    torch.cuda.init()
    grid = lib.w8a8_probe_mainloop_workgroups()
    if grid < 1:
        raise RuntimeError("cannot read the compute-unit count")
    src = torch.empty(2 << 20, dtype=torch.int8, device="cuda")
    sink = torch.empty(grid * 512, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    stages = 2048
    ops = 2.0 * 256 * 256 * 128 * grid * stages
    rand = torch.randint(-127, 128, (src.numel(),), dtype=torch.int8,
                         generator=torch.Generator().manual_seed(1234))
    results = {}
    for name, data, refill in (("constant", None, 1), ("random", rand, 1),
                               ("random_no_refill", rand, 0)):
        if data is None:
            src.fill_(1)
        else:
            src.copy_(data)

        def call():
            rc = lib.w8a8_probe_mainloop(src.data_ptr(), src.numel(), stages, refill,
                                         sink.data_ptr(), sink.numel(), stream.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"w8a8_probe_mainloop failed ({rc})")

        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        call()
        e0.record(stream)
        call()
        e1.record(stream)
        torch.cuda.synchronize()
        # >= 200 ms of load first: the engine clock ramps over ~150 ms
        for _ in range(max(3, int(200.0 / max(e0.elapsed_time(e1), 0.01)))):
            call()
        reps = 20
        e0.record(stream)
        for _ in range(reps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        results[name] = {"us_per_launch": round(ms * 1e3, 1),
                         "us_per_stage": round(ms * 1e3 / stages, 4),
                         "tops": round(ops / (ms * 1e-3) / 1e12, 1),
                         "frac_of_int8_peak": round(ops / (ms * 1e-3) / 5.0e15, 4)}
        if verbose:
            print(f"{name:18s} {results[name]}", flush=True)
    return {"workgroups": grid, "stages": stages, "results": results}


class ClockStamps:
    """Average shader clock over a region of one stream's work, from the probe
    library's stamp kernel (one workgroup per CU records its CU id, the shader
    clock counter and the 100 MHz real-time counter) launched before and after
    the region. None when the probe library is not built."""

    def __init__(self, stream):
        import ctypes
        import torch
        path = os.path.join(ROOT, "w8a8_int8_quantized_token_amd", "libw8a8_probe.so")
        self.ok = os.path.exists(path)
        if not self.ok:
            return
        self.lib = ctypes.CDLL(path)
        self.lib.w8a8_probe_clock_stamp.restype = ctypes.c_int
        self.lib.w8a8_probe_clock_stamp.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                                    ctypes.c_void_p]
        self.lib.w8a8_probe_mainloop_workgroups.restype = ctypes.c_int
        self.wg = max(1, self.lib.w8a8_probe_mainloop_workgroups())
        self.buf = [torch.zeros(4 * self.wg, dtype=torch.int64, device="cuda") for _ in range(2)]
        self.stream = stream

    def stamp(self, which: int) -> None:
        if self.ok:
            b = self.buf[which]
            rc = self.lib.w8a8_probe_clock_stamp(b.data_ptr(), b.numel(), self.wg,
                                                 self.stream.cuda_stream)
            if rc != 0:
                self.ok = False

    def ghz(self):
        """Mean over CUs of (shader cycles / real time) between the stamps."""
        if not self.ok:
            return None
        a = self.buf[0].view(-1, 4).cpu().numpy()
        b = self.buf[1].view(-1, 4).cpu().numpy()
        first_a, first_b = {}, {}
        for rec, d in ((a, first_a), (b, first_b)):
            for key, t, r, _ in rec:
                d.setdefault(int(key), (int(t), int(r)))
        rates = []
        for key, (t0, r0) in first_a.items():
            if key in first_b:
                t1, r1 = first_b[key]
                if r1 > r0 and t1 > t0:
                    rates.append((t1 - t0) / ((r1 - r0) * 10.0))      # cycles per ns = GHz
        if not rates:
            return None
        return {"ghz_mean": round(float(np.mean(rates)), 4),
                "ghz_min": round(float(np.min(rates)), 4),
                "ghz_max": round(float(np.max(rates)), 4), "cus": len(rates)}


def mainloop_ceiling() -> None:
    res = measure_mainloop_ceiling(verbose=True)
    if res is None:
        sys.exit("libw8a8_probe.so is missing: build it with __graft_entry__.build()")
    print(json.dumps({"probe": "gemm_mainloop", "workgroups": res["workgroups"],
                      "stages": res["stages"], "block_tile": [256, 256, 128],
                      "peak_tops": 5000.0, "results": res["results"]}), flush=True)


def rel_error_vs_fp32_linear(wl, x, w, gamma, mod_scale, mod_shift, bias, out) -> float:
    """Relative Frobenius error of the W8A8 step's BF16 output against a
    float32 Linear (torch, on the GPU) of the same unquantised BF16 input:
    after the step's norm prologue, rounded to BF16 as the fused kernels do
    before quantising, with the bias and the GELU (erf form) where the step
    has them. An informational figure of the quantisation noise, not a parity
    check (the parity tests compare with the oracle)."""
    import torch
    xf = x.float()
    if wl.norm:
        r = torch.rsqrt(xf.double().square().mean(1, keepdim=True) + wl.eps).float()
        y = ((xf * r) * gamma.float()).bfloat16().float()
    elif wl.layernorm:
        xd = xf.double()
        mu = xd.mean(1, keepdim=True)
        r = torch.rsqrt((xd - mu).square().mean(1, keepdim=True) + wl.eps).float()
        y = ((xf - mu.float()) * r).bfloat16().float()
        y = (y * (1.0 + mod_scale.float()).bfloat16().float()).bfloat16().float()
        y = (y + mod_shift.float()).bfloat16().float()
    else:
        y = xf
    del xf
    ref = torch.nn.functional.linear(y, w.float())
    del y
    if bias is not None:
        ref += bias.float()
    if wl.gelu:
        ref = torch.nn.functional.gelu(ref)
    err = float(torch.linalg.vector_norm((out.float() - ref).double()))
    rel = err / float(torch.linalg.vector_norm(ref.double()))
    del ref
    torch.cuda.empty_cache()
    return round(rel, 5)


def source_hash(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "w8a8_int8_quantized_token_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, workload: str, src_hash: str):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, or None
    if there is none or the kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != src_hash:
        return None
    return rec.get("hbm_bytes_per_launch")


def load_counters(kernel: str, workload: str, src_hash: str):
    """MFMA and clock counters of one launch from a committed rocprofv3 --pmc
    summary (profiles/mfma_<kernel>_<workload>.json), or None if there is none
    or the kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"mfma_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != src_hash:
        return None
    return {k: rec[k] for k in ("mfma_busy_frac", "clock_ghz", "frac_of_peak_at_clock",
                                "mfma_ops_counted", "source") if k in rec}


def main():
    args = parse()
    if args.summarize:
        import profile_summary
        profile_summary.main(args.summarize, os.path.join(ROOT, "profiles"),
                             source_hash(*GEMM_SOURCES),
                             source_hash("quant.hip", "device_common.hpp"))
        return
    if args.copy_calib:
        copy_calibration(args.steps)
        return
    if args.ceiling:
        mainloop_ceiling()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the W8A8 Linear is "
              "token-parallel and needs no collectives (several GPUs would each take their own token "
              "rows, with the quantised weight replicated).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as W
    import w8a8_int8_quantized_token_amd as w8

    wl = W.WORKLOADS[args.workload]
    M, N, K = wl.M, wl.N, wl.K
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    t0 = time.perf_counter()
    x_host = W.x_bits(wl)
    w_host = W.w_bits(wl)
    gamma = up(W.gamma_bits(wl)) if wl.norm else None
    mod_scale = up(W.mod_bits(wl, "mod_scale")) if wl.layernorm else None
    mod_shift = up(W.mod_bits(wl, "mod_shift")) if wl.layernorm else None
    bias = up(W.bias_bits(wl)) if wl.bias_std > 0 else None
    xs = [up(x_host)]
    for _ in range(N_ROTATE - 1):
        xs.append(xs[0].clone())
    w_bf16 = up(w_host)
    gen_s = time.perf_counter() - t0

    # ---- init-time weight quantisation (not part of a step) -----------------
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    if wl.blockwise:
        qw, sw = w8.w8a8_quant_rows(w_bf16, 128, 128)
    else:
        qw, sw = w8.w8a8_quant_rows(w_bf16)
    ev[1].record(stream)
    torch.cuda.synchronize()
    wquant_ms = ev[0].elapsed_time(ev[1])

    qa = torch.empty((M, K), dtype=torch.int8, device=dev)
    if wl.blockwise:
        sa = torch.empty((M, K // 128), dtype=torch.float32, device=dev)
    else:
        sa = torch.empty((M,), dtype=torch.float32, device=dev)
    inv = torch.empty((M,), dtype=torch.float32, device=dev)
    mean = torch.empty((M,), dtype=torch.float32, device=dev)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

    if wl.norm:
        quant_name = "rmsnorm_quant"
        def quant(x):
            w8.w8a8_rmsnorm_quant(x, gamma, wl.eps, q=qa, scale=sa, inv_rms=inv)
        quant_bytes = 3 * M * K + 4 * M + 2 * K + 4 * M     # read x, gamma; write q, scale, inv_rms
    elif wl.layernorm:
        quant_name = "layernorm_quant"
        def quant(x):
            w8.w8a8_layernorm_quant(x, wl.eps, mod_scale=mod_scale, mod_shift=mod_shift, q=qa,
                                    scale=sa, mean=mean, rstd=inv)
        # read x, the two modulation vectors; write q, scale, mean, rstd
        quant_bytes = 3 * M * K + 4 * K + 4 * M + 8 * M
    elif wl.blockwise:
        quant_name = "quant_rows_1x128"
        def quant(x):
            w8.w8a8_quant_rows(x, 1, 128, q=qa, scale=sa)
        quant_bytes = 3 * M * K + 4 * M * (K // 128)
    else:
        quant_name = "quant_rows"
        def quant(x):
            w8.w8a8_quant_rows(x, q=qa, scale=sa)
        quant_bytes = 3 * M * K + 4 * M

    if wl.blockwise:
        gemm_name = "gemm_blockwise" + ("_t160" if w8.tile_channels(M, N, K, True) == 160 else "")
        def gemm(_i=0):
            w8.w8a8_gemm_blockwise(qa, qw, sa, sw, out=out)
    else:
        # the epilogue's extras (bias, GELU) and, where the library splits K
        # (few tokens), its two passes all count as the GEMM
        gemm_name = ("gemm_postscale" + ("_bias" if bias is not None else "")
                     + ("_gelu" if wl.gelu else "")
                     + ("_splitk" if w8.splitk_parts(M, N, K) > 1 else
                        ("_t160" if w8.tile_channels(M, N, K) == 160 else "")))
        def gemm(_i=0):
            w8.w8a8_gemm_postscale(qa, qw, sa, sw, out=out, bias=bias, gelu=wl.gelu)

    ops = 2 * M * N * K
    # Untimed load: the --warmup steps, then more steps until at least
    # PRELOAD_MS of wall time has passed (the engine clock ramps over
    # ~150 ms of load; a step count alone can leave it short of steady state).
    # Everything the timed region needs is set up first (the clock probe's
    # first launch loads its code object, some ms of host time): an idle gap
    # between the pre-load and the timed steps lets the clock drop, and the
    # first timed steps then run up to a quarter slower while it recovers.
    clock = ClockStamps(stream)
    clock.stamp(0)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t_pre = time.perf_counter()
    done = 0
    while True:
        for _ in range(5):
            quant(xs[done % N_ROTATE])
            gemm()
            done += 1
        torch.cuda.synchronize()
        if done >= args.warmup and (time.perf_counter() - t_pre) * 1e3 >= args.preload_ms:
            break
    preload_ms = (time.perf_counter() - t_pre) * 1e3

    torch.cuda.synchronize()
    t_start = time.perf_counter()
    clock.stamp(0)
    for i in range(args.steps):
        e = evs[i]
        e[0].record(stream)
        quant(xs[i % N_ROTATE])
        e[1].record(stream)
        gemm()
        e[2].record(stream)
    clock.stamp(1)
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t_start
    quant_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    gemm_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])
    step_ms = np.array([e[0].elapsed_time(e[2]) for e in evs])
    ms_per_step = wall_s * 1e3 / args.steps

    # Each kernel alone, back to back between one event pair on the launch
    # stream, right after the timed steps: its average launch duration
    # without the gaps that a per-launch event pair adds (a few us, which
    # matter for kernels of tens of us). These give the roofline figures.
    def back_to_back(fn, least=10):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = max(least, int(args.b2b_ms / max(float(gemm_ms.mean()), 1e-3)) if fn is gemm else 30)
        e0.record(stream)
        for i in range(reps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps, reps

    quant_b2b_ms, _ = back_to_back(lambda i: quant(xs[i % N_ROTATE]))
    gemm_b2b_ms, gemm_reps = back_to_back(gemm)

    gemm_avg = gemm_b2b_ms
    gemm_tops = ops / (gemm_avg * 1e-3) / 1e12
    quant_avg = float(quant_ms.mean())
    quant_gbs = quant_bytes / (quant_avg * 1e-3) / 1e9
    value = ops / (ms_per_step * 1e-3) / 1e12

    gemm_hash = source_hash(*GEMM_SOURCES)
    traffic = load_traffic(gemm_name, args.workload, gemm_hash)

    extra = {
        "gemm_ms_avg": round(gemm_avg, 4), "gemm_back_to_back_launches": gemm_reps,
        "gemm_ms_in_step_avg": round(float(gemm_ms.mean()), 4),
        "gemm_ms_in_step_min": round(float(gemm_ms.min()), 4),
        "gemm_tops": round(gemm_tops, 1), "gemm_frac_int8_peak": round(gemm_tops / INT8_PEAK_TOPS, 4),
        f"{quant_name}_ms_avg": round(quant_b2b_ms, 4),
        f"{quant_name}_gbs": round(quant_bytes / (quant_b2b_ms * 1e-3) / 1e9, 1),
        f"{quant_name}_frac_hbm_peak": round(quant_bytes / (quant_b2b_ms * 1e-3) / 1e9
                                             / HBM_PEAK_GBS, 4),
        f"{quant_name}_ms_in_step": round(quant_avg, 4), f"{quant_name}_gbs_in_step": round(quant_gbs, 1),
        "event_step_ms_avg": round(float(step_ms.mean()), 4),
        "weight_quant_ms": round(wquant_ms, 4), "input_gen_s": round(gen_s, 1),
        "preload_ms": round(preload_ms, 1), "preload_steps": done,
    }
    clk = clock.ghz()
    if clk is not None:
        # the shader clock over the timed region, and the GEMM's rate over the
        # peak at that clock (the share of cycles its MFMAs were busy)
        extra["shader_clock_timed_region"] = clk
        extra["gemm_frac_of_peak_at_measured_clock"] = round(
            gemm_tops / (INT8_PEAK_TOPS * clk["ghz_mean"] / 2.4), 4)
    mfma = load_counters(gemm_name, args.workload, source_hash(*GEMM_SOURCES))
    if mfma is not None:
        extra["gemm_counters"] = mfma

    # ---- the pages' yardstick: torch's BF16 Linear on the same shape ---------
    if not args.no_bf16:
        wt = w_bf16
        def bf16_linear(x):
            y = torch.nn.functional.linear(x, wt, bias)
            return torch.nn.functional.gelu(y) if wl.gelu else y
        for i in range(3):
            bf16_linear(xs[i % N_ROTATE])
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 10
        e0.record(stream)
        for i in range(reps):
            bf16_linear(xs[i % N_ROTATE])
        e1.record(stream)
        torch.cuda.synchronize()
        bf16_ms = e0.elapsed_time(e1) / reps
        extra["torch_bf16_linear_ms"] = round(bf16_ms, 4)
        extra["speedup_vs_bf16_linear"] = round(bf16_ms / float(step_ms.mean()), 3)
        # informational accuracy of the step's output (every rotated input
        # holds the same values, so `out` is the W8A8 Linear of xs[0])
        extra["rel_frobenius_error_vs_fp32_linear"] = rel_error_vs_fp32_linear(
            wl, xs[0], w_bf16, gamma, mod_scale, mod_shift, bias, out)

    # ---- the post-scale kernel's own main loop on this GPU, as a yardstick
    # for roofline.frac (the chip's power limit caps it on random operands) --
    if gemm_name.startswith("gemm_postscale") and not args.no_ceiling:
        try:
            ceil = measure_mainloop_ceiling()
        except RuntimeError as e:     # the probe is a yardstick, not the product
            ceil = None
            extra["mainloop_ceiling_error"] = str(e)
        if ceil is not None:
            fr = {k: v["frac_of_int8_peak"] for k, v in ceil["results"].items()}
            extra["mainloop_ceiling_frac"] = fr
            extra["gemm_frac_of_mainloop_ceiling_random"] = round(
                gemm_tops / INT8_PEAK_TOPS / fr["random"], 4)

    # ---- CPU oracle on a bounded sample of the same workload -----------------
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(wl, x_host, w_host, args.cpu_seconds)

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": args.workload, "M": M, "N": N, "K": K,
                   "step": f"{quant_name}+{gemm_name}", "weights": "int8, quantised at init"},
        "roofline": {"bound": "mfma", "achieved": round(gemm_tops, 1), "peak": INT8_PEAK_TOPS,
                     "unit": "TOP/s", "frac": round(gemm_tops / INT8_PEAK_TOPS, 4),
                     "traffic": traffic, "kernel": gemm_name, "ops_per_launch": ops},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, x_host, w_host, budget_s):
    """The oracle, as it stands, on as many leading token rows as fit the time
    budget, on every core of this process's affinity mask: the row chunk's
    quantisation (and norm) runs as one oracle call per sub-chunk on a thread
    pool (numpy releases the GIL), the GEMM and epilogue as one oracle call on
    the chunk with BLAS threads set to the same count."""
    import concurrent.futures as cf
    import oracle as O
    import workloads as W
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=cores)
    except Exception:  # pragma: no cover
        limiter = None
    pool = cf.ThreadPoolExecutor(max_workers=cores)
    t0 = time.perf_counter()
    if wl.blockwise:
        qw, sw = O.quantize_groups(w_host, 128, 128)
    else:
        qw, sw = O.quantize_rows(w_host)
    t_w = time.perf_counter() - t0
    b = W.bias_bits(wl) if wl.bias_std > 0 else None
    g = W.gamma_bits(wl) if wl.norm else None
    msc = W.mod_bits(wl, "mod_scale") if wl.layernorm else None
    msh = W.mod_bits(wl, "mod_shift") if wl.layernorm else None

    def quant_part(x):
        if wl.norm:
            qa, sa, _ = O.rmsnorm_quant(x, g, wl.eps)
        elif wl.layernorm:
            qa, sa, _, _ = O.layernorm_quant(x, wl.eps, scale_bits=msc, shift_bits=msh)
        elif wl.blockwise:
            qa, sa = O.quantize_groups(x, 1, 128)
        else:
            qa, sa = O.quantize_rows(x)
        return qa, sa

    def epilogue(acc, sa):
        if wl.gelu:
            return O.postscale_gelu_bf16(acc, sa, sw, b)
        if b is not None:
            return O.postscale_bias_bf16(acc, sa, sw, b)
        return O.postscale_bf16(acc, sa, sw)

    rows_done = 0
    chunk = 256
    t_path = 0.0
    n_rows = min(wl.M, x_host.shape[0])
    while rows_done < n_rows and t_path < budget_s:
        r1 = min(rows_done + chunk, n_rows)
        x = x_host[rows_done:r1]
        t1 = time.perf_counter()
        bounds = np.linspace(0, x.shape[0], min(cores, max(1, x.shape[0] // 16)) + 1).astype(int)
        res = list(pool.map(lambda ab: quant_part(x[ab[0]:ab[1]]), zip(bounds[:-1], bounds[1:])))
        qa = np.concatenate([r[0] for r in res])
        sa = np.concatenate([r[1] for r in res])
        if wl.blockwise:
            O.gemm_blockwise_bf16(qa, sa, qw, sw)
        else:
            epilogue(O.gemm_i32(qa, qw), sa)
        t_path += time.perf_counter() - t1
        rows_done = r1
        chunk = min(chunk * 2, 4096)
    pool.shutdown()
    if limiter is not None and hasattr(limiter, "restore_original_limits"):
        limiter.restore_original_limits()
    ops = 2 * rows_done * wl.N * wl.K
    return {"value": round(ops / t_path / 1e12, 5), "unit": "TOP/s", "cores": cores,
            "kind": "oracle", "cpu": cpu_model(),
            "sample": f"first {rows_done} of {wl.M} token rows through the whole per-call path "
                      f"({t_path:.1f} s); weight quant of all {wl.N} rows took {t_w:.1f} s, excluded"}


if __name__ == "__main__":
    main()
