"""Concurrent calls from several host threads, each on its own stream.

The C ABI keeps no per-call state on the host beyond a thread-local error
string and per-device caches of device queries, so calls from different
threads on different streams must give exactly the single-thread results:
per-token quant codes and scales, LayerNorm + modulation codes (checked
against the oracle from the statistics the kernel reports, as in the
single-thread test), and post-scale GEMM outputs, one pass and split over K
into workspaces taken on each thread's stream. Everything is compared with
the oracle ("TurboDiffusion Integration Notes", "Reused Components", W8A8
Linear and FastNorm bullets; "Differences From TurboDiffusion", paragraph
under the table).
"""
from __future__ import annotations

import threading

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
import w8a8_int8_quantized_token_amd as w8
from tests.gpu_util import (bf16_from_dev, bf16_to_dev, check_inv_rms, check_ln_mean, from_dev,
                            log, to_dev)

pytestmark = pytest.mark.gpu

THREADS = 4
REPEATS = 3
QUANT_SHAPE = (96, 4096)
LN_SHAPE = (64, 4096)
# (M, N, K, parts): the library's choice, a forced split, the single pass
GEMMS = [(200, 1024, 3072, 8), (129, 1280, 4096, 0), (300, 768, 1024, 1)]


def _inputs(t: int):
    base = 700 + 40 * t
    inp = {"x": W.random_bits(QUANT_SHAPE, base, std=2.0),
           "ln": W.random_bits(LN_SHAPE, base + 1, std=1.5, mean=0.3),
           "sc": W.random_bits((LN_SHAPE[1],), base + 2, std=0.2),
           "sh": W.random_bits((LN_SHAPE[1],), base + 3, std=0.2)}
    for i, (M, N, K, _) in enumerate(GEMMS):
        inp[f"qa{i}"] = W.random_int8((M, K), base + 10 + 4 * i)
        inp[f"qw{i}"] = W.random_int8((N, K), base + 11 + 4 * i)
        inp[f"sa{i}"] = W.random_scales((M,), base + 12 + 4 * i)
        inp[f"sw{i}"] = W.random_scales((N,), base + 13 + 4 * i, lo=1e-5, hi=1e-3)
    return inp


def _run(inp, results, errors, t, barrier):
    try:
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            dev = {k: (bf16_to_dev(v) if v.dtype == np.uint16 else to_dev(v))
                   for k, v in inp.items()}
            torch.cuda.current_stream().synchronize()
            barrier.wait(timeout=60)            # every thread issues at once
            out = []
            for _ in range(REPEATS):
                q, sc = w8.w8a8_quant_rows(dev["x"])
                lq, ls, lmu, lr = w8.w8a8_layernorm_quant(dev["ln"], 1e-6, mod_scale=dev["sc"],
                                                          mod_shift=dev["sh"])
                gs = [w8.w8a8_gemm_postscale(dev[f"qa{i}"], dev[f"qw{i}"], dev[f"sa{i}"],
                                             dev[f"sw{i}"], parts=p)
                      for i, (_, _, _, p) in enumerate(GEMMS)]
                out.append((q, sc, lq, ls, lmu, lr, gs))
            torch.cuda.current_stream().synchronize()
            results[t] = [(from_dev(q), from_dev(sc), from_dev(lq), from_dev(ls), from_dev(lmu),
                           from_dev(lr), [bf16_from_dev(g) for g in gs])
                          for q, sc, lq, ls, lmu, lr, gs in out]
    except BaseException as e:                  # reported by the main thread
        errors[t] = e
        barrier.abort()                         # no other thread waits for this one


def test_threads_on_own_streams_match_the_oracle():
    inputs = [_inputs(t) for t in range(THREADS)]
    results, errors = [None] * THREADS, [None] * THREADS
    barrier = threading.Barrier(THREADS)
    log(f"{THREADS} threads x {REPEATS} rounds of quant, LayerNorm quant and 3 GEMMs")
    threads = [threading.Thread(target=_run, args=(inputs[t], results, errors, t, barrier),
                                daemon=True) for t in range(THREADS)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a thread did not finish"
    for e in errors:
        if e is not None:
            raise e
    for t in range(THREADS):
        inp = inputs[t]
        qo, so = O.quantize_rows(inp["x"])
        refs = [O.postscale_bf16(O.gemm_i32(inp[f"qa{i}"], inp[f"qw{i}"]), inp[f"sa{i}"],
                                 inp[f"sw{i}"]) for i in range(len(GEMMS))]
        mu_ref, r_ref = O.layernorm_stats(inp["ln"], 1e-6)
        first = results[t][0]
        for rnd, (q, sc, lq, ls, lmu, lr, gs) in enumerate(results[t]):
            assert np.array_equal(q, qo) and np.array_equal(sc.view(np.uint32), so.view(np.uint32))
            check_ln_mean(lmu, mu_ref, O.bf16_to_f32(inp["ln"]))
            check_inv_rms(lr, r_ref, LN_SHAPE[1])
            lqo, lso, _, _ = O.layernorm_quant(inp["ln"], 1e-6, None, None, inp["sc"], inp["sh"],
                                               mu=lmu, r=lr)
            assert np.array_equal(lq, lqo) and np.array_equal(ls.view(np.uint32),
                                                              lso.view(np.uint32))
            # the statistics' reduction order is fixed within the kernel, so
            # every round repeats the first bit for bit
            assert np.array_equal(lmu, first[4]) and np.array_equal(lr, first[5])
            for i, g in enumerate(gs):
                assert np.array_equal(g, refs[i]), (t, rnd, GEMMS[i])
    log("  all threads exact")
