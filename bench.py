#!/usr/bin/env python3
"""Benchmark of the bifocal RoPE attention hot path on one MI355X.

A step is one bifocal prefill of the Qwen3-4B-shaped 128K workload (32 query heads,
8 KV heads, head dim 128, L = 131072, w_pretrained = 32768 so G = 4, w0 = 4096,
theta = 1e6, outlier channels), inputs resident in HBM.  The same run also times the
Qwen3-8B-shaped decode workload (256 consecutive steps ending at position 131071 over
a 128K standard-RoPE cache) and reports it in the "decode" object.

Prints one JSON line on stdout; progress goes to stderr.
  value      prefill TFLOP/s counted as causal-attention FLOPs plus the second score
             set over the local window: F = 4*D*Hq*sum_i(i+1) + 2*D*Hq*sum_i min(i+1, w0)
  roofline   the prefill kernel against the dense bf16 MFMA peak (2500 TFLOP/s)
  decode     KV GB/s = bytes of K and V read per step / step time, against 8000 GB/s
  decode_batch  a batch of 8 sequences of 16K rows each in one bifocal_decode_batch call
             per step (the same K + V bytes per step as the 128K sequence)
  other_prefills  the Qwen3-1.7B-shaped 32K layer with G = 1 and the Qwen3-8B-shaped
             ragged batch (98427 + 40001 tokens, G = 4 and 2 per sequence): ms per call,
             TFLOP/s counted the same way and the fraction of the bf16 peak
  rope_apply the standard-RoPE rotation of the 128K query tensor in place: us per call,
             GB/s (every element read and written once) and the fraction of 8000 GB/s
  three_pass the literal inclusion-exclusion form of the same prefill (local/window,
             remote/causal and remote/window passes merged by their LSEs): time and the
             ratio to the fused call
  vanilla    the same calls with w0 >= L (every pair local, i.e. causal attention with
             standard RoPE, no remote branch): prefill and decode times and the bifocal /
             vanilla ratios, the local analogue of the pages' overhead figures
  cpu_baseline  the CPU oracle timed on sampled query rows, extrapolated by pair count;
             also the host (CPU model, cores), the small prefill workload run whole and two
             sampled steps of the 128K decode workload
  executed_mfma  matrix-core FLOPs actually issued per launch (SQ_INSTS_VALU_MFMA_MOPS_*
             counters, profiles/prefill_counters.json) over the measured time, with the
             MFMA-busy and VALU/MFMA co-execution shares; null when the kernel source
             changed after the counters were taken
  ms_median  median prefill call time (ms_per_step is the mean over the timed calls)
  traffic    HBM bytes per launch of the timed kernel from rocprofv3 FETCH_SIZE and
             WRITE_SIZE counters (profiles/hbm_traffic.json), scaled by what the same
             counters read for a plain 1 GiB device copy (``--only copy``); null when
             the kernel source changed after the counters were taken.
"""
from __future__ import annotations

import argparse
import contextlib
import gc
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# queue_primed: every timed region starts with one untimed call enqueued just before its
# start event.  After the synchronize that precedes it the GPU is idle, so without that
# call the start event would also time the host's submission of the first timed call
# (Python, binding, launch: about 0.1 ms, i.e. about 20 us per call over the five
# rope_apply calls and 0.3-1 us per decode step).  With it, the start event completes when
# the priming call's kernels do, and the timed calls are already queued behind it: the
# region holds exactly the timed calls, back to back, as in a serving loop.


@contextlib.contextmanager
def quiet_host():
    """A timed region without Python's cyclic garbage collector: a full collection after
    the large setups can pause the submitting thread for tens of milliseconds, which a
    launch-rate-bound loop (decode) would otherwise count as GPU time."""
    gc.collect()
    gc.disable()
    try:
        yield
    finally:
        gc.enable()


# Files that decide the timed kernels' machine code (sources and the build flags).
KERNEL_SOURCES = {
    "prefill": ["dynamic_rope_context_amd/csrc/prefill_mfma.hip",
                "dynamic_rope_context_amd/csrc/prefill_args.h",
                "dynamic_rope_context_amd/csrc/mfma_util.h",
                "dynamic_rope_context_amd/csrc/bf_common.h",
                "dynamic_rope_context_amd/build.py"],
    "decode": ["dynamic_rope_context_amd/csrc/decode_mfma.hip",
               "dynamic_rope_context_amd/csrc/decode.hip",
               "dynamic_rope_context_amd/csrc/decode_args.h",
               "dynamic_rope_context_amd/csrc/mfma_util.h",
               "dynamic_rope_context_amd/csrc/bf_common.h",
               "dynamic_rope_context_amd/build.py"],
}


def source_hash(kind):
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def hbm_traffic(kind):
    """Bytes moved to/from HBM per launch of the timed kernel, from the committed
    counter summary; None if absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
        k = rec[kind]
        if k["source_sha256"] != source_hash(kind):
            return None
        c = rec["copy"]
        f_fac = c["bytes_read"] / (c["FETCH_SIZE_KiB"] * 1024.0)
        w_fac = c["bytes_written"] / (c["WRITE_SIZE_KiB"] * 1024.0)
        return (k["FETCH_SIZE_KiB"] * f_fac + k["WRITE_SIZE_KiB"] * w_fac) * 1024.0
    except (OSError, KeyError, ValueError, ZeroDivisionError):
        return None


def mfma_counters(kind="prefill"):
    """Executed MFMA FLOPs per launch and the MFMA busy / co-execution shares of the
    timed kernel, from the committed counter summary; None if absent or taken on a
    different kernel source."""
    path = os.path.join(ROOT, "profiles", "prefill_counters.json")
    try:
        with open(path) as f:
            rec = json.load(f)
        if rec["source_sha256"] != source_hash(kind):
            return None
        return rec["derived"]
    except (OSError, KeyError, ValueError):
        return None


def bench_copy(torch, mib, reps):
    """A plain device copy of known size: the calibration run for the HBM byte counters."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    return {"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "launches": reps}


def prefill_flops(seqlens, w0, Hq, D):
    pc = sum(L * (L + 1) // 2 for L in seqlens)
    pw = 0
    for L in seqlens:
        m = min(L, w0)
        pw += m * (m + 1) // 2 + (L - m) * w0
    return 4 * D * Hq * pc + 2 * D * Hq * pw, 4 * D * Hq * pc


def bench_prefill(bf, torch, W, steps, warmup, w0=None, three_pass=False,
                  name="qwen3_4b_128k"):
    """w0 overrides the window (w0 >= L: vanilla mode, every pair local); three_pass
    times the literal inclusion-exclusion form (three passes + LSE merge)."""
    w = W.get(name)
    if w0 is not None:
        import dataclasses
        w = dataclasses.replace(w, w0=w0)
    T = w.total_tokens
    q, k, v = W.raw_inputs_torch(w, "cuda")
    # standard RoPE at each sequence's positions, built with the library's own rope_apply
    cu = [int(c) for c in w.cu_seqlens]
    for b in range(len(cu) - 1):
        bf.rope_apply(q[cu[b]:cu[b + 1]], w.theta)
        bf.rope_apply(k[cu[b]:cu[b + 1]], w.theta)
    out = torch.empty_like(q)
    lse = torch.empty((w.Hq, T), dtype=torch.float32, device="cuda")
    op = bf.OP_PREFILL_IE if three_pass else bf.OP_PREFILL
    ws = bf.Workspace.for_op(op, max(w.seqlens), w.Hq, w.Hkv, w.D,
                             total_tokens=T, num_seqs=len(w.seqlens))
    fn = bf.bifocal_prefill_ie if three_pass else bf.bifocal_prefill
    call = lambda: fn(q, k, v, cu, w.w0, w.w_pretrained, w.theta, out=out, lse=lse, workspace=ws)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    with quiet_host():
        call()  # primes the queue (see queue_primed)
        ev[0].record(stream)
        for i in range(steps):
            call()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
    per_call = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    ms = ev[0].elapsed_time(ev[steps]) / steps
    F, Fc = prefill_flops(w.seqlens, w.w0, w.Hq, w.D)
    assert bool(torch.isfinite(out).all())
    return w, ms, F, Fc, float(np.median(per_call))


def bench_other_prefills(bf, torch, W, steps, warmup):
    """The Qwen3-1.7B 32K layer (G = 1: every pair local) and the Qwen3-8B ragged layer
    (two sequences, G = 4 and 2) on the GPU: time per call, counted TFLOP/s (the same F
    definition as the headline) and its fraction of the bf16 dense peak."""
    out = {}
    for name in ("qwen3_1p7b_32k_g1", "qwen3_8b_ragged"):
        log(f"prefill: {name}")
        w, ms, F, Fc, ms_med = bench_prefill(bf, torch, W, steps, warmup, name=name)
        tf = F / (ms * 1e-3) / 1e12
        out[name] = {"seqlens": list(w.seqlens), "ms_per_call": round(ms, 4),
                     "ms_median": round(ms_med, 4), "flops_per_call": F,
                     "tflops": round(tf, 3), "causal_tflops": round(Fc / (ms * 1e-3) / 1e12, 3),
                     "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
        log(f"prefill {name}: {ms:.3f} ms/call, {tf:.1f} TFLOP/s counted")
        torch.cuda.empty_cache()
    return out


def bench_rope_apply(bf, torch, W, steps, warmup):
    """rope_apply in place on the 128K workload's query tensor [131072, 32, 128] bf16:
    every element read and written once, against the HBM peak."""
    w = W.get("qwen3_4b_128k")
    x = torch.randn((w.total_tokens, w.Hq, w.D), device="cuda").to(torch.bfloat16)
    for _ in range(warmup):
        bf.rope_apply(x, w.theta)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with quiet_host():
        bf.rope_apply(x, w.theta)  # primes the queue (see queue_primed)
        e0.record(stream)
        for _ in range(steps):
            bf.rope_apply(x, w.theta)
        e1.record(stream)
        torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / steps * 1e3
    nbytes = 2.0 * x.numel() * x.element_size()
    gbs = nbytes / (us * 1e-6) / 1e9
    del x
    torch.cuda.empty_cache()
    return {"tensor": [w.total_tokens, w.Hq, w.D], "dtype": "bf16", "us_per_call": round(us, 2),
            "bytes_per_call": nbytes, "GBps": round(gbs, 1),
            "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}


def bench_decode(bf, torch, W, passes, warmup, w0=None):
    """w0 overrides the window (w0 > pos: vanilla mode, every key local)."""
    w = W.get("qwen3_8b_decode_128k")
    if w0 is not None:
        import dataclasses
        w = dataclasses.replace(w, w0=w0)
    q, k, v = W.raw_inputs_torch(w, "cuda")
    bf.rope_apply(k, w.theta)
    positions = w.decode_positions()
    pos_t = torch.as_tensor(positions.astype(np.int32), device="cuda")
    bf.rope_apply(q, w.theta, pos=pos_t)  # query of step t at its own position
    ws = bf.Workspace.for_op(bf.OP_DECODE, w.cache_len, w.Hq, w.Hkv, w.D)
    o = torch.empty((w.Hq, w.D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.Hq,), dtype=torch.float32, device="cuda")

    def one_pass():
        for t, pos in enumerate(positions):
            bf.bifocal_decode(q[t], k, v, int(pos), w.w0, w.w_pretrained, w.theta, out=o,
                              lse=lse, workspace=ws)
    for _ in range(warmup):
        one_pass()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with quiet_host():
        bf.bifocal_decode(q[-1], k, v, int(positions[-1]), w.w0, w.w_pretrained, w.theta,
                          out=o, lse=lse, workspace=ws)  # primes the queue (see queue_primed)
        e0.record(stream)
        for _ in range(passes):
            one_pass()
        e1.record(stream)
        torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / (passes * len(positions))
    kv_bytes = float(np.mean([2 * (p + 1) * w.Hkv * w.D * 2 for p in positions]))
    return w, ms_step, kv_bytes


def bench_decode_batch(bf, torch, W, passes, warmup, B=8, S=16384):
    """Batched decode: B sequences of the decode layer's shape, each at position S - 1 of
    its own S-row cache (the same K + V bytes per step as one 128K sequence)."""
    w = W.get("qwen3_8b_decode_128k")
    g = torch.Generator(device="cuda").manual_seed(w.seed + 7)
    k = torch.randn((B, S, w.Hkv, w.D), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((B, S, w.Hkv, w.D), generator=g, device="cuda").to(torch.bfloat16)
    q = torch.randn((B, w.Hq, w.D), generator=g, device="cuda").to(torch.bfloat16)
    for b in range(B):
        bf.rope_apply(k[b], w.theta)
    # each query at its sequence's position S - 1
    bf.rope_apply(q, w.theta, pos=torch.full((B,), S - 1, dtype=torch.int32, device="cuda"))
    positions = [S - 1] * B
    ws = bf.Workspace.for_op(bf.OP_DECODE, S, w.Hq, w.Hkv, w.D, num_seqs=B)
    o = torch.empty_like(q)
    lse = torch.empty((B, w.Hq), dtype=torch.float32, device="cuda")
    steps = 64

    def one_pass():
        for _ in range(steps):
            bf.bifocal_decode_batch(q, k, v, positions, w.w0, w.w_pretrained, w.theta, out=o,
                                    lse=lse, workspace=ws)
    for _ in range(warmup):
        one_pass()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with quiet_host():
        bf.bifocal_decode_batch(q, k, v, positions, w.w0, w.w_pretrained, w.theta, out=o,
                                lse=lse, workspace=ws)  # primes the queue (see queue_primed)
        e0.record(stream)
        for _ in range(passes):
            one_pass()
        e1.record(stream)
        torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / (passes * steps) * 1e3
    kv = 2.0 * B * S * w.Hkv * w.D * 2
    return {"batch": B, "cache_rows_each": S, "us_per_step": round(us, 2),
            "kv_GBps": round(kv / (us * 1e-6) / 1e9, 1),
            "frac_of_hbm_peak": round(kv / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}


def cpu_baseline(W, F, n_uniform=200):
    """The oracle as it stands, on sampled query rows of the 128K workload (all 32
    heads), extrapolated to the whole prefill by the number of causal pairs."""
    from oracle.bifocal_ref import bifocal_rows, rope_rotate
    w = W.get("qwen3_4b_128k")
    L = w.total_tokens
    q, k, v = W.raw_prefill_inputs(w)
    rows = W.sample_rows(L, w.w0, n_uniform, seed=w.seed, tile=64)
    pos = np.arange(L)
    Qs = rope_rotate(q[rows], rows, w.theta).astype(np.float32)
    Ks = np.empty_like(k)
    for c0 in range(0, L, 16384):
        Ks[c0:c0 + 16384] = rope_rotate(k[c0:c0 + 16384], pos[c0:c0 + 16384], w.theta)
    Qs, Ks, V = W.round_to_bf16(Qs), W.round_to_bf16(Ks), W.round_to_bf16(v)
    del q, k, v
    threads = os.cpu_count()
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        if info:
            threads = max(int(i.get("num_threads", 1)) for i in info)
    except Exception:
        pass
    t0 = time.perf_counter()
    bifocal_rows(Qs, Ks, V, rows, w.w0, w.w_pretrained, w.theta, q_given_rows=True)
    t = time.perf_counter() - t0
    pairs_sampled = float(np.sum(rows + 1))
    pairs_total = L * (L + 1) / 2.0
    t_full = t * pairs_total / pairs_sampled
    out = {"value": F / t_full / 1e12, "unit": "TFLOP/s", "cores": int(threads),
           "kind": "oracle",
           "sample": f"{len(rows)} query rows x {w.Hq} heads of qwen3_4b_128k "
                     f"({t:.1f} s), extrapolated by causal pair count to all "
                     f"{L} rows (t_full = {t_full:.0f} s)",
           "host": host_info()}
    out.update(cpu_other_configs(W))
    return out


def host_info():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "affinity_cores": affinity}


def _oracle_sampled(W, name, n_uniform):
    """The oracle on sampled rows of each sequence of a prefill workload, for the first
    quarter of the query heads, extrapolated per sequence by its causal pair count and
    by the head count."""
    from oracle.bifocal_ref import bifocal_rows, rope_rotate
    w = W.get(name)
    q, k, v = W.raw_prefill_inputs(w)
    t_sample = t_full = 0.0
    nrows = 0
    heads = list(range(max(1, w.Hq // 4)))
    for b, L in enumerate(w.seqlens):
        s0 = int(w.cu_seqlens[b])
        rows = W.sample_rows(L, w.w0, n_uniform, seed=w.seed + b, tile=64)
        pos = np.arange(L)
        Qs = W.round_to_bf16(rope_rotate(q[s0 + rows][:, :len(heads)], rows, w.theta)
                             .astype(np.float32))
        nkv = (heads[-1] // (w.Hq // w.Hkv)) + 1  # KV heads the timed query heads read
        Ks = np.empty((L, nkv, w.D), dtype=np.float32)
        for c0 in range(0, L, 16384):
            c1 = min(L, c0 + 16384)
            Ks[c0:c1] = rope_rotate(k[s0 + c0:s0 + c1, :nkv], pos[c0:c1], w.theta)
        Ks, V = W.round_to_bf16(Ks), W.round_to_bf16(v[s0:s0 + L, :nkv])
        t0 = time.perf_counter()
        bifocal_rows(Qs, Ks, V, rows, w.w0, w.w_pretrained, w.theta, q_given_rows=True,
                     heads=heads)
        t = time.perf_counter() - t0
        t_sample += t
        nrows += len(rows)
        t_full += t * (L * (L + 1) / 2.0) / float(np.sum(rows + 1)) * (w.Hq / len(heads))
    return {"sampled_rows": nrows, "heads": f"{len(heads)} of {w.Hq}",
            "t_sample_s": round(t_sample, 2), "t_full_s_extrapolated": round(t_full, 1)}


def cpu_other_configs(W):
    """The oracle on the small prefill workload (whole, wall clock), on sampled rows of
    the 32K (G = 1) and ragged prefill workloads (extrapolated by pair count), and on
    the first and last of the 256 steps of the 128K decode workload, extrapolated to
    all 256 (each step rotates the whole 128K cache in float64: seconds per step)."""
    from oracle.bifocal_ref import bifocal_decode_ref, bifocal_prefill_ref, rope_rotate
    res = {}
    w = W.get("tiny_f32")
    q, k, v = W.raw_prefill_inputs(w)
    pos = np.concatenate([np.arange(L) for L in w.seqlens])
    Q = rope_rotate(q, pos, w.theta).astype(np.float32)
    K = rope_rotate(k, pos, w.theta).astype(np.float32)
    t0 = time.perf_counter()
    bifocal_prefill_ref(Q, K, v.astype(np.float32), [int(c) for c in w.cu_seqlens], w.w0,
                        w.w_pretrained, w.theta)
    res["tiny_f32_full_s"] = round(time.perf_counter() - t0, 3)
    for name in ("qwen3_1p7b_32k_g1", "qwen3_8b_ragged"):
        res[name] = _oracle_sampled(W, name, n_uniform=32)
    w = W.get("qwen3_8b_decode_128k")
    q, k, v = W.raw_decode_inputs(w)
    S = k.shape[0]
    Kc = np.empty(k.shape, dtype=np.float32)
    for c0 in range(0, S, 16384):
        Kc[c0:c0 + 16384] = W.round_to_bf16(
            rope_rotate(k[c0:c0 + 16384], np.arange(c0, min(S, c0 + 16384)), w.theta))
    Vc = W.round_to_bf16(v)
    del k, v
    positions = w.decode_positions()
    idx = [0, len(positions) - 1]
    t0 = time.perf_counter()
    for i in idx:
        p = int(positions[i])
        qs = W.round_to_bf16(rope_rotate(q[i][None], [p], w.theta)[0])
        bifocal_decode_ref(qs, Kc, Vc, p, w.w0, w.w_pretrained, w.theta)
    t = time.perf_counter() - t0
    res["decode_128k"] = {"s_per_step": round(t / len(idx), 3),
                          "s_per_256_steps": round(t / len(idx) * len(positions), 1),
                          "sample": f"steps at positions {int(positions[idx[0]])} and "
                                    f"{int(positions[idx[-1]])}, x {len(positions) // len(idx)}"}
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--decode-passes", type=int, default=2,
                    help="timed passes of the 256-step decode workload")
    ap.add_argument("--decode-warmup", type=int, default=1)
    ap.add_argument("--only", choices=["all", "prefill", "decode", "copy"], default="all")
    ap.add_argument("--copy-mib", type=int, default=1024,
                    help="--only copy: bytes copied per launch, MiB")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-vanilla", action="store_true",
                    help="skip the vanilla-mode (w0 >= L) comparison runs")
    ap.add_argument("--no-three-pass", action="store_true",
                    help="skip the three-pass inclusion-exclusion comparison run")
    ap.add_argument("--no-decode-batch", action="store_true",
                    help="skip the batched decode run (8 sequences x 16K rows)")
    ap.add_argument("--no-other-prefills", action="store_true",
                    help="skip the 32K (G = 1) and ragged prefill workloads")
    ap.add_argument("--no-rope", action="store_true", help="skip the rope_apply run")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import dynamic_rope_context_amd as bf
    import workloads as W
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    bf.lib()

    result = {}
    if args.only == "copy":
        print(json.dumps(bench_copy(torch, args.copy_mib, args.steps)), flush=True)
        return
    if args.only in ("all", "prefill"):
        log("prefill: qwen3_4b_128k")
        w, ms, F, Fc, ms_med = bench_prefill(bf, torch, W, args.steps, args.warmup)
        tflops = F / (ms * 1e-3) / 1e12
        log(f"prefill: {ms:.2f} ms/call, {tflops:.1f} TFLOP/s counted, "
            f"{Fc / (ms * 1e-3) / 1e12:.1f} TFLOP/s causal-only")
        result.update({
            "metric": "bifocal prefill TFLOP/s (% bf16 MFMA peak) at 128K; decode KV GB/s",
            "value": round(tflops, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded normal q/k/v with outlier channels; no weights)",
            "config": {"workload": "qwen3_4b_128k", "batch": 1, "seq_len": w.total_tokens,
                       "Hq": w.Hq, "Hkv": w.Hkv, "head_dim": w.D, "w0": w.w0,
                       "w_pretrained": w.w_pretrained, "G": 4, "theta": w.theta},
            "flops_per_step": F, "causal_flops_per_step": Fc,
            "causal_tflops": round(Fc / (ms * 1e-3) / 1e12, 3),
            "ms_median": round(ms_med, 4),
            "roofline": {"bound": "mfma", "achieved": round(tflops, 3),
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                         "traffic": hbm_traffic("prefill")},
        })
        mc = mfma_counters("prefill")
        if mc is not None:
            # matrix-core work actually issued (straddling tiles score twice, masked and
            # padded lanes, the hi/lo correction step), from SQ_INSTS_VALU_MFMA_MOPS_*
            result["executed_mfma"] = {
                "flops_per_launch": mc["executed_flops"],
                "tflops": round(mc["executed_flops"] / (ms * 1e-3) / 1e12, 3),
                "ratio_to_counted": round(mc["executed_flops"] / F, 4),
                "mfma_busy_frac": mc["mfma_busy_frac"],
                "valu_mfma_coexec_frac": mc["coexec_frac"]}
        else:
            result["executed_mfma"] = None
    if args.only in ("all", "decode"):
        log("decode: qwen3_8b_decode_128k, 256 steps per pass")
        w, ms_step, kv_bytes = bench_decode(bf, torch, W, args.decode_passes,
                                            args.decode_warmup)
        gbs = kv_bytes / (ms_step * 1e-3) / 1e9
        log(f"decode: {ms_step * 1e3:.1f} us/step, {gbs:.0f} GB/s of K+V")
        dec = {"workload": "qwen3_8b_decode_128k", "steps_per_pass": w.decode_steps,
               "passes": args.decode_passes, "us_per_step": round(ms_step * 1e3, 2),
               "kv_bytes_per_step": kv_bytes, "kv_GBps": round(gbs, 1),
               "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                            "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                            "traffic": hbm_traffic("decode")}}
        if not args.no_decode_batch:
            log("decode batch: 8 sequences x 16K rows per call")
            dec["batch"] = bench_decode_batch(bf, torch, W, args.decode_passes,
                                              args.decode_warmup)
            log(f"decode batch: {dec['batch']['us_per_step']} us/step, "
                f"{dec['batch']['kv_GBps']} GB/s")
        if "metric" in result:
            result["decode"] = dec
        else:
            result.update({"metric": "bifocal decode KV GB/s at 128K", "value": dec["kv_GBps"],
                           "unit": "GB/s", "n_gpus": 1, "steps": args.decode_passes,
                           "warmup": 1, "ms_per_step": round(ms_step * w.decode_steps, 4),
                           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
                           "dtype": "bf16", "data": "synthetic",
                           "config": {"workload": "qwen3_8b_decode_128k"},
                           "roofline": dec["roofline"], "decode_batch": dec.get("batch")})
    if not args.no_other_prefills and args.only in ("all", "prefill"):
        result["other_prefills"] = bench_other_prefills(bf, torch, W, args.steps, args.warmup)
    if not args.no_rope and args.only in ("all", "prefill"):
        log("rope_apply: 128K query tensor")
        result["rope_apply"] = bench_rope_apply(bf, torch, W, args.steps, args.warmup)
        log(f"rope_apply: {result['rope_apply']}")
    if not args.no_three_pass and args.only in ("all", "prefill"):
        log("three-pass prefill: qwen3_4b_128k, passes A, B, C + merge")
        _, tms, _, _, _ = bench_prefill(bf, torch, W, args.steps, args.warmup, three_pass=True)
        result["three_pass"] = {"prefill_ms": round(tms, 4),
                                "time_ratio_vs_fused": round(tms / result["ms_per_step"], 4)}
        log(f"three-pass prefill: {tms:.2f} ms, {tms / result['ms_per_step']:.3f}x the fused call")
    if not args.no_vanilla and args.only in ("all", "prefill", "decode"):
        van = {"mode": "same kernels with w0 >= L: every pair local (standard RoPE), "
                       "remote branch empty"}
        if args.only in ("all", "prefill"):
            log("vanilla prefill: qwen3_4b_128k with w0 = L")
            wv, vms, _, Fc, _ = bench_prefill(bf, torch, W, args.steps, args.warmup,
                                              w0=W.get("qwen3_4b_128k").total_tokens)
            van.update({"prefill_ms": round(vms, 4),
                        "prefill_causal_tflops": round(Fc / (vms * 1e-3) / 1e12, 3),
                        "prefill_time_ratio": round(result["ms_per_step"] / vms, 4)})
            log(f"vanilla prefill: {vms:.2f} ms, bifocal/vanilla time "
                f"{van['prefill_time_ratio']:.3f}")
        if args.only in ("all", "decode"):
            log("vanilla decode: qwen3_8b_decode_128k with w0 = cache length")
            wv, vms_step, _ = bench_decode(bf, torch, W, args.decode_passes, args.decode_warmup,
                                           w0=W.get("qwen3_8b_decode_128k").cache_len)
            us_b = (result["decode"]["us_per_step"] if "decode" in result
                    else result["ms_per_step"] / W.get("qwen3_8b_decode_128k").decode_steps * 1e3)
            van.update({"decode_us_per_step": round(vms_step * 1e3, 2),
                        "decode_overhead": round(us_b / (vms_step * 1e3) - 1.0, 4)})
            log(f"vanilla decode: {vms_step * 1e3:.1f} us/step, bifocal overhead "
                f"{100 * van['decode_overhead']:.1f}%")
        result["vanilla"] = van
    if args.only in ("all", "prefill") and not args.no_cpu_baseline:
        log("cpu baseline: oracle on sampled rows")
        result["cpu_baseline"] = cpu_baseline(W, result["flops_per_step"])
        log(f"cpu baseline: {result['cpu_baseline']}")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
