#!/usr/bin/env python3
"""Throughput of the attention hot path on one MI355X.

One step runs every stage of the path once, each on its own workload:
  * prefill  : bf16 causal attention with per-row lse, B=4, H=32, N=4096, d=128
               (shaped like one 7B decoder layer);
  * paged    : kv_append through a block table + attn_decode_paged, bf16, B=64,
               H_q=32, H_kv=8, d=128, cached lengths uniform in [128, 8192];
  * contig   : kv_append + attn_decode on a contiguous cache, bf16, B=32, H_q=64,
               H_kv=8, d=128, cached lengths uniform in [1024, 32768];
  * chunk    : kv_append of 512 new tokens per sequence + attn_prefill_paged
               (chunked prefill against the paged cache), bf16, B=16, H_q=32,
               H_kv=8, d=128, cached prefixes uniform in [0, 4096];
  * fp8      : kv_append_fp8 + attn_decode_paged_fp8, the paged workload with
               the cache stored as OCP FP8 E4M3 (KV GB/s counts 1-byte values);
  * int8     : kv_append_int8 + attn_decode_paged_int8, the same with an int8
               cache and per-channel scales;
  * int4     : kv_append_int4 + attn_decode_paged_int4, the same with an int4
               cache (half a byte per value);
  * fp8 prefill: attn_prefill_fp8 on the causal prefill workload with FP8
               E4M3 Q, K, V (V widened in the call, Q K^T on FP8 MFMA);
  * f16 prefill: fp16 non-causal attention, B=1, H=8, N=1024, d=64 (a small
               case: fewer query blocks of 128 rows than CUs, so the key tiles
               of each 32-row block are split over the waves of a workgroup).
Inputs are seeded synthetic tensors already resident in HBM.  Each kernel call
is bracketed by HIP events on the stream it runs on.

Printed: ONE JSON line.  ``value`` is the prefill rate in TFLOP/s (algorithmic
FLOPs: 4*d per visible query/key pair); the decode legs report KV GB/s (bytes of
every valid cached K and V row, read once) in their own objects.
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

METRIC = "prefill attn TFLOP/s & decode KV GB/s on 1 MI355X (fraction of peak)"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense FP8 MFMA
# FP8 prefill: Q K^T (half the FLOPs) on FP8 MFMA, P V (the other half) on bf16
# MFMA, so its peak is the rate at which both halves would run at their peaks
PEAK_FP8_PREFILL_TFLOPS = 1.0 / (0.5 / PEAK_FP8_TFLOPS + 0.5 / PEAK_BF16_TFLOPS)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "kv_cache_flashattention_attn_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if the kernel is unchanged."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    data = json.load(open(path))
    rec = data.get(kernel)
    if not rec or rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def to_dev(x, dtype, torch):
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()
    t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16)


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return 1


def host_info() -> dict:
    """The host the oracle ran on: CPU model, cores this process may run on
    (sched_getaffinity), and the BLAS threads the oracle's matrix products used
    (its elementwise work is single-threaded)."""
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
        affinity = os.cpu_count() or 1
    return {"cpu_model": model, "affinity_cores": affinity, "blas_threads": blas_threads()}


def block_pool_leg() -> dict:
    """Host side of the paged cache: the serving simulation on the chat workload
    (contiguous max_len reservations vs 16-token blocks from the native pool)
    and the native pool's cost per sequence-step of reserve_batch."""
    import synth
    from kv_cache_flashattention_attn_amd import serving_sim
    from kv_cache_flashattention_attn_amd.block_pool import BlockPool

    c = synth.CHAT_SIM
    prompts, outputs = synth.chat_requests(c)
    t0 = time.perf_counter()
    sims = {s: serving_sim.simulate(prompts, outputs, c.memory_tokens, c.max_len, s)
            for s in ("contiguous", "paged")}
    sim_s = time.perf_counter() - t0
    B, steps = 256, 2048
    mb = steps // 16 + 1
    pool = BlockPool(B * mb)
    table = np.full((B, mb), -1, np.int32)
    lens = np.zeros(B, np.int32)
    t0 = time.perf_counter()
    for _ in range(steps):
        pool.reserve_batch(table, lens, lens + 1)
        lens += 1
    dt = time.perf_counter() - t0
    keep = ("utilization_held", "utilization_budget", "mean_running", "peak_running", "steps", "preemptions")
    out = {"workload": c.name, "sim_seconds": round(sim_s, 2),
           "reserve_ns_per_sequence_step": round(dt / (B * steps) * 1e9, 1),
           "reserve_batch": f"{steps} steps x {B} sequences, one token each"}
    for s, r in sims.items():
        out[s] = {k: (round(r[k], 4) if isinstance(r[k], float) else r[k]) for k in keep}
    out["concurrency_gain"] = round(sims["paged"]["mean_running"] / sims["contiguous"]["mean_running"], 3)
    return out


def sample_clock(run, seconds: float, torch):
    """Run ``run()`` back to back for ``seconds`` while a thread reads the GPU's
    current graphics clock and socket power (amdsmi GPU metrics, every 10 ms).
    Returns the medians over the second half of the samples (the clock settles
    after the first few hundred ms), or None when amdsmi is unavailable."""
    try:
        import threading
        import amdsmi
        amdsmi.amdsmi_init()
        handle = amdsmi.amdsmi_get_processor_handles()[0]
        amdsmi.amdsmi_get_gpu_metrics_info(handle)
    except Exception as e:  # metrics are optional context, never a reason to fail
        log(f"GPU clock not recorded: {e!r}")
        return None
    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            try:
                m = amdsmi.amdsmi_get_gpu_metrics_info(handle)
                clk, pw = m.get("current_gfxclk"), m.get("current_socket_power")
                if isinstance(clk, (int, float)) and isinstance(pw, (int, float)):
                    samples.append((clk, pw))
            except Exception:
                pass
            time.sleep(0.01)

    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            run()
        torch.cuda.synchronize()
    stop.set()
    th.join()
    tail = samples[len(samples) // 2:]
    if not tail:
        return None
    return {"gfxclk_mhz": float(np.median([c for c, _ in tail])),
            "socket_power_w": float(np.median([p for _, p in tail])), "samples": len(tail)}


def cpu_baseline(seconds: float, prefill_case, prefill_raw, paged_case, paged_inp):
    """The fp64 oracle as it stands, on a bounded sample of the same workloads."""
    import oracle
    out = {}
    # prefill: whole (b, h) heads of the causal workload, one at a time
    t0 = time.perf_counter()
    flops = 0.0
    heads = 0
    c = prefill_case
    while time.perf_counter() - t0 < seconds / 2 and heads < c.B * c.H_q:
        b, h = divmod(heads, c.H_q)
        Q = oracle.decode_bits(prefill_raw["q"][b:b + 1, h:h + 1], c.dtype)
        K = oracle.decode_bits(prefill_raw["k"][b:b + 1, h:h + 1], c.dtype)
        V = oracle.decode_bits(prefill_raw["v"][b:b + 1, h:h + 1], c.dtype)
        oracle.one_shot(Q, K, V, c.sm_scale, causal=True)
        flops += 4.0 * c.d * c.N * (c.N + 1) / 2
        heads += 1
    dt = time.perf_counter() - t0
    host = host_info()
    out["prefill"] = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": host["blas_threads"], "kind": "oracle",
                      "sample": f"{heads} of {c.B * c.H_q} (batch, head) pairs of the causal prefill, "
                                f"one_shot in fp64, {dt:.1f} s", "host": host}
    # decode: whole sequences of the paged workload (append + gather + attend)
    t0 = time.perf_counter()
    nbytes = 0
    seqs = 0
    pc = paged_case
    pcache = oracle.PagedCache(paged_inp["k_pool"], paged_inp["v_pool"], paged_inp["block_table"])
    copy_s = time.perf_counter() - t0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds / 2 and seqs < pc.B:
        b = seqs
        heads = [(b, h) for h in range(pc.H_q)]
        oracle.decode_step(pcache, paged_inp["q"], paged_inp["k_new"], paged_inp["v_new"], paged_inp["lens"],
                           pc.sm_scale, pc.dtype, heads=heads)
        nbytes += (int(paged_inp["lens"][b]) + pc.n_new) * pc.H_kv * pc.d * 2 * 2
        seqs += 1
    dt = time.perf_counter() - t0
    out["decode"] = {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": host["blas_threads"], "kind": "oracle",
                     "sample": f"{seqs} of {pc.B} sequences of the paged decode (append, gather, attend "
                               f"all {pc.H_q} query heads) in fp64, {dt:.1f} s (+{copy_s:.1f} s pool copy)",
                     "host": host}
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=20.0, help="oracle time budget (0 = skip)")
    ap.add_argument("--clock-seconds", type=float, default=1.5,
                    help="per leg: run prefill, then paged decode, alone this long while sampling "
                         "the GPU clock (0 = skip)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB read + 1 GiB write kernel (scale for HBM byte counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        log("bench.py measures one GPU only: this build has no multi-GPU path "
            "(prefill and decode would shard by head / sequence with no exchange).")
        return 2

    import torch
    import synth
    import kv_cache_flashattention_attn_amd as K
    K.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev_props = torch.cuda.get_device_properties(0)

    # ---------------- inputs ----------------
    t_gen = time.perf_counter()
    pcase = synth.PREFILL_BF16_CAUSAL
    praw = synth.prefill_inputs(pcase)
    q, k, v = (to_dev(praw[n], pcase.dtype, torch) for n in ("q", "k", "v"))
    o = torch.empty_like(q)
    lse = torch.empty((pcase.B, pcase.H_q, pcase.N), dtype=torch.float32, device="cuda")
    # the fp16 non-causal prefill 1x8x1024x64 (a small case: 64 query blocks of 128 rows)
    scase = synth.PREFILL_F16
    sraw = synth.prefill_inputs(scase)
    q2, k2, v2 = (to_dev(sraw[n], scase.dtype, torch) for n in ("q", "k", "v"))
    o2 = torch.empty_like(q2)
    del sraw
    log(f"prefill inputs ready ({time.perf_counter() - t_gen:.1f} s)")
    # the same workload with FP8 E4M3 inputs
    f8 = synth.fp8_prefill_inputs(pcase)
    q8, k8, v8 = (torch.from_numpy(f8[n]).cuda() for n in ("q", "k", "v"))
    del f8
    o8 = torch.empty(q8.shape, dtype=torch.bfloat16, device="cuda")
    lse8 = torch.empty_like(lse)

    gcase = synth.DECODE_PAGED
    ginp = synth.decode_inputs(gcase)
    g = {n: to_dev(ginp[n], gcase.dtype, torch) for n in ("q", "k_new", "v_new", "k_pool", "v_pool")}
    g_table = torch.from_numpy(ginp["block_table"]).cuda()
    g_lens = torch.from_numpy(ginp["lens"]).cuda()
    g_seq = g_lens + gcase.n_new
    g_ws = torch.empty(K.attn_decode_workspace_bytes(gcase.B, gcase.H_q, gcase.max_blocks * 16, gcase.d),
                       dtype=torch.uint8, device="cuda")
    g_out = torch.empty_like(g["q"])
    g_bytes = synth.kv_bytes_read(ginp["lens"] + gcase.n_new, gcase.H_kv, gcase.d, gcase.dtype)
    log(f"paged decode inputs ready ({time.perf_counter() - t_gen:.1f} s)")

    ccase = synth.DECODE_CONTIG
    cinp = synth.decode_inputs(ccase)
    cdev = {n: to_dev(cinp[n], ccase.dtype, torch) for n in ("q", "k_new", "v_new", "k_cache", "v_cache")}
    c_lens = torch.from_numpy(cinp["lens"]).cuda()
    c_seq = c_lens + ccase.n_new
    c_ws = torch.empty(K.attn_decode_workspace_bytes(ccase.B, ccase.H_q, ccase.max_len, ccase.d),
                       dtype=torch.uint8, device="cuda")
    c_out = torch.empty_like(cdev["q"])
    c_bytes = synth.kv_bytes_read(cinp["lens"] + ccase.n_new, ccase.H_kv, ccase.d, ccase.dtype)
    c_lens_np = cinp["lens"]
    del cinp
    log(f"contiguous decode inputs ready ({time.perf_counter() - t_gen:.1f} s)")

    # chunked prefill against a paged cache (beyond the five workloads)
    kcase = synth.CHUNK_PAGED
    kinp = synth.chunk_inputs(kcase)
    kd = {n: to_dev(kinp[n], kcase.dtype, torch) for n in ("q", "k_new", "v_new", "k_pool", "v_pool")}
    k_table = torch.from_numpy(kinp["block_table"]).cuda()
    k_lens = torch.from_numpy(kinp["lens"]).cuda()
    k_out = torch.empty_like(kd["q"])
    k_lse = torch.empty(kd["q"].shape[:3], dtype=torch.float32, device="cuda")
    k_flops = synth.chunk_flops(kinp["lens"], kcase.n_new, kcase.H_q, kcase.d, causal=True)
    del kinp
    log(f"chunk prefill inputs ready ({time.perf_counter() - t_gen:.1f} s)")

    # the paged decode workload over an 8-bit (FP8 E4M3) cache: same q, new rows,
    # lengths, block table and workspace as the bf16 paged leg
    fcase = gcase
    finp = synth.fp8_decode_inputs(fcase, base=ginp)
    f_kp = torch.from_numpy(finp["k_pool"]).cuda()
    f_vp = torch.from_numpy(finp["v_pool"]).cuda()
    f_out = torch.empty_like(g["q"])
    f_bytes = int(np.sum((finp["lens"] + fcase.n_new).astype(np.int64))) * fcase.H_kv * fcase.d * 2  # 1 byte each
    del finp
    # ... and over an int8 cache with per-channel scales
    iinp = synth.int8_decode_inputs(gcase, base=ginp)
    i_kp = torch.from_numpy(iinp["k_pool"]).cuda()
    i_vp = torch.from_numpy(iinp["v_pool"]).cuda()
    i_ks = torch.from_numpy(iinp["k_scales"]).cuda()
    i_vs = torch.from_numpy(iinp["v_scales"]).cuda()
    i_out = torch.empty_like(g["q"])
    del iinp
    # ... and over an int4 cache (two codes per byte)
    i4inp = synth.int4_decode_inputs(gcase, base=ginp)
    i4_kp = torch.from_numpy(i4inp["k_pool"]).cuda()
    i4_vp = torch.from_numpy(i4inp["v_pool"]).cuda()
    i4_ks = torch.from_numpy(i4inp["k_scales"]).cuda()
    i4_vs = torch.from_numpy(i4inp["v_scales"]).cuda()
    i4_out = torch.empty_like(g["q"])
    del i4inp
    log(f"fp8 decode inputs ready ({time.perf_counter() - t_gen:.1f} s)")
    torch.cuda.synchronize()

    legs = ["prefill", "paged_append", "paged_decode", "contig_append", "contig_decode", "chunk_append",
            "chunk_prefill", "fp8_append", "fp8_decode", "int8_append", "int8_decode", "fp8_prefill",
            "int4_append", "int4_decode", "f16_prefill"]

    def step(ev=None):
        def rec(i):
            if ev is not None:
                ev[i].record()
        rec(0)
        K.attn_prefill(q, k, v, causal=True, scale=pcase.sm_scale, return_lse=True, out=o, lse=lse)
        rec(1)
        K.kv_append(g["k_pool"], g["v_pool"], g["k_new"], g["v_new"], g_lens, g_table)
        rec(2)
        K.attn_decode_paged(g["q"], g["k_pool"], g["v_pool"], g_table, g_seq, scale=gcase.sm_scale,
                            workspace=g_ws, out=g_out)
        rec(3)
        K.kv_append(cdev["k_cache"], cdev["v_cache"], cdev["k_new"], cdev["v_new"], c_lens)
        rec(4)
        K.attn_decode(cdev["q"], cdev["k_cache"], cdev["v_cache"], c_seq, scale=ccase.sm_scale,
                      workspace=c_ws, out=c_out)
        rec(5)
        K.kv_append(kd["k_pool"], kd["v_pool"], kd["k_new"], kd["v_new"], k_lens, k_table)
        rec(6)
        K.attn_prefill_paged(kd["q"], kd["k_pool"], kd["v_pool"], k_table, k_lens, causal=True,
                             scale=kcase.sm_scale, return_lse=True, out=k_out, lse=k_lse)
        rec(7)
        K.kv_append_fp8(f_kp, f_vp, g["k_new"], g["v_new"], g_lens, g_table, synth.FP8_K_SCALE,
                        synth.FP8_V_SCALE)
        rec(8)
        K.attn_decode_paged_fp8(g["q"], f_kp, f_vp, g_table, g_seq, k_scale=synth.FP8_K_SCALE,
                                v_scale=synth.FP8_V_SCALE, scale=fcase.sm_scale, workspace=g_ws, out=f_out)
        rec(9)
        K.kv_append_int8(i_kp, i_vp, g["k_new"], g["v_new"], g_lens, g_table, i_ks, i_vs)
        rec(10)
        K.attn_decode_paged_int8(g["q"], i_kp, i_vp, g_table, g_seq, i_ks, i_vs, scale=fcase.sm_scale,
                                 workspace=g_ws, out=i_out)
        rec(11)
        K.attn_prefill_fp8(q8, k8, v8, causal=True, scale=pcase.sm_scale, q_scale=synth.FP8_Q_SCALE,
                           k_scale=synth.FP8_K_SCALE, v_scale=synth.FP8_V_SCALE,
                           return_lse=True, out=o8, lse=lse8)
        rec(12)
        K.kv_append_int4(i4_kp, i4_vp, g["k_new"], g["v_new"], g_lens, g_table, i4_ks, i4_vs)
        rec(13)
        K.attn_decode_paged_int4(g["q"], i4_kp, i4_vp, g_table, g_seq, i4_ks, i4_vs, scale=fcase.sm_scale,
                                 workspace=g_ws, out=i4_out)
        rec(14)
        K.attn_prefill(q2, k2, v2, causal=False, scale=scase.sm_scale, out=o2)
        rec(15)

    if args.calibrate_copy:
        # torch's elementwise multiply: reads 2^30 bytes, writes 2^30 bytes per launch
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(legs) + 1)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for s in range(args.steps):
        step(events[s])
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    per = {name: [] for name in legs}
    for ev in events:
        for i, name in enumerate(legs):
            per[name].append(ev[i].elapsed_time(ev[i + 1]))
    ms = {name: float(np.mean(x)) for name, x in per.items()}
    med = {name: float(np.median(x)) for name, x in per.items()}
    p10 = {name: float(np.percentile(x, 10)) for name, x in per.items()}
    p90 = {name: float(np.percentile(x, 90)) for name, x in per.items()}

    def spread(name):
        return {"ms_p10": round(p10[name], 4), "ms_p90": round(p90[name], 4)}
    flags = K.attn_device_error_flags()
    if flags:
        log(f"WARNING: device error flags {flags}")

    pf_flops = pcase.flops()
    pf_tflops = pf_flops / (ms["prefill"] * 1e-3) / 1e12
    g_gbs = g_bytes / (ms["paged_decode"] * 1e-3) / 1e9
    c_gbs = c_bytes / (ms["contig_decode"] * 1e-3) / 1e9
    k_tflops = k_flops / (ms["chunk_prefill"] * 1e-3) / 1e12
    f_gbs = f_bytes / (ms["fp8_decode"] * 1e-3) / 1e9
    i_gbs = f_bytes / (ms["int8_decode"] * 1e-3) / 1e9  # same 1-byte cache
    p8_tflops = pf_flops / (ms["fp8_prefill"] * 1e-3) / 1e12
    i4_bytes = f_bytes // 2  # half a byte per value
    i4_gbs = i4_bytes / (ms["int4_decode"] * 1e-3) / 1e9
    s_tflops = scase.flops() / (ms["f16_prefill"] * 1e-3) / 1e12

    def roof(bound, achieved, peak, unit, kernel, per_unit):
        return {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": measured_traffic(kernel), "kernel": kernel,
                "per_launch": per_unit}

    result = {
        "metric": METRIC,
        "value": round(pf_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1), SFC64)",
        "config": {"workload": pcase.name, "B": pcase.B, "H_q": pcase.H_q, "H_kv": pcase.H_kv, "N": pcase.N,
                   "d": pcase.d, "causal": True, "lse": True, "parallelism": "none (1 GPU)"},
        "roofline": roof("mfma", pf_tflops, PEAK_BF16_TFLOPS, "TFLOP/s", "prefill_mfma_kernel<BF16,128,causal>",
                         {"flops": pf_flops, "ms_mean": round(ms["prefill"], 4), "ms_median": round(med["prefill"], 4),
                          **spread("prefill")}),
        "decode_paged": {
            "value": round(g_gbs, 1), "unit": "GB/s", "workload": gcase.name,
            "kv_bytes": g_bytes, "ms_mean": round(ms["paged_decode"], 4), "ms_median": round(med["paged_decode"], 4),
            **spread("paged_decode"),
            "append_ms": round(ms["paged_append"], 4),
            "roofline": roof("hbm", g_gbs, PEAK_HBM_GBS, "GB/s", "decode_mfma_kernel<BF16,128,paged>+merge",
                             {"bytes": g_bytes}),
        },
        "decode_contig": {
            "value": round(c_gbs, 1), "unit": "GB/s", "workload": ccase.name,
            "kv_bytes": c_bytes, "ms_mean": round(ms["contig_decode"], 4), "ms_median": round(med["contig_decode"], 4),
            **spread("contig_decode"),
            "append_ms": round(ms["contig_append"], 4),
            "roofline": roof("hbm", c_gbs, PEAK_HBM_GBS, "GB/s", "decode_mfma_kernel<BF16,128,contig>+merge",
                             {"bytes": c_bytes}),
        },
        "chunk_prefill_paged": {
            "value": round(k_tflops, 2), "unit": "TFLOP/s", "workload": kcase.name,
            "flops": k_flops, "ms_mean": round(ms["chunk_prefill"], 4), "ms_median": round(med["chunk_prefill"], 4),
            **spread("chunk_prefill"),
            "append_ms": round(ms["chunk_append"], 4),
            "roofline": roof("mfma", k_tflops, PEAK_BF16_TFLOPS, "TFLOP/s",
                             "prefill_mfma_kernel<BF16,128,causal,paged>", {"flops": k_flops}),
        },
        "decode_paged_fp8": {
            "value": round(f_gbs, 1), "unit": "GB/s", "workload": fcase.name + " (E4M3 cache)",
            "kv_bytes": f_bytes, "ms_mean": round(ms["fp8_decode"], 4), "ms_median": round(med["fp8_decode"], 4),
            **spread("fp8_decode"),
            "append_ms": round(ms["fp8_append"], 4),
            "speedup_vs_bf16_cache": round(ms["paged_decode"] / ms["fp8_decode"], 3),
            "roofline": roof("hbm", f_gbs, PEAK_HBM_GBS, "GB/s", "decode_mfma_kernel<BF16,128,paged,fp8>+merge",
                             {"bytes": f_bytes}),
        },
        "decode_paged_int8": {
            "value": round(i_gbs, 1), "unit": "GB/s", "workload": fcase.name + " (int8 cache, per-channel scales)",
            "kv_bytes": f_bytes, "ms_mean": round(ms["int8_decode"], 4), "ms_median": round(med["int8_decode"], 4),
            **spread("int8_decode"),
            "append_ms": round(ms["int8_append"], 4),
            "speedup_vs_bf16_cache": round(ms["paged_decode"] / ms["int8_decode"], 3),
            "roofline": roof("hbm", i_gbs, PEAK_HBM_GBS, "GB/s",
                             "decode_mfma_kernel<BF16,128,paged,int8>+merge", {"bytes": f_bytes}),
        },
        "decode_paged_int4": {
            "value": round(i4_gbs, 1), "unit": "GB/s", "workload": fcase.name + " (int4 cache, per-channel scales)",
            "kv_bytes": i4_bytes, "ms_mean": round(ms["int4_decode"], 4), "ms_median": round(med["int4_decode"], 4),
            **spread("int4_decode"),
            "append_ms": round(ms["int4_append"], 4),
            "speedup_vs_bf16_cache": round(ms["paged_decode"] / ms["int4_decode"], 3),
            "roofline": roof("hbm", i4_gbs, PEAK_HBM_GBS, "GB/s",
                             "decode_mfma_kernel<BF16,128,paged,int4>+merge", {"bytes": i4_bytes}),
        },
        "prefill_fp8": {
            "value": round(p8_tflops, 2), "unit": "TFLOP/s", "workload": pcase.name + " (FP8 E4M3 Q, K, V)",
            "flops": pf_flops, "ms_mean": round(ms["fp8_prefill"], 4), "ms_median": round(med["fp8_prefill"], 4),
            **spread("fp8_prefill"),
            "speedup_vs_bf16": round(ms["prefill"] / ms["fp8_prefill"], 3),
            "roofline": roof("mfma", p8_tflops, round(PEAK_FP8_PREFILL_TFLOPS, 1), "TFLOP/s",
                             "prefill_mfma_kernel<BF16,128,causal,fp8>", {"flops": pf_flops}),
        },
        "prefill_f16_small": {
            "value": round(s_tflops, 2), "unit": "TFLOP/s", "workload": scase.name + " (non-causal, no lse)",
            "flops": scase.flops(), "ms_mean": round(ms["f16_prefill"], 4), "ms_median": round(med["f16_prefill"], 4),
            **spread("f16_prefill"),
            "note": "256 workgroups of 32 query rows, each splitting the key tiles over its 4 waves",
            "roofline": roof("mfma", s_tflops, PEAK_BF16_TFLOPS, "TFLOP/s", "prefill_small_kernel<F16,64,noncausal>",
                             {"flops": scase.flops()}),
        },
        "device": {"name": dev_props.name, "cus": dev_props.multi_processor_count},
        "device_error_flags": flags,
        "kernel_source_hash": kernel_source_hash(),
    }
    # clock and power while one leg runs alone (after the timed steps; context
    # for the fractions of peak, which assume the 2.4 GHz peak clock)
    if args.clock_seconds > 0:
        clk_pf = sample_clock(lambda: K.attn_prefill(q, k, v, causal=True, scale=pcase.sm_scale, return_lse=True,
                                                     out=o, lse=lse), args.clock_seconds, torch)
        clk_dec = sample_clock(lambda: K.attn_decode_paged(g["q"], g["k_pool"], g["v_pool"], g_table, g_seq,
                                                           scale=gcase.sm_scale, workspace=g_ws, out=g_out),
                               args.clock_seconds, torch)
        result["clock"] = {"prefill": clk_pf, "decode_paged": clk_dec, "peak_gfxclk_mhz": 2400,
                           "source": "amdsmi current_gfxclk / current_socket_power, sampled every 10 ms while "
                                     "the leg runs alone after the timed steps; median of the second half"}
    result["block_pool"] = block_pool_leg()
    if args.cpu_seconds > 0:
        log("timing the CPU oracle on a bounded sample ...")
        cb = cpu_baseline(args.cpu_seconds, pcase, praw, gcase, ginp)
        result["cpu_baseline"] = cb["prefill"]
        result["decode_paged"]["cpu_baseline"] = cb["decode"]
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
