"""Benchmark: ring-attention forward on one MI355X, the 128k GQA causal zigzag workload.

One step is the whole hot path on one batch of synthetic input already resident
in HBM: zigzag permute of q, k, v into rank-major order, the simulated 8-rank
ring (every rank's query block against all 8 KV blocks, with the double-buffered
block copies), and the inverse permute of out and lse. ``value`` is useful
TFLOP/s: 4*D flops per (query, key) pair the causal mask allows, over the
wall-clock time of the K timed steps.

The JSON line also carries the attention kernel's roofline (its summed launch
time from HIP events recorded on its own stream during the timed steps, against
the bf16 dense MFMA peak) and the fp64 CPU oracle timed on a bounded sample of
the same workload (a baseline, not the target).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
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

METRIC = "ring-attn fwd useful TFLOP/s & % bf16 MFMA peak, S=131072 GQA causal zigzag"
# MI355X published figures: 256 CUs x 2.4 GHz x 4096 dense bf16 flops/CU/clk, HBM3E 8 TB/s.
# The bench re-reads the CU count and clock on the device (peak_derivation) and
# confirms the flops/CU/clk with the matrix-core probe.
BF16_FLOPS_PER_CU_CLK = 4096
PEAK_BF16_TFLOPS = 256 * 2.4e9 * BF16_FLOPS_PER_CU_CLK / 1e12
PEAK_FP32_MFMA_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


# Hardware byte counts of the attention kernel (rocprofv3 FETCH_SIZE / WRITE_SIZE
# passes, scaled by a plain-copy calibration) live in this summary; they are
# reported only while the kernel sources still hash to what was profiled.
PMC_SUMMARY = os.path.join(ROOT, "profiles", "attn_fwd_bf16_gqa128k_pmc.txt")
KERNEL_SOURCES = ("attn_fwd.hip", "attn_fwd_w64_phases.h", "attn_common.h", "attn_fwd_args.h")
# The same for the backward kernels, per block pair (one dk/dv + one dq launch).
BWD_PMC_SUMMARY = os.path.join(ROOT, "profiles", "attn_bwd_bf16_gqa128k_pmc.txt")
BWD_KERNEL_SOURCES = ("attn_bwd.hip", "attn_bwd_dkdv_loop.h", "attn_bwd_dq_w64_loop.h",
                      "attn_common.h", "attn_bwd_args.h")


def kernel_sources_sha256(sources=KERNEL_SOURCES) -> str:
    """SHA-256 of a kernel's source files and of the compiler flags its .hip
    file is built with (a flag can change the kernel as much as an edit)."""
    import hashlib
    from ring_context_parallelism_flash_amd import build as ra_build
    h = hashlib.sha256()
    for name in sources:
        with open(os.path.join(ROOT, "ring_context_parallelism_flash_amd", "csrc", name), "rb") as f:
            h.update(f.read())
        if name.endswith(".hip"):
            # include paths name the checkout's directory, which differs from
            # machine to machine; hash them relative to the repository root
            flags = [f.replace(ROOT, "<root>") for f in ra_build.FLAGS + ra_build.EXTRA.get(name, [])]
            h.update(" ".join(flags).encode())
    return h.hexdigest()


def measured_traffic(workload_name: str, summary=PMC_SUMMARY, sources=KERNEL_SOURCES):
    """HBM bytes per launch (per block pair for the backward) from a committed
    counter summary, or (None, reason) when it does not describe this
    workload or these sources."""
    try:
        kv = {}
        with open(summary) as f:
            for line in f:
                if line.startswith("@ ") and "=" in line:
                    key, val = line[2:].split("=", 1)
                    kv[key.strip()] = val.strip()
        if kv.get("workload") != workload_name:
            return None, "no counter summary for this workload"
        if kv.get("sources_sha256") != kernel_sources_sha256(sources):
            return None, "kernel sources changed since the counters were taken"
        return int(float(kv["traffic_bytes_per_launch"])), summary[len(ROOT) + 1:]
    except (OSError, KeyError, ValueError) as e:
        return None, f"counter summary unreadable: {e}"


def bwd_kernel_name(w):
    """The dk/dv and dq kernels a backward block pair of workload w launches
    (the one-wave-per-SIMD ones for D = 128; dq's needs whole 64-key tiles)."""
    block = w.S // (2 * w.N) if w.layout == "zigzag" else w.S // w.N
    if w.D != 128:
        return f"attn_bwd_dkdv<{w.D}> + attn_bwd_dq<{w.D}>"
    return "attn_bwd_dkdv_w32 + " + ("attn_bwd_dq_w64" if block % 64 == 0 else "attn_bwd_dq<128>")


def fwd_kernel_name(w, block_keys=None) -> str:
    """The forward kernel a launch on key blocks of `block_keys` keys (default:
    the zigzag half chunk S / 2N) runs: D = 128 bf16 blocks of whole 64-key
    tiles run the one-wave-per-SIMD kernel."""
    if w.dtype != "bf16":
        return f"attn_fwd_f32<{w.D}>"
    ck = w.S // (2 * w.N) if block_keys is None else block_keys
    if w.D == 128 and ck % 64 == 0:
        return "attn_fwd_bf16_w64"
    return f"attn_fwd_bf16<{w.D}>"


def useful_pairs(S: int, causal: bool) -> int:
    """Allowed (query, key) pairs of one head over the whole sequence."""
    return S * (S + 1) // 2 if causal else S * S


def useful_flops(w) -> float:
    return 4.0 * w.D * w.B * w.Hq * useful_pairs(w.S, w.causal)


def baseline_rows(w, rows_per_head: int):
    """[Hq, R] sorted rows per head: the first and last row of every chunk of
    the 2N-chunk split, and ``rows_per_head`` rows drawn per head from the
    rest with numpy.random.default_rng([seed, head])."""
    import numpy as np
    c = w.S // (2 * w.N)
    fixed = np.unique(np.concatenate([np.arange(2 * w.N) * c, np.arange(1, 2 * w.N + 1) * c - 1]))
    rest = np.setdiff1d(np.arange(w.S), fixed)
    n = min(rows_per_head, len(rest))
    return np.stack([np.sort(np.concatenate(
        [fixed, np.random.default_rng([w.seed, h]).choice(rest, n, replace=False)]))
        for h in range(w.Hq)])


def cpu_baseline(w, q, k, v, out_gpu, lse_gpu, rows_per_head: int):
    """Time the unmodified fp64 oracle on seeded rows of every head, run over
    a process pool of the host's cores (oracle.pool: groups of sorted rows,
    each against the keys its last row can see), and compare those rows with
    the GPU result."""
    import numpy as np
    from oracle import pool
    rows = baseline_rows(w, rows_per_head)
    n_workers = pool.workers()
    t0 = time.perf_counter()
    ref_out, ref_lse = pool.pooled_attention(q, k, v, causal=w.causal, rows=rows,
                                             n_workers=n_workers)
    dt = time.perf_counter() - t0
    pairs = float(np.sum(rows + 1)) if w.causal else float(rows.size) * w.S
    useful = 4.0 * w.D * w.B * pairs
    idx = [np.asarray(r) for r in rows]
    go = np.stack([out_gpu[0, h, idx[h]].double().numpy() for h in range(w.Hq)])
    gl = np.stack([lse_gpu[0, h, idx[h]].double().numpy() for h in range(w.Hq)])
    err = np.abs(go - ref_out)
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        affinity = os.cpu_count() or 1
    return {
        "value": useful / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": n_workers,
        "kind": "oracle",
        "sample": (f"{rows.shape[1]} rows per head ({rows_per_head} seeded random + every "
                   f"chunk's first and last row) x {w.Hq} heads of {w.name}, numpy fp64, "
                   f"{n_workers} single-threaded worker processes ({affinity} CPUs in the "
                   f"affinity mask); {useful / 1e12:.3f} useful TFLOP in {dt:.1f} s"),
        "parity_vs_gpu": {"rows": int(rows.size), "out_max_abs": float(err.max()),
                          "out_mean_abs": float(err.mean()),
                          "lse_max_abs": float(np.abs(gl - ref_lse).max())},
    }


def peak_derivation(dev):
    """The bf16 dense peak from the device's own figures: compute units x
    maximum shader clock x flops per CU per clock, the last confirmed by the
    library's matrix-core probe (register-fed MFMAs, two waves per SIMD)."""
    import ring_context_parallelism_flash_amd as ra
    cus, khz = ra.ra_device_info()
    probe = ra.ra_mfma_probe_bf16(iters=100000, device=dev)
    derived = cus * khz * 1e3 * BF16_FLOPS_PER_CU_CLK / 1e12
    return {
        "compute_units": cus,
        "max_clock_mhz": khz / 1e3,
        "flops_per_cu_clk": BF16_FLOPS_PER_CU_CLK,
        "derived_tflops": round(derived, 1),
        "published_tflops": round(PEAK_BF16_TFLOPS, 1),
        "probe": {"flops_per_cu_clk": round(probe["flops_per_cu_clk"], 1),
                  "clock_mhz": round(probe["clock_mhz"], 1),
                  "chip_tflops": round(probe["chip_tflops"], 1),
                  "mfma_per_wave": 4 * probe["iters"]},
    }


def copy_overlap(kernel_trace_csv: str) -> dict:
    """From a rocprofv3 kernel trace (csv): the ring's block copies (the
    runtime's copyBuffer kernels) and how much of their time passes while an
    attention kernel runs."""
    import csv
    att, cp = [], []
    with open(kernel_trace_csv) as f:
        for r in csv.DictReader(f):
            iv = (int(r["Start_Timestamp"]), int(r["End_Timestamp"]))
            name = r["Kernel_Name"]
            if "attn_fwd" in name or "attn_bwd" in name:
                att.append(iv)
            elif "copyBuffer" in name:
                cp.append(iv)
    att.sort()
    merged = []
    for a, b in att:
        if merged and a <= merged[-1][1]:
            merged[-1][1] = max(merged[-1][1], b)
        else:
            merged.append([a, b])
    import bisect
    starts = [m[0] for m in merged]
    total = covered = 0
    for a, b in cp:
        total += b - a
        i = max(0, bisect.bisect_right(starts, a) - 1)
        while i < len(merged) and merged[i][0] < b:
            covered += max(0, min(b, merged[i][1]) - max(a, merged[i][0]))
            i += 1
    return {"copies": len(cp), "copy_ms": total / 1e6, "copy_ms_under_attention": covered / 1e6,
            "overlap_frac": covered / total if total else None,
            "attention_launches": len(att)}


def aux_bandwidth(w, q, dev):
    """HBM rates of the layout permute (one q-sized permute, read + write), of
    the lse merge (one rank's fp32 running state) and of the Ulysses
    all-to-all (q-sized, both directions), timed with events."""
    import torch
    import ring_context_parallelism_flash_amd as ra
    permute = ra.ra_striped_permute if w.layout == "striped" else ra.ra_zigzag_permute
    dst = torch.empty_like(q)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    permute(q, dst, w.N)
    e0.record()
    for _ in range(5):
        permute(q, dst, w.N)
    e1.record()
    torch.cuda.synchronize()
    perm_gbs = 2 * q.numel() * q.element_size() * 5 / (e0.elapsed_time(e1) / 1e3) / 1e9
    del dst
    rows = w.B * w.Hq * (w.S // w.N)
    mo = torch.randn(rows, w.D, device=dev)
    ml = torch.randn(rows, device=dev)
    mob, mlb = torch.randn_like(mo), torch.randn_like(ml)
    ra.ra_lse_merge(mo, ml, mob, mlb)
    e0.record()
    for _ in range(5):
        ra.ra_lse_merge(mo, ml, mob, mlb)
    e1.record()
    torch.cuda.synchronize()
    merge_gbs = (3 * rows * w.D + 3 * rows) * 4 * 5 / (e0.elapsed_time(e1) / 1e3) / 1e9
    del mo, ml, mob, mlb
    res = {f"{'striped' if w.layout == 'striped' else 'zigzag'}_permute_GBs": round(perm_gbs, 1),
           "lse_merge_GBs": round(merge_gbs, 1), "hbm_peak_GBs": PEAK_HBM_GBS,
           "permute_bytes": 2 * q.numel() * q.element_size(),
           "lse_merge_bytes": (3 * rows * w.D + 3 * rows) * 4}
    # Ulysses all-to-all of q's bytes taken as the N ranks' sequence slices
    # [N, B, S/N, Hq, D], forward and back (the Ulysses step's q and out moves)
    P = w.N
    if w.Hq % P == 0 and w.S % P == 0:
        src = q.view(P, w.B, w.S // P, w.Hq, w.D)
        mid = torch.empty((P, w.B, w.Hq // P, w.S, w.D), dtype=q.dtype, device=dev)
        back = torch.empty_like(src)
        for inverse, a, b in ((False, src, mid), (True, mid, back)):
            ra.ra_ulysses_all_to_all(a, b, P, inverse=inverse)
            e0.record()
            for _ in range(5):
                ra.ra_ulysses_all_to_all(a, b, P, inverse=inverse)
            e1.record()
            torch.cuda.synchronize()
            gbs = 2 * q.numel() * q.element_size() * 5 / (e0.elapsed_time(e1) / 1e3) / 1e9
            res["ulysses_all_to_all_inverse_GBs" if inverse else "ulysses_all_to_all_GBs"] = \
                round(gbs, 1)
        if not torch.equal(back, src):
            raise RuntimeError("all-to-all forward and back did not restore q")
        del mid, back
    return res


def bench_backward(args, w, q, k, v, runner, out, lse) -> int:
    """One step = permute q, k, v, out, dout, lse into rank-major order, the ring
    backward (all N ranks x N steps, fp32 accumulation, bf16 gradients), and the
    inverse permute of dq, dk, dv. The forward runs once, untimed, for out/lse.
    Useful work: 10*D flops per allowed pair (scores recomputed + four products)."""
    import torch
    import ring_context_parallelism_flash_amd as ra
    import workloads
    dev = q.device
    runner(q, k, v, out, lse)
    dout = workloads.make_random(q.shape, w.seed + 500, q.dtype).to(dev)
    B, Hq, S, D = q.shape
    ws = torch.empty(ra.ra_ring_sim_bwd_workspace_bytes(B, Hq, w.Hkv, S, D, q.dtype, w.N),
                     dtype=torch.uint8, device=dev)

    def step():
        return ra.ring_attention_sim_backward(q, k, v, out, lse, dout, N=w.N, layout=w.layout,
                                              causal=w.causal, workspace=ws)

    print(f"bench: backward warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ra.ra_kernel_timing_enable(True)
    ra.ra_kernel_timing_read()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    k_ms, launches, k_flops = ra.ra_kernel_timing_read()
    ra.ra_kernel_timing_enable(False)
    print(f"bench: timed {args.steps} backward steps in {t1 - t0:.3f} s", file=sys.stderr, flush=True)
    flops_step = 2.5 * useful_flops(w)   # 10*D per pair against the forward's 4*D
    traffic, traffic_src = measured_traffic(w.name, BWD_PMC_SUMMARY, BWD_KERNEL_SOURCES)
    ms_step = (t1 - t0) * 1e3 / args.steps
    value = flops_step / (ms_step / 1e3) / 1e12
    achieved = k_flops / (k_ms / 1e3) / 1e12 if k_ms > 0 else 0.0
    line = {
        "metric": f"ring-attn bwd useful TFLOP/s, {w.name}",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded iid normal q/k/v/dout, k x0.5, bf16)",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D, "S": w.S,
                   "virtual_ranks": w.N, "layout": w.layout, "causal": w.causal,
                   "pass": "backward"},
        "pct_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "useful_flops_per_step": flops_step,
        "roofline": {
            "kernel": bwd_kernel_name(w),
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": round(PEAK_BF16_TFLOPS, 1),
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "traffic_unit": "HBM bytes per block pair, dk/dv + dq launch (FETCH_SIZE x2.0 + "
                            "WRITE_SIZE x1.0)",
            "traffic_source": traffic_src,
            "launches_per_step": launches // max(args.steps, 1),
            "kernel_ms_per_step": round(k_ms / max(args.steps, 1), 3),
        },
        "flops_check": {"closed_form": flops_step, "library_count": k_flops / max(args.steps, 1)},
    }
    print(json.dumps(line), flush=True)
    calibration_copy(args, dev)
    return 0


def calibration_copy(args, dev):
    """One plain device copy of a known size, a reference for byte counters."""
    import torch
    if args.copy_calibration_mib <= 0:
        return
    n = args.copy_calibration_mib << 20
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(f"bench: calibration copy of {n} bytes done", file=sys.stderr, flush=True)


def bench_ulysses(args, w, q_cpu, k_cpu, v_cpu, dev) -> int:
    """One step = the Ulysses forward of P = w.N ranks on one GPU: the all-to-all
    of q, k, v (sequence slices -> head slices), each rank's attention over the
    whole sequence for its Hq/P heads (the cast to bf16 fused), and the
    all-to-all of the output back. The inputs are the ranks' sequence slices
    [P, B, S/P, H, D], laid out once before timing. Useful work as for the ring:
    4*D flops per allowed pair."""
    import torch
    import ring_context_parallelism_flash_amd as ra
    P = w.N

    def shard(x):
        B, H, S, D = x.shape
        return x.permute(0, 2, 1, 3).reshape(B, P, S // P, H, D).permute(1, 0, 2, 3, 4).contiguous()

    q, k, v = (shard(t).to(dev) for t in (q_cpu, k_cpu, v_cpu))
    out = torch.empty_like(q)
    lse = torch.empty((P, w.B, w.Hq // P, w.S), dtype=torch.float32, device=dev)
    ws = torch.empty(ra.ra_ulysses_sim_workspace_bytes(w.B, w.Hq, w.Hkv, w.S, w.D, q.dtype, P),
                     dtype=torch.uint8, device=dev)

    def step():
        ra.ra_ulysses_sim_fwd(q, k, v, out, lse, P=P, causal=w.causal, workspace=ws)

    print(f"bench: ulysses warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ra.ra_kernel_timing_enable(True)
    ra.ra_kernel_timing_read()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    k_ms, launches, k_flops = ra.ra_kernel_timing_read()
    ra.ra_kernel_timing_enable(False)
    print(f"bench: timed {args.steps} ulysses steps in {t1 - t0:.3f} s", file=sys.stderr,
          flush=True)
    # all-to-all bandwidth: one q-sized first all-to-all, timed with events
    dst = torch.empty((P, w.B, w.Hq // P, w.S, w.D), dtype=q.dtype, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        ra.ra_ulysses_all_to_all(q, dst, P)
    e1.record()
    torch.cuda.synchronize()
    a2a_gbs = 2 * q.numel() * q.element_size() * 5 / (e0.elapsed_time(e1) / 1e3) / 1e9
    del dst

    flops_step = useful_flops(w)
    ms_step = (t1 - t0) * 1e3 / args.steps
    value = flops_step / (ms_step / 1e3) / 1e12
    achieved = k_flops / (k_ms / 1e3) / 1e12 if k_ms > 0 else 0.0
    line = {
        "metric": f"ulysses attn fwd useful TFLOP/s, {w.name}",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded iid normal q/k/v, k x0.5, bf16)",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D, "S": w.S,
                   "virtual_ranks": P, "layout": "ulysses", "causal": w.causal},
        "pct_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "useful_flops_per_step": flops_step,
        "roofline": {
            "kernel": fwd_kernel_name(w, w.S),
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": round(PEAK_BF16_TFLOPS, 1),
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": None,
            "traffic_source": "no counter summary for this workload",
            "launches_per_step": launches // max(args.steps, 1),
            "avg_launch_ms": round(k_ms / max(launches, 1), 4),
            "flops_per_launch": k_flops / max(launches, 1),
            "kernel_ms_per_step": round(k_ms / max(args.steps, 1), 3),
        },
        "aux_kernels": {"ulysses_all_to_all_GBs": round(a2a_gbs, 1), "hbm_peak_GBs": PEAK_HBM_GBS},
        "flops_check": {"closed_form": flops_step, "library_count": k_flops / max(args.steps, 1)},
    }
    if not args.no_cpu_baseline:
        print("bench: cpu baseline (fp64 oracle)", file=sys.stderr, flush=True)
        o = out.cpu().permute(1, 0, 2, 3, 4).reshape(w.B, w.S, w.Hq, w.D).permute(0, 2, 1, 3)
        l_ = lse.cpu().permute(1, 0, 2, 3).reshape(w.B, w.Hq, w.S)
        line["cpu_baseline"] = cpu_baseline(w, q_cpu, k_cpu, v_cpu, o, l_, args.cpu_rows)
    print(json.dumps(line), flush=True)
    return 0


def bench_usp(args, w, q_cpu, k_cpu, v_cpu, dev) -> int:
    """One step = unified sequence parallelism on P_r = N / P_u nodes of P_u
    devices, simulated on one GPU: the intra-node all-to-all of q, k, v, the
    ring across the nodes for every head group, and the reverse all-to-all.
    Inputs are laid out once, before timing, as the devices' slices (the
    node token lists of the ring layout, split across each node's devices).
    Useful work as for the ring: 4*D flops per allowed pair."""
    import torch
    import ring_context_parallelism_flash_amd as ra
    P_u, P_r = w.P_u, w.N // w.P_u
    perm = {"zigzag": ra.ra_zigzag_permute, "striped": ra.ra_striped_permute}.get(w.ring_layout)

    def shard(x):
        x = x.to(dev)
        if perm is not None:                      # sequence order -> node-major order
            y = torch.empty_like(x)
            perm(x, y, P_r)
            x = y
        B, H, S, D = x.shape
        return (x.permute(0, 2, 1, 3).reshape(B, P_r * P_u, S // (P_r * P_u), H, D)
                .permute(1, 0, 2, 3, 4).contiguous())

    q, k, v = (shard(t) for t in (q_cpu, k_cpu, v_cpu))
    out = torch.empty_like(q)
    lse = torch.empty((P_u, w.B, w.Hq // P_u, w.S), dtype=torch.float32, device=dev)
    ws = torch.empty(ra.ra_usp_sim_workspace_bytes(w.B, w.Hq, w.Hkv, w.S, w.D, q.dtype, P_u, P_r),
                     dtype=torch.uint8, device=dev)
    copy = torch.cuda.Stream(device=dev)

    def step():
        ra.ra_usp_sim_fwd(q, k, v, out, lse, P_u=P_u, P_r=P_r, layout=w.ring_layout,
                          causal=w.causal, workspace=ws, copy_stream=copy)

    print(f"bench: usp warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ra.ra_kernel_timing_enable(True)
    ra.ra_kernel_timing_read()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    k_ms, launches, k_flops = ra.ra_kernel_timing_read()
    ra.ra_kernel_timing_enable(False)
    print(f"bench: timed {args.steps} usp steps in {t1 - t0:.3f} s", file=sys.stderr, flush=True)
    flops_step = useful_flops(w)
    ms_step = (t1 - t0) * 1e3 / args.steps
    value = flops_step / (ms_step / 1e3) / 1e12
    achieved = k_flops / (k_ms / 1e3) / 1e12 if k_ms > 0 else 0.0
    line = {
        "metric": f"usp attn fwd useful TFLOP/s, {w.name}",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded iid normal q/k/v, k x0.5, bf16)",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D, "S": w.S,
                   "virtual_devices": w.N, "nodes": P_r, "devices_per_node": P_u,
                   "ring_layout": w.ring_layout, "causal": w.causal},
        "pct_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "useful_flops_per_step": flops_step,
        "roofline": {
            "kernel": fwd_kernel_name(w, w.S // (2 * P_r)),
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": round(PEAK_BF16_TFLOPS, 1),
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": None,
            "traffic_source": "no counter summary for this workload",
            "launches_per_step": launches // max(args.steps, 1),
            "avg_launch_ms": round(k_ms / max(launches, 1), 4),
            "flops_per_launch": k_flops / max(launches, 1),
            "kernel_ms_per_step": round(k_ms / max(args.steps, 1), 3),
        },
        "flops_check": {"closed_form": flops_step, "library_count": k_flops / max(args.steps, 1)},
    }
    if not args.no_cpu_baseline:
        print("bench: cpu baseline (fp64 oracle)", file=sys.stderr, flush=True)
        node_major = torch.empty(w.S, dtype=torch.long)
        pos = torch.arange(w.S, dtype=torch.float32, device=dev)[None, None, :, None]
        if perm is not None:
            y = torch.empty_like(pos)
            perm(pos, y, P_r)
            pos = y
        node_major = pos[0, 0, :, 0].long().cpu()              # node-major -> position
        inv = torch.empty_like(node_major)
        inv[node_major] = torch.arange(w.S)
        o = out.cpu().permute(1, 0, 2, 3, 4).reshape(w.B, w.S, w.Hq, w.D)[:, inv]
        o = o.permute(0, 2, 1, 3)
        l_ = lse.cpu().permute(1, 0, 2, 3).reshape(w.B, w.Hq, w.S)[:, :, inv]
        line["cpu_baseline"] = cpu_baseline(w, q_cpu, k_cpu, v_cpu, o, l_, args.cpu_rows)
    print(json.dumps(line), flush=True)
    return 0


def main(argv=None) -> int:
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=5)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--workload", default=None, help="workload name (default: the 128k GQA one)")
    p.add_argument("--cpu-rows", type=int, default=4096,
                   help="seeded random rows per head for the CPU oracle (plus chunk boundaries)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--backward", action="store_true",
                   help="time the ring backward (dq, dk, dv of a seeded dout) instead of the forward")
    p.add_argument("--copy-calibration-mib", type=int, default=0,
                   help="finish with one plain device copy of this many MiB (a known-size "
                        "reference for hardware byte counters)")
    p.add_argument("--aux-only", action="store_true",
                   help="only the permute, lse-merge and all-to-all kernels (for "
                        "hardware-counter runs)")
    p.add_argument("--trace-overlap", metavar="KERNEL_TRACE_CSV", default=None,
                   help="print the block copies' overlap with attention kernels in a "
                        "rocprofv3 kernel trace and exit (no GPU use)")
    args = p.parse_args(argv)
    if args.trace_overlap:
        print(json.dumps(copy_overlap(args.trace_overlap)), flush=True)
        return 0
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: measures one GPU only -- the N ranks of the ring (and the devices "
              "of the Ulysses / USP grids) are simulated on a single MI355X; run with --gpus 1.",
              file=sys.stderr)
        return 2

    import torch
    import ring_context_parallelism_flash_amd as ra
    import workloads

    w = workloads.BY_NAME[args.workload] if args.workload else workloads.HEADLINE
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"bench: generating {w.name} inputs", file=sys.stderr, flush=True)
    q_cpu, k_cpu, v_cpu = workloads.make_inputs(w)
    if w.layout == "ulysses":
        if args.backward:
            print("bench.py: no backward for the Ulysses workload", file=sys.stderr)
            return 2
        return bench_ulysses(args, w, q_cpu, k_cpu, v_cpu, dev)
    if w.layout == "usp":
        if args.backward:
            print("bench.py: no backward for the USP workload", file=sys.stderr)
            return 2
        return bench_usp(args, w, q_cpu, k_cpu, v_cpu, dev)
    q, k, v = (t.to(dev) for t in (q_cpu, k_cpu, v_cpu))
    if args.aux_only:
        print(json.dumps({"workload": w.name, "aux_kernels": aux_bandwidth(w, q, dev)}),
              flush=True)
        calibration_copy(args, dev)
        return 0
    runner = ra.RingRunner(w.B, w.Hq, w.Hkv, w.S, w.D, q.dtype, w.N, w.layout, w.causal,
                           device=dev)
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.S), dtype=torch.float32, device=dev)

    if args.backward:
        return bench_backward(args, w, q, k, v, runner, out, lse)
    print(f"bench: warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        runner(q, k, v, out, lse)
    torch.cuda.synchronize()

    ra.ra_kernel_timing_enable(True)
    ra.ra_kernel_timing_read()  # clear
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        runner(q, k, v, out, lse)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    k_ms, launches, k_flops = ra.ra_kernel_timing_read()
    ra.ra_kernel_timing_enable(False)
    print(f"bench: timed {args.steps} steps in {t1 - t0:.3f} s", file=sys.stderr, flush=True)

    flops_step = useful_flops(w)
    lib_flops_step = k_flops / max(args.steps, 1)
    ms_step = (t1 - t0) * 1e3 / args.steps
    value = flops_step / (ms_step / 1e3) / 1e12

    # ring alone (inputs already in rank-major order), for the record
    qr, kr, vr = runner.permute_inputs(q, k, v)
    torch.cuda.synchronize()
    r0 = time.perf_counter()
    for _ in range(args.steps):
        runner.ring(qr, kr, vr)
    torch.cuda.synchronize()
    ring_ms = (time.perf_counter() - r0) * 1e3 / args.steps

    aux = aux_bandwidth(w, q, dev)
    peak_info = peak_derivation(dev) if w.dtype == "bf16" else None

    achieved = k_flops / (k_ms / 1e3) / 1e12 if k_ms > 0 else 0.0
    traffic, traffic_src = measured_traffic(w.name)
    bf16 = w.dtype == "bf16"
    peak = PEAK_BF16_TFLOPS if bf16 else PEAK_FP32_MFMA_TFLOPS
    line = {
        "metric": METRIC if w is workloads.HEADLINE else f"ring-attn fwd useful TFLOP/s, {w.name}",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf16 else "f32",
        "data": "synthetic (seeded iid normal q/k/v, k x0.5, bf16)",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D, "S": w.S,
                   "virtual_ranks": w.N, "layout": w.layout, "causal": w.causal},
        "pct_peak": round(100.0 * value / peak, 2),
        "useful_flops_per_step": flops_step,
        "roofline": {
            "kernel": fwd_kernel_name(w),
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": round(peak, 1),
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": traffic,
            "traffic_unit": "HBM bytes per launch (FETCH_SIZE x2.0 + WRITE_SIZE x1.0)",
            "traffic_source": traffic_src,
            "launches_per_step": launches // max(args.steps, 1),
            "avg_launch_ms": round(k_ms / max(launches, 1), 4),
            "flops_per_launch": k_flops / max(launches, 1),
            "kernel_ms_per_step": round(k_ms / max(args.steps, 1), 3),
        },
        "ring_only_ms": round(ring_ms, 3),
        "aux_kernels": aux,
        "flops_check": {"closed_form": flops_step, "library_count": lib_flops_step},
    }
    if peak_info is not None:
        line["peak_derivation"] = peak_info
    if not args.no_cpu_baseline:
        print("bench: cpu baseline (fp64 oracle)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(w, q_cpu, k_cpu, v_cpu, out.cpu(), lse.cpu(),
                                            args.cpu_rows)
    print(json.dumps(line), flush=True)
    calibration_copy(args, dev)
    return 0


if __name__ == "__main__":
    sys.exit(main())
