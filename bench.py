"""Attention-forward throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one attn_fwd call (the whole hot path) over one batch of the
causal multi-head workload B=2, H=32, N=8192, d=128 (bf16), with Q, K, V
already resident in HBM.  Throughput counts 4*d FLOPs per unmasked score
("Efficient attention: long context and sub-quadratic variants", section
"The quadratic wall, stated concretely"), never the masked entries a tile
computes and discards.  Prints one JSON line.

The same line also carries, as secondary figures, the backward (attn_bwd:
dQ, dK, dV) timed on the same workload, at 10*d FLOPs per unmasked score
(S, dP, dV, dQ, dK: five 2*d contractions), and the paged decode
(attn_decode_paged) on the decode workloads in HBM GB/s (the visible K and V
rows once, q, o, lse and the page-table entries), and the packed-sequence
forward with structured masks (attn_fwd_varlen) at 4*d FLOPs per visible
score, and the FP8 forward (attn_fwd_fp8) against the dense fp8 peak.
"""

from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s (bf16, d=128, causal/window) and % of MFMA peak"
MAIN = "c2_causal_mha"
OTHERS = ["c2_causal_mha_sharp", "c3_causal_window", "c4_causal_gqa", "c5_long_causal",
          "c5_long_window"]
BWD_OTHERS = ["c4_causal_gqa"]
DECODE = ["d1_decode_gqa_128k", "d2_decode_mha_8k", "d3_decode_window_spec4",
          "d4_decode_mqa_128k", "d5_decode_gqa16_spec4"]
VARLEN = ["v1_packed_causal_gqa", "l1_longformer_4k"]
FP8_OTHERS = ["c4_causal_gqa", "c5_long_causal"]
CSRC = os.path.join(ROOT, "exact_tiled_attention_attn_amd", "csrc")
KERNEL_SRC = os.path.join(CSRC, "attn_fwd.hip")
# source of each kind of kernel the line times (the forward's also serves the
# packed-sequence forward); every kernel also compiles the shared device helpers
KERNEL_SOURCES = {"fwd": "attn_fwd.hip", "varlen": "attn_fwd.hip", "bwd": "attn_bwd.hip",
                  "fp8": "attn_fp8.hip", "decode": "attn_decode.hip"}
KERNEL_HEADERS = [os.path.join(CSRC, "attn_device.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def fwd_kernel_name(d: int, variant: int) -> str:
    """The forward kernel a launch runs: variants 3 and 4 (and the default at
    d = 128) are the ping-pong kernel, 1 and 2 (and the default at d = 64)
    the lockstep one."""
    v = variant if variant != 0 else (1 if d == 64 else 4)
    return "attn_fwd_pp_kernel" if v in (3, 4) else "attn_fwd_kernel"


def kernel_sha(kind: str = "fwd") -> str:
    """sha256[:16] of one kind of kernel's code (KERNEL_SOURCES; the forward's
    is KERNEL_SRC): its source and the device header it includes, with //
    comments, trailing blanks and empty lines removed, and the device compile
    flags other than include paths (which name the directory the repository
    sits in).  A comment edit or a move of the repository keeps stored counter
    data valid; any change to the code or the flags invalidates it."""
    from exact_tiled_attention_attn_amd.build import DEVICE_ONLY, COMMON
    src = KERNEL_SRC if kind == "fwd" else os.path.join(CSRC, KERNEL_SOURCES[kind])
    code = []
    for path in [src] + KERNEL_HEADERS:
        with open(path) as f:
            for line in f:
                line = line.split("//", 1)[0].rstrip()
                if line:
                    code.append(line)
    code.append(" ".join(f for f in COMMON + DEVICE_ONLY if not f.startswith("-I")))
    return hashlib.sha256("\n".join(code).encode()).hexdigest()[:16]


def device_inputs(w, torch):
    from exact_tiled_attention_attn_amd.inputs import make_qkv
    q, k, v = make_qkv(w.B, w.Hq, w.Hkv, w.N, w.d, w.seed)
    if w.q_mult != 1.0:
        q = (q.float() * w.q_mult).to(torch.bfloat16)
    dev = torch.device("cuda:0")
    return q.to(dev), k.to(dev), v.to(dev), (q, k, v)


def run_timed(launch, steps, warmup, seconds, torch, stream, sync_every=8):
    """Warm up (at least `warmup` calls and at least `seconds` of them: the
    clock ramps up over the first milliseconds of sustained load), then time
    `steps` back-to-back calls between two events on `stream`.

    The region is bracketed by synchronisations, and nothing stands between
    the first synchronisation and the first timed launch but the start
    event: after even a few milliseconds of idling the GPU runs the next
    tens of calls measurably slower.  So Python's cyclic garbage collector
    is off from the start of the warmup to the end (a collection there would
    idle the GPU, and the events would count that time as well).  Returns
    (event ms per call, host wall ms per call)."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    gc.collect()
    gc.disable()
    try:
        t_end = time.perf_counter() + seconds
        n = 0
        while n < warmup or time.perf_counter() < t_end:
            launch()
            n += 1
            if n % sync_every == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(steps):
            launch()
        e1.record(stream)
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    finally:
        gc.enable()
    return e0.elapsed_time(e1) / steps, wall_ms


def time_workload(w, steps, warmup, variant, torch, attn):
    """Returns (wall ms/step, event ms/launch, host tensors)."""
    q, k, v, host = device_inputs(w, torch)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream()

    def launch():
        st = attn.attn_fwd_ex(q, k, v, o, lse, w.B, w.Hq, w.Hkv, w.N, w.d, w.sm_scale,
                              int(w.causal), w.window, variant, stream)
        if st != 0:
            raise RuntimeError(f"attn_fwd_ex: {attn.attn_status_string(st)}")

    ev_ms, wall_ms = run_timed(launch, steps, warmup, 0.5, torch, stream)
    del q, k, v, o, lse
    return wall_ms, ev_ms, host


def time_backward(w, steps, warmup, torch, attn):
    """attn_bwd (Delta, dQ, dK/dV kernels) on the workload, with o and lse
    from attn_fwd.  Returns event ms per call."""
    from exact_tiled_attention_attn_amd.inputs import make_dout
    q, k, v, _ = device_inputs(w, torch)
    do = make_dout(w.B, w.Hq, w.N, w.d, w.seed + 100).to(q.device)
    o, lse = attn.fwd(q, k, v, causal=w.causal, window=w.window, scale=w.sm_scale)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty((attn.attn_bwd_workspace_size(w.B, w.Hq, w.N) // 4,), dtype=torch.float32,
                     device=q.device)
    stream = torch.cuda.current_stream()

    def launch():
        st = attn.attn_bwd(q, k, v, o, lse, do, dq, dk, dv, ws, w.B, w.Hq, w.Hkv, w.N, w.d,
                           w.sm_scale, int(w.causal), w.window, stream)
        if st != 0:
            raise RuntimeError(f"attn_bwd: {attn.attn_status_string(st)}")

    ev_ms, _ = run_timed(launch, steps, warmup, 0.5, torch, stream, sync_every=4)
    del q, k, v, do, o, lse, dq, dk, dv, ws
    return ev_ms


def time_decode(w, steps, warmup, torch, attn):
    """attn_decode_paged on a decode workload.  Returns (event ms per call,
    the sequence lengths)."""
    from exact_tiled_attention_attn_amd.inputs import decode_lengths, make_decode_q, make_paged_kv
    lens = decode_lengths(w.B, w.max_len, w.seed)
    kc, vc, table = make_paged_kv(lens, w.Hkv, w.d, w.page_size, seed=w.seed)
    dev = torch.device("cuda:0")
    kc, vc, table = kc.to(dev), vc.to(dev), table.to(dev)
    q = make_decode_q(w.B, w.Hq, w.T, w.d, seed=w.seed + 1).to(dev)
    lt = torch.tensor(lens, dtype=torch.int32, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.T), dtype=torch.float32, device=dev)
    nws = attn.attn_decode_workspace_size(w.B, w.Hq, w.Hkv, w.T, w.d, w.page_size, w.max_len,
                                          w.window)
    ws = torch.empty((max(nws, 16) // 4,), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def launch():
        st = attn.attn_decode_paged(q, kc, vc, table, lt, o, lse, ws, w.B, w.Hq, w.Hkv, w.T, w.d,
                                    w.page_size, kc.shape[0], table.shape[1], w.max_len,
                                    w.sm_scale, w.window, stream)
        if st != 0:
            raise RuntimeError(f"attn_decode_paged: {attn.attn_status_string(st)}")

    ev_ms, _ = run_timed(launch, steps, warmup, 0.3, torch, stream)
    del q, kc, vc, table, lt, o, lse, ws
    return ev_ms, lens


def time_varlen(w, steps, warmup, torch, attn):
    """attn_fwd_varlen on a packed workload.  Returns event ms per call."""
    from exact_tiled_attention_attn_amd.inputs import make_packed_qkv
    q, k, v, cu = make_packed_qkv(list(w.lens), w.Hq, w.Hkv, w.d, seed=w.seed)
    dev = torch.device("cuda:0")
    q, k, v, cu = q.to(dev), k.to(dev), v.to(dev), cu.to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.Hq, w.total), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    B, max_len = len(w.lens), max(w.lens)

    def launch():
        st = attn.attn_fwd_varlen(q, k, v, o, lse, cu, B, max_len, w.total, w.Hq, w.Hkv, w.d,
                                  w.sm_scale, int(w.causal), w.window, w.radius, w.n_global,
                                  stream)
        if st != 0:
            raise RuntimeError(f"attn_fwd_varlen: {attn.attn_status_string(st)}")

    ev_ms, _ = run_timed(launch, steps, warmup, 0.3, torch, stream)
    del q, k, v, cu, o, lse
    return ev_ms


def time_fp8(w, steps, warmup, torch, attn):
    """attn_fwd_fp8 on a dense workload (inputs packed once by
    attn_fp8_quantize, which is timed separately).  Returns (forward event
    ms per call, quantize ms per call)."""
    q, k, v, _ = device_inputs(w, torch)
    q8, k8, vt8, sc = attn.fp8_quantize(q, k, v)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream()

    def launch():
        st = attn.attn_fwd_fp8(q8, k8, vt8, sc, o, lse, w.B, w.Hq, w.Hkv, w.N, w.d, w.sm_scale,
                               int(w.causal), w.window, stream)
        if st != 0:
            raise RuntimeError(f"attn_fwd_fp8: {attn.attn_status_string(st)}")

    def quant():
        st = attn.attn_fp8_quantize(q, k, v, q8, k8, vt8, sc, w.B, w.Hq, w.Hkv, w.N, w.d, stream)
        if st != 0:
            raise RuntimeError(f"attn_fp8_quantize: {attn.attn_status_string(st)}")

    em, _ = run_timed(launch, steps, warmup, 0.3, torch, stream)
    qm, _ = run_timed(quant, steps, warmup, 0.3, torch, stream)
    del q, k, v, q8, k8, vt8, sc, o, lse
    return em, qm


def cpu_baseline(w, host, seconds):
    """The float64 oracle on the host cores, on the same workload: the whole
    workload when it fits in about 2 * `seconds`, else a seeded sample of
    rows over as many (batch, head) slices as fit."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from exact_tiled_attention_attn_amd.inputs import sample_rows
    from exact_tiled_attention_attn_amd.workloads import visible_scores_per_head
    from oracle import attention_rows

    q, k, v = (t.float().numpy() for t in host)
    cores = len(os.sched_getaffinity(0))
    G = w.Hq // w.Hkv

    def visible(i):
        hi = i + 1 if w.causal else w.N
        lo = max(0, i - w.window + 1) if w.window > 0 else 0
        return hi - lo

    with threadpool_limits(limits=1, user_api="blas"):
        probe = sample_rows(w.N, 256, seed=w.seed * 7919, edges=())
        t0 = time.perf_counter()
        attention_rows(q[:1, :1], k[:1, :1], v[:1, :1], w.sm_scale, w.causal, w.window,
                       rows=probe)
        rate = sum(visible(int(i)) for i in probe) / (time.perf_counter() - t0)  # scores/s/core
        full_scores = w.B * w.Hq * visible_scores_per_head(w.N, w.causal, w.window)
        if full_scores / (rate * cores) <= 2 * seconds:
            rows, nslices, what = None, w.B * w.Hq, "the whole workload (every row of every head)"
            scores = full_scores
        else:
            rows = sample_rows(w.N, 2048, seed=w.seed * 7919, edges=())
            per_slice = sum(visible(int(i)) for i in rows)
            nslices = int(max(1, min(w.B * w.Hq, seconds * rate * cores / per_slice)))
            scores = per_slice * nslices
            what = (f"{nslices} (batch, head) slices x {len(rows)} seeded random query rows")
        heads = list(range(nslices))
        qs = np.stack([q[h // w.Hq, h % w.Hq] for h in heads])[None]
        ks = np.stack([k[h // w.Hq, (h % w.Hq) // G] for h in heads])[None]
        vs = np.stack([v[h // w.Hq, (h % w.Hq) // G] for h in heads])[None]
        # repeat the sample until about `seconds` of CPU time have passed, so
        # a workload that the host finishes quickly is still timed stably
        reps = 0
        t0 = time.perf_counter()
        while True:
            attention_rows(qs, ks, vs, w.sm_scale, w.causal, w.window, rows=rows, workers=cores)
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= seconds or dt * (reps + 1) / reps > 2 * seconds:
                break
    if reps > 1:
        what += f", {reps} passes"
    scores *= reps
    flops = 4 * w.d * scores
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"{w.name}: {what} ({scores} unmasked scores), float64 NumPy, one BLAS "
                   f"thread per worker, {cores} worker threads, {dt:.1f} s"),
        "seconds": dt,
        "cpu": _cpu_model(),
    }


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor()


def fwd_key(name, variant):
    """traffic.json key of a forward workload under a kernel variant."""
    return name if variant == 0 else f"{name}@v{variant}"


def traffic_for(key, sha):
    """HBM bytes per call from the committed counter summary (entry `key`:
    a forward workload's name, or "bwd:", "fp8:", "varlen:", "decode:" and
    the workload's name), if they were taken on the current source of that
    kernel (`sha`); else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get("workloads", {}).get(key)
    if not e or e.get("kernel_source_sha") != sha:
        return None
    return e.get("hbm_bytes_per_call")


# Dense matrix-core FLOP per compute unit and clock: v_mfma_f32_32x32x16_bf16
# does 32 x 32 x 16 multiply-adds (32 768 FLOP) and issues every 32 clocks on
# each of a CU's 4 SIMDs (32.0 busy cycles per MFMA in the counters); the
# dense fp8 rate is twice that (the published fp8 and bf16 peaks are 2 : 1).
BF16_FLOP_PER_CU_CLK = 32 * 32 * 16 * 2 // 32 * 4
FP8_FLOP_PER_CU_CLK = 2 * BF16_FLOP_PER_CU_CLK


def derive_peaks(info, published_bf16, published_fp8):
    """Peak dense MFMA rates of the device bench.py runs on, from what the HIP
    runtime reports (compute units, peak engine clock) and the FLOP per CU
    and clock above, with the published figures beside them."""
    cus, clock_khz, mem_khz, bus_bits = info
    if cus <= 0 or clock_khz <= 0:
        raise RuntimeError(f"device reports {cus} CUs at {clock_khz} kHz")
    bf16 = cus * clock_khz * 1e3 * BF16_FLOP_PER_CU_CLK / 1e12
    return {"bf16_tflops": round(bf16, 1),
            "fp8_tflops": round(bf16 * FP8_FLOP_PER_CU_CLK / BF16_FLOP_PER_CU_CLK, 1),
            "cus": cus, "max_clock_mhz": clock_khz / 1e3,
            "bf16_flop_per_cu_clock": BF16_FLOP_PER_CU_CLK,
            "fp8_flop_per_cu_clock": FP8_FLOP_PER_CU_CLK,
            "source": "hipDeviceAttributeMultiprocessorCount x hipDeviceAttributeClockRate x "
                      "FLOP/CU/clock of v_mfma_f32_32x32x16_bf16 (fp8: twice that)",
            "published_bf16_tflops": published_bf16, "published_fp8_tflops": published_fp8,
            "memory_clock_mhz": mem_khz / 1e3, "memory_bus_bits": bus_bits}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--variant", type=int, default=0)
    ap.add_argument("--workload", default=MAIN)
    ap.add_argument("--no-others", action="store_true", help="time only the main workload")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-bwd", action="store_true", help="skip the backward timing")
    ap.add_argument("--no-decode", action="store_true", help="skip the paged-decode timing")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8 forward timing")
    ap.add_argument("--no-varlen", action="store_true",
                    help="skip the packed-sequence / structured-mask timing")
    ap.add_argument("--varlen-case", default=None,
                    help="time only this packed-sequence / structured-mask workload")
    ap.add_argument("--decode-case", default=None, help="time only this paged-decode workload")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for HBM counter scaling)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch

    from exact_tiled_attention_attn_amd import attn
    from exact_tiled_attention_attn_amd.workloads import (DECODE_WORKLOADS, MI355X_BF16_DENSE_TFLOPS,
                                                          MI355X_FP8_DENSE_TFLOPS,
                                                          MI355X_HBM_GBPS, VARLEN_WORKLOADS,
                                                          WORKLOADS, algorithmic_bytes, bwd_flops,
                                                          decode_bytes, flops, varlen_flops)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    attn.load_library()
    props = torch.cuda.get_device_properties(0)
    peaks = derive_peaks(attn.attn_device_info(0), MI355X_BF16_DENSE_TFLOPS,
                         MI355X_FP8_DENSE_TFLOPS)
    peak, fp8_peak = peaks["bf16_tflops"], peaks["fp8_tflops"]

    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    w = WORKLOADS[args.workload]
    log(f"timing {w.name} variant {args.variant} ({attn.attn_variant_name(args.variant)})")
    wall_ms, ev_ms, host = time_workload(w, args.steps, args.warmup, args.variant, torch, attn)
    f = flops(w)
    value = f / (wall_ms * 1e-3) / 1e12
    achieved = f / (ev_ms * 1e-3) / 1e12
    sha = kernel_sha()
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: Q, K, V i.i.d. N(0,1) rounded to bf16, seeded",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N,
                   "d": w.d, "causal": w.causal, "window": w.window,
                   "variant": attn.attn_variant_name(args.variant)},
        "pct_of_peak": round(100.0 * value / peak, 2),
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": traffic_for(fwd_key(w.name, args.variant), sha),
            "kernel": fwd_kernel_name(w.d, args.variant),
            "avg_launch_ms": round(ev_ms, 4),
            "flops_per_launch": f,
            "algorithmic_bytes_per_launch": algorithmic_bytes(w),
        },
        "device": {"name": props.name, "cus": props.multi_processor_count,
                   "arch": getattr(props, "gcnArchName", "")},
        "peak_derivation": peaks,
        "kernel_source_sha": sha,
    }
    if not args.no_others:
        others = {}
        for name in OTHERS:
            ow = WORKLOADS[name]
            log(f"timing {name}")
            steps = max(3, args.steps // 4) if ow.N >= 131072 else args.steps
            wm, em, _ = time_workload(ow, steps, max(1, args.warmup // 2), args.variant, torch,
                                      attn)
            of = flops(ow)
            others[name] = {"tflops": round(of / (em * 1e-3) / 1e12, 2),
                            "pct_of_peak": round(100 * of / (em * 1e-3) / 1e12 / peak, 2),
                            "ms": round(em, 4), "steps": steps,
                            "traffic": traffic_for(fwd_key(name, args.variant), sha),
                            "algorithmic_bytes": algorithmic_bytes(ow)}
            torch.cuda.empty_cache()
        out["other_workloads"] = others
    if not args.no_bwd:
        bw = {}
        for name in [w.name] + ([] if args.no_others else BWD_OTHERS):
            bwl = WORKLOADS[name]
            log(f"timing backward {name}")
            em = time_backward(bwl, max(3, args.steps // 2), max(1, args.warmup // 2), torch,
                               attn)
            bf = bwd_flops(bwl)
            bw[name] = {"tflops": round(bf / (em * 1e-3) / 1e12, 2),
                        "pct_of_peak": round(100 * bf / (em * 1e-3) / 1e12 / peak, 2),
                        "ms": round(em, 4), "flops_per_call": bf,
                        "traffic": traffic_for("bwd:" + name, kernel_sha("bwd"))}
            torch.cuda.empty_cache()
        out["backward"] = bw
    if not args.no_fp8:
        f8 = {}
        for name in [w.name] + ([] if args.no_others else FP8_OTHERS):
            fw = WORKLOADS[name]
            log(f"timing fp8 {name}")
            em, qm = time_fp8(fw, args.steps, max(1, args.warmup // 2), torch, attn)
            ff = flops(fw)
            f8[name] = {"tflops": round(ff / (em * 1e-3) / 1e12, 2),
                        "pct_of_fp8_peak": round(100 * ff / (em * 1e-3) / 1e12 / fp8_peak,
                                                 2),
                        "ms": round(em, 4), "quantize_ms": round(qm, 4),
                        "traffic": traffic_for("fp8:" + name, kernel_sha("fp8"))}
            torch.cuda.empty_cache()
        out["fp8"] = f8
    if not args.no_varlen:
        var = {}
        for name in ([args.varlen_case] if args.varlen_case else
                     VARLEN if not args.no_others else VARLEN[:1]):
            vw = VARLEN_WORKLOADS[name]
            log(f"timing varlen {name}")
            em = time_varlen(vw, args.steps, max(1, args.warmup // 2), torch, attn)
            vf = varlen_flops(vw)
            var[name] = {"tflops": round(vf / (em * 1e-3) / 1e12, 2),
                         "pct_of_peak": round(100 * vf / (em * 1e-3) / 1e12 / peak, 2),
                         "ms": round(em, 4), "flops_per_call": vf,
                         "traffic": traffic_for("varlen:" + name, kernel_sha("varlen"))}
            torch.cuda.empty_cache()
        out["varlen"] = var
    if not args.no_decode:
        dec = {}
        for name in ([args.decode_case] if args.decode_case else
                     DECODE if not args.no_others else DECODE[:1]):
            dw = DECODE_WORKLOADS[name]
            log(f"timing decode {name}")
            em, lens = time_decode(dw, args.steps, max(1, args.warmup // 2), torch, attn)
            nb = decode_bytes(dw, lens)
            dec[name] = {"GB/s": round(nb / (em * 1e-3) / 1e9, 1),
                         "frac_of_hbm_peak": round(nb / (em * 1e-3) / 1e9 / MI355X_HBM_GBPS, 4),
                         "ms": round(em, 4), "bytes_per_call": nb, "seq_lens": lens,
                         "traffic": traffic_for("decode:" + name, kernel_sha("decode"))}
            torch.cuda.empty_cache()
        out["decode"] = dec
    if not args.no_cpu:
        log(f"oracle CPU baseline (~{args.cpu_seconds:.0f} s)")
        out["cpu_baseline"] = cpu_baseline(w, host, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
