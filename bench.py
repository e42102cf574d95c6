"""Throughput of the GDN streaming core on one MI355X.

Workload: one GDN layer on one 720p streaming chunk -- B=1 stream, H=20 heads,
d_k = d_v = 112, T = 2640 tokens (3 latent frames x 22 x 40 tokens), bf16
q/k/v/o, fp32 gates and state.  One step = the forward scan from the carried
state (committed back to the cache) plus the reverse scan inside the chunk.
Inputs are synthetic (seeded) and already resident in HBM; by default they
rotate over enough buffer sets that the live set exceeds the 256 MB MALL, so
every step streams from HBM.

Prints one JSON line.  `value` is tokens per second per layer (T / step time).
`roofline` is for the step, the launch pair gdn_prep_kernel + gdn_scan_kernel
that one gdn_chunk_bidir call runs: the algorithmic bytes of the step over
`ms_per_step`.  Algorithmic bytes per token-head: q, k, v read once and o
written (224 B each in bf16) plus the two fp32 gates; a bidirectional call also
writes o_rev; the forward scan reads and writes the 112x112 fp32 state of each
head once.  `roofline.kernels` splits those bytes between the two kernels (the
prep reads q, k, a, beta; the scan reads v and the state and writes o, o_rev and
the state) and gives each kernel's average duration from HIP events on its
launch stream, its duration in the committed rocprofv3 trace, and its HBM
traffic from the committed FETCH_SIZE / WRITE_SIZE counter runs (null once the
kernel source has changed since they were taken).
`--mode long` times the same call on a 21-frame clip (T = 18480 tokens: 289
dependent sub-chunk steps per head), a secondary line beside the headline.
`cpu_baseline` times the fp64 CPU oracle on the host cores over the same
workload (the oracle is a test reference, not a tuned CPU implementation), and
once more on one core.
`measured_peaks` states what this machine reaches with plain kernels of our own
(a 1 GiB device copy, a dense bf16 MFMA loop) beside the vendor peaks the
fractions are quoted against.
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

METRIC = "GDN tokens/s per layer at 2640-token 720p chunk; % of MFMA/HBM roofline"
B, H, D, T = 1, 20, 112, 2640
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16
BYTES_PER_TOKEN_HEAD = 4 * D * 2 + 2 * 4     # one scan: q, k, v, o in bf16 + a, beta in fp32
BIDIR_BYTES_PER_TOKEN_HEAD = 5 * D * 2 + 2 * 4   # both scans in one call: q, k, v once, o and o_rev
STATE_BYTES = B * H * D * D * 4
FLOPS_PER_TOKEN_HEAD = 6 * D * D             # S k, rank-1 update, S q
T_LONG = 21 * 880                            # 21 latent frames of 22 x 40 tokens
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gdn_step_720p.json")
TRACE_FILE = os.path.join(ROOT, "profiles", "trace_gdn_step_720p.json")
KERNEL_SRC = os.path.join(ROOT, "gated_deltanet_streaming_amd", "csrc", "gdn_kernels.hip")
ATTN_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_attn_720p.json")
ATTN_TRACE_FILE = os.path.join(ROOT, "profiles", "trace_attn_720p.json")
ATTN_KERNEL_SRC = os.path.join(ROOT, "gated_deltanet_streaming_amd", "csrc", "gdn_attention.hip")
LOWP_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm_e4m3_720p.json")
LOWP_TRACE_FILE = os.path.join(ROOT, "profiles", "trace_gemm_e4m3_720p.json")
LOWP_KERNEL_SRC = os.path.join(ROOT, "gated_deltanet_streaming_amd", "csrc", "gdn_lowp.hip")
MFMA_FP8_PEAK_TFLOPS = 5000.0    # dense fp8
KERNEL_NAMES = ("gdn_prep_kernel", "gdn_scan_kernel", "attn_kernel", "attn_append_kernel", "gemm_e4m3_kernel",
                "quantize_rows_vec_kernel", "quantize_rows_kernel")


def kernel_source_hash(src: str = KERNEL_SRC) -> str:
    with open(src, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def algorithmic_bytes(mode: str, t: int = T) -> int:
    """Bytes a whole step (forward with carried state + reverse) must move at least."""
    if mode in ("bidir", "long"):
        return B * t * H * BIDIR_BYTES_PER_TOKEN_HEAD + 2 * STATE_BYTES
    per_scan = B * t * H * BYTES_PER_TOKEN_HEAD
    return 2 * per_scan + 2 * STATE_BYTES


def kernel_byte_shares(t: int = T) -> dict:
    """The algorithmic bytes of one bidirectional call split between its two kernels: the prep
    reads q, k (bf16) and a, beta (fp32); the scan reads v and the carried state and writes o,
    o_rev and the state.  The shares add up to algorithmic_bytes("bidir", t)."""
    prep = B * t * H * (2 * D * 2 + 2 * 4)
    scan = B * t * H * (3 * D * 2) + 2 * STATE_BYTES
    return {"gdn_prep_kernel": prep, "gdn_scan_kernel": scan}


def _load_record(path: str, src: str = KERNEL_SRC):
    """A committed rocprofv3 summary record, if it was taken on the current kernel source."""
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != kernel_source_hash(src):
        return None
    return rec


def load_traffic(path: str = TRAFFIC_FILE, src: str = KERNEL_SRC):
    """HBM bytes per dispatch of each kernel from the committed FETCH_SIZE / WRITE_SIZE runs,
    {kernel: bytes}, if they were taken on the current kernel source; else None."""
    rec = _load_record(path, src)
    if rec is None:
        return None
    return {k: v["bytes_per_dispatch"] for k, v in rec["kernels"].items()}


def load_trace(path: str = TRACE_FILE, src: str = KERNEL_SRC):
    """Average duration (us) of each kernel in the committed kernel trace, if it was taken on the
    current kernel source; else None."""
    rec = _load_record(path, src)
    if rec is None:
        return None
    return {k: v["average_us"] for k, v in rec["kernels"].items()}


def _short_kernel_name(name: str) -> str:
    for k in KERNEL_NAMES:
        if k in name:
            return k
    return name


def summarize_rocprof(kind: str, dirs, out_path: str, src: str) -> None:
    """Write the committed summary record of rocprofv3 csv output.

    kind "traffic": dirs = (FETCH_SIZE run, WRITE_SIZE run) of a bench run with --copy-probe; the
    counters of each kernel (median over its dispatches, KiB) are scaled by what the same counter
    reads for the 256 MiB device copy (bytes read, bytes written).  kind "trace": dirs = (trace
    run,); the kernel_stats average of each kernel."""
    import csv
    import glob
    import statistics

    def rows(d, pattern):
        files = glob.glob(os.path.join(d, "**", pattern), recursive=True)
        if not files:
            raise SystemExit(f"no {pattern} under {d}")
        out = []
        for fn in files:
            with open(fn) as f:
                out.extend(csv.DictReader(f))
        return out

    rec = {"kernel_source_sha256_16": kernel_source_hash(src), "kernels": {}}
    if kind == "trace":
        for r in rows(dirs[0], "*kernel_stats.csv"):
            k = _short_kernel_name(r["Name"])
            if k in KERNEL_NAMES:
                rec["kernels"][k] = {"calls": int(r["Calls"]), "average_us": round(float(r["AverageNs"]) / 1e3, 3),
                                     "min_us": round(float(r["MinNs"]) / 1e3, 3),
                                     "max_us": round(float(r["MaxNs"]) / 1e3, 3)}
    else:
        per = {}
        copy_bytes = 256 * 1024 * 1024
        for d, counter in zip(dirs, ("FETCH_SIZE", "WRITE_SIZE")):
            vals = {}
            for r in rows(d, "*counter_collection.csv"):
                if r["Counter_Name"] != counter:
                    continue
                vals.setdefault((r["Kernel_Name"], r["Dispatch_Id"]), 0.0)
                vals[(r["Kernel_Name"], r["Dispatch_Id"])] += float(r["Counter_Value"])
            by_kernel = {}
            for (name, _), v in vals.items():
                by_kernel.setdefault(name, []).append(v)
            copy = [statistics.median(v) for n, v in by_kernel.items() if "copyBuffer" in n]
            if not copy:
                raise SystemExit(f"{counter}: no copy-probe dispatch in {d} (run the bench with --copy-probe)")
            # the copy reads and writes copy_bytes: scale = bytes per counter unit (KiB)
            rec[f"{counter.lower()}_scale_bytes_per_unit"] = copy_bytes / copy[0]
            rec[f"copy_probe_{counter}_KiB"] = copy[0]
            for n, v in by_kernel.items():
                k = _short_kernel_name(n)
                if k in KERNEL_NAMES:
                    per.setdefault(k, {})[counter] = (statistics.median(v), len(v))
        for k, c in per.items():
            f_kib, n = c.get("FETCH_SIZE", (0.0, 0))
            w_kib, _ = c.get("WRITE_SIZE", (0.0, 0))
            rec["kernels"][k] = {"dispatches": n, "fetch_KiB": f_kib, "write_KiB": w_kib,
                                 "bytes_per_dispatch": int(f_kib * rec["fetch_size_scale_bytes_per_unit"]
                                                           + w_kib * rec["write_size_scale_bytes_per_unit"])}
    with open(out_path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


def cpu_baseline(d, threads, t=T):
    import oracle
    oracle.build(force=False)

    def rate(nthreads, budget_s, max_reps):
        reps, t0 = 0, time.perf_counter()
        while reps < max_reps and (reps < 1 or time.perf_counter() - t0 < budget_s):
            oracle.forward(d["q"], d["k"], d["v"], d["a"], d["beta"], d["S0"], threads=nthreads)
            oracle.reverse(d["q"], d["k"], d["v"], d["a"], d["beta"], threads=nthreads)
            reps += 1
        return reps, (time.perf_counter() - t0) / reps

    reps, dt = rate(threads, 12.0, 500)
    reps1, dt1 = rate(1, 3.0, 4)
    return {"value": round(t / dt, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"the full workload, {reps} repeats: forward + reverse fp64 scans of B={B} H={H} "
                      f"d={D} T={t} ({dt:.3f} s per step)",
            "single_core": {"value": round(t / dt1, 1), "cores": 1,
                            "sample": f"the same step on one thread, {reps1} repeats ({dt1:.3f} s per step)"}}


def measured_peaks(torch, dev):
    """A 1 GiB device-to-device copy (512 MiB read + 512 MiB written, beyond the 256 MB MALL) and a
    dense bf16 MFMA loop (two wavefronts per SIMD), both hand-written HIP in libgdn_peaks.so."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "gated_deltanet_streaming_amd", "libgdn_peaks.so"))
    lib.gdn_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_void_p, ctypes.POINTER(ctypes.c_float)]
    lib.gdn_peak_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_double)]
    stream = torch.cuda.current_stream(dev).cuda_stream
    half = 512 * 1024 * 1024
    src = torch.empty(half, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1)
    copy_gbs = {}
    for form, name in ((0, "grid_stride"), (1, "one_vector_per_thread")):
        ms = ctypes.c_float()
        if lib.gdn_peak_copy(src.data_ptr(), dst.data_ptr(), half, 20, form, stream, ctypes.byref(ms)) != 0:
            raise RuntimeError("copy probe failed")
        copy_gbs[name] = round(2 * half / (ms.value * 1e-3) / 1e9, 1)
    best = max(copy_gbs.values())
    del src, dst
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    blocks = 2 * cus
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    mms, flops = ctypes.c_float(), ctypes.c_double()
    if lib.gdn_peak_mfma_bf16(blocks, 2000, 10, out.data_ptr(), stream, ctypes.byref(mms), ctypes.byref(flops)) != 0:
        raise RuntimeError("MFMA probe failed")
    torch.cuda.synchronize()
    tflops = flops.value / (mms.value * 1e-3) / 1e12
    return {"hbm_copy_GBs": best, "hbm_copy_frac_of_vendor": round(best / HBM_PEAK_GBS, 4), "hbm_copy_forms": copy_gbs,
            "mfma_bf16_TFLOPs": round(tflops, 1), "mfma_bf16_frac_of_vendor": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "compute_units": cus,
            "how": "copy: 1 GiB moved per launch (read + write), average of 20, the better of two kernel forms; "
                   "MFMA: 16x16x32 bf16, 8 independent "
                   "chains per wavefront, 2 wavefronts per SIMD, average of 10 launches"}


def measured_peaks_lowp(torch, dev):
    """A dense fp8 (E4M3) MFMA loop (two wavefronts per SIMD) and the LDS read rate of 16-byte reads (eight
    wavefronts per CU, no bank conflicts), both hand-written HIP in libgdn_peaks.so: the MFMA rate the fp8
    GEMM is quoted against, and the LDS rate that bounds it."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "gated_deltanet_streaming_amd", "libgdn_peaks.so"))
    for fn in (lib.gdn_peak_mfma_fp8, lib.gdn_peak_lds_read):
        fn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                       ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_double)]
    stream = torch.cuda.current_stream(dev).cuda_stream
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    out = torch.empty(2 * cus * 512, dtype=torch.float32, device=dev)
    ms, amount = ctypes.c_float(), ctypes.c_double()
    if lib.gdn_peak_mfma_fp8(2 * cus, 2000, 10, out.data_ptr(), stream, ctypes.byref(ms), ctypes.byref(amount)) != 0:
        raise RuntimeError("fp8 MFMA probe failed")
    fp8 = amount.value / (ms.value * 1e-3) / 1e12
    if lib.gdn_peak_lds_read(cus, 2000, 10, out.data_ptr(), stream, ctypes.byref(ms), ctypes.byref(amount)) != 0:
        raise RuntimeError("LDS probe failed")
    torch.cuda.synchronize()
    lds = amount.value / (ms.value * 1e-3)
    return {"mfma_fp8_TFLOPs": round(fp8, 1), "mfma_fp8_frac_of_vendor": round(fp8 / MFMA_FP8_PEAK_TFLOPS, 4),
            "lds_read_GBs_per_cu": round(lds / cus / 1e9, 1),
            "lds_read_bytes_per_clock_per_cu_at_2400MHz": round(lds / cus / 2.4e9, 1), "compute_units": cus,
            "how": "fp8: 16x16x128 E4M3 MFMAs, 8 independent chains per wavefront, 2 wavefronts per SIMD; LDS: 16-byte "
                   "reads of 1 KB contiguous per wavefront instruction, 8 wavefronts per CU, one workgroup per CU"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--mode", choices=["bidir", "separate", "long", "backward", "attention", "lowp", "split"], default="bidir",
                    help="bidir: one gdn_chunk_bidir call per step; separate: forward then reverse calls; "
                         "long: gdn_chunk_bidir on a 21-frame clip (T = 18480); "
                         "backward: the gradients of both scans of the pair (gdn_chunk_backward); "
                         "attention: the softmax block's sink + window attention (gdn_attn_chunk); "
                         "lowp: the GDN block's fused q/k/v projection as an E4M3 GEMM (gdn_quantize_rows_e4m3 + "
                         "gdn_gemm_e4m3); "
                         "split: the forward scan of a 21-frame clip with few stream-heads, plain "
                         "(gdn_chunk_forward) against the time split (gdn_chunk_forward_split)")
    ap.add_argument("--split-heads", type=int, default=1, help="heads of the split mode's single stream")
    ap.add_argument("--sets", type=int, default=6, help="rotating input/output buffer sets (1 = warm)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-peaks", action="store_true", help="skip the copy / MFMA peak probes")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a 256 MiB device copy (reference for counter scaling)")
    ap.add_argument("--summarize", nargs="+", metavar=("KIND", "DIR"),
                    help="no GPU run: write the committed summary record of rocprofv3 csv output; "
                         "'traffic FETCH_DIR WRITE_DIR [attn|lowp]' or 'trace TRACE_DIR [attn|lowp]'")
    args = ap.parse_args()

    if args.summarize:
        kind, rest = args.summarize[0], args.summarize[1:]
        tag = rest[-1] if rest and rest[-1] in ("attn", "lowp") else None
        dirs = rest[:-1] if tag else rest
        if kind not in ("traffic", "trace") or len(dirs) != (2 if kind == "traffic" else 1):
            raise SystemExit("--summarize traffic FETCH_DIR WRITE_DIR [attn|lowp] | trace TRACE_DIR [attn|lowp]")
        if tag == "attn":
            out = ATTN_TRAFFIC_FILE if kind == "traffic" else ATTN_TRACE_FILE
            src = ATTN_KERNEL_SRC
        elif tag == "lowp":
            out = LOWP_TRAFFIC_FILE if kind == "traffic" else LOWP_TRACE_FILE
            src = LOWP_KERNEL_SRC
        else:
            out, src = (TRAFFIC_FILE if kind == "traffic" else TRACE_FILE), KERNEL_SRC
        return summarize_rocprof(kind, dirs, out, src)

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (this path needs no "
              "multi-GPU exchange; see the sharding notes).", file=sys.stderr)
        sys.exit(2)

    if args.mode == "backward":
        return main_backward(args)
    if args.mode == "attention":
        return main_attention(args)
    if args.mode == "lowp":
        return main_lowp(args)
    if args.mode == "split":
        return main_split(args)

    import numpy as np
    import torch

    import gdn_inputs
    from gated_deltanet_streaming_amd import binding as gb

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t_run = T_LONG if args.mode == "long" else T
    nsets = min(args.sets, 3) if args.mode == "long" else args.sets   # 3 long sets: 620 MB live
    d = gdn_inputs.batch(1, B, t_run, H, D, with_state=True)

    sets = []
    for i in range(nsets):
        # distinct values per set (the first set is the seeded workload itself)
        di = d if i == 0 else gdn_inputs.batch(1, B, t_run, H, D, chunk=i)
        qi = {k: torch.from_numpy(di[k]).to(dev, torch.bfloat16) for k in ("q", "k", "v")}
        qi["a"] = torch.from_numpy(di["a"]).to(dev)
        qi["beta"] = torch.from_numpy(di["beta"]).to(dev)
        qi["o"] = torch.empty_like(qi["v"])
        qi["o_rev"] = torch.empty_like(qi["v"])
        sets.append(qi)

    s = gb.Stream(B, H, D, D, t_run, device=0)
    s.state_set(torch.from_numpy(d["S0"]).to(dev))
    stream = torch.cuda.current_stream(dev)

    def step(i):
        x = sets[i % len(sets)]
        if args.mode in ("bidir", "long"):
            s.bidir(x["q"], x["k"], x["v"], x["a"], x["beta"], x["o"], x["o_rev"], stream=stream)
        else:
            s.forward(x["q"], x["k"], x["v"], x["a"], x["beta"], x["o"], stream=stream)
            s.reverse(x["q"], x["k"], x["v"], x["a"], x["beta"], x["o_rev"], stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: exactly `steps` steps, no per-kernel events
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_events = e0.elapsed_time(e1)
    ms_per_step = wall * 1e3 / args.steps
    print(f"# timed {args.steps} steps: wall {wall * 1e3:.3f} ms, events {ms_events:.3f} ms", file=sys.stderr,
          flush=True)

    # per-call distribution: events around every step (a separate pass, so the timed
    # region above carries no per-step events)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        evs[i][0].record(stream)
        step(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    per_call = np.array([a.elapsed_time(b) for a, b in evs])
    p10, p50, p90 = (float(x) for x in np.percentile(per_call, [10, 50, 90]))

    # warm: the same buffer set every step
    torch.cuda.synchronize()
    w1 = time.perf_counter()
    for i in range(args.steps):
        step(0)
    torch.cuda.synchronize()
    warm_ms = (time.perf_counter() - w1) * 1e3 / args.steps

    # second pass over the same steps with per-kernel HIP events on the launch stream
    gb.gdn_profile(s.handle, True)
    gb.gdn_profile_read(s.handle, reset=True)
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    prof = gb.gdn_profile_read(s.handle, reset=True)
    gb.gdn_profile(s.handle, False)
    scan_ms, scan_n = prof["scan"]
    prep_ms, prep_n = prof["prep"]
    scan_avg_ms = scan_ms / max(scan_n, 1)
    prep_avg_ms = prep_ms / max(prep_n, 1)

    if args.copy_probe:
        src = torch.empty(64 * 1024 * 1024, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    alg_bytes = algorithmic_bytes(args.mode, t_run)
    launches_per_step = scan_n / args.steps
    step_gbs = alg_bytes / (ms_per_step * 1e-3) / 1e9
    flops = 2 * B * t_run * H * FLOPS_PER_TOKEN_HEAD
    headline = args.mode == "bidir" and args.sets >= 6
    # the committed trace and counter records describe the headline run only
    traffic = load_traffic() if headline else None
    trace = load_trace() if headline else None
    kernels = {}
    if args.mode in ("bidir", "long"):
        for k, share in kernel_byte_shares(t_run).items():
            ev_ms = prep_avg_ms if k == "gdn_prep_kernel" else scan_avg_ms
            kernels[k] = {
                "algorithmic_bytes": share,
                "avg_us_events": round(ev_ms * 1e3, 3),
                "achieved_GBs_events": round(share / (ev_ms * 1e-3) / 1e9, 1),
                "avg_us_trace": trace.get(k) if trace else None,
                "traffic": traffic.get(k) if traffic else None,
            }
    step_traffic = sum(v["traffic"] for v in kernels.values()) if traffic and kernels else None

    out = {
        "metric": METRIC,
        "value": round(t_run / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": ("21-frame clip (18480 tokens), one GDN layer: forward scan from the carried state + "
                         "reverse scan" if args.mode == "long" else
                         "720p streaming chunk, one GDN layer: forward scan from the carried state + "
                         "intra-chunk reverse scan"),
            "B": B, "H": H, "d_k": D, "d_v": D, "T": t_run, "subchunk": 64,
            "call": "gdn_chunk_forward + gdn_chunk_reverse" if args.mode == "separate" else "gdn_chunk_bidir",
            "buffers": f"{nsets} rotating sets ({'cold: live set > 256 MB MALL' if nsets * t_run >= 6 * T else 'warm'})",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(step_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(step_gbs / HBM_PEAK_GBS, 4),
            "traffic": step_traffic,
            "kernel": "step: gdn_prep_kernel + gdn_scan_kernel",
            "algorithmic_bytes_per_step": alg_bytes,
            "kernels": kernels,
            "note": "achieved = algorithmic bytes of the step / ms_per_step; traffic = the kernels' scaled "
                    "FETCH_SIZE + WRITE_SIZE per dispatch from the committed counter runs",
        },
        "step_detail": {
            "mfma_bf16_frac": round(flops / (ms_per_step * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 5),
            "launches_per_step": launches_per_step,
            "event_ms_per_step": round(ms_events / args.steps, 5),
            "per_call_ms_p10_p50_p90": [round(p10, 5), round(p50, 5), round(p90, 5)],
            "warm_ms_per_step": round(warm_ms, 5),
            "target_tokens_per_s": 108e6 if args.mode == "bidir" else None,
        },
    }
    if not args.no_peaks:
        out["measured_peaks"] = measured_peaks(torch, dev)
    if not args.no_cpu:
        # the host share of one GPU: OMP_NUM_THREADS when set (16 on the GPU machines), else the affinity mask
        threads = min(len(os.sched_getaffinity(0)), int(os.environ.get("OMP_NUM_THREADS", "0")) or 1 << 30)
        out["cpu_baseline"] = cpu_baseline(d, threads, t_run)
    s.close()
    print(json.dumps(out), flush=True)


def main_split(args):
    """The causal forward scan of the 21-frame clip (T = 18480, 289 steps of 64 tokens) for one stream
    of `--split-heads` heads of 112: the plain call against the time split at several segment
    counts.  Every call starts from the same cached state (GDN_NO_COMMIT); inputs resident in HBM."""
    import numpy as np
    import torch

    import gdn_inputs
    import oracle
    from gated_deltanet_streaming_amd import binding as gb

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    Hs, t_run = args.split_heads, T_LONG
    d = gdn_inputs.batch(1, 1, t_run, Hs, D, with_state=True)
    x = {k: torch.from_numpy(d[k]).to(dev, torch.bfloat16) for k in ("q", "k", "v")}
    x["a"] = torch.from_numpy(d["a"]).to(dev)
    x["beta"] = torch.from_numpy(d["beta"]).to(dev)
    o = torch.empty_like(x["v"])
    s = gb.Stream(1, Hs, D, D, t_run, device=0)
    s.state_set(torch.from_numpy(d["S0"]).to(dev))
    stream = torch.cuda.current_stream(dev)

    def call(seg):
        if seg == 1:
            s.forward(x["q"], x["k"], x["v"], x["a"], x["beta"], o, flags=gb.GDN_NO_COMMIT, stream=stream)
        else:
            s.forward_split(x["q"], x["k"], x["v"], x["a"], x["beta"], o, seg, flags=gb.GDN_NO_COMMIT, stream=stream)

    steps = max(args.steps // 4, 10)
    by_seg = {}
    for seg in (1, 4, 8, 16, 32, 48, 72):
        for _ in range(max(args.warmup // 4, 3)):
            call(seg)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            call(seg)
        e1.record(stream)
        torch.cuda.synchronize()
        by_seg[seg] = e0.elapsed_time(e1) / steps
    best = min((v, k) for k, v in by_seg.items() if k > 1)
    ms, seg_best = best
    alg = Hs * (t_run * (3 * 2 * D + 2 * D + 8) + 2 * D * D * 4)
    out = {
        "metric": "GDN causal forward scan tokens/s, one stream, few heads, 21-frame clip (time split)",
        "value": t_run / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": max(args.warmup // 4, 3), "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "21-frame clip, one stream, forward scan from a carried state", "B": 1, "H": Hs,
                   "d_k": D, "d_v": D, "T": t_run, "subchunk": 64, "call": "gdn_chunk_forward_split",
                   "segments": seg_best},
        "plain_ms": by_seg[1], "speedup_vs_plain": by_seg[1] / ms,
        "ms_by_segments": {str(k): round(v, 4) for k, v in by_seg.items()},
        "roofline": {"bound": "hbm", "achieved": alg / (ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "traffic": None,
                     "note": "algorithmic bytes of the forward scan (q, k, v, o, gates, the state in and out) / call time"},
    }
    if not args.no_cpu:
        oracle.build(force=False)
        threads = min(16, os.cpu_count() or 1)
        reps, t0 = 0, time.perf_counter()
        while reps < 3 or time.perf_counter() - t0 < 5.0:
            oracle.forward(d["q"], d["k"], d["v"], d["a"], d["beta"], d["S0"], threads=threads)
            reps += 1
        per = (time.perf_counter() - t0) / reps
        out["cpu_baseline"] = {"value": round(t_run / per, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
                               "sample": f"the full workload, {reps} repeats of the fp64 forward scan ({per:.3f} s each)"}
    print(json.dumps(out), flush=True)


def main_backward(args):
    """Gradients of both scans of the 720p pair (forward from the carried state, reverse from
    zero) in one gdn_chunk_backward_bidir call: a token-sequential fp32 path, bound by its serial chain
    of T steps per (head, row block), reported against the HBM roofline of its bytes."""
    import numpy as np
    import torch

    import gdn_inputs
    from gated_deltanet_streaming_amd import binding as gb

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d = gdn_inputs.batch(1, B, T, H, D, with_state=True)
    rng = np.random.default_rng(2)
    x = {k: torch.from_numpy(d[k]).to(dev, torch.bfloat16) for k in ("q", "k", "v")}
    a = torch.from_numpy(d["a"]).to(dev)
    beta = torch.from_numpy(d["beta"]).to(dev)
    S0 = torch.from_numpy(d["S0"]).to(dev)
    dO = [torch.from_numpy(rng.standard_normal((B, T, H, D)).astype(np.float32)).to(dev, torch.bfloat16) for _ in range(2)]
    dSf = torch.from_numpy(rng.standard_normal((B, H, D, D)).astype(np.float32)).to(dev)
    s = gb.Stream(B, H, D, D, T, device=0)
    stream = torch.cuda.current_stream(dev)

    gf, gr = s._grad_buffers(x["q"], x["v"]), s._grad_buffers(x["q"], x["v"])

    def step():
        gb.gdn_chunk_backward_bidir(s.handle, x["q"], x["k"], x["v"], a, beta, dO[0], dO[1], gf, gr, d_state=dSf,
                                    state0=S0, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - w0) * 1e3 / args.steps
    gb.gdn_profile(s.handle, True)
    gb.gdn_profile_read(s.handle, reset=True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    prof = gb.gdn_profile_read(s.handle, reset=True)
    gb.gdn_profile(s.handle, False)
    bwd_ms, bwd_n = prof["backward"]
    launch_ms = bwd_ms / max(bwd_n, 1)
    # per scan and token-head: q, k, v, d_o read (bf16), a and beta read, dq, dk, dv written (fp32),
    # da and dbeta written; per scan and head: start state, final-state gradient and start-state
    # gradient (fp32) for the forward scan, the start-state gradient for the reverse one
    per_tok = 4 * D * 2 + 2 * 4 + 3 * D * 4 + 2 * 4
    alg_bytes = 2 * B * T * H * per_tok + 4 * B * H * D * D * 4
    # one timed launch pair (rows + reduce) computes both scans' gradients
    achieved = alg_bytes / (launch_ms * 1e-3) / 1e9
    out = {
        "metric": "GDN backward (gradients of the forward and reverse scans) tokens/s per layer at 2640-token 720p chunk",
        "value": round(T / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": "720p streaming chunk, one GDN layer: gradients of the forward scan (carried "
                               "state) and of the intra-chunk reverse scan", "B": B, "H": H, "d_k": D, "d_v": D,
                   "T": T, "call": "gdn_chunk_backward_bidir", "path": "token-sequential fp32"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 5), "traffic": None, "kernel": "gdn_bwd_rows_kernel + "
                     "gdn_bwd_reduce_kernel", "kernel_avg_us": round(launch_ms * 1e3, 1),
                     "algorithmic_bytes_per_launch": int(alg_bytes),
                     "note": "latency-bound by the serial chain of T tokens per (head, 4-row block)"},
    }
    if not args.no_cpu:
        import oracle
        oracle.build(force=False)
        hs = 2   # bounded sample: 2 of the H heads, the full 2640 tokens, both scans
        sl = {k: d[k][:, :, :hs] for k in ("q", "k", "v", "a", "beta")}
        dOs = [t[:, :, :hs].float().cpu().numpy() for t in dO]
        threads = min(len(os.sched_getaffinity(0)), hs)
        t0 = time.perf_counter()
        oracle.backward(sl["q"], sl["k"], sl["v"], sl["a"], sl["beta"], dOs[0], d["S0"][:, :hs],
                        dSf[:, :hs].cpu().numpy(), threads=threads)
        oracle.backward(sl["q"], sl["k"], sl["v"], sl["a"], sl["beta"], dOs[1], None, None, reverse=True,
                        threads=threads)
        dt = (time.perf_counter() - t0) * H / hs
        out["cpu_baseline"] = {"value": round(T / dt, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
                               "sample": f"{hs} of {H} heads, full {T} tokens, both scans' gradients, scaled "
                                         f"to {H} heads ({dt:.1f} s per step)"}
    s.close()
    print(json.dumps(out), flush=True)


ATTN_SINK, ATTN_WINDOW = 880, 2640   # one latent frame of sink, one chunk of window


def main_attention(args):
    """The softmax block of the hybrid DiT at the 720p layer shape in steady state: every step
    is one committed gdn_attn_chunk call on a 2640-token chunk whose queries attend over
    880 sink + 2640 window + 2640 chunk = 6160 keys (attention kernel plus cache append),
    reported against the bf16 MFMA roofline of its algorithmic flops."""
    import numpy as np
    import torch

    import gdn_inputs
    from gated_deltanet_streaming_amd import binding as gb

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    nsets = max(1, args.sets)
    sets = []
    for i in range(nsets):
        d = gdn_inputs.attn_chunk(i, B, T, H, D)
        sets.append([torch.from_numpy(d[k]).to(dev, torch.bfloat16) for k in ("q", "k", "v")])
    outs = [torch.empty((B, T, H, D), dtype=torch.bfloat16, device=dev) for _ in range(nsets)]
    att = gb.WindowAttention(B, H, D, ATTN_SINK, ATTN_WINDOW, T, device=0)
    stream = torch.cuda.current_stream(dev)
    for i in range(2):                       # fill the sink and the window
        att.chunk(*sets[i % nsets], outs[0], stream=stream)
    L = ATTN_SINK + ATTN_WINDOW + T
    n = [0]

    def step():
        i = n[0] % nsets
        n[0] += 1
        att.chunk(*sets[i], outs[i], stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert att.cache_len() == (ATTN_SINK, ATTN_WINDOW)
    w0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - w0) * 1e3 / args.steps
    gb.gdn_attn_profile(att.handle, True)
    gb.gdn_attn_profile_read(att.handle, reset=True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    k_ms, k_n = gb.gdn_attn_profile_read(att.handle, reset=True)
    gb.gdn_attn_profile(att.handle, False)
    if args.copy_probe:   # a 256 MiB device copy: the reference that scales the byte counters
        src = torch.empty(64 * 1024 * 1024, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    launch_ms = k_ms / max(k_n, 1)
    flops = 4.0 * B * H * T * L * D          # q.k and p.v, 2 flops per multiply-add
    achieved = flops / (launch_ms * 1e-3) / 1e12
    out = {
        "metric": "softmax-block (sink + window attention) tokens/s per layer at 2640-token 720p chunk",
        "value": round(T / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "720p streaming chunk, one softmax block in steady state: 2640 queries over "
                               "880 sink + 2640 window + 2640 chunk keys", "B": B, "H": H, "d": D, "T": T,
                   "sink": ATTN_SINK, "window": ATTN_WINDOW, "keys": L, "call": "gdn_attn_chunk (commit)"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": (load_traffic(ATTN_TRAFFIC_FILE, ATTN_KERNEL_SRC) or {}).get("attn_kernel"),
                     "kernel": "attn_kernel", "kernel_avg_us": round(launch_ms * 1e3, 1),
                     "algorithmic_flops_per_launch": flops},
    }
    if not args.no_cpu:
        from oracle.window_attn import SinkWindowAttention
        import threadpoolctl
        hs = H   # the whole steady-state chunk (about 73 GFLOP in fp64: seconds on the host)
        ref = SinkWindowAttention(ATTN_SINK, ATTN_WINDOW)
        for i in range(2):
            d = gdn_inputs.attn_chunk(i, B, T, H, D)
            ref.chunk(d["q"][:, :1, :hs], d["k"][:, :, :hs], d["v"][:, :, :hs])
        d = gdn_inputs.attn_chunk(2, B, T, H, D)
        reps, t0 = 0, time.perf_counter()
        while reps == 0 or time.perf_counter() - t0 < 10.0:   # about 10 s of host work, uncommitted calls
            ref.chunk(d["q"][:, :, :hs], d["k"][:, :, :hs], d["v"][:, :, :hs], commit=False)
            reps += 1
        dt = (time.perf_counter() - t0) / reps * H / hs
        blas = [p["num_threads"] for p in threadpoolctl.threadpool_info() if p.get("user_api") == "blas"]
        out["cpu_baseline"] = {"value": round(T / dt, 1), "unit": "tokens/s",
                               "cores": max(blas) if blas else 1, "kind": "oracle",
                               "sample": f"{hs} of {H} heads of one steady-state chunk ({L} keys), numpy fp64 "
                                         f"matmuls, {reps} repetitions ({dt:.2f} s per step)"}
    att.close()
    print(json.dumps(out), flush=True)


def main_lowp(args):
    """The GDN block's fused q/k/v projection at the 720p layer shape as an FP8 (E4M3) GEMM: X [2640 tokens x
    2240] bf16 times W [6720 = 3 x 2240 features x 2240]^T, weights quantised once beforehand (as a deployed model
    stores them).  One step = per-token quantisation of X (gdn_quantize_rows_e4m3) + the GEMM (gdn_gemm_e4m3),
    bf16 out.  The roofline is the GEMM kernel's: 2 M N K flops per launch against the dense fp8 peak."""
    import numpy as np
    import torch

    import gdn_inputs
    from gated_deltanet_streaming_amd import binding as gb

    M, K, N = T, H * D, 3 * H * D
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    nsets = max(1, args.sets)
    xs, ys = [], []
    x0, w = gdn_inputs.proj_inputs(0, M, K, N)
    for i in range(nsets):
        xi = x0 if i == 0 else gdn_inputs.proj_inputs(i, M, K, N)[0]
        xs.append(torch.from_numpy(xi.astype(np.float32)).to(dev, torch.bfloat16))
        ys.append(torch.empty((M, N), dtype=torch.bfloat16, device=dev))
    wq, ws = gb.quantize_rows_e4m3(torch.from_numpy(w.astype(np.float32)).to(dev, torch.bfloat16))
    xq = [gb.e4m3_codes_empty(M, K, dev) for _ in range(nsets)]
    xsc = [torch.empty(M, dtype=torch.float32, device=dev) for _ in range(nsets)]
    stream = torch.cuda.current_stream(dev)
    n = [0]

    def step():
        i = n[0] % nsets
        n[0] += 1
        gb.quantize_rows_e4m3(xs[i], codes=xq[i], scales=xsc[i], stream=stream)
        gb.gemm_e4m3(xq[i], xsc[i], wq, ws, ys[i], stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - w0) * 1e3 / args.steps
    # the GEMM kernel alone, HIP events on its launch stream (the current stream)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for j in range(args.steps):
        gb.gemm_e4m3(xq[j % nsets], xsc[j % nsets], wq, ws, ys[j % nsets], stream=stream)
    ev1.record(stream)
    ev1.synchronize()
    gemm_ms = ev0.elapsed_time(ev1) / args.steps
    ev0.record(stream)
    for j in range(args.steps):
        gb.quantize_rows_e4m3(xs[j % nsets], codes=xq[j % nsets], scales=xsc[j % nsets], stream=stream)
    ev1.record(stream)
    ev1.synchronize()
    quant_ms = ev0.elapsed_time(ev1) / args.steps
    if args.copy_probe:   # a 256 MiB device copy: the reference that scales the byte counters
        src = torch.empty(64 * 1024 * 1024, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    flops = 2.0 * M * N * K
    achieved = flops / (gemm_ms * 1e-3) / 1e12
    quant_bytes = M * K * 2 + M * K + M * 4            # bf16 X read, codes and scales written
    gemm_bytes = M * K + N * K + (M + N) * 4 + M * N * 2   # codes and scales read once, bf16 Y written
    traffic = load_traffic(LOWP_TRAFFIC_FILE, LOWP_KERNEL_SRC) or {}
    trace = load_trace(LOWP_TRACE_FILE, LOWP_KERNEL_SRC) or {}
    out = {
        "metric": "GDN block q/k/v projection tokens/s at 2640-token 720p chunk (E4M3 GEMM); % of fp8 MFMA roofline",
        "value": round(M / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8-e4m3 (fp32 accumulate, bf16 out)", "data": "synthetic",
        "config": {"workload": "720p streaming chunk, the GDN block's fused q/k/v projection: 2640 tokens x 2240 "
                               "in, 6720 out", "M": M, "K": K, "N": N,
                   "call": "gdn_quantize_rows_e4m3 (activations) + gdn_gemm_e4m3; weights quantised once"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_FP8_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_FP8_PEAK_TFLOPS, 4),
                     "traffic": traffic.get("gemm_e4m3_kernel"),
                     "kernel": "gemm_e4m3_kernel", "kernel_avg_us": round(gemm_ms * 1e3, 2),
                     "trace_avg_us": trace.get("gemm_e4m3_kernel"),
                     "algorithmic_flops_per_launch": flops, "algorithmic_bytes_per_launch": gemm_bytes,
                     "quantize": {"kernel": "quantize_rows_vec_kernel", "kernel_avg_us": round(quant_ms * 1e3, 2),
                                  "trace_avg_us": trace.get("quantize_rows_vec_kernel"),
                                  "algorithmic_bytes_per_launch": quant_bytes, "bound": "hbm",
                                  "achieved_GBs": round(quant_bytes / (quant_ms * 1e-3) / 1e9, 1),
                                  "traffic": traffic.get("quantize_rows_vec_kernel")}},
    }
    if not args.no_peaks:
        out["measured_peaks"] = measured_peaks_lowp(torch, dev)
    if not args.no_cpu:
        from oracle import lowp_gemm
        import threadpoolctl
        rows = 512   # a bounded sample: 512 of the 2640 tokens against the whole weight
        xr = x0[:rows].astype(np.float32)
        wcodes, wscales = lowp_gemm.quantize_rows(w.astype(np.float32))
        reps, t0 = 0, time.perf_counter()
        while reps == 0 or time.perf_counter() - t0 < 10.0:
            c, sc = lowp_gemm.quantize_rows(xr)
            lowp_gemm.bf16_round(lowp_gemm.gemm_e4m3(c, sc, wcodes, wscales))
            reps += 1
        dt = (time.perf_counter() - t0) / reps
        blas = [p["num_threads"] for p in threadpoolctl.threadpool_info() if p.get("user_api") == "blas"]
        out["cpu_baseline"] = {"value": round(rows / dt, 1), "unit": "tokens/s",
                               "cores": max(blas) if blas else 1, "kind": "oracle",
                               "sample": f"{rows} of {M} tokens: per-row quantisation + fp64 GEMM of the decoded "
                                         f"codes against all {N} features, {reps} repetitions ({dt:.2f} s each)"}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
