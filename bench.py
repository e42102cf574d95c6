"""Throughput of the GDN streaming core on one MI355X.

Workload: one GDN layer on one 720p streaming chunk -- B=1 stream, H=20 heads,
d_k = d_v = 112, T = 2640 tokens (3 latent frames x 22 x 40 tokens), bf16
q/k/v/o, fp32 gates and state.  One step = the forward scan from the carried
state (committed back to the cache) plus the reverse scan inside the chunk.
Inputs are synthetic (seeded) and already resident in HBM; by default they
rotate over enough buffer sets that the live set exceeds the 256 MB MALL, so
every step streams from HBM.

Prints one JSON line.  `value` is tokens per second per layer (T / step time).
`roofline` is for the dominant kernel (the chunk scan): the algorithmic bytes of
the call it serves over its average duration from HIP events recorded on its
launch stream.  Algorithmic bytes per token-head: q, k, v read once and o
written (224 B each in bf16) plus the two fp32 gates; a bidirectional call also
writes o_rev; the forward scan reads and writes the 112x112 fp32 state of each
head once.
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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_scan_720p.json")
KERNEL_SRC = os.path.join(ROOT, "gated_deltanet_streaming_amd", "csrc", "gdn_kernels.hip")
ATTN_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_attn_720p.json")
ATTN_KERNEL_SRC = os.path.join(ROOT, "gated_deltanet_streaming_amd", "csrc", "gdn_attention.hip")


def kernel_source_hash(src: str = KERNEL_SRC) -> str:
    with open(src, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def algorithmic_bytes(mode: str) -> int:
    """Bytes a whole step (forward with carried state + reverse) must move at least."""
    if mode == "bidir":
        return B * T * H * BIDIR_BYTES_PER_TOKEN_HEAD + 2 * STATE_BYTES
    per_scan = B * T * H * BYTES_PER_TOKEN_HEAD
    return 2 * per_scan + 2 * STATE_BYTES


def load_traffic(path: str = TRAFFIC_FILE, src: str = KERNEL_SRC):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3 counter runs,
    if they were taken on the current kernel source; else None."""
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != kernel_source_hash(src):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(d, threads):
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
    return {"value": round(T / dt, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"the full workload, {reps} repeats: forward + reverse fp64 scans of B={B} H={H} "
                      f"d={D} T={T} ({dt:.3f} s per step)",
            "single_core": {"value": round(T / dt1, 1), "cores": 1,
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--mode", choices=["bidir", "separate", "backward", "attention"], default="bidir",
                    help="bidir: one gdn_chunk_bidir call per step; separate: forward then reverse calls; "
                         "backward: the gradients of both scans of the pair (gdn_chunk_backward); "
                         "attention: the softmax block's sink + window attention (gdn_attn_chunk)")
    ap.add_argument("--sets", type=int, default=6, help="rotating input/output buffer sets (1 = warm)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-peaks", action="store_true", help="skip the copy / MFMA peak probes")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a 256 MiB device copy (reference for counter scaling)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (this path needs no "
              "multi-GPU exchange; see the sharding notes).", file=sys.stderr)
        sys.exit(2)

    if args.mode == "backward":
        return main_backward(args)
    if args.mode == "attention":
        return main_attention(args)

    import numpy as np
    import torch

    import gdn_inputs
    from gated_deltanet_streaming_amd import binding as gb

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d = gdn_inputs.batch(1, B, T, H, D, with_state=True)

    sets = []
    for i in range(args.sets):
        # distinct values per set (the first set is the seeded workload itself)
        di = d if i == 0 else gdn_inputs.batch(1, B, T, H, D, chunk=i)
        qi = {k: torch.from_numpy(di[k]).to(dev, torch.bfloat16) for k in ("q", "k", "v")}
        qi["a"] = torch.from_numpy(di["a"]).to(dev)
        qi["beta"] = torch.from_numpy(di["beta"]).to(dev)
        qi["o"] = torch.empty_like(qi["v"])
        qi["o_rev"] = torch.empty_like(qi["v"])
        sets.append(qi)

    s = gb.Stream(B, H, D, D, T, device=0)
    s.state_set(torch.from_numpy(d["S0"]).to(dev))
    stream = torch.cuda.current_stream(dev)

    def step(i):
        x = sets[i % len(sets)]
        if args.mode == "bidir":
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

    alg_bytes = algorithmic_bytes(args.mode)
    launches_per_step = scan_n / args.steps
    bytes_per_scan_launch = alg_bytes / launches_per_step
    achieved_gbs = bytes_per_scan_launch / (scan_avg_ms * 1e-3) / 1e9
    step_gbs = alg_bytes / (ms_per_step * 1e-3) / 1e9
    flops = 2 * B * T * H * FLOPS_PER_TOKEN_HEAD
    traffic = load_traffic()

    out = {
        "metric": METRIC,
        "value": round(T / (ms_per_step * 1e-3), 1),
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
            "workload": "720p streaming chunk, one GDN layer: forward scan from the carried state + "
                        "intra-chunk reverse scan",
            "B": B, "H": H, "d_k": D, "d_v": D, "T": T, "subchunk": 64,
            "call": "gdn_chunk_bidir" if args.mode == "bidir" else "gdn_chunk_forward + gdn_chunk_reverse",
            "buffers": f"{args.sets} rotating sets ({'cold: live set > 256 MB MALL' if args.sets >= 6 else 'warm'})",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": "gdn_scan_kernel",
            "kernel_avg_us": round(scan_avg_ms * 1e3, 3),
            "algorithmic_bytes_per_launch": int(bytes_per_scan_launch),
        },
        "step_roofline": {
            "algorithmic_bytes_per_step": alg_bytes,
            "achieved_GBs": round(step_gbs, 1),
            "hbm_frac": round(step_gbs / HBM_PEAK_GBS, 4),
            "mfma_bf16_frac": round(flops / (ms_per_step * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 5),
            "prep_avg_us": round(prep_avg_ms * 1e3, 3),
            "scan_avg_us": round(scan_avg_ms * 1e3, 3),
            "event_ms_per_step": round(ms_events / args.steps, 5),
            "per_call_ms_p10_p50_p90": [round(p10, 5), round(p50, 5), round(p90, 5)],
            "warm_ms_per_step": round(warm_ms, 5),
            "target_tokens_per_s": 108e6,
        },
    }
    if not args.no_peaks:
        out["measured_peaks"] = measured_peaks(torch, dev)
    if not args.no_cpu:
        # the host share of one GPU: OMP_NUM_THREADS when set (16 on the GPU machines), else the affinity mask
        threads = min(len(os.sched_getaffinity(0)), int(os.environ.get("OMP_NUM_THREADS", "0")) or 1 << 30)
        out["cpu_baseline"] = cpu_baseline(d, threads)
    s.close()
    print(json.dumps(out), flush=True)


def main_backward(args):
    """Gradients of both scans of the 720p pair (forward from the carried state, reverse from
    zero) through gdn_chunk_backward: a token-sequential fp32 path, bound by its serial chain
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

    def step():
        s.backward(x["q"], x["k"], x["v"], a, beta, dO[0], d_state=dSf, state0=S0, stream=stream)
        s.backward(x["q"], x["k"], x["v"], a, beta, dO[1], reverse=True, stream=stream)

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
    achieved = alg_bytes / 2 / (launch_ms * 1e-3) / 1e9
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
                   "T": T, "call": "gdn_chunk_backward x 2", "path": "token-sequential fp32"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 5), "traffic": None, "kernel": "gdn_bwd_rows_kernel + "
                     "gdn_bwd_reduce_kernel", "kernel_avg_us": round(launch_ms * 1e3, 1),
                     "algorithmic_bytes_per_launch": int(alg_bytes / 2),
                     "note": "latency-bound by the serial chain of T tokens per (head, 16-row block)"},
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
                     "traffic": load_traffic(ATTN_TRAFFIC_FILE, ATTN_KERNEL_SRC),
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


if __name__ == "__main__":
    main()
