#!/usr/bin/env python3
"""Benchmark: grouped / pointer-array bf16 GEMM, W4A16 GEMM and implicit-GEMM
conv fprop on one MI355X.

A step is one pointer-array GEMM launch over L = 16 separately allocated
M = N = K = 1024 bf16 problems (beta = 0): the library's dense mainloop run
by its persistent scheduler.  The inputs rotate through enough distinct
copies that every step reads its operands from HBM, not from the 256 MB
Infinity Cache.  The JSON line also reports the other workloads (grouped
fp16, MoE grouped bf16, W4A16 at M = 16 / 128 / 1024 / 4096, conv fprop),
each against its own roofline, and the fp64 CPU oracle timed on a bounded
sample of the headline workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MFMA_16 = 2516.6  # TFLOP/s, dense fp16 / bf16: 256 CU x 4096 FLOP/clk x 2.4 GHz
PEAK_MFMA_8 = 5033.2  # TFLOP/s, dense fp8: twice the 16-bit rate
PEAK_HBM = 8000.0  # GB/s
# HBM bytes per launch of the headline kernel: rocprofv3 FETCH_SIZE and WRITE_SIZE of the headline command,
# each scaled by what the same counter reads for a plain 256 MiB device copy (FETCH x 1.99973, WRITE x 1.0);
# summary and commands in profiles/k_gemm_ptr_array_256x256_bf16_ptr_array_L16_1024.md.  Valid for the
# kernel named here only.
HEADLINE_KERNEL = "k_gemm_ptr_array<TileCfg<256,256,4,2,64,2,5>, bf16, false>"
HEADLINE_TRAFFIC_BYTES = 100992876
HEADLINE_PROFILE = "k_gemm_ptr_array_256x256_bf16_ptr_array_L16_1024.md"
# GRBM_GUI_ACTIVE cycles (summed over the 8 XCDs) / 8 / kernel time of the headline kernel in that profile's
# counter run, where every dispatch is serialized by the profiler
HEADLINE_PMC_CLOCK_MHZ = 2401
MALL_BYTES = 256 << 20
ROTATE_TARGET = 512 << 20
METRIC = "TFLOP/s and % of MFMA peak: grouped bf16 GEMM, w4a16 GEMM, conv fprop"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def copies_for(ws_bytes: int) -> int:
    return 1 if ws_bytes >= ROTATE_TARGET else int(math.ceil(ROTATE_TARGET / ws_bytes))


RAMP_MS = 50.0


def time_launches(torch, fn, n_copies, warmup, group=1, min_window_ms=2.0, windows=7, ramp_ms=RAMP_MS):
    """Per-launch time of fn (cycling over the rotating copies), HIP events on the launch stream.

    After `warmup` untimed launches, untimed back-to-back launches continue until they have taken at least
    `ramp_ms` of GPU time: after an idle spell the same launches run up to 20% slower for the first 15-20 ms
    of load, until the device's power management settles, and the timed region starts once it has.  Then one untimed calibration window of `group` launches, and
    the loop times `windows` windows; each is a whole number of `group`-launch runs, enough to last at least
    min_window_ms.  Returns the median per-launch time over the windows (ms) with the spread, the window size
    and the number of ramp launches."""
    i = 0
    for _ in range(warmup):
        fn(i % n_copies)
        i += 1
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ramped, ramp_launches, chunk = 0.0, 0, max(group, 8)
    while ramped < ramp_ms:
        s.record()
        for _ in range(chunk):
            fn(i % n_copies)
            i += 1
        e.record()
        torch.cuda.synchronize()
        ramped += s.elapsed_time(e)
        ramp_launches += chunk

    def window(n):
        nonlocal i
        torch.cuda.synchronize()
        s.record()
        for _ in range(n):
            fn(i % n_copies)
            i += 1
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e)

    reps = max(1, int(math.ceil(min_window_ms / max(window(group), 1e-3))))
    n = group * reps
    per = sorted(window(n) / n for _ in range(windows))
    return {"ms": per[len(per) // 2], "min_ms": per[0], "max_ms": per[-1], "windows": windows,
            "launches_per_window": n, "ramp_launches": ramp_launches}


def time_isolated_kernels(torch, gmi, fn, n_copies, launches):
    """Median execution time (ms) of the GEMM kernel launched on an otherwise idle stream: each call is
    synchronized before the next, and its kernel stamps its own event pair at its start and end
    (gmi.time_next_gemm, which launches it through hipExtLaunchKernel), as a kernel trace times it."""
    k0 = [torch.cuda.Event(enable_timing=True) for _ in range(launches)]
    k1 = [torch.cuda.Event(enable_timing=True) for _ in range(launches)]
    for e in k0 + k1:
        e.record()  # torch creates the HIP event on its first record
    torch.cuda.synchronize()
    for i in range(launches):
        gmi.time_next_gemm(k0[i], k1[i])
        fn(i % n_copies)
        torch.cuda.synchronize()
    gmi.time_next_gemm(None, None)
    return sorted(a.elapsed_time(b) for a, b in zip(k0, k1))[launches // 2]


def copy_ref(torch, dev, args):
    """With --copy-ref, one plain 256 MiB device-to-device copy: a kernel of known traffic that calibrates
    the hardware byte counters."""
    if args.copy_ref:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst


def roof(flops, bytes_, t, peak=PEAK_MFMA_16, bound=None):
    """Rates and roofline fractions of one workload from its time_launches record; `bound` is the roof
    that is closer (the larger of the two fractions) unless given ("launch" for latency-bound calls)."""
    ms = t["ms"]
    sec = ms * 1e-3
    tf = flops / sec / 1e12
    gbs = bytes_ / sec / 1e9
    f_mfma, f_hbm = tf / peak, gbs / PEAK_HBM
    return dict(us=round(ms * 1e3, 3), us_min=round(t["min_ms"] * 1e3, 3), us_max=round(t["max_ms"] * 1e3, 3),
                launches_per_window=t["launches_per_window"], ramp_launches=t["ramp_launches"], tflops=round(tf, 2),
                frac_mfma=round(f_mfma, 4),
                gbps=round(gbs, 1), frac_hbm=round(f_hbm, 4), roofline_frac=round(max(f_mfma, f_hbm), 4),
                bound=bound or ("mfma" if f_mfma >= f_hbm else "hbm"))


def t16(torch, bits, dtype, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(dtype).to(dev)


def shader_clock(torch, fn, n_copies, seconds=1.5):
    """Shader clock under the headline load, for context next to the fixed 2.4 GHz of the peak: the headline
    launches run back to back for about `seconds` while `amd-smi metric -c` samples the graphics clock from
    another process (median of the samples, MHz).  The clock that rocprofv3 derives for the same kernel
    (GRBM_GUI_ACTIVE cycles over the kernel time) is recorded beside it."""
    import subprocess
    import threading

    samples, errors = [], []

    def gfx_mhz(obj):
        # every "gfx_<i>" entry's current clock, in MHz, wherever it sits in the JSON
        out = []
        if isinstance(obj, dict):
            for k, v in obj.items():
                if str(k).lower().startswith("gfx") and isinstance(v, dict) and "clk" in v:
                    c = v["clk"]
                    c = c.get("value") if isinstance(c, dict) else c
                    try:
                        out.append(float(str(c).split()[0]))
                    except ValueError:
                        pass
                else:
                    out += gfx_mhz(v)
        elif isinstance(obj, list):
            for v in obj:
                out += gfx_mhz(v)
        return out

    stop = threading.Event()

    def sampler():
        while not stop.is_set():
            try:
                r = subprocess.run(["amd-smi", "metric", "-g", "0", "-c", "--json"], capture_output=True, text=True,
                                   timeout=10)
                v = gfx_mhz(json.loads(r.stdout)) if r.returncode == 0 else []
                if v:
                    samples.append(max(v))
                else:
                    errors.append((r.stderr or r.stdout).strip()[:200])
            except Exception as exc:  # a missing or failing tool leaves the clock unreported
                errors.append(repr(exc)[:200])
            stop.wait(0.2)

    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    t0, i = time.perf_counter(), 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(50):
            fn(i % n_copies)
            i += 1
        torch.cuda.synchronize()
    stop.set()
    th.join(timeout=15)
    pmc = {"mhz": HEADLINE_PMC_CLOCK_MHZ, "source": "rocprofv3 GRBM_GUI_ACTIVE / 8 XCDs / kernel duration of the "
                                                    "headline kernel with the profiler serializing dispatches, "
                                                    "profiles/" + HEADLINE_PROFILE}
    if not samples:
        return {"amd_smi_mhz": None, "amd_smi_error": errors[-1] if errors else "no sample", "pmc": pmc}
    samples.sort()
    return {"amd_smi_mhz": samples[len(samples) // 2], "amd_smi_samples": len(samples), "pmc": pmc}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


# --------------------------------------------------------------------------
def setup_ptr_array(torch, gmi, gi, dev, L=16, M=1024, N=1024, K=1024):
    A, B = gi.ptr_array_bf16(L=L, M=M, N=N, K=K)
    ws = 3 * L * M * K * 2
    R = copies_for(ws)
    sets = []
    for r in range(R):
        Ad = [t16(torch, a, torch.bfloat16, dev) for a in A]
        Bd = [t16(torch, b, torch.bfloat16, dev) for b in B]
        Dd = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(L)]
        sets.append((gmi.pointer_array(Ad, dev), gmi.pointer_array(Bd, dev), gmi.pointer_array(Dd, dev), Ad, Bd, Dd))

    def fn(i):
        pa, pb, pd = sets[i][:3]
        gmi.gemm_ptr_array(L, M, N, K, pa, K, pb, K, None, N, pd, N, torch.bfloat16, 1.0, 0.0)

    return fn, R, 2.0 * L * M * N * K, ws, (A, B, sets)


def cpu_baseline(gi, A, B, budget_s=12.0):
    """The oracle, as it stands, on batches of the headline workload (cycling
    over the 16) until about budget_s of host time has been spent."""
    import oracle

    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    done, flops, t0 = 0, 0.0, time.perf_counter()
    while True:
        oracle.gemm(A[done % len(A)], B[done % len(B)], dtype="bf16")
        done += 1
        flops += 2.0 * A[0].shape[0] * B[0].shape[0] * A[0].shape[1]
        if time.perf_counter() - t0 > budget_s:
            break
    sec = time.perf_counter() - t0
    return {"value": round(flops / sec / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "cpu": cpu_model(),
            "logical_cpus": os.cpu_count(), "kind": "oracle",
            "sample": f"{done} batch products of 1024^3 bf16 inputs in fp64 (cycling over the 16 batches), "
                      f"{sec:.1f} s"}


def bench_moe(torch, gmi, gi, dev, out):
    """The MoE grouped bf16 layer, host table and device-held group sizes."""
    # 3. MoE grouped bf16, 16384 tokens over 128 experts, N 2048, K 4096
    counts = gi.moe_counts()
    N, K = 2048, 4096
    A = t16(torch, gi.moe_activations(), torch.bfloat16, dev)
    D = torch.empty((int(counts.sum()), N), dtype=torch.bfloat16, device=dev)
    Bw = [t16(torch, gi.moe_expert_weight(g), torch.bfloat16, dev) for g in range(len(counts))]
    off = np.concatenate([[0], np.cumsum(counts)])
    table = gmi.make_problems([A[off[g]:off[g + 1]] for g in range(128)], Bw, [None] * 128,
                              [D[off[g]:off[g + 1]] for g in range(128)])
    wsb = torch.empty(gmi.workspace_bytes(128), dtype=torch.uint8, device=dev)
    fl = 2.0 * counts.sum() * N * K
    by = 2 * (counts.sum() * K + int((counts > 0).sum()) * N * K + counts.sum() * N)
    tm = time_launches(torch, lambda i: gmi.gemm_grouped_raw(table, 128, gmi.GMI_BF16, 1.0, 0.0, wsb), 1, 3)
    out["moe_grouped_bf16"] = roof(fl, by, tm)
    # the same layer with the group sizes held on the device (row offsets; a
    # table-building launch, then the GEMM): no host round trip
    B3 = torch.stack(Bw)
    del Bw
    offs = torch.tensor(off.astype(np.int32), device=dev)
    tm = time_launches(torch, lambda i: gmi.gemm_grouped_offsets(offs, A, B3, D, workspace=wsb), 1, 3)
    out["moe_grouped_offsets_bf16"] = roof(fl, by, tm)
    del B3, A, D
    torch.cuda.empty_cache()
    log("bench: MoE grouped done")
    return counts, off


def bench_moe_w4(torch, gmi, gi, dev, out):
    # 4b. MoE decode step with 4-bit experts: 128 routed rows over 128 experts
    # (N 2048, K 4096, g 128), bf16, int4 with zero points, sizes on the device
    w4_counts = gi.moe_w4_counts()
    E, N, K = len(w4_counts), 2048, 4096
    experts = [gi.moe_w4_expert(e) for e in range(E)]
    wpp = torch.stack([gmi.prepack_w4(torch.from_numpy(w).to(dev), N, K) for w, _, _ in experts])
    Sx = torch.stack([t16(torch, s, torch.bfloat16, dev) for _, s, _ in experts])
    Zx = torch.stack([torch.from_numpy(z).to(dev) for _, _, z in experts])
    del experts
    Xm = t16(torch, gi.moe_w4_activations(rows=int(w4_counts.sum())), torch.bfloat16, dev)
    Ym = torch.empty((Xm.shape[0], N), dtype=torch.bfloat16, device=dev)
    offs = torch.tensor(np.concatenate([[0], np.cumsum(w4_counts)]).astype(np.int32), device=dev)
    live = int((w4_counts > 0).sum())
    by = live * (N * K // 2 + (K // 128) * N * 2 + (K // 128) * N // 2) + 2 * int(w4_counts.sum()) * (K + N)
    R = copies_for(by)
    sets = [(wpp, Sx, Zx)] + [(wpp.clone(), Sx.clone(), Zx.clone()) for _ in range(R - 1)]

    def fn(i, sets=sets):
        w, s, z = sets[i]
        gmi.gemm_mixed_grouped(offs, Xm, w, s, z, 128, N, w_type="int4", Y=Ym)

    tm = time_launches(torch, fn, R, 5)
    out["moe_w4_decode_bf16"] = dict(roof(2.0 * int(w4_counts.sum()) * N * K, by, tm), experts_live=live)
    del Xm, Ym
    # 4c. the same experts on a prefill batch: 16384 rows routed like the bf16 MoE layer (groups above 32 rows
    # take the tiled launch, the rest the decode launch)
    p_counts = gi.moe_w4_counts(rows=16384)
    Xp = t16(torch, gi.moe_w4_activations(rows=16384), torch.bfloat16, dev)
    Yp = torch.empty((16384, N), dtype=torch.bfloat16, device=dev)
    p_offs = torch.tensor(np.concatenate([[0], np.cumsum(p_counts)]).astype(np.int32), device=dev)
    p_live = int((p_counts > 0).sum())
    p_by = p_live * (N * K // 2 + (K // 128) * N * 2 + (K // 128) * N // 2) + 2 * 16384 * (K + N)

    def fnp(i, sets=sets):
        w, s, z = sets[i]
        gmi.gemm_mixed_grouped(p_offs, Xp, w, s, z, 128, N, w_type="int4", Y=Yp)

    tm = time_launches(torch, fnp, R, 3)
    out["moe_w4_prefill_bf16"] = dict(roof(2.0 * 16384 * N * K, p_by, tm), experts_live=p_live)
    del sets, wpp, Sx, Zx, Xp, Yp
    torch.cuda.empty_cache()
    log("bench: MoE W4 decode and prefill done")


def bench_conv(torch, gmi, gi, dev, out):
    """Conv fprop, dgrad and wgrad of one 3x3 layer."""
    # 5. conv fprop bf16 32x56x56x256, 3x3x256 -> 256, pad 1
    x, wf = gi.conv_fprop_bf16()
    xd, wd = t16(torch, x, torch.bfloat16, dev), t16(torch, wf, torch.bfloat16, dev)
    ws = 2 * (x.size + wf.size + 32 * 56 * 56 * 256)
    R = copies_for(ws)
    sets = [(xd.clone(), wd.clone(), torch.empty((32, 56, 56, 256), dtype=torch.bfloat16, device=dev))
            for _ in range(R)]
    tm = time_launches(torch, lambda i: gmi.conv2d_fprop(sets[i][0], sets[i][1], pad=(1, 1), y=sets[i][2]), R, 5)
    out["conv_fprop_bf16"] = roof(2.0 * 100352 * 256 * 2304, ws, tm)
    # the same layer with its bias and ReLU fused into the epilogue
    bd = t16(torch, gi.conv_bias(), torch.bfloat16, dev)
    tm = time_launches(torch, lambda i: gmi.conv2d_fprop(sets[i][0], sets[i][1], pad=(1, 1), y=sets[i][2], bias=bd,
                                                         act="relu"), R, 5)
    out["conv_fprop_bias_relu_bf16"] = roof(2.0 * 100352 * 256 * 2304, ws + 512, tm)
    # the data gradient of the same layer (dy of the forward output's shape; the filter rearranged each call)
    wsd = torch.empty(gmi.lib().gmi_conv2d_dgrad_workspace_bytes(256, 256, 3, 3), dtype=torch.uint8, device=dev)
    tm = time_launches(torch, lambda i: gmi.conv2d_dgrad(sets[i][2], sets[i][1], 56, 56, pad=(1, 1), dx=sets[i][0],
                                                         workspace=wsd), R, 5)
    out["conv_dgrad_bf16"] = roof(2.0 * 100352 * 256 * 2304, ws, tm)
    # the data gradient of the same layer at stride 2 (dy 32 x 28 x 28 x 256 back to 56 x 56): the four output
    # phases in one launch, each with only the taps that reach it; FLOPs of the forward view (every tap of every
    # dy pixel)
    dy2 = [torch.empty((32, 28, 28, 256), dtype=torch.bfloat16, device=dev).normal_() for _ in range(R)]
    tm = time_launches(torch, lambda i: gmi.conv2d_dgrad(dy2[i], sets[i][1], 56, 56, pad=(1, 1), stride=(2, 2),
                                                         dx=sets[i][0], workspace=wsd), R, 5)
    out["conv_dgrad_stride2_bf16"] = roof(2.0 * 32 * 28 * 28 * 256 * 2304, 2 * (32 * 28 * 28 * 256 + wf.size)
                                          + 2 * x.size, tm)
    del dy2
    # and its weight gradient (x and dy of the same shapes; transposes and the split sum included)
    dws = torch.empty((256, 3, 3, 256), dtype=torch.bfloat16, device=dev)
    wsw = torch.empty(gmi.conv2d_wgrad_workspace_bytes((32, 56, 56, 256), (32, 56, 56, 256), 3, 3, (1, 1)),
                      dtype=torch.uint8, device=dev)
    tm = time_launches(torch, lambda i: gmi.conv2d_wgrad(sets[i][0], sets[i][2], 3, 3, pad=(1, 1), dw=dws,
                                                         workspace=wsw), R, 3)
    out["conv_wgrad_bf16"] = roof(2.0 * 100352 * 256 * 2304, ws, tm)
    log("bench: conv done")
    del sets
    torch.cuda.empty_cache()


def bench_w4(torch, gmi, gi, dev, out):
    """W4A16 at M = 16 / 128 / 1024 / 4096 (fp16, uint4 with zero points) and the bf16 / int4 mixed-input lines."""
    # 4. W4A16, N = K = 8192, g = 128
    w = gi.w4a16(M=16)
    base_pp = gmi.prepack_w4(torch.from_numpy(w["W"]).to(dev), 8192, 8192)
    S = t16(torch, w["scales"], torch.float16, dev)
    Z = torch.from_numpy(w["zeros"]).to(dev)
    for M in (16, 128, 1024, 4096):
        X = t16(torch, gi.w4a16(M=M, N=16, K=8192)["X"], torch.float16, dev)
        ws = 8192 * 8192 // 2 + S.numel() * 2 + Z.numel() + 2 * M * 8192 * 2
        R = copies_for(ws)
        sets = [(base_pp.clone(), S.clone(), Z.clone(), X.clone(), torch.empty((M, 8192), dtype=torch.float16,
                                                                                device=dev)) for _ in range(R)]

        wsp = torch.empty(gmi.w4a16_workspace_bytes(M, 8192, 8192), dtype=torch.uint8, device=dev)

        def fn(i, sets=sets, wsp=wsp):
            pp, s, z, x, y = sets[i]
            gmi.gemm_w4a16(x, pp, s, z, 128, 8192, Y=y, workspace=wsp)

        tm = time_launches(torch, fn, R, 5)
        out[f"w4a16_M{M}"] = roof(2.0 * M * 8192 * 8192, ws, tm)
        del sets
    # the same shapes with bf16 activations and scales, int4 weights with zero points
    Sb = S.float().to(torch.bfloat16)
    for M in (16, 48, 128, 1024):
        X = t16(torch, gi.w4a16(M=M, N=16, K=8192)["X"], torch.float16, dev).float().to(torch.bfloat16)
        ws = 8192 * 8192 // 2 + Sb.numel() * 2 + Z.numel() + 2 * M * 8192 * 2
        R = copies_for(ws)
        sets = [(base_pp.clone(), Sb.clone(), Z.clone(), X.clone(), torch.empty((M, 8192), dtype=torch.bfloat16,
                                                                                 device=dev)) for _ in range(R)]
        wsp = torch.empty(gmi.w4a16_workspace_bytes(M, 8192, 8192), dtype=torch.uint8, device=dev)

        def fn(i, sets=sets, wsp=wsp):
            pp, s, z, x, y = sets[i]
            gmi.gemm_mixed(x, pp, s, z, 128, 8192, w_type="int4", Y=y, workspace=wsp)

        tm = time_launches(torch, fn, R, 5)
        out[f"mixed_bf16_int4_M{M}"] = roof(2.0 * M * 8192 * 8192, ws, tm)
        del sets
    log("bench: W4A16 done")


def bench_fp8(torch, gmi, gi, dev, out):
    """fp8 (E4M3) inputs, bf16 results: the pointer-array headline shape and the MoE layer."""
    counts = gi.moe_counts()
    off = np.concatenate([[0], np.cumsum(counts)])
    A8, B8 = gi.ptr_array_f8(L=16)
    ws = 16 * (1024 * 1024 + 1024 * 1024 + 1024 * 1024 * 2)  # A, B fp8 read once; D bf16 written once
    R = copies_for(ws)
    f8 = torch.float8_e4m3fn
    sets = []
    for r in range(R):
        Ad = [torch.from_numpy(a).view(f8).to(dev) for a in A8]
        Bd = [torch.from_numpy(b).view(f8).to(dev) for b in B8]
        Dd = [torch.empty((1024, 1024), dtype=torch.bfloat16, device=dev) for _ in range(16)]
        sets.append([gmi.pointer_array(x, dev) for x in (Ad, Bd, Dd)] + [Ad, Bd, Dd])
    tm = time_launches(torch, lambda i: gmi.gemm_ptr_array(16, 1024, 1024, 1024, sets[i][0], 1024, sets[i][1], 1024,
                                                           None, 1024, sets[i][2], 1024, gmi.GMI_F8E4M3, 1.0, 0.0),
                       R, 10)
    out["ptr_array_fp8"] = roof(2.0 * 16 * 1024 ** 3, ws, tm, PEAK_MFMA_8)
    del sets, A8, B8
    N, K = 2048, 4096
    A = torch.from_numpy(gi.moe_activations_f8()).view(f8).to(dev)
    D = torch.empty((int(counts.sum()), N), dtype=torch.bfloat16, device=dev)
    Bw = [torch.from_numpy(gi.moe_expert_weight_f8(g)).view(f8).to(dev) for g in range(len(counts))]
    table = gmi.make_problems([A[off[g]:off[g + 1]] for g in range(128)], Bw, [None] * 128,
                              [D[off[g]:off[g + 1]] for g in range(128)])
    wsb = torch.empty(gmi.workspace_bytes(128), dtype=torch.uint8, device=dev)
    fl = 2.0 * counts.sum() * N * K
    by = counts.sum() * K + int((counts > 0).sum()) * N * K + 2 * counts.sum() * N
    tm = time_launches(torch, lambda i: gmi.gemm_grouped_raw(table, 128, gmi.GMI_F8E4M3, 1.0, 0.0, wsb), 1, 3)
    out["moe_grouped_fp8"] = roof(fl, by, tm, PEAK_MFMA_8)
    del Bw, A, D
    torch.cuda.empty_cache()
    log("bench: fp8 done")


def bench_workloads(torch, gmi, gi, dev, args):
    out = {}
    # 1. grouped fp16, 4 groups, beta 0.5 (launch-latency bound)
    probs = gi.grouped_f16()
    As = [t16(torch, p["A"], torch.float16, dev) for p in probs]
    Bs = [t16(torch, p["B"], torch.float16, dev) for p in probs]
    Cs = [t16(torch, p["C"], torch.float16, dev) for p in probs]
    Ds = [torch.empty((p["M"], p["N"]), dtype=torch.float16, device=dev) for p in probs]
    table = gmi.make_problems(As, Bs, Cs, Ds)
    wsb = torch.empty(gmi.workspace_bytes(4), dtype=torch.uint8, device=dev)
    fl = sum(2.0 * p["M"] * p["N"] * p["K"] for p in probs)
    by = sum(2 * (p["M"] * p["K"] + p["N"] * p["K"] + 2 * p["M"] * p["N"]) for p in probs)
    tm = time_launches(torch, lambda i: gmi.gemm_grouped_raw(table, 4, gmi.GMI_F16, 1.0, 0.5, wsb), 1, 20)
    out["grouped_f16_4groups"] = roof(fl, by, tm, bound="launch")
    log("bench: grouped fp16 done")

    bench_moe(torch, gmi, gi, dev, out)

    bench_w4(torch, gmi, gi, dev, out)

    bench_moe_w4(torch, gmi, gi, dev, out)

    bench_conv(torch, gmi, gi, dev, out)

    bench_fp8(torch, gmi, gi, dev, out)
    return out


def decode_only(torch, gmi, gi, dev, args):
    """The W4A16 M = 16 line of the workloads alone: rotating copies, HIP events over the timed launches."""
    M, N, K, g = 16, 8192, 8192, 128
    w = gi.w4a16(M=M, N=N, K=K, group=g)
    pp = gmi.prepack_w4(torch.from_numpy(w["W"]).to(dev), N, K)
    S = t16(torch, w["scales"], torch.float16, dev)
    Z = torch.from_numpy(w["zeros"]).to(dev)
    X = t16(torch, w["X"], torch.float16, dev)
    ws = N * K // 2 + S.numel() * 2 + Z.numel() + 2 * M * (N + K)
    R = copies_for(ws)
    sets = [(pp.clone(), S.clone(), Z.clone(), X.clone(), torch.empty((M, N), dtype=torch.float16, device=dev))
            for _ in range(R)]
    wsp = torch.empty(gmi.w4a16_workspace_bytes(M, N, K), dtype=torch.uint8, device=dev)
    fn = lambda i: gmi.gemm_w4a16(sets[i][3], sets[i][0], sets[i][1], sets[i][2], g, N, Y=sets[i][4], workspace=wsp)
    tm = time_launches(torch, fn, R, args.warmup, group=args.steps)
    copy_ref(torch, dev, args)
    line = dict(workload=f"w4a16 decode M={M} N={N} K={K} g={g}", steps=args.steps, warmup=args.warmup,
                algorithmic_bytes=ws, copies=R, **roof(2.0 * M * N * K, ws, tm))
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--headline-only", action="store_true", help="skip the other workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode-only", action="store_true",
                    help="time only the W4A16 decode workload (M = 16, N = K = 8192, g = 128) and print one line "
                         "for it (for the decode kernel's profiles)")
    ap.add_argument("--only", choices=["moe", "moe_w4", "conv", "w4", "fp8"],
                    help="time only the bf16 MoE layers, the 4-bit MoE layers, the conv layers or the W4A16 / mixed-input "
                         "lines or the fp8 lines and print their lines (for those kernels' profiles)")
    ap.add_argument("--no-clock-sample", action="store_true",
                    help="skip the 1.5 s of back-to-back headline launches that sample the shader clock (for "
                         "counter runs, which serialize every launch)")
    ap.add_argument("--copy-ref", action="store_true",
                    help="after the timed region, run one plain 256 MiB device copy (a known-size kernel that "
                         "calibrates hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this library's kernels run on a single device and there is no "
              "multi-GPU path to time (--gpus must be 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import gmi_inputs as gi
    import grouped_mixed_input_amd as gmi

    if not gmi.LIB_PATH.exists():
        from __graft_entry__ import build

        build()
    gmi.lib()
    dev = torch.device("cuda:0")
    if args.decode_only:
        decode_only(torch, gmi, gi, dev, args)
        return
    if args.only:
        out = {}
        {"moe": bench_moe, "moe_w4": bench_moe_w4, "conv": bench_conv, "w4": bench_w4, "fp8": bench_fp8}[args.only](torch, gmi, gi, dev, out)
        copy_ref(torch, dev, args)
        print(json.dumps(out), flush=True)
        return
    log("bench: building inputs")
    fn, R, flops, ws, keep = setup_ptr_array(torch, gmi, gi, dev)
    log(f"bench: headline rotates {R} copies of {ws / 2**20:.0f} MiB")
    # W untimed warm-up steps, an untimed ramp of back-to-back steps (at least RAMP_MS of GPU time, while the
    # device settles after idling), then windows of whole K-step runs (each window at least 2 ms, bracketed by
    # synchronizations); the step time is the median over the windows
    tm = time_launches(torch, fn, R, args.warmup, group=args.steps)
    ms = tm["ms"]
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"bench: headline {ms * 1e3:.1f} us/step (median of {tm['windows']} windows of {tm['launches_per_window']} "
        f"steps; {tm['min_ms'] * 1e3:.1f} to {tm['max_ms'] * 1e3:.1f}), {tflops:.1f} TFLOP/s")
    iso_ms = time_isolated_kernels(torch, gmi, fn, R, 200)
    log(f"bench: headline kernel alone on an idle stream {iso_ms * 1e3:.1f} us (median of 200 kernel-stamped "
        f"launches), {flops / (iso_ms * 1e-3) / 1e12:.1f} TFLOP/s")
    clock = None if args.no_clock_sample else shader_clock(torch, fn, R)
    log(f"bench: shader clock under the headline load {clock}")

    result = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "pointer-array bf16 GEMM, L=16 separately allocated M=N=K=1024 problems, "
                               "beta=0, fp32 accumulate, bf16 D", "L": 16, "M": 1024, "N": 1024, "K": 1024,
                   "cache": f"cold: {R} rotating copies of the {ws / 2**20:.0f} MiB working set"},
        "timing": {"ramp_ms": RAMP_MS, "ramp_steps": tm["ramp_launches"], "windows": tm["windows"],
                   "steps_per_window": tm["launches_per_window"],
                   "us_per_step_median": round(ms * 1e3, 3), "us_per_step_min": round(tm["min_ms"] * 1e3, 3),
                   "us_per_step_max": round(tm["max_ms"] * 1e3, 3)},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_MFMA_16, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_MFMA_16, 4), "launch_us": round(ms * 1e3, 3),
                     "isolated_kernel_us": round(iso_ms * 1e3, 3),
                     "achieved_basis": "algorithmic FLOPs per launch / the timed region's time per launch (HIP "
                                       "events on the launch stream, median window); back to back the kernels "
                                       "leave no gap, so this is the kernel's own duration in the timed region. "
                                       "isolated_kernel_us: the same kernel launched alone on an idle stream, "
                                       "timed by event stamps at its own start and end (gmi_time_next_gemm)",
                     "traffic": HEADLINE_TRAFFIC_BYTES,
                     "traffic_unit": "HBM bytes per launch", "algorithmic_bytes": 3 * 16 * 1024 * 1024 * 2,
                     "kernel": HEADLINE_KERNEL, "clock": clock},
    }
    copy_ref(torch, dev, args)
    if not args.headline_only:
        result["workloads"] = bench_workloads(torch, gmi, gi, dev, args)
    if not args.no_cpu_baseline:
        log("bench: timing the oracle on the host")
        result["cpu_baseline"] = cpu_baseline(gi, keep[0], keep[1])
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
