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
# each scaled by what the same counter reads for a plain 256 MiB device copy (FETCH x 1.99972, WRITE x 1.0);
# summary and commands in profiles/k_gemm_ptr_array_256x256_bf16_ptr_array_L16_1024.md.  Valid for the
# kernel named here only.
HEADLINE_KERNEL = "k_gemm_ptr_array<TileCfg<256,256,4,2,64,2,5>, bf16, false>"
HEADLINE_TRAFFIC_BYTES = 101441928
MALL_BYTES = 256 << 20
ROTATE_TARGET = 512 << 20
METRIC = "TFLOP/s and % of MFMA peak: grouped bf16 GEMM, w4a16 GEMM, conv fprop"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def copies_for(ws_bytes: int) -> int:
    return 1 if ws_bytes >= ROTATE_TARGET else int(math.ceil(ROTATE_TARGET / ws_bytes))


def time_launches(torch, fn, n_copies, warmup, iters):
    """Average ms per launch over `iters` back-to-back launches (cycling over
    the rotating copies), HIP events on the launch stream."""
    for i in range(warmup):
        fn(i % n_copies)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for i in range(iters):
        fn(i % n_copies)
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / iters


def copy_ref(torch, dev, args):
    """With --copy-ref, one plain 256 MiB device-to-device copy: a kernel of known traffic that calibrates
    the hardware byte counters."""
    if args.copy_ref:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst


def roof(flops, bytes_, ms, peak=PEAK_MFMA_16):
    t = ms * 1e-3
    tf = flops / t / 1e12
    gbs = bytes_ / t / 1e9
    return dict(us=round(ms * 1e3, 3), tflops=round(tf, 2), frac_mfma=round(tf / peak, 4),
                gbps=round(gbs, 1), frac_hbm=round(gbs / PEAK_HBM, 4),
                roofline_frac=round(max(flops / (peak * 1e12), bytes_ / (PEAK_HBM * 1e9)) / t, 4))


def t16(torch, bits, dtype, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(dtype).to(dev)


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
    return {"value": round(flops / sec / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
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
    ms = time_launches(torch, lambda i: gmi.gemm_grouped_raw(table, 128, gmi.GMI_BF16, 1.0, 0.0, wsb), 1, 3, 10)
    out["moe_grouped_bf16"] = dict(roof(fl, by, ms), bound="hbm")
    # the same layer with the group sizes held on the device (row offsets; a
    # table-building launch, then the GEMM): no host round trip
    B3 = torch.stack(Bw)
    del Bw
    offs = torch.tensor(off.astype(np.int32), device=dev)
    ms = time_launches(torch, lambda i: gmi.gemm_grouped_offsets(offs, A, B3, D, workspace=wsb), 1, 3, 10)
    out["moe_grouped_offsets_bf16"] = dict(roof(fl, by, ms), bound="hbm")
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

    ms = time_launches(torch, fn, R, 5, max(50, 2 * R))
    out["moe_w4_decode_bf16"] = dict(roof(2.0 * int(w4_counts.sum()) * N * K, by, ms), bound="hbm", experts_live=live)
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

    ms = time_launches(torch, fnp, R, 3, max(10, 2 * R))
    out["moe_w4_prefill_bf16"] = dict(roof(2.0 * 16384 * N * K, p_by, ms), bound="mfma", experts_live=p_live)
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
    ms = time_launches(torch, lambda i: gmi.conv2d_fprop(sets[i][0], sets[i][1], pad=(1, 1), y=sets[i][2]), R, 5,
                       max(20, 2 * R))
    out["conv_fprop_bf16"] = dict(roof(2.0 * 100352 * 256 * 2304, ws, ms), bound="mfma")
    # the same layer with its bias and ReLU fused into the epilogue
    bd = t16(torch, gi.conv_bias(), torch.bfloat16, dev)
    ms = time_launches(torch, lambda i: gmi.conv2d_fprop(sets[i][0], sets[i][1], pad=(1, 1), y=sets[i][2], bias=bd,
                                                         act="relu"), R, 5, max(20, 2 * R))
    out["conv_fprop_bias_relu_bf16"] = dict(roof(2.0 * 100352 * 256 * 2304, ws + 512, ms), bound="mfma")
    # the data gradient of the same layer (dy of the forward output's shape; the filter rearranged each call)
    wsd = torch.empty(gmi.lib().gmi_conv2d_dgrad_workspace_bytes(256, 256, 3, 3), dtype=torch.uint8, device=dev)
    ms = time_launches(torch, lambda i: gmi.conv2d_dgrad(sets[i][2], sets[i][1], 56, 56, pad=(1, 1), dx=sets[i][0],
                                                         workspace=wsd), R, 5, max(20, 2 * R))
    out["conv_dgrad_bf16"] = dict(roof(2.0 * 100352 * 256 * 2304, ws, ms), bound="mfma")
    # and its weight gradient (x and dy of the same shapes; transposes and the split sum included)
    dws = torch.empty((256, 3, 3, 256), dtype=torch.bfloat16, device=dev)
    wsw = torch.empty(gmi.conv2d_wgrad_workspace_bytes((32, 56, 56, 256), (32, 56, 56, 256), 3, 3, (1, 1)),
                      dtype=torch.uint8, device=dev)
    ms = time_launches(torch, lambda i: gmi.conv2d_wgrad(sets[i][0], sets[i][2], 3, 3, pad=(1, 1), dw=dws,
                                                         workspace=wsw), R, 3, max(10, 2 * R))
    out["conv_wgrad_bf16"] = dict(roof(2.0 * 100352 * 256 * 2304, ws, ms), bound="mfma")
    log("bench: conv done")
    del sets
    torch.cuda.empty_cache()


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
    ms = time_launches(torch, lambda i: gmi.gemm_grouped_raw(table, 4, gmi.GMI_F16, 1.0, 0.5, wsb), 1, 20, 500)
    out["grouped_f16_4groups"] = dict(roof(fl, by, ms), bound="launch")
    log("bench: grouped fp16 done")

    counts, off = bench_moe(torch, gmi, gi, dev, out)

    # 4. W4A16, N = K = 8192, g = 128
    w = gi.w4a16(M=16)
    base_pp = gmi.prepack_w4(torch.from_numpy(w["W"]).to(dev), 8192, 8192)
    S = t16(torch, w["scales"], torch.float16, dev)
    Z = torch.from_numpy(w["zeros"]).to(dev)
    rx = np.random.default_rng(0)
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

        ms = time_launches(torch, fn, R, 5, max(20, R * 2))
        bound = "hbm" if M <= 64 else "mfma"
        out[f"w4a16_M{M}"] = dict(roof(2.0 * M * 8192 * 8192, ws, ms), bound=bound)
        del sets
    del rx
    # the same shapes with bf16 activations and scales, int4 weights with zero points
    Sb = S.float().to(torch.bfloat16)
    for M in (16, 1024):
        X = t16(torch, gi.w4a16(M=M, N=16, K=8192)["X"], torch.float16, dev).float().to(torch.bfloat16)
        ws = 8192 * 8192 // 2 + Sb.numel() * 2 + Z.numel() + 2 * M * 8192 * 2
        R = copies_for(ws)
        sets = [(base_pp.clone(), Sb.clone(), Z.clone(), X.clone(), torch.empty((M, 8192), dtype=torch.bfloat16,
                                                                                 device=dev)) for _ in range(R)]
        wsp = torch.empty(gmi.w4a16_workspace_bytes(M, 8192, 8192), dtype=torch.uint8, device=dev)

        def fn(i, sets=sets, wsp=wsp):
            pp, s, z, x, y = sets[i]
            gmi.gemm_mixed(x, pp, s, z, 128, 8192, w_type="int4", Y=y, workspace=wsp)

        ms = time_launches(torch, fn, R, 5, max(20, R * 2))
        out[f"mixed_bf16_int4_M{M}"] = dict(roof(2.0 * M * 8192 * 8192, ws, ms), bound="hbm" if M <= 64 else "mfma")
        del sets
    log("bench: W4A16 done")

    bench_moe_w4(torch, gmi, gi, dev, out)

    bench_conv(torch, gmi, gi, dev, out)

    # 6. fp8 (E4M3) inputs, bf16 results: the pointer-array headline shape and the MoE layer
    A8, B8 = gi.ptr_array_f8(L=16)
    ws = 16 * (2 * 1024 * 1024 + 2 * 1024 * 1024 * 2)
    R = copies_for(ws)
    f8 = torch.float8_e4m3fn
    sets = []
    for r in range(R):
        Ad = [torch.from_numpy(a).view(f8).to(dev) for a in A8]
        Bd = [torch.from_numpy(b).view(f8).to(dev) for b in B8]
        Dd = [torch.empty((1024, 1024), dtype=torch.bfloat16, device=dev) for _ in range(16)]
        sets.append([gmi.pointer_array(x, dev) for x in (Ad, Bd, Dd)] + [Ad, Bd, Dd])
    ms = time_launches(torch, lambda i: gmi.gemm_ptr_array(16, 1024, 1024, 1024, sets[i][0], 1024, sets[i][1], 1024,
                                                           None, 1024, sets[i][2], 1024, gmi.GMI_F8E4M3, 1.0, 0.0),
                       R, 10, max(50, 2 * R))
    out["ptr_array_fp8"] = dict(roof(2.0 * 16 * 1024 ** 3, ws, ms, PEAK_MFMA_8), bound="hbm")
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
    ms = time_launches(torch, lambda i: gmi.gemm_grouped_raw(table, 128, gmi.GMI_F8E4M3, 1.0, 0.0, wsb), 1, 3, 10)
    out["moe_grouped_fp8"] = dict(roof(fl, by, ms, PEAK_MFMA_8), bound="hbm")
    del Bw, A, D
    torch.cuda.empty_cache()
    log("bench: fp8 done")
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
    ms = time_launches(torch, fn, R, args.warmup, args.steps)
    copy_ref(torch, dev, args)
    line = dict(workload=f"w4a16 decode M={M} N={N} K={K} g={g}", steps=args.steps, warmup=args.warmup,
                us=round(ms * 1e3, 3), algorithmic_bytes=ws, gbps=round(ws / (ms * 1e-3) / 1e9, 1),
                frac_hbm=round(ws / (ms * 1e-3) / (PEAK_HBM * 1e9), 4), copies=R)
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
    ap.add_argument("--only", choices=["moe", "moe_w4", "conv"],
                    help="time only the bf16 MoE layers, the 4-bit MoE layers or the conv layers and print their lines (for those "
                         "kernels' profiles)")
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
        {"moe": bench_moe, "moe_w4": bench_moe_w4, "conv": bench_conv}[args.only](torch, gmi, gi, dev, out)
        copy_ref(torch, dev, args)
        print(json.dumps(out), flush=True)
        return
    log("bench: building inputs")
    fn, R, flops, ws, keep = setup_ptr_array(torch, gmi, gi, dev)
    log(f"bench: headline rotates {R} copies of {ws / 2**20:.0f} MiB")
    for i in range(args.warmup):
        fn(i % R)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(args.steps):
        fn(i % R)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"bench: headline {ms * 1e3:.1f} us/step, {tflops:.1f} TFLOP/s")

    result = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "pointer-array bf16 GEMM, L=16 separately allocated M=N=K=1024 problems, "
                               "beta=0, fp32 accumulate, bf16 D", "L": 16, "M": 1024, "N": 1024, "K": 1024,
                   "cache": f"cold: {R} rotating copies of the {ws / 2**20:.0f} MiB working set"},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_MFMA_16, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_MFMA_16, 4), "traffic": HEADLINE_TRAFFIC_BYTES,
                     "traffic_unit": "HBM bytes per launch", "algorithmic_bytes": 3 * 16 * 1024 * 1024 * 2,
                     "kernel": HEADLINE_KERNEL},
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
