#!/usr/bin/env python3
"""Benchmark of the block-scaled FP8 linear on one MI355X (gfx950).

One step = the FP8 linear of the prefill-shaped workload: act_quant of
x bf16 [4096, 7168] (1x128 blocks, float32 scales) followed by the
block-scaled FP8 GEMM with W e4m3 [18432, 7168] (128x128 scales), bf16 out.
`value` is that step's throughput in TFLOP/s (2*M*N*K per step).  The other
rows of the hot path -- the decode-shaped linear (GB/s), act_quant in both
scale formats, weight_dequant, the two small GEMMs of the ue8m0 workload, the
prefill down-projection, the grouped MoE GEMMs, the MoE dispatch and
combine around them, and the BF16 path (weight dequantised inside a bf16
GEMM) -- are timed as secondary rows in the same run.

Inputs are seeded synthetic tensors (block_scaled_fp8_03_amd.inputs), drawn on
the device and resident in HBM before timing.  Warmup runs at least W steps and
at least WARMUP_MIN_S seconds: under sustained MFMA load the clocks take tens of
milliseconds to settle (a GEMM's duration drifts by ~25% over its first
~30 ms), and the timed region is meant to see the steady state.  Kernel durations come from HIP
events recorded on the stream the kernels run on; HBM-bound rows cycle through
enough copies of their inputs that the 256 MB Infinity Cache cannot hold them.
Secondary rows are timed as one replay of a HIP graph holding K back-to-back
launches, so short kernels are not paced by the host's per-launch cost.
The CPU baseline is the oracle (binary64 C + OpenMP) on a bounded sample of
the same workload, timed on the host cores, plus the oracle's wall time on
each other hot-path row's shape (`per_op`), with the CPU model recorded.

Usage: python bench.py [--gpus 1] [--steps 50] [--warmup 10]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import block_scaled_fp8_03_amd as fp8bs  # noqa: E402
from block_scaled_fp8_03_amd import inputs  # noqa: E402

PEAK_FP8_TFLOPS = 5000.0       # MI355X dense FP8 MFMA
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense BF16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
MALL_BYTES = 256 << 20         # Infinity Cache
ROTATE_FOOTPRINT = 2 * MALL_BYTES

# The prefill GEMM call is two kernels on one stream: 1024 tiles of 256x256
# (128x64 per wave, 2 LDS stages, 8 waves, activation scales in chunks) in four
# full rounds over the 256 CUs, then the last 2048 columns as 512 tiles of
# 128x128 (64x64 per wave, 4 waves, 2 stages, two workgroups per CU) in one
# more round.  The roofline is for the whole call, timed as one launch.
GEMM_KERNEL = ("gemm_tile_kernel<256,256,128,64,2,8,2,true,false,1,false> x 1024 tiles + "
               "gemm_tile_kernel<128,128,64,64,2,4,2,true,false,2,false> x 512 tiles")
GEMM_SOURCE = os.path.join(ROOT, "block_scaled_fp8_03_amd", "csrc", "gemm.hip")
# HBM traffic of one prefill GEMM call (both kernels) from the rocprofv3
# FETCH_SIZE and WRITE_SIZE runs (scaled by the 1 GiB copy calibration; see
# profiles/), valid only for the gemm.hip source whose SHA-256 is recorded
# with it.
GEMM_TRAFFIC = {"source_sha256": "da45023d687673a77190564d99ae8bd98338de51b3955455a73dadfcef282995",
                "fetch_bytes": 868753818, "write_bytes": 151034880}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------- algorithmic work

def act_quant_bytes(M, K):
    return 2 * M * K + M * K + 4 * M * (K // 128)


def dequant_bytes(N, K):
    return N * K + 4 * (-(-N // 128)) * (-(-K // 128)) + 2 * N * K


def gemm_bytes(M, N, K, out_bytes=2):
    return M * K + 4 * M * (K // 128) + N * K + 4 * (-(-N // 128)) * (K // 128) + out_bytes * M * N


def moe_bytes(R, N, K, active_experts, out_bytes=2):
    per_expert = N * K + 4 * (-(-N // 128)) * (K // 128)
    return R * K + 4 * R * (K // 128) + active_experts * per_expert + out_bytes * R * N


# ------------------------------------------------------------------ timing

WARMUP_MIN_S = 0.25


def warm(launch, copies, warmup):
    """At least `warmup` calls and at least WARMUP_MIN_S seconds of them."""
    t0 = time.perf_counter()
    i = 0
    while i < warmup or time.perf_counter() - t0 < WARMUP_MIN_S:
        launch(i % copies)
        i += 1
        if i % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def timed(launch, copies, steps, warmup, graph=True):
    """Average duration (us) of `launch(i)` over `steps` back-to-back launches
    on one stream, bracketed by one event pair.  With graph=True (the
    secondary rows) the launches are first captured into a HIP graph and the
    timed region is one replay of it, so the host's per-launch cost (Python
    and ctypes, several us) does not pace short kernels; the headline GEMM is
    timed with plain launches."""
    warm(launch, copies, warmup)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                launch(i % copies)
        g.replay()                                 # first replay uploads the graph
        torch.cuda.synchronize()
        start.record()
        g.replay()
        end.record()
        torch.cuda.synchronize()
        del g
        return start.elapsed_time(end) * 1e3 / steps
    start.record()
    for i in range(steps):
        launch(i % copies)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) * 1e3 / steps


def n_copies(bytes_per_copy):
    return max(1, min(16, -(-ROTATE_FOOTPRINT // max(1, bytes_per_copy))))


def quantised_weight(N, K, seed, dev):
    w = inputs.normal_bf16_device((N, K), 0.02, seed, dev)
    q, s = fp8bs.weight_quant(w)
    return q, s


# ------------------------------------------------------------------ rows

def row_result(name, us, flops=None, nbytes=None, bound="hbm", extra=None):
    r = {"us": round(us, 3)}
    if flops:
        r["tflops"] = round(flops / us / 1e6, 2)
    if nbytes:
        r["gbs"] = round(nbytes / us / 1e3, 1)
        r["bytes"] = int(nbytes)
    if bound == "hbm":
        r["bound"] = "hbm"
        r["frac"] = round(nbytes / us / 1e3 / PEAK_HBM_GBS, 4)
    elif bound == "mfma":
        r["bound"] = "mfma"
        r["frac"] = round(flops / us / 1e6 / PEAK_FP8_TFLOPS, 4)
    if extra:
        r.update(extra)
    log(f"  {name:28s} {json.dumps(r)}")
    return r


def bench_linear_step(M, N, K, sid, steps, warmup, dev, fmt="fp32"):
    """The FP8 linear (act_quant then GEMM) of one workload.  Returns the wall
    time per step over the timed region, and each kernel's average duration
    from its own back-to-back timed region."""
    x = inputs.normal_bf16_device((M, K), 1.0, inputs.seed_for(sid, 0), dev)
    q, s = quantised_weight(N, K, inputs.seed_for(sid, 1), dev)
    xq = torch.empty((M, K), dtype=torch.float8_e4m3fn, device=dev)
    xs = torch.empty((M, K // 128), dtype=torch.float32, device=dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

    def step(_=0):
        fp8bs.fp8bs_act_quant(x, xq, xs, fmt)
        fp8bs.fp8bs_gemm(xq, xs, q, s, y)
    warm(step, 1, warmup)
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    aq = timed(lambda c: fp8bs.fp8bs_act_quant(x, xq, xs, fmt), 1, steps, warmup, graph=False)
    gm = timed(lambda c: fp8bs.fp8bs_gemm(xq, xs, q, s, y), 1, steps, warmup, graph=False)
    return wall_ms, aq, gm, (x, q, s)


def bench_linear_step_rotated(M, N, K, sid, steps, warmup, dev):
    """The headline step with x and W cycled over enough copies that the
    Infinity Cache cannot hold them (the headline step reuses one x and one
    W, which stay cache-resident); graph-replayed."""
    copies = n_copies(2 * M * K + N * K)
    xs = [inputs.normal_bf16_device((M, K), 1.0, inputs.seed_for(sid, 0) + 100 * c, dev)
          for c in range(copies)]
    ws = [quantised_weight(N, K, inputs.seed_for(sid, 1) + 100 * c, dev) for c in range(copies)]
    xq = torch.empty((M, K), dtype=torch.float8_e4m3fn, device=dev)
    xsc = torch.empty((M, K // 128), dtype=torch.float32, device=dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

    def step(c):
        fp8bs.fp8bs_act_quant(xs[c], xq, xsc, "fp32")
        fp8bs.fp8bs_gemm(xq, xsc, ws[c][0], ws[c][1], y)
    us = timed(step, copies, steps, warmup)
    del xs, ws
    return us, copies


def bench_decode(steps, warmup, dev, out):
    cfg = inputs.DECODE
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    x = inputs.normal_bf16((M, K), 1.0, inputs.seed_for(inputs.SEED_DECODE, 0), outlier_frac=0.01,
                           outlier_mult=50.0).to(dev)
    copies = n_copies(N * K)
    ws = [quantised_weight(N, K, inputs.seed_for(inputs.SEED_DECODE, 1) + 100 * c, dev) for c in range(copies)]
    xq, xs = fp8bs.act_quant(x)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    us = timed(lambda c: fp8bs.fp8bs_gemm(xq, xs, ws[c][0], ws[c][1], y), copies, steps, warmup)
    out["decode_gemm_32x18432x7168"] = row_result(
        "decode gemm", us, 2 * M * N * K, gemm_bytes(M, N, K), "hbm", {"weight_copies": copies})
    aq_us = timed(lambda c: fp8bs.fp8bs_act_quant(x, xq, xs, "fp32"), 1, steps, warmup)
    out["decode_act_quant_32x7168"] = row_result("decode act_quant", aq_us, None,
                                                 act_quant_bytes(M, K), "hbm")

    def step(c):
        fp8bs.fp8bs_act_quant(x, xq, xs, "fp32")
        fp8bs.fp8bs_gemm(xq, xs, ws[c][0], ws[c][1], y)
    st_us = timed(step, copies, steps, warmup)
    out["decode_linear_step"] = row_result(
        "decode linear step", st_us, 2 * M * N * K,
        act_quant_bytes(M, K) + gemm_bytes(M, N, K), "hbm")
    del ws


def bench_act_quant(steps, warmup, dev, out):
    for (M, K, fmt, sid) in [(4096, 7168, "fp32", inputs.SEED_PREFILL), (4096, 18432, "fp32", inputs.SEED_PREFILL),
                             (32768, 2048, "fp32", inputs.SEED_MOE), (1024, 7168, "ue8m0", inputs.SEED_UE8M0)]:
        nb = act_quant_bytes(M, K)
        copies = n_copies(nb)
        xs_in = [inputs.normal_bf16_device((M, K), 1.0, inputs.seed_for(sid, 50 + c), dev)
                 for c in range(copies)]
        qs = [torch.empty((M, K), dtype=torch.float8_e4m3fn, device=dev) for _ in range(copies)]
        ss = [torch.empty((M, K // 128), dtype=torch.float32, device=dev) for _ in range(copies)]
        us = timed(lambda c: fp8bs.fp8bs_act_quant(xs_in[c], qs[c], ss[c], fmt), copies, steps, warmup)
        out[f"act_quant_{M}x{K}_{fmt}"] = row_result(f"act_quant {M}x{K} {fmt}", us, None, nb, "hbm",
                                                     {"copies": copies})
        del xs_in, qs, ss
        # reference: a plain device copy moving the same bytes (half read, half
        # written), rotated and timed the same way -- what a streaming kernel of
        # this size reaches on this GPU
        half = nb // 2 // 16 * 16
        srcs = [torch.empty(half, dtype=torch.uint8, device=dev) for _ in range(copies)]
        dsts = [torch.empty(half, dtype=torch.uint8, device=dev) for _ in range(copies)]
        us = timed(lambda c: dsts[c].copy_(srcs[c]), copies, steps, warmup)
        out[f"copy_reference_{M}x{K}"] = row_result(f"device copy, bytes of {M}x{K}", us, None, 2 * half,
                                                    "hbm", {"copies": copies})
        del srcs, dsts


def bench_dequant(steps, warmup, dev, out):
    N, K = 18432, 7168
    nb = dequant_bytes(N, K)
    copies = n_copies(nb)
    ws = [quantised_weight(N, K, inputs.seed_for(inputs.SEED_UE8M0, 1) + 100 * c, dev) for c in range(copies)]
    ys = [torch.empty((N, K), dtype=torch.bfloat16, device=dev) for _ in range(copies)]
    us = timed(lambda c: fp8bs.fp8bs_weight_dequant(ws[c][0], ws[c][1], ys[c]), copies, steps, warmup)
    out["weight_dequant_18432x7168"] = row_result("weight_dequant", us, None, nb, "hbm",
                                                  {"copies": copies})
    del ws, ys


def bench_small_gemms(steps, warmup, dev, out):
    M = 1024
    for (N, K, tid) in [(1536, 7168, 2), (16384, 512, 4)]:
        x = inputs.normal_bf16_device((M, K), 1.0, inputs.seed_for(inputs.SEED_UE8M0, tid), dev)
        xq, xs = fp8bs.act_quant(x, "ue8m0")
        nb = gemm_bytes(M, N, K)
        copies = n_copies(nb)
        ws = [quantised_weight(N, K, inputs.seed_for(inputs.SEED_UE8M0, tid + 1) + 100 * c, dev) for c in range(copies)]
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        us = timed(lambda c: fp8bs.fp8bs_gemm(xq, xs, ws[c][0], ws[c][1], y), copies, steps, warmup)
        ai = 2 * M * N * K / nb
        out[f"gemm_{M}x{N}x{K}_ue8m0"] = row_result(
            f"gemm {M}x{N}x{K}", us, 2 * M * N * K, nb, "mfma" if ai > 629 else "hbm",
            {"copies": copies})
        del ws


def bench_moe(steps, warmup, dev, out):
    cfg = inputs.MOE
    E, T, topk = cfg["experts"], cfg["tokens"], cfg["topk"]
    route = inputs.zipf_topk_routing(T, E, topk, cfg["zipf_s"], inputs.seed_for(inputs.SEED_MOE, 9))
    off = torch.from_numpy(route["offsets"]).to(dev)
    R = int(route["offsets"][-1])
    active = int((route["counts"] > 0).sum())
    tok_idx = torch.from_numpy(route["token"]).to(dev)
    for proj, tid in (("up", 2), ("down", 3)):
        N, K = cfg[proj]["N"], cfg[proj]["K"]
        if proj == "up":
            tok = inputs.normal_bf16_device((T, K), 1.0, inputs.seed_for(inputs.SEED_MOE, 0), dev)
            x = tok.index_select(0, tok_idx)
            del tok
        else:
            x = inputs.normal_bf16_device((R, K), 1.0, inputs.seed_for(inputs.SEED_MOE, 1), dev)
        xq, xs = fp8bs.act_quant(x)
        w = inputs.normal_bf16_device((E * N, K), 0.02, inputs.seed_for(inputs.SEED_MOE, tid), dev)
        bq, bs = fp8bs.weight_quant(w)
        del w
        bq, bs = bq.view(E, N, K), bs.view(E, N // 128, K // 128)
        y = torch.empty((R, N), dtype=torch.bfloat16, device=dev)
        us = timed(lambda c: fp8bs.fp8bs_moe_gemm(xq, xs, bq, bs, off, y), 1, steps, warmup)
        out[f"moe_{proj}_{R}x{N}x{K}_E{E}"] = row_result(
            f"moe {proj}", us, 2 * R * N * K, moe_bytes(R, N, K, active), "hbm",
            {"active_experts": active})
        del bq, bs, y, x, xq, xs


def bench_moe_dispatch(steps, warmup, dev, out):
    """The steps around the expert GEMMs on the MoE workload: the route
    (counting sort of the 4096 x 8 expert ids), the expert inputs (act_quant of
    each token written to its 8 routed rows) and the combine of the
    down-projection output [32768, 7168] into 4096 tokens."""
    cfg = inputs.MOE
    E, T, topk = cfg["experts"], cfg["tokens"], cfg["topk"]
    g = inputs.zipf_topk_routing(T, E, topk, cfg["zipf_s"], inputs.seed_for(inputs.SEED_MOE, 9))
    idx = torch.from_numpy(g["choice"].astype(np.int32)).to(dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    row_token = torch.empty(T * topk, dtype=torch.int32, device=dev)
    row_of = torch.empty((T, topk), dtype=torch.int32, device=dev)
    ws = torch.empty(fp8bs.lib().fp8bs_moe_route_workspace_size(T, topk, E), dtype=torch.uint8,
                     device=dev)
    us = timed(lambda c: fp8bs.fp8bs_moe_route(idx, E, offsets, row_token, row_of, ws), 1, steps,
               warmup)
    route_bytes = 4 * T * topk + 4 * (E + 1) + 4 * T * topk + 4 * T * topk
    out[f"moe_route_{T}x{topk}_E{E}"] = row_result("moe route", us, None, route_bytes, "hbm")
    R = T * topk
    K, N = cfg["up"]["K"], cfg["down"]["N"]
    nb = 2 * T * K + R * K + 4 * R * (K // 128) + 4 * T * topk
    copies = n_copies(nb)
    xs = [inputs.normal_bf16_device((T, K), 1.0, inputs.seed_for(inputs.SEED_MOE, 60 + c), dev) for c in range(copies)]
    qs = [torch.empty((R, K), dtype=torch.float8_e4m3fn, device=dev) for _ in range(copies)]
    ss = [torch.empty((R, K // 128), dtype=torch.float32, device=dev) for _ in range(copies)]
    us = timed(lambda c: fp8bs.fp8bs_moe_quant_scatter(xs[c], row_of, qs[c], ss[c]), copies, steps,
               warmup)
    out[f"moe_quant_scatter_{T}x{K}_to_{R}"] = row_result("moe quant_scatter", us, None, nb, "hbm",
                                                          {"copies": copies})
    del xs, qs, ss
    nb = 2 * R * N + 8 * T * topk + 2 * T * N
    copies = n_copies(nb)
    outs = [inputs.normal_bf16_device((R, N), 1.0, inputs.seed_for(inputs.SEED_MOE, 70 + c), dev) for c in range(copies)]
    w = torch.from_numpy(inputs.routing_weights(T, topk, inputs.seed_for(inputs.SEED_MOE, 6))).to(dev)
    ys = [torch.empty((T, N), dtype=torch.bfloat16, device=dev) for _ in range(copies)]
    us = timed(lambda c: fp8bs.fp8bs_moe_combine(outs[c], w, row_of, ys[c]), copies, steps, warmup)
    out[f"moe_combine_{R}x{N}_to_{T}"] = row_result("moe combine", us, None, nb, "hbm",
                                                    {"copies": copies})
    del outs, ys


def bench_w8a16(steps, warmup, dev, out):
    """The BF16 path of the linear (weight dequantised in registers, bf16
    MFMA) on the prefill and decode shapes, against the bf16 MFMA peak (prefill)
    and HBM (decode)."""
    for (M, N, K, sid, bound) in [(4096, 18432, 7168, inputs.SEED_PREFILL, "mfma_bf16"),
                                  (32, 18432, 7168, inputs.SEED_DECODE, "hbm")]:
        x = inputs.normal_bf16_device((M, K), 1.0, inputs.seed_for(sid, 20), dev)
        nb = 2 * M * K + N * K + 4 * (-(-N // 128)) * (K // 128) + 2 * M * N
        copies = n_copies(N * K) if bound == "hbm" else 1
        ws = [quantised_weight(N, K, inputs.seed_for(sid, 21) + 100 * c, dev) for c in range(copies)]
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        us = timed(lambda c: fp8bs.fp8bs_w8a16_gemm(x, ws[c][0], ws[c][1], y), copies, steps, warmup)
        r = row_result(f"w8a16 gemm {M}x{N}x{K}", us, 2 * M * N * K, nb,
                       "hbm" if bound == "hbm" else None, {"copies": copies})
        if bound == "mfma_bf16":
            r["bound"] = "mfma_bf16"
            r["frac"] = round(2 * M * N * K / us / 1e6 / PEAK_BF16_TFLOPS, 4)
        out[f"w8a16_gemm_{M}x{N}x{K}"] = r
        del ws, x, y


def bench_ue8m0(steps, warmup, dev, out):
    """The ue8m0 fast path (power-of-two scales applied by the scaled MFMA) on
    the prefill GEMM and on the two GEMM shapes of the ue8m0 workload."""
    for (M, N, K, sid, tx, tw) in [(4096, 18432, 7168, inputs.SEED_PREFILL, 0, 1), (1024, 1536, 7168, inputs.SEED_UE8M0, 2, 3),
                                   (1024, 16384, 512, 5, 4, 5)]:
        x = inputs.normal_bf16_device((M, K), 1.0, inputs.seed_for(sid, tx), dev)
        xq, xs = fp8bs.act_quant(x, "ue8m0")
        del x
        nb = gemm_bytes(M, N, K)
        copies = 1 if M == 4096 else n_copies(nb)
        ws = []
        for c in range(copies):
            w = inputs.normal_bf16_device((N, K), 0.02, inputs.seed_for(sid, tw) + 100 * c, dev)
            ws.append(fp8bs.weight_quant(w, "ue8m0"))
            del w
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        us = timed(lambda c: fp8bs.fp8bs_gemm(xq, xs, ws[c][0], ws[c][1], y, ue8m0=True), copies,
                   steps, warmup)
        ai = 2 * M * N * K / nb
        out[f"gemm_ue8m0_scaled_mfma_{M}x{N}x{K}"] = row_result(
            f"gemm ue8m0 {M}x{N}x{K}", us, 2 * M * N * K, nb, "mfma" if ai > 629 else "hbm",
            {"copies": copies})
        del ws, xq, xs, y


def mla_bytes(side, T, H, dn, dv, R, out_bytes=2):
    """Algorithmic bytes of one MLA absorb launch: the wkv_b half the side
    reads (codes + scales), the bf16 input, the output."""
    rows = dn if side == "key" else dv
    w = H * rows * R + 4 * (H * rows // 128) * (R // 128)
    width, ncol = (dn, R) if side == "key" else (R, dv)
    return w + 2 * T * H * width + out_bytes * T * H * ncol


def bench_mla(steps, warmup, dev, out):
    """The MLA absorb products with an FP8 wkv_b (128 heads, dn = dv = 128,
    kv_lora_rank 512) at a decode batch and a prefill chunk; HBM-bound."""
    m = inputs.MLA
    H, dn, dv, R = m["heads"], m["dn"], m["dv"], m["R"]
    for T in (m["decode_tokens"], m["prefill_tokens"]):
        for side in ("key", "value"):
            nb = mla_bytes(side, T, H, dn, dv, R)
            copies = n_copies(nb)
            width = dn if side == "key" else R
            sets = []
            for c in range(copies):
                w = inputs.normal_bf16_device((H * (dn + dv), R), 0.02,
                                              inputs.seed_for(m["seed_id"], 1) + 100 * c, dev)
                q, sc = fp8bs.weight_quant(w)
                del w
                x = inputs.normal_bf16_device((T, H, width), 1.0, inputs.seed_for(m["seed_id"], 3) + 100 * c, dev)
                sets.append((x, q, sc))
            y = torch.empty((T, H, R if side == "key" else dv), dtype=torch.bfloat16, device=dev)
            fn = fp8bs.fp8bs_mla_absorb_key if side == "key" else fp8bs.fp8bs_mla_absorb_value
            us = timed(lambda c: fn(sets[c][0], sets[c][1], sets[c][2], y, dn, dv), copies, steps, warmup)
            flops = 2 * T * H * dn * R if side == "key" else 2 * T * H * R * dv
            out[f"mla_absorb_{side}_T{T}_H{H}"] = row_result(
                f"mla {side} T={T}", us, flops, nb, "hbm", {"copies": copies})
            del sets, y


def bench_vendor(steps, warmup, dev, out):
    """Context, not part of the path: the vendor library's plain FP8 GEMM
    (hipBLASLt through torch._scaled_mm, one per-tensor scale, so no block
    scales and no per-K-block fold) next to this library's GEMM with float32
    block scales and with ue8m0 scales, on the same codes, timed the same way
    (graph replays, no rotation), at the prefill up and down shapes and at
    4096 x 16384 x 7168, whose 256 x 256 tiles fill whole rounds of the CUs."""
    one = torch.ones((), dtype=torch.float32, device=dev)
    for (M, N, K) in [(4096, 18432, 7168), (4096, 7168, 18432), (4096, 16384, 7168)]:
        x = inputs.normal_bf16_device((M, K), 1.0, inputs.seed_for(inputs.SEED_PREFILL, 20), dev)
        w = inputs.normal_bf16_device((N, K), 0.02, inputs.seed_for(inputs.SEED_PREFILL, 21), dev)
        xq, xs = fp8bs.act_quant(x)
        xe, xse = fp8bs.act_quant(x, "ue8m0")
        wq, ws = fp8bs.weight_quant(w)
        we, wse = fp8bs.weight_quant(w, "ue8m0")
        del x, w
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        flops = 2 * M * N * K
        tag = f"{M}x{N}x{K}"
        us = timed(lambda c: torch._scaled_mm(xq, wq.t(), scale_a=one, scale_b=one,
                                              out_dtype=torch.bfloat16), 1, steps, warmup)
        out[f"vendor_hipblaslt_plain_fp8_{tag}"] = row_result(
            f"hipBLASLt plain fp8 {tag}", us, flops, None, "mfma",
            {"note": "torch._scaled_mm, per-tensor scales: context, not this library"})
        us = timed(lambda c: fp8bs.fp8bs_gemm(xq, xs, wq, ws, y), 1, steps, warmup)
        out[f"vendor_cmp_fp8bs_fp32_scales_{tag}"] = row_result(f"fp8bs fp32 scales {tag}", us, flops,
                                                                 None, "mfma")
        us = timed(lambda c: fp8bs.fp8bs_gemm(xe, xse, we, wse, y, ue8m0=True), 1, steps, warmup)
        out[f"vendor_cmp_fp8bs_ue8m0_{tag}"] = row_result(f"fp8bs ue8m0 {tag}", us, flops, None, "mfma")
        del xq, xs, xe, xse, wq, ws, we, wse, y
        torch.cuda.empty_cache()


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(x_dev, w_dev, budget_s, dev):
    """The oracle (binary64 C + OpenMP over all host threads) timed on the
    host cores.  Headline `value`: act_quant of a row sample of the prefill
    linear's x, then all N outputs of each sampled row, W quantised by the
    oracle itself from the same bf16 draw.  `per_op`: wall time of the
    oracle on each other hot-path row's workload shape (whole, or the sample
    stated), with seeded inputs of the same shapes and distributions."""
    import oracle
    oracle.build()
    per_op = {}

    def clock(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    def op(name, dt, work, unit, sample):
        per_op[name] = {"ms": round(dt * 1e3, 2), unit: round(work / dt / 1e9, 3), "sample": sample}
        log(f"  cpu {name:28s} {per_op[name]}")

    # act_quant, both formats (full tensors)
    for (M, K, fmt, sid) in [(4096, 7168, oracle.FMT_FP32, inputs.SEED_PREFILL),
                             (1024, 7168, oracle.FMT_UE8M0, inputs.SEED_UE8M0),
                             (32, 7168, oracle.FMT_FP32, inputs.SEED_DECODE)]:
        xb = inputs.bf16_bits(inputs.normal_bf16_device((M, K), 1.0, inputs.seed_for(sid, 50), dev).cpu())
        dt = clock(lambda: oracle.act_quant(xb, fmt))
        op(f"act_quant_{M}x{K}_{'ue8m0' if fmt else 'fp32'}", dt, act_quant_bytes(M, K), "gbs", "whole")
    # weight_dequant [18432, 7168] (whole)
    wq, ws = quantised_weight(18432, 7168, inputs.seed_for(inputs.SEED_UE8M0, 1), dev)
    q, sc = wq.view(torch.uint8).cpu().numpy(), ws.cpu().numpy()
    del wq, ws
    dt = clock(lambda: oracle.weight_dequant(q, sc))
    op("weight_dequant_18432x7168", dt, dequant_bytes(18432, 7168), "gbs", "whole")
    del q, sc
    # decode GEMM and the two GEMMs of the ue8m0 workload (whole)
    for (M, N, K, fmt) in [(32, 18432, 7168, oracle.FMT_FP32), (1024, 1536, 7168, oracle.FMT_UE8M0),
                           (1024, 16384, 512, oracle.FMT_UE8M0)]:
        xb = inputs.bf16_bits(inputs.normal_bf16_device((M, K), 1.0, inputs.seed_for(inputs.SEED_UE8M0, 2), dev).cpu())
        wb = inputs.bf16_bits(inputs.normal_bf16_device((N, K), 0.02, inputs.seed_for(inputs.SEED_UE8M0, 3), dev).cpu())
        a, a_s = oracle.act_quant(xb, fmt)
        b, b_s = oracle.weight_quant(wb)
        dt = clock(lambda: oracle.gemm(a, a_s, b, b_s))
        op(f"gemm_{M}x{N}x{K}", dt, 2 * M * N * K, "gflops", "whole")
    # grouped MoE up projection on 16 of the 256 experts: every 16th in
    # order of row count, so the sample spans the Zipf distribution
    cfg = inputs.MOE
    E, T, topk, N, K = cfg["experts"], cfg["tokens"], cfg["topk"], cfg["up"]["N"], cfg["up"]["K"]
    route = inputs.zipf_topk_routing(T, E, topk, cfg["zipf_s"], inputs.seed_for(inputs.SEED_MOE, 9))
    counts = np.diff(route["offsets"])
    pick = np.sort(np.argsort(counts, kind="stable")[::16])
    rows = int(counts[pick].sum())
    xb = inputs.bf16_bits(inputs.normal_bf16_device((rows, K), 1.0, inputs.seed_for(inputs.SEED_MOE, 0), dev).cpu())
    a, a_s = oracle.act_quant(xb, oracle.FMT_FP32)
    wb = inputs.bf16_bits(inputs.normal_bf16_device((len(pick) * N, K), 0.02, inputs.seed_for(inputs.SEED_MOE, 2),
                                                    dev).cpu())
    b, b_s = oracle.weight_quant(wb)
    off = np.concatenate([[0], np.cumsum(counts[pick])]).astype(np.int32)
    dt = clock(lambda: oracle.moe_gemm(a, a_s, b.reshape(len(pick), N, K),
                                       b_s.reshape(len(pick), N // 128, K // 128), off))
    op("moe_up_16_of_256_experts", dt, 2 * rows * N * K, "gflops",
       f"every 16th expert by row count of the Zipf routing ({rows} of {T * topk} rows)")
    del a, b, wb, xb

    # headline: the prefill linear on a row sample
    M, K = x_dev.shape
    N = w_dev.shape[0]
    b, b_s = oracle.weight_quant(inputs.bf16_bits(w_dev.cpu()))
    xb = inputs.bf16_bits(x_dev.cpu())

    def run(r):
        t0 = time.perf_counter()
        a, a_s = oracle.act_quant(xb[:r], oracle.FMT_FP32)
        oracle.gemm(a, a_s, b, b_s)
        return time.perf_counter() - t0

    dt0 = run(2) / 2                               # calibration
    rows = int(min(M, max(2, budget_s / max(dt0, 1e-4))))
    dt = run(rows)
    flops = 2 * rows * N * K
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "cpu_model": cpu_model(), "logical_cpus": os.cpu_count(),
            "sample": f"act_quant + binary64 block-scaled GEMM of the first {rows} of the {M} rows "
                      f"of the prefill linear (all {N} outputs per row, K={K}); {dt:.1f} s",
            "per_op": per_op}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--rows", default="all", help="secondary rows: all, none, or a comma list of "
                    "decode,act_quant,dequant,small,moe,dispatch,w8a16,ue8m0,mla,down,rotated,vendor "
                    "(vendor: the vendor library's plain FP8 GEMM next to this one's, for context)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a plain 1 GiB device copy (known traffic) so hardware byte "
                         "counters collected over this run can be scaled against it")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the block-scaled FP8 linear runs on a single MI355X here "
              "(no sharding, no collectives); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    fp8bs.lib()                                    # fails loudly if the library is missing
    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cfg = inputs.PREFILL
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    log(f"prefill fp8 linear M={M} N={N} K={K}: {args.warmup} warmup + {args.steps} timed steps")
    wall_ms, aq_us, gm_us, prefill_inputs = bench_linear_step(M, N, K, inputs.SEED_PREFILL, args.steps, args.warmup, dev)
    flops = 2 * M * N * K
    value = flops / (wall_ms * 1e-3) / 1e12
    rows = {}
    rows["prefill_up_act_quant_4096x7168"] = row_result("prefill act_quant", aq_us, None,
                                                        act_quant_bytes(M, K), "hbm")
    rows["prefill_up_gemm_4096x18432x7168"] = row_result("prefill gemm", gm_us, flops,
                                                         gemm_bytes(M, N, K), "mfma")
    sel = set(["decode", "act_quant", "dequant", "small", "moe", "dispatch", "w8a16", "ue8m0",
             "mla", "down", "rotated", "vendor"]) if args.rows == "all" else (
        set() if args.rows == "none" else set(args.rows.split(",")))
    if "down" in sel:
        d = cfg["down"]
        w2, a2, g2, _ = bench_linear_step(d["M"], d["N"], d["K"], inputs.SEED_PREFILL, args.steps, args.warmup, dev)
        rows["prefill_down_gemm_4096x7168x18432"] = row_result(
            "prefill down gemm", g2, 2 * d["M"] * d["N"] * d["K"], gemm_bytes(d["M"], d["N"], d["K"]),
            "mfma")
    if "rotated" in sel:
        r_us, r_copies = bench_linear_step_rotated(M, N, K, inputs.SEED_PREFILL, args.steps, args.warmup, dev)
        rows["prefill_linear_step_rotated"] = row_result(
            "prefill step, rotated", r_us, flops, act_quant_bytes(M, K) + gemm_bytes(M, N, K), "mfma",
            {"copies": r_copies})
    if "decode" in sel:
        bench_decode(args.steps, args.warmup, dev, rows)
    if "act_quant" in sel:
        bench_act_quant(args.steps, args.warmup, dev, rows)
    if "dequant" in sel:
        bench_dequant(args.steps, args.warmup, dev, rows)
    if "small" in sel:
        bench_small_gemms(args.steps, args.warmup, dev, rows)
    if "moe" in sel:
        bench_moe(args.steps, args.warmup, dev, rows)
    if "dispatch" in sel:
        bench_moe_dispatch(args.steps, args.warmup, dev, rows)
    if "w8a16" in sel:
        bench_w8a16(args.steps, args.warmup, dev, rows)
    if "ue8m0" in sel:
        bench_ue8m0(args.steps, args.warmup, dev, rows)
    if "mla" in sel:
        bench_mla(args.steps, args.warmup, dev, rows)
    if "vendor" in sel:
        try:
            bench_vendor(args.steps, args.warmup, dev, rows)
        except Exception as e:                     # context only: never fail the run for it
            rows["vendor_hipblaslt_plain_fp8"] = {"error": f"{type(e).__name__}: {e}"[:200]}
            torch.cuda.empty_cache()
    torch.cuda.empty_cache()

    gemm_tflops = flops / gm_us / 1e6
    traffic = None
    if GEMM_TRAFFIC["source_sha256"] is not None:
        import hashlib
        with open(GEMM_SOURCE, "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() == GEMM_TRAFFIC["source_sha256"]:
                traffic = GEMM_TRAFFIC["fetch_bytes"] + GEMM_TRAFFIC["write_bytes"]
    result = {
        "metric": "FP8 block-scaled GEMM TFLOP/s @M=4096,K=7168,N=18432; GB/s @M=32 decode",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": "prefill fp8 linear: act_quant x bf16 [4096,7168] + block-scaled FP8 "
                               "GEMM with W e4m3 [18432,7168], bf16 out",
                   "M": M, "N": N, "K": K, "block": 128, "scale_fmt": "fp32"},
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 2), "peak": PEAK_FP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tflops / PEAK_FP8_TFLOPS, 4),
                     "traffic": traffic, "kernel": GEMM_KERNEL,
                     "us_per_launch": round(gm_us, 3)},
    }
    if "decode_gemm_32x18432x7168" in rows:
        result["decode_gbs"] = rows["decode_gemm_32x18432x7168"]["gbs"]
    result["rows"] = rows
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle on a row sample (~{args.cpu_seconds:.0f} s)")
        px, _, _ = prefill_inputs
        w_bf16 = inputs.normal_bf16_device((N, K), 0.02, inputs.seed_for(inputs.SEED_PREFILL, 1), dev)
        result["cpu_baseline"] = cpu_baseline(px, w_bf16, args.cpu_seconds, dev)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
