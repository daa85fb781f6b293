#!/usr/bin/env python3
"""Throughput of the fine-grained FP8 GEMM path on one MI355X.

One step = the whole hot path over one batch: online 1x128 quantisation of the
activations X, online 128x128 quantisation of the weight W, and the
block-scaled FP8 GEMM with per-128-K-chunk FP32 promotion, Y = X W^T in bf16.
Inputs are resident in HBM before timing starts; outputs are preallocated.

Default workload: the large heavy-tail Fprop, X bf16 [16384, 7168] ~ Student-t(3),
W bf16 [18432, 7168] ~ N(0, 0.02), Y bf16 [16384, 18432].

Prints one JSON line: value = 2 M N K / step time (TFLOP/s including both
quantisers), plus the GEMM kernel's roofline (HIP-event time of the kernel
alone, on the stream it runs on) and the CPU oracle timed on a bounded sample
of the same workload. Kernels timed alone report the mean, median, p10 and p90
of --kernel-reps launches; the quantisers are also compared with the measured
streaming ceiling of their traffic (2 bytes read, 1 written per element), and
the probes measure what the promotion costs the matrix unit (clock) and how the
unit accumulates (report section 3.3.2's K = 4096 experiment).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP8 block-scaled GEMM TFLOP/s incl. quant (% of MFMA FP8 peak); quant GB/s"
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense FP8 MFMA (published)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E (published)

WORKLOADS = {
    "large": ("large heavy-tail fprop", 16384, 18432, 7168),
    "dense": ("dense fprop", 4096, 2048, 7168),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-ms", type=float, default=500.0,
                    help="untimed steps run back to back for this long before the warm-up steps: the GPU's "
                         "clock needs tens of milliseconds of sustained load to reach its steady state")
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="large")
    ap.add_argument("--kernel-reps", type=int, default=50, help="reps of each kernel timed alone")
    ap.add_argument("--no-probes", action="store_true", help="skip the ceilings and the matrix-unit probes")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip timing the dense, backward and MoE configurations' kernels")
    ap.add_argument("--cpu-rows", type=int, default=2048, help="oracle sample: rows of X")
    ap.add_argument("--cpu-wrows", type=int, default=8192, help="oracle sample: rows of W")
    ap.add_argument("--leg", choices=LEGS, default=None,
                    help="only launch one kernel of the bench (after one untimed launch) --leg-reps times: "
                         "the command the counter summaries under profiles/ are taken with")
    ap.add_argument("--leg-reps", type=int, default=5)
    ap.add_argument("--status-table", metavar="JSON", default=None,
                    help="print the measured-status rows (markdown) of a file holding this script's JSON line")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (reference for HBM byte counters)")
    return ap.parse_args()


def calibrate_copy():
    """A plain copy of known size: under rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE its
    readings give the factor between the counters and bytes moved."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read": n, "bytes_written": n, "reps": 3}), flush=True)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def status_table(path):
    """Markdown rows of the measured status, generated from a bench JSON line (the last
    line of `path` that parses as one), so that no figure is copied by hand."""
    d = None
    for line in open(path).read().splitlines():
        try:
            v = json.loads(line)
        except ValueError:
            continue
        if isinstance(v, dict) and "roofline" in v:
            d = v
    if d is None:
        raise SystemExit(f"{path}: no bench JSON line")

    def spread(st):
        return f"median {st['median']:.1f}, p10 {st['p10']:.1f}, p90 {st['p90']:.1f}" if st else ""

    def pct(x):
        return f"{100 * x:.1f}%"

    rows = []
    r, b, o, v = d["roofline"], d["breakdown"], d.get("other_configs", {}), d.get("variants", {})
    clk = (f"; {pct(r['frac_at_measured_clock'])} of the peak at the measured {r['clock_ghz']:.3f} GHz"
           if r.get("clock_ghz") else "")
    rows.append(("a6–a8 Fprop GEMM, large (16384×18432×7168)", r["kernel"],
                 f"{r['avg_us']:.1f} µs ({spread(r.get('us_stats'))}), {r['achieved']:.0f} TFLOP/s = "
                 f"{pct(r['frac'])} of 5.0 PF{clk}"))
    rows.append(("step: quant X + quant W + GEMM", "three kernels",
                 f"{d['ms_per_step']:.3f} ms, **{d['value']:.0f} TFLOP/s incl. quant = {pct(b['frac_of_fp8_peak_incl_quant'])}"
                 f" of 5.0 PF**"))
    for key, name, kern in (("quant_act", "a1–a3 activation 1×128 quantisation, X [16384, 7168]", "quant_act_rows_kernel"),
                            ("quant_w", "a4 weight 128×128 quantisation, W [18432, 7168]", "quant_w2_kernel")):
        rows.append((name, kern, f"{b[key + '_us']:.1f} µs cold ({spread(b.get(key + '_us_stats'))}), "
                                 f"{b[key + '_GBps'] / 1000:.2f} TB/s = {pct(b[key + '_frac_hbm'])} of 8 TB/s, "
                                 f"{pct(b[key + '_frac_ceiling'])} of the measured 2:1 streaming ceiling"))
    if "quant_act_128x1" in o:
        q = o["quant_act_128x1"]
        rows.append(("a5 128×1 token-direction quantisation, X [4096, 7168]", "quant_act_cols_kernel",
                     f"{q['us']:.1f} µs cold, {q['GBps'] / 1000:.2f} TB/s = {pct(q['frac_hbm'])} of 8 TB/s"
                     + (f", {pct(q['frac_ceiling'])} of the measured 2:1 streaming ceiling at this size"
                        if q.get("frac_ceiling") else "")))
    for key, name, kern in (("dense_fprop", "a6–a8 Fprop GEMM, dense (4096×2048×7168)", "gemm_kernel<FPROP>, 256×128 tiles"),
                            ("dgrad", "a6–a8 Dgrad GEMM (4096×7168×2048)", "gemm_kernel<DGRAD>, 256×224 tiles"),
                            ("wgrad", "a6–a8 Wgrad GEMM (2048×7168×4096, fp32 out)", "gemm_kernel<WGRAD>, 256×224 tiles")):
        if key in o:
            g = o[key]
            rows.append((name, kern, f"{g['us']:.1f} µs, {g['TFLOPs']:.0f} TFLOP/s = {pct(g['frac_fp8_peak'])} of 5.0 PF"))
    if "moe_grouped" in o:
        g = o["moe_grouped"]
        rows.append(("a9 grouped MoE Fprop (8 experts, 54 400 padded rows)", "gemm_kernel<FPROP, grouped>",
                     f"{g['us']:.1f} µs, {g['TFLOPs_routed_rows']:.0f} TFLOP/s on the routed rows = "
                     f"{pct(g['frac_fp8_peak_routed'])} of 5.0 PF"))
    if "requant_t_us" in b:
        rows.append(("NEXT-1 cache re-quantisation 1×128 → 128×1, X [16384, 7168]", "requant_t_kernel",
                     f"{b['requant_t_us']:.1f} µs cold, {b['requant_t_GBps'] / 1000:.2f} TB/s = "
                     f"{pct(b['requant_t_frac_hbm'])} of 8 TB/s"
                     + (f", {pct(b['requant_t_frac_ceiling'])} of the measured rate of a device copy of the same codes"
                        if "requant_t_frac_ceiling" in b else "")))
    if "e5m6_cache" in v:
        g = v["e5m6_cache"]
        rows.append(("A11 E5M6 activation cache 1×128, X [16384, 7168]", g["kernel"],
                     f"cache {g['cache_us']:.1f} µs cold, {g['cache_GBps'] / 1000:.2f} TB/s = {pct(g['cache_frac_hbm'])}"
                     f" of 8 TB/s; read back {g['read_back_us']:.1f} µs, {g['read_back_GBps'] / 1000:.2f} TB/s = "
                     f"{pct(g['read_back_frac_hbm'])}"))
        if "to_128x1_us" in g:
            rows.append(("A11 E5M6 cache → 128×1 FP8 tiles (backward operand), X [16384, 7168]", g["to_128x1_kernel"],
                         f"{g['to_128x1_us']:.1f} µs cold, {g['to_128x1_GBps'] / 1000:.2f} TB/s = "
                         f"{pct(g['to_128x1_frac_hbm'])} of 8 TB/s"))
    if "pow2_scales" in v:
        g = v["pow2_scales"]
        rows.append(("NEXT-2 power-of-two scales (large fprop)", g["kernel"],
                     f"GEMM {g['gemm_us']:.1f} µs, {g['gemm_TFLOPs']:.0f} TFLOP/s = {pct(g['gemm_TFLOPs'] / PEAK_FP8_TFLOPS)}"
                     f" of 5.0 PF; step {g['ms_per_step']:.3f} ms, {g['value']:.0f} TFLOP/s incl. quant"))
    if "producer_fusion" in v:
        g = v["producer_fusion"]
        rows.append(("NEXT-3 producer fusion (large fprop)", g["kernel"],
                     f"fused {g['fused_us']:.1f} µs against {g['separate_us']:.1f} µs for GEMM + quantiser of its output;"
                     f" {g['hbm_bytes_saved'] / 1e9:.2f} GB less HBM traffic per launch"))
    if "decode_grouped" in v:
        g = v["decode_grouped"]
        rows.append(("NEXT-4 decode grouped Fprop (853 rows, 8 × [2048, 7168])", g["kernel"],
                     f"{g['us']:.1f} µs cold ({spread(g.get('us_stats'))}), {g['GBps'] / 1000:.2f} TB/s = "
                     f"{pct(g['roofline']['frac'])} of 8 TB/s"
                     + (f"; without workspace (64-column full-K workgroups) {g['full_k_us']:.1f} µs"
                        if "full_k_us" in g else "")))
    c = d.get("cpu_baseline")
    if c:
        rows.append(("CPU oracle (numpy)", "oracle/", f"{c['value'] * 1000:.1f} GFLOP/s on {c['cores']} host threads ({c['sample']})"))
    print("| row | kernel | measured |")
    print("|---|---|---|")
    for row in rows:
        print("| " + " | ".join(row) + " |")


# kernels that --leg launches alone (each on the workload the bench times it on)
LEGS = ("fprop", "fprop_pow2", "quant_x", "quant_w", "dense", "dgrad", "wgrad", "qcol", "decode", "decode_fullk",
        "mfma_stream",
        "cache_e5m6", "uncache_e5m6", "requant_e5m6", "requant", "requant_exact", "grouped")


def run_leg(args):
    """Launch one kernel of the bench on its workload: one untimed launch, then
    --leg-reps launches, each timed by HIP events on its stream (the quantisers
    and the decode GEMM after a 512 MB read that evicts the MALL, as in the full
    bench), after about 300 ms of untimed launches that bring the clock to its
    sustained-load value. Under rocprofv3 the named kernel's dispatches are the
    last --leg-reps of its name; the operands' own quantisation runs first."""
    import torch

    import fp8_fine_grained_fp8bq_amd as fb
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(0)
    sp = torch.cuda.current_stream(dev).cuda_stream
    leg = args.leg
    cold = leg in ("quant_x", "quant_w", "qcol", "decode", "decode_fullk", "cache_e5m6", "uncache_e5m6",
                   "requant_e5m6", "requant", "requant_exact")
    flush = torch.ones(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev) if cold else None
    flops = nbytes = None

    def dev16(a):
        return torch.from_numpy(a.view(np.int16)).to(dev)

    if leg in ("cache_e5m6", "uncache_e5m6", "requant_e5m6"):
        cfg = workloads.large_fprop()
        _, M, _, K = WORKLOADS["large"]
        x = dev16(cfg.x)
        ldq_e = (K * 3 // 2 + 15) // 16 * 16
        xe = torch.empty((M, ldq_e), dtype=torch.uint8, device=dev)
        xes = torch.empty((K // 128, M), dtype=torch.float32, device=dev)
        yb = torch.empty((M, K), dtype=torch.int16, device=dev)
        nbytes = M * K * 2 + M * (K * 3 // 2) + M * (K // 128) * 4

        def cache():
            fb.fp8bq_cache_e5m6_1x128(x.data_ptr(), M, K, K, xe.data_ptr(), ldq_e, xes.data_ptr(), M, sp)

        def uncache():
            fb.fp8bq_uncache_e5m6_1x128(xe.data_ptr(), M, K, ldq_e, xes.data_ptr(), M, yb.data_ptr(), K, sp)

        def requant():
            fb.fp8bq_requant_e5m6_t_128x1(xe.data_ptr(), M, K, ldq_e, xes.data_ptr(), M, xet.data_ptr(), M,
                                          xets.data_ptr(), K, sp)
        if leg == "cache_e5m6":
            fn = cache
        elif leg == "uncache_e5m6":
            cache()
            fn = uncache
        else:
            xet = torch.empty((K, M), dtype=torch.uint8, device=dev)
            xets = torch.empty((M // 128, K), dtype=torch.float32, device=dev)
            nbytes = M * (K * 3 // 2) + M * (K // 128) * 4 + K * M + (M // 128) * K * 4
            cache()
            fn = requant
    elif leg in ("requant", "requant_exact"):
        # the power-of-two (or, requant_exact, the absmax/448) FP8 cache of X,
        # re-quantised to transposed 128x1 tiles
        cfg = workloads.large_fprop()
        _, M, _, K = WORKLOADS["large"]
        x = dev16(cfg.x)
        xq = torch.empty((M, K), dtype=torch.uint8, device=dev)
        xs = torch.empty((K // 128, M), dtype=torch.float32, device=dev)
        xqt = torch.empty((K, M), dtype=torch.uint8, device=dev)
        xst = torch.empty((M // 128, K), dtype=torch.float32, device=dev)
        fb.fp8bq_quant_act_1x128(x.data_ptr(), M, K, K, fb.ACT_ROWWISE | (0 if leg == "requant_exact" else fb.SCALE_POW2),
                                 xq.data_ptr(), K, xs.data_ptr(), M, sp)
        nbytes = 2 * M * K + 2 * (M * (K // 128) * 4)

        def fn():
            fb.fp8bq_requant_t_128x1(xq.data_ptr(), M, K, K, xs.data_ptr(), M, xqt.data_ptr(), M, xst.data_ptr(), K,
                                     0 if leg == "requant_exact" else fb.SCALE_POW2, sp)
    elif leg == "grouped":
        # MoE grouped Fprop: 8 local experts, Zipf top-8 routing, rows padded to 128
        moe = workloads.moe_fprop()
        G_m, N_m, K_m = moe.w.shape
        m_m = int(moe.row_off[-1])
        g_xq, g_xs = fb.quant_act_1x128(dev16(moe.x))
        g_wq = torch.empty((G_m, N_m, K_m), dtype=torch.uint8, device=dev)
        g_ws = torch.empty((G_m, N_m // 128, K_m // 128), dtype=torch.float32, device=dev)
        for e in range(G_m):
            q_e, s_e, _ = fb.quant_w_128x128(dev16(moe.w[e]))
            g_wq[e].copy_(q_e)
            g_ws[e].copy_(s_e)
        g_y = torch.empty((m_m, N_m), dtype=torch.bfloat16, device=dev)
        g_off = [int(v) for v in moe.row_off]
        flops = 2.0 * float(np.sum(moe.real_rows)) * N_m * K_m

        def fn():
            fb.fp8bq_grouped_gemm(G_m, g_off, N_m, K_m, g_xq.data_ptr(), K_m, g_xs.data_ptr(), m_m, g_wq.data_ptr(),
                                  K_m, g_ws.data_ptr(), K_m // 128, g_y.data_ptr(), N_m, 0, sp)
    elif leg in ("fprop", "fprop_pow2", "quant_x", "quant_w"):
        cfg = workloads.large_fprop()
        _, M, N, K = WORKLOADS["large"]
        x, w = dev16(cfg.x), dev16(cfg.w)
        fl = fb.SCALE_POW2 if leg == "fprop_pow2" else 0
        xq = torch.empty((M, K), dtype=torch.uint8, device=dev)
        xs = torch.empty((K // 128, M), dtype=torch.float32, device=dev)
        wq = torch.empty((N, K), dtype=torch.uint8, device=dev)
        ws = torch.empty((N // 128, K // 128), dtype=torch.float32, device=dev)
        y = torch.empty((M, N), dtype=torch.int16, device=dev)

        def qx():
            fb.fp8bq_quant_act_1x128(x.data_ptr(), M, K, K, fb.ACT_ROWWISE | fl, xq.data_ptr(), K, xs.data_ptr(), M, sp)

        def qw():
            fb.fp8bq_quant_w_128x128(w.data_ptr(), N, K, K, wq.data_ptr(), K, ws.data_ptr(), K // 128, None, N, fl, sp)

        def gemm():
            fb.fp8bq_gemm(fb.FPROP | fl, M, N, K, xq.data_ptr(), K, xs.data_ptr(), M, wq.data_ptr(), K,
                          ws.data_ptr(), K // 128, y.data_ptr(), N, sp)

        if leg == "quant_x":
            fn, nbytes = qx, M * K * 3 + (K // 128) * M * 4
        elif leg == "quant_w":
            fn, nbytes = qw, N * K * 3 + (N // 128) * (K // 128) * 4
        else:
            qx()
            qw()
            fn, flops = gemm, 2.0 * M * N * K
    elif leg in ("dense", "dgrad", "wgrad", "qcol"):
        dn = workloads.dense_fprop()
        o_x, o_w = dev16(dn.x), dev16(dn.w)
        Md, Nd, Kd = dn.x.shape[0], dn.w.shape[0], dn.x.shape[1]
        flops = 2.0 * Md * Nd * Kd
        if leg == "dense":
            o_xq, o_xs = fb.quant_act_1x128(o_x)
            o_wq, o_ws, _ = fb.quant_w_128x128(o_w)
            o_y = torch.empty((Md, Nd), dtype=torch.bfloat16, device=dev)

            def fn():
                fb.fp8bq_gemm(fb.FPROP, Md, Nd, Kd, o_xq.data_ptr(), Kd, o_xs.data_ptr(), Md, o_wq.data_ptr(), Kd,
                              o_ws.data_ptr(), Kd // 128, o_y.data_ptr(), Nd, sp)
        elif leg == "dgrad":
            o_dy = dev16(workloads.backward_dy())
            o_wq, o_ws, o_wqt = fb.quant_w_128x128(o_w, transposed_copy=True)
            o_dq, o_ds = fb.quant_act_1x128(o_dy)
            o_dx = torch.empty((Md, Kd), dtype=torch.bfloat16, device=dev)

            def fn():
                fb.fp8bq_gemm(fb.DGRAD, Md, Kd, Nd, o_dq.data_ptr(), Nd, o_ds.data_ptr(), Md, o_wqt.data_ptr(), Nd,
                              o_ws.data_ptr(), Kd // 128, o_dx.data_ptr(), Kd, sp)
        else:
            o_xqt = torch.empty((Kd, Md), dtype=torch.uint8, device=dev)
            o_xst = torch.empty((Md // 128, Kd), dtype=torch.float32, device=dev)

            def qcol_x():
                fb.fp8bq_quant_act_1x128(o_x.data_ptr(), Md, Kd, Kd, fb.ACT_COLWISE, o_xqt.data_ptr(), Md,
                                         o_xst.data_ptr(), Kd, sp)
            if leg == "qcol":
                fn, flops, nbytes = qcol_x, None, Md * Kd * 3 + (Md // 128) * Kd * 4
            else:
                o_dy = dev16(workloads.backward_dy())
                o_dqt = torch.empty((Nd, Md), dtype=torch.uint8, device=dev)
                o_dst = torch.empty((Md // 128, Nd), dtype=torch.float32, device=dev)
                fb.fp8bq_quant_act_1x128(o_dy.data_ptr(), Md, Nd, Nd, fb.ACT_COLWISE, o_dqt.data_ptr(), Md,
                                         o_dst.data_ptr(), Nd, sp)
                qcol_x()
                o_dw = torch.empty((Nd, Kd), dtype=torch.float32, device=dev)

                def fn():
                    fb.fp8bq_gemm(fb.WGRAD, Nd, Kd, Md, o_dqt.data_ptr(), Md, o_dst.data_ptr(), Nd, o_xqt.data_ptr(),
                                  Md, o_xst.data_ptr(), Kd, o_dw.data_ptr(), Kd, sp)
    elif leg in ("decode", "decode_fullk"):
        dec = workloads.moe_decode()
        G_d, N_d, K_d = dec.w.shape
        m_d = int(dec.row_off[-1])
        d_xq, d_xs = fb.quant_act_1x128(dev16(dec.x))
        d_wq = torch.empty((G_d, N_d, K_d), dtype=torch.uint8, device=dev)
        d_ws = torch.empty((G_d, N_d // 128, K_d // 128), dtype=torch.float32, device=dev)
        for e in range(G_d):
            q_e, s_e, _ = fb.quant_w_128x128(dev16(dec.w[e]))
            d_wq[e].copy_(q_e)
            d_ws[e].copy_(s_e)
        d_y = torch.empty((m_d, N_d), dtype=torch.bfloat16, device=dev)
        d_off = [int(v) for v in dec.row_off]
        nbytes = (G_d * N_d * K_d + G_d * (N_d // 128) * (K_d // 128) * 4 + m_d * K_d + m_d * (K_d // 128) * 4
                  + m_d * N_d * 2)

        d_need = fb.fp8bq_grouped_gemm_decode_workspace_size(G_d, d_off, N_d, K_d)
        d_wsp = fb.decode_workspace(d_need, dev)

        def fn():
            if leg == "decode":
                fb.fp8bq_grouped_gemm_decode_ws(G_d, d_off, N_d, K_d, d_xq.data_ptr(), K_d, d_xs.data_ptr(), m_d,
                                                d_wq.data_ptr(), K_d, d_ws.data_ptr(), K_d // 128, d_y.data_ptr(),
                                                N_d, d_wsp.data_ptr(), d_wsp.numel(), 0, sp)
            else:
                fb.fp8bq_grouped_gemm_decode(G_d, d_off, N_d, K_d, d_xq.data_ptr(), K_d, d_xs.data_ptr(), m_d,
                                             d_wq.data_ptr(), K_d, d_ws.data_ptr(), K_d // 128, d_y.data_ptr(), N_d,
                                             0, sp)
    else:   # mfma_stream: the matrix-unit probe without promotion (reference for the busy counters)
        from fp8_fine_grained_fp8bq_amd import probe
        codes = torch.randint(0, 0x7F, (1 << 22,), dtype=torch.uint8, device=dev)
        pscales = torch.full((64,), 1e-3, dtype=torch.float32, device=dev)
        sink = torch.empty((256 * 512,), dtype=torch.float32, device=dev)
        ticks = torch.zeros((512,), dtype=torch.int64, device=dev)
        iters = 2000
        flops = 2.0 * 16 * 16 * 128 * 32 * 8 * 256 * iters

        def fn():
            probe.fp8bq_probe_mfma_stream(0, iters, 256, codes.data_ptr(), pscales.data_ptr(), sink.data_ptr(),
                                          ticks.data_ptr(), sp)

    fn()
    torch.cuda.synchronize()
    # bring the clock to its sustained-load value first (untimed launches, about 300 ms)
    t0 = time.perf_counter()
    fn()
    torch.cuda.synchronize()
    first = max(time.perf_counter() - t0, 1e-5)
    for _ in range(min(400, int(0.3 / first) + 1)):
        if cold:
            flush.sum()
        fn()
    torch.cuda.synchronize()
    us = []
    for _ in range(args.leg_reps):
        if cold:
            flush.sum()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        us.append(a.elapsed_time(b) * 1e3)
    med = float(np.median(us))
    out = {"leg": leg, "reps": args.leg_reps, "us_median": round(med, 2), "us": [round(u, 2) for u in us]}
    if flops:
        out["TFLOPs"] = round(flops / (med * 1e-6) / 1e12, 1)
        out["flops_per_launch"] = flops
    if nbytes:
        out["GBps"] = round(nbytes / med / 1e3, 1)
        out["bytes_per_launch"] = nbytes
    print(json.dumps(out), flush=True)


# every file whose change alters the GEMM kernel's code (the counters taken for one
# build do not describe another)
GEMM_SOURCES = ["fp8_fine_grained_fp8bq_amd/csrc/gemm_kernels.h", "fp8_fine_grained_fp8bq_amd/csrc/gemm.hip",
                "fp8_fine_grained_fp8bq_amd/csrc/fp8_codec.h", "fp8_fine_grained_fp8bq_amd/csrc/internal.h",
                "fp8_fine_grained_fp8bq_amd/build.py"]


def gemm_sources_sha256() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in GEMM_SOURCES:
        h.update(rel.encode())
        h.update(open(os.path.join(ROOT, rel), "rb").read())
    return h.hexdigest()


def profile_values(name: str) -> dict:
    """Machine-readable `key: value` lines of a committed rocprofv3 summary, or {}
    when the GEMM sources have changed since it was taken (or it is missing)."""
    path = os.path.join(ROOT, "profiles", name)
    try:
        kv = dict(line.split(": ", 1) for line in open(path).read().splitlines()
                  if line.startswith("gemm_") and ": " in line)
    except OSError:
        return {}
    if kv.get("gemm_sources_sha256", "").strip() != gemm_sources_sha256():
        return {}
    return kv


def gemm_traffic():
    """HBM bytes per GEMM launch from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE, copy-calibrated), or None when stale or missing."""
    kv = profile_values("large_fprop_hbm_traffic.md")
    try:
        return int(kv["gemm_fetch_bytes_per_launch"]) + int(kv["gemm_write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def gemm_clock_ghz():
    """Shader clock under the GEMM from the committed counter summary
    (GRBM_GUI_ACTIVE per XCD / kernel duration), or None when stale or missing."""
    kv = profile_values("large_fprop_mfma_counters.md")
    try:
        return float(kv["gemm_clock_ghz"])
    except (KeyError, ValueError):
        return None


def stats(durs):
    d = np.asarray(durs, dtype=np.float64)
    return {"mean": float(d.mean()), "median": float(np.median(d)), "p10": float(np.percentile(d, 10)),
            "p90": float(np.percentile(d, 90)), "n": int(d.size)}


def rnd(st, nd=2):
    return {k: (round(v, nd) if isinstance(v, float) else v) for k, v in st.items()}


def cpu_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [d.get("num_threads", 1) for d in threadpool_info() if d.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return os.cpu_count() or 1


def main():
    args = parse()
    if args.status_table:
        status_table(args.status_table)
        return
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.leg:
        run_leg(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported by this build "
              "(the path is single-GPU; see the sharding notes in the design document).", flush=True)
        sys.exit(2)

    import torch

    import fp8_fine_grained_fp8bq_amd as fb
    import workloads

    name, M, N, K = WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream

    t0 = time.perf_counter()
    cfg = workloads.large_fprop() if args.workload == "large" else workloads.dense_fprop()
    log(f"[bench] generated {cfg.name} in {time.perf_counter() - t0:.1f}s")
    x = torch.from_numpy(cfg.x.view(np.int16)).to(dev)
    w = torch.from_numpy(cfg.w.view(np.int16)).to(dev)
    xq = torch.empty((M, K), dtype=torch.uint8, device=dev)
    xs = torch.empty((K // 128, M), dtype=torch.float32, device=dev)
    wq = torch.empty((N, K), dtype=torch.uint8, device=dev)
    ws = torch.empty((N // 128, K // 128), dtype=torch.float32, device=dev)
    y = torch.empty((M, N), dtype=torch.int16, device=dev)
    # > 256 MB MALL; read (not written) before each cold kernel, so no dirty lines are
    # left whose write-back would land inside the timed kernel
    flush = torch.ones(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def quant_x():
        fb.fp8bq_quant_act_1x128(x.data_ptr(), M, K, K, fb.ACT_ROWWISE, xq.data_ptr(), K, xs.data_ptr(), M, sp)

    def quant_w():
        fb.fp8bq_quant_w_128x128(w.data_ptr(), N, K, K, wq.data_ptr(), K, ws.data_ptr(), K // 128, None, N, 0, sp)

    def gemm():
        fb.fp8bq_gemm(fb.FPROP, M, N, K, xq.data_ptr(), K, xs.data_ptr(), M, wq.data_ptr(), K,
                      ws.data_ptr(), K // 128, y.data_ptr(), N, sp)

    def step():
        quant_x()
        quant_w()
        gemm()

    # the same step with power-of-two scales (the matrix instruction applies them)
    def quant_x_p2():
        fb.fp8bq_quant_act_1x128(x.data_ptr(), M, K, K, fb.ACT_ROWWISE | fb.SCALE_POW2, xq.data_ptr(), K,
                                 xs.data_ptr(), M, sp)

    def quant_w_p2():
        fb.fp8bq_quant_w_128x128(w.data_ptr(), N, K, K, wq.data_ptr(), K, ws.data_ptr(), K // 128, None, N,
                                 fb.SCALE_POW2, sp)

    def gemm_p2():
        fb.fp8bq_gemm(fb.FPROP | fb.SCALE_POW2, M, N, K, xq.data_ptr(), K, xs.data_ptr(), M, wq.data_ptr(), K,
                      ws.data_ptr(), K // 128, y.data_ptr(), N, sp)

    def step_p2():
        quant_x_p2()
        quant_w_p2()
        gemm_p2()

    # bring the GPU to its sustained-load clock first: a kernel timed after idling
    # runs up to ~15% slower than the same kernel after ~50 ms of back-to-back work
    def settle(ms):
        s0, n = time.perf_counter(), 0
        while (time.perf_counter() - s0) * 1e3 < ms:
            for _ in range(5):
                step()
            n += 5
            torch.cuda.synchronize()
        return n

    settle_steps = settle(args.settle_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] settled with {settle_steps} steps, warmup {args.warmup} steps done")

    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = ev0.elapsed_time(ev1) / args.steps
    flops = 2.0 * M * N * K
    value = flops / (ms_step * 1e-3) / 1e12
    log(f"[bench] {args.steps} steps: {ms_step:.3f} ms/step (wall {wall * 1e3 / args.steps:.3f}), {value:.1f} TFLOP/s")

    # each kernel alone; the quantisers after a 512 MB read that evicts the MALL
    # reps are queued back to back (no host wait between them, so the GPU does not
    # idle), after steps that bring the clock back up from any idle time before.
    # Warm short kernels (batch=True) are timed by one event pair around all reps:
    # a pair around each launch adds 6-13 us of dispatch gap to a 60-90 us kernel.
    def time_kernel(fn, reps, cold, batch=False):
        fn()                        # first touch of any buffer it writes happens outside the timing
        settle(min(150.0, args.settle_ms))
        if batch and not cold:
            # ten groups of back-to-back launches, one event pair per group: the
            # statistics are over group means
            groups, per = 10, max(1, reps // 10)
            evs = []
            for _ in range(groups):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                for _ in range(per):
                    fn()
                b.record(stream)
                evs.append((a, b))
            torch.cuda.synchronize()
            st = stats([a.elapsed_time(b) * 1e3 / per for a, b in evs])
            st["launches_per_sample"] = per
            return st
        evs = []
        for _ in range(reps):
            if cold:
                flush.sum()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            evs.append((a, b))
        torch.cuda.synchronize()
        return stats([a.elapsed_time(b) * 1e3 for a, b in evs])

    # power-of-two variant: the same number of timed steps
    for _ in range(args.warmup):
        step_p2()
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        step_p2()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_step_p2 = ev0.elapsed_time(ev1) / args.steps
    st_tg_p2 = time_kernel(gemm_p2, args.kernel_reps, False)
    tg_p2 = st_tg_p2["mean"]
    log(f"[bench] power-of-two scales: {ms_step_p2:.3f} ms/step, GEMM {tg_p2:.1f} us")

    # transposing re-quantisation (1x128 -> 128x1) of the power-of-two cache of X,
    # in buffers of its own (time_kernel's settling steps rewrite xq / xs with
    # the absmax/448 cache)
    xq_c = torch.empty((M, K), dtype=torch.uint8, device=dev)
    xs_c = torch.empty((K // 128, M), dtype=torch.float32, device=dev)
    fb.fp8bq_quant_act_1x128(x.data_ptr(), M, K, K, fb.ACT_ROWWISE | fb.SCALE_POW2, xq_c.data_ptr(), K,
                             xs_c.data_ptr(), M, sp)
    xqt = torch.empty((K, M), dtype=torch.uint8, device=dev)
    xst = torch.empty((M // 128, K), dtype=torch.float32, device=dev)

    def requant():
        fb.fp8bq_requant_t_128x1(xq_c.data_ptr(), M, K, K, xs_c.data_ptr(), M, xqt.data_ptr(), M, xst.data_ptr(),
                                 K, fb.SCALE_POW2, sp)

    requant()
    st_t_rq = time_kernel(requant, args.kernel_reps, True)
    t_rq = st_t_rq["mean"]
    bytes_rq = 2 * M * K + 2 * (M * (K // 128) * 4)
    # its ceiling: the runtime's device copy of the same code bytes (read 1 B, write
    # 1 B per element; the re-quantisation also moves the scales, 0.8% more bytes)

    def copy_codes():
        xqt.view(-1).copy_(xq_c.view(-1))

    st_cp_rq = time_kernel(copy_codes, args.kernel_reps, True)
    log(f"[bench] requant 1x128 -> 128x1: {t_rq:.1f} us ({bytes_rq / t_rq / 1e3:.0f} GB/s); "
        f"copy of the codes {st_cp_rq['mean']:.1f} us")
    del xqt, xst, xq_c, xs_c

    # E5M6 activation cache of X (1x128 tiles, power-of-two scales, 12-bit codes
    # packed two per 3 bytes) and its inverse, both cold
    nb_e = K * 3 // 2
    ldq_e = (nb_e + 15) // 16 * 16
    xe = torch.empty((M, ldq_e), dtype=torch.uint8, device=dev)
    xes = torch.empty((K // 128, M), dtype=torch.float32, device=dev)

    def cache_e5m6():
        fb.fp8bq_cache_e5m6_1x128(x.data_ptr(), M, K, K, xe.data_ptr(), ldq_e, xes.data_ptr(), M, sp)

    def uncache_e5m6():
        fb.fp8bq_uncache_e5m6_1x128(xe.data_ptr(), M, K, ldq_e, xes.data_ptr(), M, y.data_ptr(), K, sp)

    cache_e5m6()
    st_t_ce = time_kernel(cache_e5m6, args.kernel_reps, True)
    uncache_e5m6()
    st_t_ue = time_kernel(uncache_e5m6, args.kernel_reps, True)
    bytes_e5m6 = M * K * 2 + M * nb_e + M * (K // 128) * 4
    log(f"[bench] E5M6 cache {st_t_ce['mean']:.1f} us, read back {st_t_ue['mean']:.1f} us "
        f"({bytes_e5m6 / st_t_ce['mean'] / 1e3:.0f} / {bytes_e5m6 / st_t_ue['mean'] / 1e3:.0f} GB/s)")
    # the backward use of the E5M6 cache: 128x1 FP8 tiles (power-of-two scales), transposed
    xet = torch.empty((K, M), dtype=torch.uint8, device=dev)
    xets = torch.empty((M // 128, K), dtype=torch.float32, device=dev)

    def requant_e5m6():
        fb.fp8bq_requant_e5m6_t_128x1(xe.data_ptr(), M, K, ldq_e, xes.data_ptr(), M, xet.data_ptr(), M,
                                      xets.data_ptr(), K, sp)

    cache_e5m6()
    requant_e5m6()
    st_t_re = time_kernel(requant_e5m6, args.kernel_reps, True)
    bytes_re = M * nb_e + M * (K // 128) * 4 + K * M + (M // 128) * K * 4
    log(f"[bench] E5M6 cache -> 128x1 FP8: {st_t_re['mean']:.1f} us ({bytes_re / st_t_re['mean'] / 1e3:.0f} GB/s)")
    del xe, xes, xet, xets

    # producer fusion: the GEMM quantises its own output (1x128 tiles) for the
    # next GEMM, against the GEMM followed by the quantiser of its bf16 output
    yq = torch.empty((M, N), dtype=torch.uint8, device=dev)
    ysq = torch.empty((N // 128, M), dtype=torch.float32, device=dev)

    def gemm_quant_out():
        fb.fp8bq_gemm_quant(fb.FPROP, M, N, K, xq.data_ptr(), K, xs.data_ptr(), M, wq.data_ptr(), K,
                            ws.data_ptr(), K // 128, None, N, yq.data_ptr(), N, ysq.data_ptr(), M, 0, sp)

    def gemm_then_quant():
        gemm()
        fb.fp8bq_quant_act_1x128(y.data_ptr(), M, N, N, fb.ACT_ROWWISE, yq.data_ptr(), N, ysq.data_ptr(), M, sp)

    quant_x()
    quant_w()
    gemm_quant_out()
    gemm_then_quant()
    st_t_fq = time_kernel(gemm_quant_out, args.kernel_reps, False)
    t_fq = st_t_fq["mean"]
    st_t_sq = time_kernel(gemm_then_quant, args.kernel_reps, False)
    t_sq = st_t_sq["mean"]
    log(f"[bench] GEMM + output quantisation: fused {t_fq:.1f} us, separate {t_sq:.1f} us")

    # decode-shape grouped Fprop (memory-bound): 256 tokens routed top-8, the 8 local
    # experts' rows unpadded; timed cold (MALL evicted), as weights are in a real decode step
    dec = workloads.moe_decode()
    G_d, N_d, K_d = dec.w.shape
    m_d = int(dec.row_off[-1])
    d_xq, d_xs = fb.quant_act_1x128(torch.from_numpy(dec.x.view(np.int16)).to(dev))
    d_wq = torch.empty((G_d, N_d, K_d), dtype=torch.uint8, device=dev)
    d_ws = torch.empty((G_d, N_d // 128, K_d // 128), dtype=torch.float32, device=dev)
    for e in range(G_d):
        q_e, s_e, _ = fb.quant_w_128x128(torch.from_numpy(dec.w[e].view(np.int16)).to(dev))
        d_wq[e].copy_(q_e)
        d_ws[e].copy_(s_e)
    d_y = torch.empty((m_d, N_d), dtype=torch.bfloat16, device=dev)
    d_off = [int(v) for v in dec.row_off]

    # the workspace form (experts above 32 rows as 128-column half-K pairs); its
    # workspace is allocated and zeroed here, outside the timed region
    d_need = fb.fp8bq_grouped_gemm_decode_workspace_size(G_d, d_off, N_d, K_d)
    d_wsp = fb.decode_workspace(d_need, dev)

    def decode():
        fb.fp8bq_grouped_gemm_decode_ws(G_d, d_off, N_d, K_d, d_xq.data_ptr(), K_d, d_xs.data_ptr(), m_d,
                                        d_wq.data_ptr(), K_d, d_ws.data_ptr(), K_d // 128, d_y.data_ptr(), N_d,
                                        d_wsp.data_ptr(), d_wsp.numel(), 0, sp)

    def decode_fullk():
        fb.fp8bq_grouped_gemm_decode(G_d, d_off, N_d, K_d, d_xq.data_ptr(), K_d, d_xs.data_ptr(), m_d,
                                     d_wq.data_ptr(), K_d, d_ws.data_ptr(), K_d // 128, d_y.data_ptr(), N_d, 0, sp)

    decode_fullk()
    st_t_dec0 = time_kernel(decode_fullk, args.kernel_reps, True)
    decode()
    st_t_dec = time_kernel(decode, args.kernel_reps, True)
    t_dec = st_t_dec["mean"]
    bytes_dec = (G_d * N_d * K_d + G_d * (N_d // 128) * (K_d // 128) * 4 + m_d * K_d + m_d * (K_d // 128) * 4
                 + m_d * N_d * 2)
    log(f"[bench] decode grouped Fprop ({m_d} rows): {t_dec:.1f} us ({bytes_dec / t_dec / 1e3:.0f} GB/s)")

    # the other configurations' kernels, each timed alone (GEMMs warm, quantisers cold):
    # dense fprop, the backward pair (Dgrad, Wgrad with token-direction 128x1
    # quantisation) and the MoE grouped fprop
    others = {}
    if not args.no_other_configs:
        t0 = time.perf_counter()
        dn = workloads.dense_fprop()
        dyb = workloads.backward_dy()
        moe = workloads.moe_fprop()
        log(f"[bench] generated the other configurations in {time.perf_counter() - t0:.1f}s")
        o_x = torch.from_numpy(dn.x.view(np.int16)).to(dev)
        o_w = torch.from_numpy(dn.w.view(np.int16)).to(dev)
        o_dy = torch.from_numpy(dyb.view(np.int16)).to(dev)
        Md, Nd, Kd = dn.x.shape[0], dn.w.shape[0], dn.x.shape[1]
        o_xq, o_xs = fb.quant_act_1x128(o_x)
        o_wq, o_ws, o_wqt = fb.quant_w_128x128(o_w, transposed_copy=True)
        o_y = torch.empty((Md, Nd), dtype=torch.bfloat16, device=dev)
        o_dq, o_ds = fb.quant_act_1x128(o_dy)
        o_dx = torch.empty((Md, Kd), dtype=torch.bfloat16, device=dev)
        o_dqt = torch.empty((Nd, Md), dtype=torch.uint8, device=dev)
        o_dst = torch.empty((Md // 128, Nd), dtype=torch.float32, device=dev)
        o_xqt = torch.empty((Kd, Md), dtype=torch.uint8, device=dev)
        o_xst = torch.empty((Md // 128, Kd), dtype=torch.float32, device=dev)
        o_dw = torch.empty((Nd, Kd), dtype=torch.float32, device=dev)

        def o_fprop():
            fb.fp8bq_gemm(fb.FPROP, Md, Nd, Kd, o_xq.data_ptr(), Kd, o_xs.data_ptr(), Md, o_wq.data_ptr(), Kd,
                          o_ws.data_ptr(), Kd // 128, o_y.data_ptr(), Nd, sp)

        def o_dgrad():
            fb.fp8bq_gemm(fb.DGRAD, Md, Kd, Nd, o_dq.data_ptr(), Nd, o_ds.data_ptr(), Md, o_wqt.data_ptr(), Nd,
                          o_ws.data_ptr(), Kd // 128, o_dx.data_ptr(), Kd, sp)

        def o_qcol_dy():
            fb.fp8bq_quant_act_1x128(o_dy.data_ptr(), Md, Nd, Nd, fb.ACT_COLWISE, o_dqt.data_ptr(), Md,
                                     o_dst.data_ptr(), Nd, sp)

        def o_qcol_x():
            fb.fp8bq_quant_act_1x128(o_x.data_ptr(), Md, Kd, Kd, fb.ACT_COLWISE, o_xqt.data_ptr(), Md,
                                     o_xst.data_ptr(), Kd, sp)

        def o_wgrad():
            fb.fp8bq_gemm(fb.WGRAD, Nd, Kd, Md, o_dqt.data_ptr(), Md, o_dst.data_ptr(), Nd, o_xqt.data_ptr(), Md,
                          o_xst.data_ptr(), Kd, o_dw.data_ptr(), Kd, sp)

        for fn in (o_fprop, o_dgrad, o_qcol_dy, o_qcol_x, o_wgrad):
            fn()
        st_t_of = time_kernel(o_fprop, args.kernel_reps, False, batch=True)
        t_of = st_t_of["mean"]
        st_t_od = time_kernel(o_dgrad, args.kernel_reps, False, batch=True)
        t_od = st_t_od["mean"]
        st_t_ow = time_kernel(o_wgrad, args.kernel_reps, False, batch=True)
        t_ow = st_t_ow["mean"]
        st_t_qc = time_kernel(o_qcol_x, args.kernel_reps, True)
        t_qc = st_t_qc["mean"]
        # its ceiling at this size: the 2:1 stream over the same elements, cold
        st_s_qc = None
        if not args.no_probes:
            from fp8_fine_grained_fp8bq_amd import probe

            def o_stream_x():
                probe.fp8bq_probe_stream_2to1(o_x.data_ptr(), o_xqt.data_ptr(), Md * Kd, sp)

            st_s_qc = time_kernel(o_stream_x, args.kernel_reps, True)
        f_d = 2.0 * Md * Nd * Kd
        b_qc = Md * Kd * 3 + (Md // 128) * Kd * 4
        others["dense_fprop"] = {"what": f"GEMM {Md}x{Nd}x{Kd} (bf16 out)", "us": round(t_of, 2),
                                 "TFLOPs": round(f_d / (t_of * 1e-6) / 1e12, 1),
                                 "frac_fp8_peak": round(f_d / (t_of * 1e-6) / 1e12 / PEAK_FP8_TFLOPS, 4),
                                 "us_stats": rnd(st_t_of)}
        others["dgrad"] = {"what": f"dX = dY W: GEMM {Md}x{Kd}x{Nd} (bf16 out)", "us": round(t_od, 2),
                           "TFLOPs": round(f_d / (t_od * 1e-6) / 1e12, 1),
                           "frac_fp8_peak": round(f_d / (t_od * 1e-6) / 1e12 / PEAK_FP8_TFLOPS, 4),
                           "us_stats": rnd(st_t_od)}
        others["wgrad"] = {"what": f"dW = dY^T X: GEMM {Nd}x{Kd}x{Md} over tokens, 128x1-quantised operands (fp32 out)",
                           "us": round(t_ow, 2), "TFLOPs": round(f_d / (t_ow * 1e-6) / 1e12, 1),
                           "frac_fp8_peak": round(f_d / (t_ow * 1e-6) / 1e12 / PEAK_FP8_TFLOPS, 4),
                           "us_stats": rnd(st_t_ow)}
        others["quant_act_128x1"] = {"what": f"token-direction (128x1) quantisation of X [{Md}, {Kd}], transposed out",
                                     "us": round(t_qc, 2), "GBps": round(b_qc / t_qc / 1e3, 1),
                                     "frac_hbm": round(b_qc / t_qc / 1e3 / PEAK_HBM_GBS, 4), "us_stats": rnd(st_t_qc),
                                     "ceiling_us": round(st_s_qc["mean"], 2) if st_s_qc else None,
                                     "frac_ceiling": round(st_s_qc["mean"] / t_qc, 4) if st_s_qc else None}
        del o_x, o_w, o_dy, o_y, o_dx, o_dw
        # MoE grouped fprop (8 local experts, Zipf top-8 routing, rows padded to 128)
        G_m, N_m, K_m = moe.w.shape
        m_m = int(moe.row_off[-1])
        g_xq, g_xs = fb.quant_act_1x128(torch.from_numpy(moe.x.view(np.int16)).to(dev))
        g_wq = torch.empty((G_m, N_m, K_m), dtype=torch.uint8, device=dev)
        g_ws = torch.empty((G_m, N_m // 128, K_m // 128), dtype=torch.float32, device=dev)
        for e in range(G_m):
            q_e, s_e, _ = fb.quant_w_128x128(torch.from_numpy(moe.w[e].view(np.int16)).to(dev))
            g_wq[e].copy_(q_e)
            g_ws[e].copy_(s_e)
        g_y = torch.empty((m_m, N_m), dtype=torch.bfloat16, device=dev)
        g_off = [int(v) for v in moe.row_off]

        def o_grouped():
            fb.fp8bq_grouped_gemm(G_m, g_off, N_m, K_m, g_xq.data_ptr(), K_m, g_xs.data_ptr(), m_m, g_wq.data_ptr(),
                                  K_m, g_ws.data_ptr(), K_m // 128, g_y.data_ptr(), N_m, 0, sp)

        o_grouped()
        st_t_og = time_kernel(o_grouped, args.kernel_reps, False, batch=True)
        t_og = st_t_og["mean"]
        f_real = 2.0 * float(np.sum(moe.real_rows)) * N_m * K_m
        others["moe_grouped"] = {"what": f"{moe.name}: {m_m} rows padded to 128 per expert "
                                         f"({int(np.sum(moe.real_rows))} routed)",
                                 "us": round(t_og, 2), "TFLOPs_routed_rows": round(f_real / (t_og * 1e-6) / 1e12, 1),
                                 "TFLOPs_padded_rows": round(2.0 * m_m * N_m * K_m / (t_og * 1e-6) / 1e12, 1),
                                 "frac_fp8_peak_routed": round(f_real / (t_og * 1e-6) / 1e12 / PEAK_FP8_TFLOPS, 4),
                                 "us_stats": rnd(st_t_og)}
        log(f"[bench] other configs: dense {t_of:.1f} us, dgrad {t_od:.1f} us, wgrad {t_ow:.1f} us, "
            f"128x1 quant {t_qc:.1f} us, MoE grouped {t_og:.1f} us")

    st_tq_x = time_kernel(quant_x, args.kernel_reps, True)
    tq_x = st_tq_x["mean"]
    st_tq_w = time_kernel(quant_w, args.kernel_reps, True)
    tq_w = st_tq_w["mean"]
    st_tg = time_kernel(gemm, args.kernel_reps, False)
    tg = st_tg["mean"]
    bytes_qx = M * K * 3 + M * (K // 128) * 4
    bytes_qw = N * K * 3 + (N // 128) * (K // 128) * 4
    gemm_tflops = flops / (tg * 1e-6) / 1e12
    log(f"[bench] quant X {tq_x:.1f} us ({bytes_qx / tq_x / 1e3:.0f} GB/s), quant W {tq_w:.1f} us "
        f"({bytes_qw / tq_w / 1e3:.0f} GB/s), GEMM {tg:.1f} us ({gemm_tflops:.0f} TFLOP/s)")

    # measured ceilings of the quantisers' traffic (cold): a stream reading 2 bytes and
    # writing 1 per element with no arithmetic, and the runtime's device copy
    ceilings, probes = {}, {}
    if not args.no_probes:
        from fp8_fine_grained_fp8bq_amd import probe
        qbuf = torch.empty((N, K), dtype=torch.uint8, device=dev)

        def stream_x():
            probe.fp8bq_probe_stream_2to1(x.data_ptr(), qbuf.data_ptr(), M * K, sp)

        def stream_w():
            probe.fp8bq_probe_stream_2to1(w.data_ptr(), qbuf.data_ptr(), N * K, sp)

        cbuf = torch.empty_like(x)

        def copy_x():
            cbuf.copy_(x)

        st_sx = time_kernel(stream_x, args.kernel_reps, True)
        st_sw = time_kernel(stream_w, args.kernel_reps, True)
        st_cp = time_kernel(copy_x, args.kernel_reps, True)
        ceilings = {
            "stream_2to1_X": {"what": f"read 2 B / write 1 B per element over X [{M}, {K}], no arithmetic, cold",
                              "us": round(st_sx["mean"], 2), "GBps": round(M * K * 3 / st_sx["mean"] / 1e3, 1),
                              "us_stats": rnd(st_sx)},
            "stream_2to1_W": {"what": f"read 2 B / write 1 B per element over W [{N}, {K}], no arithmetic, cold",
                              "us": round(st_sw["mean"], 2), "GBps": round(N * K * 3 / st_sw["mean"] / 1e3, 1),
                              "us_stats": rnd(st_sw)},
            "device_copy_X": {"what": f"device-to-device copy of X ({M * K * 2 / 1e6:.0f} MB read + written), cold",
                              "us": round(st_cp["mean"], 2), "GBps": round(M * K * 4 / st_cp["mean"] / 1e3, 1),
                              "us_stats": rnd(st_cp)},
        }
        del qbuf, cbuf
        log(f"[bench] ceilings: stream 2:1 X {ceilings['stream_2to1_X']['GBps']} GB/s, "
            f"W {ceilings['stream_2to1_W']['GBps']} GB/s, copy {ceilings['device_copy_X']['GBps']} GB/s")

        # what the promotion costs the matrix unit: the same MFMA stream with and without
        # the four FMAs per instruction, the unit kept busy in both (time = clock)
        quant_x()
        codes = xq.view(-1)[: 1 << 22].clone()      # 4 MiB of the workload's own E4M3 codes
        pscales = torch.full((64,), 1e-3, dtype=torch.float32, device=dev)
        sink = torch.empty((256 * 512,), dtype=torch.float32, device=dev)
        ticks = torch.zeros((512,), dtype=torch.int64, device=dev)
        iters = 20000
        pw = {}
        for fold in (0, 1, 0, 1):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            probe.fp8bq_probe_mfma_stream(fold, iters, 256, codes.data_ptr(), pscales.data_ptr(), sink.data_ptr(),
                                          ticks.data_ptr(), sp)
            b.record(stream)
            torch.cuda.synchronize()
            us = a.elapsed_time(b) * 1e3
            tk = ticks.cpu().numpy().reshape(256, 2).astype(np.float64)
            pw[fold] = {"us": round(us, 1),
                        "TFLOPs": round(2.0 * 16 * 16 * 128 * 32 * 8 * 256 * iters / (us * 1e-6) / 1e12, 1),
                        "shader_clock_ghz": round(float(tk[:, 0].sum() / tk[:, 1].sum()) * 0.1, 3)}
        probes["promotion_power"] = {
            "what": "256 workgroups x 8 waves, each 20000 x 32 independent 16x16x128 FP8 MFMAs on register-resident "
                    "fragments; with_fold adds the exact-scale GEMM's promotion (4 FMAs per MFMA)",
            "mfma_only": pw[0], "with_fold": pw[1],
            "time_ratio": round(pw[1]["us"] / pw[0]["us"], 4),
            "clock_note": "shader clock = s_memtime ticks / s_memrealtime ticks x 0.1 GHz",
        }
        del codes, sink
        # accumulation inside the unit against promotion (report section 3.3.2): two
        # random 16 x 4096 E4M3 matrices, errors against the exact integer dot product
        from oracle import e4m3 as oe
        rng = np.random.default_rng(7)
        ah = [oe.encode((r * (448.0 / np.abs(r).max())).astype(np.float32)) for r in
              (rng.standard_normal((16, 4096)), rng.standard_normal((16, 4096)))]
        da, db = torch.from_numpy(ah[0]).to(dev), torch.from_numpy(ah[1]).to(dev)
        ch = torch.empty((16, 16), dtype=torch.float32, device=dev)
        pr = torch.empty((16, 16), dtype=torch.float32, device=dev)
        probe.fp8bq_probe_mfma_accum(da.data_ptr(), db.data_ptr(), 4096, ch.data_ptr(), pr.data_ptr(), sp)
        torch.cuda.synchronize()
        ia, ib = (np.round(oe.decode(a_) * 512.0).astype(np.int64) for a_ in ah)
        exact = (ia @ ib.T).astype(np.float64) * 2.0 ** -18
        absum = (np.abs(ia) @ np.abs(ib).T).astype(np.float64) * 2.0 ** -18
        acc = {}
        for nm, t in (("chained_in_unit", ch), ("promoted_every_128", pr)):
            err = np.abs(t.cpu().numpy().astype(np.float64) - exact)
            acc[nm] = {"max_err_over_sum_abs": float((err / absum).max()),
                       "max_rel_err": float((err[exact != 0] / np.abs(exact[exact != 0])).max())}
        probes["accumulation_k4096"] = {"what": "16x16x4096 product of two random E4M3 matrices (N(0,1) scaled to "
                                                "448): inside the matrix unit vs promoted every 128 K", **acc}
        log(f"[bench] probes: MFMA stream {pw[0]['TFLOPs']} TFLOP/s at {pw[0]['shader_clock_ghz']} GHz, with "
            f"promotion {pw[1]['TFLOPs']} at {pw[1]['shader_clock_ghz']} GHz; accumulation {acc}")

    cpu = None
    cpu_configs = {}
    if not args.no_cpu_baseline:
        from oracle import gemm as og
        from oracle import quant as oq
        r, nw = min(args.cpu_rows, M), min(args.cpu_wrows, N)
        xs_h, ws_h = cfg.x[:r], cfg.w[:nw]
        c0 = time.perf_counter()
        q0, s0 = oq.quant_act_1x128(xs_h)
        qw0, sw0 = oq.quant_w_128x128(ws_h)
        og.fprop(q0, s0, qw0, sw0)
        csec = time.perf_counter() - c0
        cpu = {"value": 2.0 * r * nw * K / csec / 1e12, "unit": "TFLOP/s", "cores": cpu_threads(),
               "kind": "oracle",
               "sample": f"quantise X[:{r}] (1x128) and W[:{nw}] (128x128), then the oracle GEMM of "
                         f"those {r}x{nw}x{K} (fp64 chunk sums, fp32 promotion); {csec:.1f} s on the host"}
        log(f"[bench] oracle sample: {csec:.1f} s -> {cpu['value'] * 1e3:.3f} GFLOP/s")
        # the oracle on a bounded sample of each other configuration: its quantisers (GB/s
        # of algorithmic bytes) and its GEMM (fp64 chunk sums, GFLOP/s)
        if others:
            def timed(fn, *a):
                c = time.perf_counter()
                out_ = fn(*a)
                return out_, time.perf_counter() - c

            dn = workloads.dense_fprop()
            dyb = workloads.backward_dy()
            rows = 512
            (qd, sd), tqa = timed(oq.quant_act_1x128, dn.x[:rows])
            (qwd, swd), tqw = timed(oq.quant_w_128x128, dn.w)
            _, tgf = timed(og.fprop, qd, sd, qwd, swd)
            cpu_configs["dense_fprop"] = {
                "sample": f"X[:{rows}] of [4096, 7168], all of W [2048, 7168]",
                "quant_act_GBps": round(rows * 7168 * 3.031 / tqa / 1e9, 3),
                "quant_w_GBps": round(2048 * 7168 * 3.0 / tqw / 1e9, 3),
                "gemm_GFLOPs": round(2.0 * rows * 2048 * 7168 / tgf / 1e9, 2)}
            (qy, sy), _ = timed(oq.quant_act_1x128, dyb[:rows])
            _, tdg = timed(og.dgrad, qy, sy, qwd, swd)
            (qyt, syt), tqc = timed(oq.quant_act_128x1, dyb[:, :256])
            (qxt, sxt), _ = timed(oq.quant_act_128x1, dn.x[:, :512])
            _, twg = timed(og.wgrad, qyt, syt, qxt, sxt)
            cpu_configs["backward_pair"] = {
                "sample": f"Dgrad on dY[:{rows}]; Wgrad dW[:256, :512] over all 4096 tokens",
                "dgrad_GFLOPs": round(2.0 * rows * 7168 * 2048 / tdg / 1e9, 2),
                "quant_act_128x1_GBps": round(4096 * 256 * 3.031 / tqc / 1e9, 3),
                "wgrad_GFLOPs": round(2.0 * 256 * 512 * 4096 / twg / 1e9, 2)}
            mo = workloads.moe_fprop()
            e0r = int(mo.real_rows[0])
            (qm, sm_), _ = timed(oq.quant_act_1x128, mo.x[:rows])
            (qwm, swm), _ = timed(oq.quant_w_128x128, mo.w[0])
            _, tmg = timed(og.fprop, qm, sm_, qwm, swm)
            cpu_configs["moe_grouped"] = {"sample": f"{rows} of expert 0's {e0r} rows against its weight",
                                          "gemm_GFLOPs": round(2.0 * rows * 2048 * 7168 / tmg / 1e9, 2)}
            log(f"[bench] oracle per configuration: {cpu_configs}")

    clk = gemm_clock_ghz() if args.workload == "large" else None
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": settle_steps,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic: seeded Student-t(3) / N(0,1)+outliers activations, N(0,0.02) weights, bf16",
        "config": {"workload": name, "M": M, "N": N, "K": K, "act_tile": "1x128", "weight_block": "128x128",
                   "fp8": "E4M3FN", "out": "bf16", "step": "quant_act + quant_w + gemm"},
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 1), "peak": PEAK_FP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tflops / PEAK_FP8_TFLOPS, 4),
                     "traffic": gemm_traffic() if args.workload == "large" else None,
                     "kernel": "gemm_kernel<FPROP>", "avg_us": round(tg, 2), "us_stats": rnd(st_tg),
                     # the 5.0 PF peak assumes 2.4 GHz; the clock under this GEMM, from the
                     # committed rocprofv3 counters (GRBM_GUI_ACTIVE / duration), scales it
                     "clock_ghz": clk,
                     "frac_at_measured_clock": (round(gemm_tflops / (PEAK_FP8_TFLOPS * clk / 2.4), 4)
                                                if clk else None)},
        "cpu_baseline": cpu,
        "cpu_baseline_per_config": cpu_configs,
        "breakdown": {
            "frac_of_fp8_peak_incl_quant": round(value / PEAK_FP8_TFLOPS, 4),
            "quant_act_us": round(tq_x, 2), "quant_act_GBps": round(bytes_qx / tq_x / 1e3, 1),
            "quant_act_frac_hbm": round(bytes_qx / tq_x / 1e3 / PEAK_HBM_GBS, 4),
            "quant_w_us": round(tq_w, 2), "quant_w_GBps": round(bytes_qw / tq_w / 1e3, 1),
            "quant_w_frac_hbm": round(bytes_qw / tq_w / 1e3 / PEAK_HBM_GBS, 4),
            "gemm_us": round(tg, 2), "gemm_TFLOPs": round(gemm_tflops, 1),
            "requant_t_us": round(t_rq, 2), "requant_t_GBps": round(bytes_rq / t_rq / 1e3, 1),
            "requant_t_frac_hbm": round(bytes_rq / t_rq / 1e3 / PEAK_HBM_GBS, 4),
            "requant_t_copy_us": round(st_cp_rq["mean"], 2),
            "requant_t_frac_ceiling": round(st_cp_rq["mean"] / t_rq, 4),
            "quant_act_frac_ceiling": (round(ceilings["stream_2to1_X"]["us"] / tq_x, 4) if ceilings else None),
            "quant_w_frac_ceiling": (round(ceilings["stream_2to1_W"]["us"] / tq_w, 4) if ceilings else None),
            "quant_act_us_stats": rnd(st_tq_x), "quant_w_us_stats": rnd(st_tq_w),
            "requant_t_us_stats": rnd(st_t_rq),
            "quant_timing": "each kernel alone after a 512 MB read (MALL evicted), one HIP event pair per launch; "
                            "us = mean; frac_ceiling = the plain 2:1 stream's time over the same elements / "
                            "the quantiser's (re-quantisation: the device copy of the same codes / its time)",
        },
        "ceilings": ceilings,
        "probes": probes,
        "other_configs": others,
        "variants": {
            "pow2_scales": {
                "what": "the same step with power-of-two scales, applied by the scaled matrix instruction",
                "value": round(flops / (ms_step_p2 * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
                "ms_per_step": round(ms_step_p2, 4), "gemm_us": round(tg_p2, 2), "gemm_us_stats": rnd(st_tg_p2),
                "gemm_TFLOPs": round(flops / (tg_p2 * 1e-6) / 1e12, 1),
                "kernel": "gemm_pow2_kernel<FPROP>",
            },
            "producer_fusion": {
                "what": "GEMM whose epilogue writes Y as E4M3 codes + 1x128 scales (no bf16 Y), against the GEMM "
                        "writing bf16 Y followed by the 1x128 quantiser of Y",
                "fused_us": round(t_fq, 2), "separate_us": round(t_sq, 2), "fused_us_stats": rnd(st_t_fq),
                "fused_TFLOPs": round(flops / (t_fq * 1e-6) / 1e12, 1),
                "hbm_bytes_saved": 4 * M * N,
                "kernel": "gemm_kernel<FPROP, QMODE=1>",
            },
            "e5m6_cache": {
                "what": f"E5M6 activation cache of X [{M}, {K}]: 1x128 tiles, power-of-two scales, 12-bit codes "
                        "packed two per 3 bytes (read 2 B, write 1.5 B per element), and reading it back to bf16; "
                        "cold",
                "cache_us": round(st_t_ce["mean"], 2), "cache_us_stats": rnd(st_t_ce),
                "cache_GBps": round(bytes_e5m6 / st_t_ce["mean"] / 1e3, 1),
                "cache_frac_hbm": round(bytes_e5m6 / st_t_ce["mean"] / 1e3 / PEAK_HBM_GBS, 4),
                "read_back_us": round(st_t_ue["mean"], 2), "read_back_us_stats": rnd(st_t_ue),
                "read_back_GBps": round(bytes_e5m6 / st_t_ue["mean"] / 1e3, 1),
                "read_back_frac_hbm": round(bytes_e5m6 / st_t_ue["mean"] / 1e3 / PEAK_HBM_GBS, 4),
                "algorithmic_bytes": bytes_e5m6,
                "kernel": "cache_e5m6_kernel / uncache_e5m6_kernel",
                "to_128x1_us": round(st_t_re["mean"], 2), "to_128x1_us_stats": rnd(st_t_re),
                "to_128x1_GBps": round(bytes_re / st_t_re["mean"] / 1e3, 1),
                "to_128x1_frac_hbm": round(bytes_re / st_t_re["mean"] / 1e3 / PEAK_HBM_GBS, 4),
                "to_128x1_algorithmic_bytes": bytes_re,
                "to_128x1_kernel": "requant_e5m6_t_kernel",
            },
            "decode_grouped": {
                "what": f"{dec.name}: rows per expert {[int(c) for c in dec.real_rows]} (unpadded), "
                        "bf16 out; HBM-bound (each expert's FP8 weight streamed once); timed cold",
                "us": round(t_dec, 2), "GBps": round(bytes_dec / t_dec / 1e3, 1), "us_stats": rnd(st_t_dec),
                "roofline": {"bound": "hbm", "achieved": round(bytes_dec / t_dec / 1e3, 1), "peak": PEAK_HBM_GBS,
                             "unit": "GB/s", "frac": round(bytes_dec / t_dec / 1e3 / PEAK_HBM_GBS, 4),
                             "traffic": None},
                "algorithmic_bytes": bytes_dec,
                "TFLOPs": round(2.0 * m_d * N_d * K_d / (t_dec * 1e-6) / 1e12, 1),
                "kernel": "gemm_decode_kernel<true> (fp8bq_grouped_gemm_decode_ws)",
                "workspace_bytes": d_need,
                "full_k_us": round(st_t_dec0["mean"], 2), "full_k_us_stats": rnd(st_t_dec0),
                "full_k_kernel": "gemm_decode_kernel<true> (fp8bq_grouped_gemm_decode, no workspace)",
            },
        },
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
