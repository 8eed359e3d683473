"""Benchmark of the NVFP4 W4A4 linear-layer hot path on one MI355X.

One step = one pass of every kernel on the path over seeded synthetic inputs
already resident in HBM:

  prefill, M = 4096 tokens
    quantize A (dynamic global scale)  -> fused GDN in-projection
        (N = 16480 = q|k|v|z|b|a, K = 5120, per-module global scales,
         sigmoid on b, -exp(A_log)*softplus(a + dt_bias) on a)
    quantize A  -> MLP gate_up (N = 2 x 17408, K = 5120, SiLU*mul; the
        epilogue also leaves partial maxima of |h|)
        -> quantize h (dynamic global scale from those maxima)
        -> down (N = 5120, K = 17408)
  decode, M = 1
    quantize A -> GEMM (N = 17408, K = 5120) on one of 8 rotating copies of
    the packed weight (8 x 50.1 MB > the 256 MB Infinity Cache)

Reported beside the timed step: the decode GEMM at M = 1, 8, 32, 64 (HIP
graph replays), and the MLP with h quantised in the gate/up epilogue
(static global scale of h) against its unfused chain, and the fused GDN
in-projection under both repairs of the per-module scale mismatch, and the
second workload: the gated delta-rule recurrence over the 4096 tokens, fed by
the in-projection's output.

value = algorithmic GEMM FLOP (2MNK) of the prefill part / its wall time
(quantizers and epilogues included), in TFLOP/s.  The decode part is
reported as weight GB/s (packed weight bytes / GEMM time).  Kernel durations
for the roofline are taken with HIP events on the stream the kernels run on,
in every other timed step; the part totals behind `value` come from the
steps in between, which record no events between kernels (each such event
delays the next kernel by about 6 us).  Durations are medians over their
steps (50 timed steps after 10 warm-up steps by default).  Weight packing is offline (done
once, outside the timed region).
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W4A4 NVFP4 GEMM TFLOP/s at M=4096 + weight GB/s at M=1; % of MI355X peak"
PEAK_F16_TFLOPS = 2500.0      # MI355X dense f16/bf16 MFMA
PEAK_FP4_TFLOPS = 10100.0     # dense FP4 MFMA (context only: NVFP4's E4M3 scales do not fit it)
PEAK_HBM_GBPS = 8000.0
DECODE_COPIES = 8
CONFIGS = ("step", "linear", "quantizer", "decode", "recurrence")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="target length of the oracle sample")
    p.add_argument("--no-decode-sweep", action="store_true", help="skip the per-M decode sweep (profiling runs)")
    p.add_argument("--decode-profile", action="store_true",
                   help="profiling run of the decode kernels only: the GEMM at M = 1, 8, 32, 64, the one-kernel "
                        "linear layer at M = 1 and the streaming-read reference, 16 eager launches each, then exit")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="after the timed region, run one plain device copy of this many MiB (counter calibration)")
    p.add_argument("--config", choices=CONFIGS, default="step",
                   help="step (default): the timed step and every measurement beside it, one JSON line in the "
                        "bench contract; the others run one measurement alone and print {config, result}: "
                        "linear (M=2048 N=K=5120 layer), quantizer (the three activation shapes), decode (the "
                        "M sweep and the streaming-read reference), recurrence (4096 tokens x 48 heads)")
    return p.parse_args()


def dev_bf16(torch, bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def setup(torch, B):
    from nvfp4_w4a4_gemm_quantize_amd import inputs
    t0 = time.time()
    gdn = inputs.gdn_inproj()
    mlp = inputs.mlp()
    dec = inputs.decode(1)
    S = {}
    S["gdn_A"] = dev_bf16(torch, gdn["A"])
    S["gdn_offs"] = [int(v) for v in gdn["seg_offsets"]]
    S["gdn_packed"], S["gdn_g"] = B.nvfp4_pack_weights(dev_bf16(torch, gdn["W"]), S["gdn_offs"])
    # the same fused weight quantised with one shared global scale (the pre-harmonised repair)
    S["gdn_packed_h"], S["gdn_g_h"] = B.nvfp4_pack_weights(dev_bf16(torch, gdn["W"]))
    S["A_log"] = torch.tensor(gdn["A_log"], device="cuda")
    S["dt_bias"] = torch.tensor(gdn["dt_bias"], device="cuda")
    S["mlp_A"] = dev_bf16(torch, mlp["A"])
    S["gu_packed"], S["gu_g"] = B.nvfp4_pack_weights(dev_bf16(torch, mlp["W_gate_up"]))
    S["dn_packed"], S["dn_g"] = B.nvfp4_pack_weights(dev_bf16(torch, mlp["W_down"]))
    S["dec_A"] = dev_bf16(torch, dec["A"])
    p, g = B.nvfp4_pack_weights(dev_bf16(torch, dec["W"]))
    S["dec_packed"] = [p] + [p.clone() for _ in range(DECODE_COPIES - 1)]
    S["dec_g"] = g
    M, K = 4096, 5120
    # preallocated outputs and quantizer buffers
    S["qa_codes"] = torch.empty((M, K // 2), dtype=torch.uint8, device="cuda")
    S["qa_scales"] = torch.empty((M, K // 16), dtype=torch.uint8, device="cuda")
    S["qa_g"] = torch.empty(1, dtype=torch.float32, device="cuda")
    S["qh_codes"] = torch.empty((M, 17408 // 2), dtype=torch.uint8, device="cuda")
    S["qh_scales"] = torch.empty((M, 17408 // 16), dtype=torch.uint8, device="cuda")
    S["qh_g"] = torch.empty(1, dtype=torch.float32, device="cuda")
    # the gate/up GEMM's partial maxima of |h| live in h's codes buffer until the quantizer reduces them
    S["qh_parts"] = S["qh_codes"].view(-1)[:4 * B.nvfp4_silu_amax_parts(M, 34816)].view(torch.int32)
    S["gdn_out"] = torch.empty((M, 16480), dtype=torch.bfloat16, device="cuda")
    S["h"] = torch.empty((M, 17408), dtype=torch.bfloat16, device="cuda")
    S["mlp_out"] = torch.empty((M, 5120), dtype=torch.bfloat16, device="cuda")
    S["qd_codes"] = torch.empty((1, K // 2), dtype=torch.uint8, device="cuda")
    S["qd_scales"] = torch.empty((1, K // 16), dtype=torch.uint8, device="cuda")
    S["qd_g"] = torch.empty(1, dtype=torch.float32, device="cuda")
    S["dec_out"] = torch.empty((1, 17408), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    S["setup_s"] = time.time() - t0
    return S


FLOP = {
    "gdn": 2 * 4096 * 16480 * 5120,
    "gate_up": 2 * 4096 * 34816 * 5120,
    "down": 2 * 4096 * 5120 * 17408,
    "decode": 2 * 1 * 17408 * 5120,
}
DECODE_W_BYTES = 17408 * 5120 * 9 // 16          # packed codes + scales: 50,135,040
DECODE_BYTES = DECODE_W_BYTES + 5120 * 9 // 16 + 17408 * 2


OUTER_EVENTS = ("prefill", "decode_all")
INNER_EVENTS = ("gdn", "gate_up", "down")


def step(torch, B, S, it, ev, inner=True):
    """One pass; ev: dict name -> (start, end) events.  The prefill and decode
    parts are always bracketed; with `inner`, each GEMM (with its tail launch)
    is bracketed too.  An event recorded between two kernels holds the next one
    back by about 6 us, so a step timed for its total records no inner events."""
    outer = (lambda name, i: ev[name][i].record()) if ev is not None else (lambda name, i: None)
    rec = outer if inner else (lambda name, i: None)
    outer("prefill", 0)
    B.nvfp4_quantize(S["gdn_A"], S["qa_g"], True, S["qa_codes"], S["qa_scales"])
    rec("gdn", 0)
    B.gemm_w4a4_fused_segments(S["qa_codes"], S["qa_scales"], S["qa_g"], S["gdn_packed"], 16480, 5120,
                               S["gdn_offs"], S["gdn_g"], ["none", "none", "none", "none", "sigmoid", "gdn_decay"],
                               S["A_log"], S["dt_bias"], out=S["gdn_out"])
    rec("gdn", 1)
    B.nvfp4_quantize(S["mlp_A"], S["qa_g"], True, S["qa_codes"], S["qa_scales"])
    rec("gate_up", 0)
    _, _, n_parts = B.gemm_w4a4_silu_mul_amax(S["qa_codes"], S["qa_scales"], S["qa_g"], S["gu_packed"], S["gu_g"],
                                              34816, 5120, h=S["h"], parts=S["qh_parts"])
    rec("gate_up", 1)
    B.nvfp4_quantize_amax_parts(S["h"], S["qh_parts"], n_parts, S["qh_g"], S["qh_codes"], S["qh_scales"])
    rec("down", 0)
    B.gemm_w4a4(S["qh_codes"], S["qh_scales"], S["qh_g"], S["dn_packed"], S["dn_g"], 5120, 17408, out=S["mlp_out"])
    rec("down", 1)
    outer("prefill", 1)
    outer("decode_all", 0)
    B.nvfp4_linear(S["dec_A"], S["dec_packed"][it % DECODE_COPIES], S["dec_g"], 17408, out=S["dec_out"],
                   a_global=S["qd_g"], a_codes=S["qd_codes"], a_scales=S["qd_scales"])
    outer("decode_all", 1)


def _graph(torch, fn):
    """Capture fn() (a sequence of library calls on the current stream) into a HIP graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                                    # warm-up on the capture stream's side, as torch requires
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def _replay_us(torch, g, calls, reps=3):
    """Mean time per captured call over `reps` replays, from events around each replay."""
    g.replay()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1000 / calls)
    return min(ts)


def decode_sweep(torch, B, S, iters=64):
    """Decode GEMM time at each M, from HIP-graph replays of `iters` back-to-back launches over the
    rotating weight copies (a Python launch loop would measure the host, not the kernel): gemm_w4a4 on an
    already quantised activation (GEMM only), and nvfp4_linear on the bf16 activation (quantize + GEMM;
    one kernel at M = 1).  Each replayed output is checked bit-for-bit against an eager launch.  The
    weight stream with no arithmetic (nvfp4_weight_stream_read, the decode kernel's loads and launch
    shape) is timed the same way: the measured ceiling for these GEMMs."""
    from nvfp4_w4a4_gemm_quantize_amd import inputs
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")

    def reads():
        for i in range(iters):
            B.nvfp4_weight_stream_read(S["dec_packed"][i % DECODE_COPIES], 17408, 5120, sink)

    g0 = _graph(torch, reads)
    stream_us = _replay_us(torch, g0, iters, reps=5)
    del g0
    out = {"stream_read_us": round(stream_us, 2), "stream_read_GBps": round(DECODE_W_BYTES / stream_us / 1e3, 1),
           "stream_read_hbm_frac": round(DECODE_W_BYTES / stream_us / 1e3 / PEAK_HBM_GBPS, 3)}
    for M in inputs.DECODE_M:
        a = dev_bf16(torch, inputs.decode(M, weights=False)["A"])
        qc, qs, qg = B.nvfp4_quantize(a)
        y = torch.empty((M, 17408), dtype=torch.bfloat16, device="cuda")
        last = S["dec_packed"][(iters - 1) % DECODE_COPIES]
        B.gemm_w4a4(qc, qs, qg, last, S["dec_g"], 17408, 5120, out=y)
        y_eager = y.clone()

        def gemms():
            for i in range(iters):
                B.gemm_w4a4(qc, qs, qg, S["dec_packed"][i % DECODE_COPIES], S["dec_g"], 17408, 5120, out=y)

        def linears():
            for i in range(iters):
                B.nvfp4_linear(a, S["dec_packed"][i % DECODE_COPIES], S["dec_g"], 17408, out=y, a_global=qg,
                               a_codes=qc, a_scales=qs)

        g1, g2 = _graph(torch, gemms), _graph(torch, linears)
        us = _replay_us(torch, g1, iters, reps=5)
        same = bool(torch.equal(y, y_eager))
        us_q = _replay_us(torch, g2, iters, reps=5)
        same = same and bool(torch.equal(y, y_eager))
        nbytes = DECODE_W_BYTES + M * (5120 * 9 // 16) + M * 17408 * 2
        out["M%d" % M] = {"gemm_us": round(us, 2), "weight_GBps": round(DECODE_W_BYTES / us / 1e3, 1),
                          "hbm_frac": round(nbytes / us / 1e3 / PEAK_HBM_GBPS, 3),
                          "gemm_over_stream_read": round(us / stream_us, 3),
                          "quantize_plus_gemm_us": round(us_q, 2),
                          "tflops": round(2 * M * 17408 * 5120 / us / 1e6, 2),
                          "graph_replay_matches_eager": same}
        del g1, g2
    return out


def decode_summary(dur, sweep):
    """The M = 1 decode figures: from the graph replays of the sweep (back-to-back launches, no
    event between kernels) when it ran, else from the timed steps' events.  The in-step event
    timing of the decode part (nvfp4_linear: quantize + GEMM in one kernel) is reported beside them."""
    in_step = {"quantize_plus_gemm_us": round(dur["decode_all"] * 1e3, 2)}
    if sweep:
        us, us_q, src = sweep["M1"]["gemm_us"], sweep["M1"]["quantize_plus_gemm_us"], "graph replay (decode sweep, M=1)"
    else:
        us, us_q, src = None, in_step["quantize_plus_gemm_us"], "timed steps, events around the decode part"
    res = {"M": 1, "gemm_us": us, "quantize_plus_gemm_us": us_q, "source": src, "in_step_events": in_step,
           "sweep": sweep}
    if us is not None:
        res.update({"weight_GBps": round(DECODE_W_BYTES / us / 1e3, 1),
                    "hbm_frac": round(DECODE_BYTES / us / 1e3 / PEAK_HBM_GBPS, 4)})
    if sweep:
        res["stream_read_us"] = sweep["stream_read_us"]
        res["gemm_over_stream_read"] = sweep["M1"]["gemm_over_stream_read"]
    return res


def linear_config(torch, B, reps=20):
    """The single linear layer, prefill (M = 2048, N = K = 5120, bf16 out): quantize A (dynamic g) +
    GEMM, and the GEMM alone, from events around `reps` back-to-back launches."""
    from nvfp4_w4a4_gemm_quantize_amd import inputs
    d = inputs.linear()
    a = dev_bf16(torch, d["A"])
    packed, wg = B.nvfp4_pack_weights(dev_bf16(torch, d["W"]))
    qc, qs, qg = B.nvfp4_quantize(a)
    y = torch.empty((2048, 5120), dtype=torch.bfloat16, device="cuda")

    def time_us(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    t_g, t_q = [], []
    for _ in range(3):
        t_g.append(time_us(lambda: B.gemm_w4a4(qc, qs, qg, packed, wg, 5120, 5120, out=y)))
        t_q.append(time_us(lambda: B.nvfp4_linear(a, packed, wg, 5120, out=y, a_global=qg, a_codes=qc, a_scales=qs)))
    t_g, t_q = min(t_g), min(t_q)
    flop = 2 * 2048 * 5120 * 5120
    return {"M": 2048, "N": 5120, "K": 5120, "gemm_us": round(t_g, 1), "tflops": round(flop / t_g / 1e6, 1),
            "mfma_frac": round(flop / t_g / 1e6 / PEAK_F16_TFLOPS, 4), "quantize_plus_gemm_us": round(t_q, 1),
            "tflops_with_quantize": round(flop / t_q / 1e6, 1)}


def quantizer_rates(torch, B, reps=20):
    """nvfp4_quantize with a dynamic global scale on the path's three activation shapes.  Algorithmic
    bytes: 2 B read + 0.5625 B written per element (codes + E4M3 scales); the amax pre-pass reads the
    tensor once more (2 B per element), given separately."""
    out = {}
    for name, (r, c) in (("A_4096x5120", (4096, 5120)), ("h_4096x17408", (4096, 17408)), ("A_1x5120", (1, 5120))):
        x = (torch.randn((r, c), device="cuda") * 3).to(torch.bfloat16)
        g = torch.empty(1, dtype=torch.float32, device="cuda")
        codes = torch.empty((r, c // 2), dtype=torch.uint8, device="cuda")
        scales = torch.empty((r, c // 16), dtype=torch.uint8, device="cuda")
        fn = lambda: B.nvfp4_quantize(x, g, True, codes, scales)
        fn()
        torch.cuda.synchronize()
        best = 1e9
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) * 1e3 / reps)
        n = r * c
        algo = n * 2 + n * 9 // 16
        out[name] = {"us": round(best, 2), "algorithmic_bytes": algo, "GBps": round(algo / best / 1e3, 1),
                     "hbm_frac": round(algo / best / 1e3 / PEAK_HBM_GBPS, 3),
                     "GBps_incl_amax_pass": round((algo + 2 * n) / best / 1e3, 1)}
        del x, codes, scales
    return out


def cpu_baseline(target_s):
    """The CPU oracle on a row sample of the same prefill workload, scaled to TFLOP/s."""
    from threadpoolctl import threadpool_limits
    from nvfp4_w4a4_gemm_quantize_amd import inputs
    from oracle import epilogue as OE
    from oracle import gemm as OG
    from oracle import quantize as OQ
    cores = min(16, len(os.sched_getaffinity(0)))
    gdn = inputs.gdn_inproj()
    offs = [int(v) for v in gdn["seg_offsets"]]
    with threadpool_limits(limits=cores):
        cw, sw, gs = OQ.quantize_segments(gdn["W"], offs)          # offline weight pack: untimed
        gcol = OG.column_global(offs[-1], offs, gs)
        t0 = time.perf_counter()
        g_a = OQ.dynamic_global_scale(gdn["A"])                    # per-tensor amax of the whole batch
        flops, spent, rows_done, r0 = 0, time.perf_counter() - t0, 0, 0
        rows = 16
        while spent < target_s and r0 + rows <= 4096:
            t0 = time.perf_counter()
            ca, sa, ga = OQ.quantize(gdn["A"][r0:r0 + rows], g_a)
            y, b = OG.gemm(ca, sa, ga, cw, sw, gcol)
            OE.sigmoid(y[:, offs[4]:offs[5]])
            OE.gdn_decay(y[:, offs[5]:offs[6]], gdn["A_log"], gdn["dt_bias"])
            spent += time.perf_counter() - t0
            flops += 2 * rows * offs[-1] * 5120
            rows_done += rows
            r0 += rows
            rows = min(rows * 2, 256)
    return {"value": round(flops / spent / 1e12, 5), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": "fused GDN in-projection (N=16480, K=5120, 6 modules, sigmoid/decay epilogues) on the "
                      "first %d of 4096 rows: numpy FP32 quantizer + fp64 dequant GEMM with the sum|a*w| bound; "
                      "%.1f s" % (rows_done, spent)}


KERNEL_SOURCES = ("nvfp4_w4a4_gemm_quantize_amd/csrc/gemm.hip", "nvfp4_w4a4_gemm_quantize_amd/csrc/nvfp4_device.h",
                  "nvfp4_w4a4_gemm_quantize_amd/csrc/kernels.h")
TRAFFIC_PROFILE = "profiles/hbm_traffic__gemm_prefill_dma_kernel__prefill_M4096.txt"
# Algorithmic bytes per launch: packed A + packed W + output (bf16).
ALGO_BYTES = {
    "gdn": 4096 * 5120 * 9 // 16 + 16480 * 5120 * 9 // 16 + 4096 * 16480 * 2,
    "gate_up": 4096 * 5120 * 9 // 16 + 34816 * 5120 * 9 // 16 + 4096 * 17408 * 2,
    "down": 4096 * 17408 * 9 // 16 + 5120 * 17408 * 9 // 16 + 4096 * 5120 * 2,
}


def kernel_source_sha256():
    """SHA-256 of the GEMM kernel sources with comments and runs of white space
    removed: an edit to comments alone leaves the kernels, and the hash, as they were."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(re.sub(r"\s+", " ", text).strip().encode())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per prefill GEMM from the committed FETCH_SIZE/WRITE_SIZE summary (copy-calibrated),
    or None when it is missing or was taken on a different kernel source."""
    path = os.path.join(ROOT, TRAFFIC_PROFILE)
    if not os.path.exists(path):
        return None
    sha, per = None, {}
    for line in open(path):
        f = line.split()
        if len(f) >= 2 and f[0] == "source_sha256":
            sha = f[1]
        elif len(f) >= 2 and f[0] == "launch":
            kv = dict(zip(f[2::2], f[3::2]))
            per[f[1]] = float(kv["fetch_bytes"]) + float(kv["write_bytes"])
    if sha != kernel_source_sha256() or set(per) != set(ALGO_BYTES):
        return None
    return per


def progress(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def mlp_fused(torch, B, S, reps=5):
    """The MLP block with h quantised in the gate/up epilogue (static global scale of h, calibrated as
    2688/amax(h) on another seeded batch through the unfused path) against the chain of the timed step
    (gate_up with |h| maxima -> bf16 h -> quantize with h's dynamic scale -> down).  Both start from the
    quantised A."""
    from nvfp4_w4a4_gemm_quantize_amd import inputs
    cal = dev_bf16(torch, inputs.mlp(seed=1, weights=False)["A"])
    B.nvfp4_quantize(cal, S["qa_g"], True, S["qa_codes"], S["qa_scales"])
    B.gemm_w4a4(S["qa_codes"], S["qa_scales"], S["qa_g"], S["gu_packed"], S["gu_g"], 34816, 5120,
                epilogue="silu_mul", out=S["h"])
    hg = torch.empty(1, dtype=torch.float32, device="cuda")
    B.nvfp4_quantize(S["h"], hg, True, S["qh_codes"], S["qh_scales"])
    del cal
    B.nvfp4_quantize(S["mlp_A"], S["qa_g"], True, S["qa_codes"], S["qa_scales"])
    y_f = torch.empty_like(S["mlp_out"])

    def unfused():
        _, _, n_parts = B.gemm_w4a4_silu_mul_amax(S["qa_codes"], S["qa_scales"], S["qa_g"], S["gu_packed"],
                                                  S["gu_g"], 34816, 5120, h=S["h"], parts=S["qh_parts"])
        B.nvfp4_quantize_amax_parts(S["h"], S["qh_parts"], n_parts, S["qh_g"], S["qh_codes"], S["qh_scales"])
        B.gemm_w4a4(S["qh_codes"], S["qh_scales"], S["qh_g"], S["dn_packed"], S["dn_g"], 5120, 17408,
                    out=S["mlp_out"])

    def gate_up_fused():
        B.gemm_w4a4_silu_mul_quantize(S["qa_codes"], S["qa_scales"], S["qa_g"], S["gu_packed"], S["gu_g"], 34816,
                                      5120, hg, h_codes=S["qh_codes"], h_scales=S["qh_scales"])

    def fused():
        gate_up_fused()
        B.gemm_w4a4(S["qh_codes"], S["qh_scales"], hg, S["dn_packed"], S["dn_g"], 5120, 17408, out=y_f)

    def time_us(fn):
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    t_u, t_f, t_g = [], [], []
    for _ in range(3):          # interleaved rounds, best of each
        t_u.append(time_us(unfused))
        t_f.append(time_us(fused))
        t_g.append(time_us(gate_up_fused))
    t_u, t_f, t_g = min(t_u), min(t_f), min(t_g)
    dev = float(torch.linalg.vector_norm((y_f.float() - S["mlp_out"].float())) /
                torch.linalg.vector_norm(S["mlp_out"].float()))
    return {"static_h_global": round(float(hg.item()), 6), "unfused_us": round(t_u, 1), "fused_us": round(t_f, 1),
            "gate_up_quantize_fused_us": round(t_g, 1), "saving_frac": round(1.0 - t_f / t_u, 4),
            "tflops_fused": round((FLOP["gate_up"] + FLOP["down"]) / t_f / 1e6, 1),
            "down_out_rel_l2_vs_unfused": round(dev, 5)}


def gdn_repairs(torch, B, S, reps=5):
    """Fused GDN in-projection under the two repairs of the per-module scale mismatch: per-segment alpha
    (the timed step) and a weight quantised with one shared global scale, run through the same segmented
    call (gates included) and as a plain single-alpha GEMM (no gates)."""
    epis = ["none", "none", "none", "none", "sigmoid", "gdn_decay"]
    nseg = len(S["gdn_offs"]) - 1
    g_rep = S["gdn_g_h"].repeat(nseg)
    B.nvfp4_quantize(S["gdn_A"], S["qa_g"], True, S["qa_codes"], S["qa_scales"])
    y2 = torch.empty_like(S["gdn_out"])

    def per_segment():
        B.gemm_w4a4_fused_segments(S["qa_codes"], S["qa_scales"], S["qa_g"], S["gdn_packed"], 16480, 5120,
                                   S["gdn_offs"], S["gdn_g"], epis, S["A_log"], S["dt_bias"], out=S["gdn_out"])

    def harmonised_gates():
        B.gemm_w4a4_fused_segments(S["qa_codes"], S["qa_scales"], S["qa_g"], S["gdn_packed_h"], 16480, 5120,
                                   S["gdn_offs"], g_rep, epis, S["A_log"], S["dt_bias"], out=y2)

    def harmonised_plain():
        B.gemm_w4a4(S["qa_codes"], S["qa_scales"], S["qa_g"], S["gdn_packed_h"], S["gdn_g_h"], 16480, 5120, out=y2)

    def time_us(fn):
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    # interleaved rounds, best of each: the chip's clock drifts with what ran just before
    t = {"per_segment_alpha_us": [], "shared_scale_segmented_us": [], "shared_scale_single_alpha_gemm_us": []}
    for _ in range(3):
        t["per_segment_alpha_us"].append(time_us(per_segment))
        t["shared_scale_segmented_us"].append(time_us(harmonised_gates))
        t["shared_scale_single_alpha_gemm_us"].append(time_us(harmonised_plain))
    out = {k: round(min(v), 1) for k, v in t.items()}
    out["shared_global_scale"] = round(float(S["gdn_g_h"].item()), 3)
    out["module_global_scales"] = [round(float(v), 3) for v in S["gdn_g"].tolist()]
    return out


def bf16_library_context(torch, reps=5):
    """Context, not part of the path: the same three prefill GEMMs as plain bf16 matrix products through
    torch (hipBLASLt), unquantised operands -- a measured practical MFMA ceiling on this GPU.  Two-
    dimensional products only (no batched kernels)."""
    import torch.nn.functional as F
    out = {}
    for name, (n, k) in (("gdn", (16480, 5120)), ("gate_up", (34816, 5120)), ("down", (5120, 17408))):
        a = torch.randn((4096, k), device="cuda").to(torch.bfloat16)
        w = (torch.randn((n, k), device="cuda") * k ** -0.5).to(torch.bfloat16)
        F.linear(a, w)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            F.linear(a, w)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        out[name] = {"us": round(us, 1), "tflops": round(2 * 4096 * n * k / us / 1e6, 1)}
        del a, w
    torch.cuda.empty_cache()
    tot = sum(FLOP[x] for x in ("gdn", "gate_up", "down")) / sum(out[x]["us"] for x in out) / 1e6
    out["all_3_tflops"] = round(tot, 1)
    return out


REC_FLOP_PER_HEAD_TOKEN = 7 * 128 * 128      # two 128x128 dot passes (2 d^2 each) + decay-and-write (3 d^2)
PEAK_F32_VECTOR_TFLOPS = 157.3                # MI355X fp32 vector (packed); 78.6 without packed FP32


def gdn_recurrence_run(torch, B, S, reps=5):
    """Second workload: the gated delta-rule recurrence of the 48 value heads over the 4096 tokens of the
    step, reading q | k | v and the gate columns straight from the fused in-projection output."""
    offs = S["gdn_offs"]
    y = S["gdn_out"]
    out = torch.empty((4096, 48 * 128), dtype=torch.bfloat16, device="cuda")

    def run():
        B.gdn_recurrence(y[:, offs[0]:offs[1]], y[:, offs[1]:offs[2]], y[:, offs[2]:offs[3]], y[:, offs[4]:offs[5]],
                         y[:, offs[5]:offs[6]], 16, 48, out_dtype=torch.bfloat16, out=out)

    run()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    tflops = REC_FLOP_PER_HEAD_TOKEN * 48 * 4096 / us / 1e6
    return {"tokens": 4096, "key_heads": 16, "value_heads": 48, "head_dim": 128, "us": round(us, 1),
            "Mtokens_per_s": round(4096 / us, 3), "tflops": round(tflops, 2),
            "roofline": {"bound": "alu", "achieved": round(tflops, 2), "peak": PEAK_F32_VECTOR_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / PEAK_F32_VECTOR_TFLOPS, 4),
                         "flop_per_head_token": REC_FLOP_PER_HEAD_TOKEN},
            "input": "the timed step's fused in-projection output (q, k, v, sigmoid and decay gate columns)"}


def copy_probe(torch, mib):
    """Untimed plain device copy of known size: the reference point that scales the HBM byte counters."""
    if mib <= 0:
        return
    nb = mib << 20
    src = torch.empty(nb, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def decode_profile(torch, B, copy_mib, launches=16):
    """The decode kernels alone, eagerly, for per-dispatch counters: W = 17408 x 5120 over DECODE_COPIES
    rotating copies (larger than the 256 MB MALL together), A at M = 1, 8, 32, 64."""
    from nvfp4_w4a4_gemm_quantize_amd import inputs
    d = inputs.decode(1)
    p, wg = B.nvfp4_pack_weights(dev_bf16(torch, d["W"]))
    copies = [p] + [p.clone() for _ in range(DECODE_COPIES - 1)]
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for i in range(launches):
        B.nvfp4_weight_stream_read(copies[i % DECODE_COPIES], 17408, 5120, sink)
    for M in (1, 8, 32, 64):
        a = dev_bf16(torch, inputs.decode(M, weights=False)["A"])
        qc, qs, qg = B.nvfp4_quantize(a)
        y = torch.empty((M, 17408), dtype=torch.bfloat16, device="cuda")
        for i in range(launches):
            B.gemm_w4a4(qc, qs, qg, copies[i % DECODE_COPIES], wg, 17408, 5120, out=y)
        if M == 1:
            for i in range(launches):
                B.nvfp4_linear(a, copies[i % DECODE_COPIES], wg, 17408, out=y, a_global=qg, a_codes=qc, a_scales=qs)
    torch.cuda.synchronize()
    copy_probe(torch, copy_mib)
    progress("decode profile launches done")
    print(json.dumps({"decode_profile": {"launches_per_kernel": launches, "M": [1, 8, 32, 64], "N": 17408,
                                         "K": 5120, "weight_copies": DECODE_COPIES}}), flush=True)


def single_config(torch, B, name):
    """One measurement on its own (bench.py --config NAME)."""
    if name == "linear":
        return linear_config(torch, B)
    if name == "quantizer":
        return quantizer_rates(torch, B)
    S = setup(torch, B)
    if name == "decode":
        return decode_sweep(torch, B, S)
    # the recurrence takes the fused in-projection's output of one step as its input
    step(torch, B, S, 0, None)
    return gdn_recurrence_run(torch, B, S)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one MI355X: the library has no multi-GPU path (the projections would shard "
              "by output columns, the down-projection by K); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    from nvfp4_w4a4_gemm_quantize_amd import binding as B
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    B.load()
    if args.decode_profile:
        decode_profile(torch, B, args.copy_probe_mib)
        return
    if args.config != "step":
        print(json.dumps({"config": args.config, "result": single_config(torch, B, args.config)}), flush=True)
        return
    S = setup(torch, B)
    progress("inputs packed and resident (%.1f s)" % S["setup_s"])
    for i in range(args.warmup):
        step(torch, B, S, i, None)
    names = list(OUTER_EVENTS + INNER_EVENTS)
    evs = [{n: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for n in names}
           for _ in range(args.steps)]
    # Even steps carry the per-GEMM events (kernel durations for the
    # roofline), odd steps only the outer ones (the part totals, free of the
    # inner events' delays); a single step carries both.
    inner = [i % 2 == 0 or args.steps == 1 for i in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(torch, B, S, i, evs[i], inner[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    progress("%d timed steps done" % args.steps)
    ins = [e for e, f in zip(evs, inner) if f]
    tot = [e for e, f in zip(evs, inner) if not f] or ins
    median_ms = lambda es, n: float(np.median([e[n][0].elapsed_time(e[n][1]) for e in es]))
    dur = {n: median_ms(tot, n) for n in OUTER_EVENTS}
    dur.update({n: median_ms(ins, n) for n in INNER_EVENTS})
    prefill_instrumented_ms = median_ms(ins, "prefill")
    prefill_flop = FLOP["gdn"] + FLOP["gate_up"] + FLOP["down"]
    value = prefill_flop / (dur["prefill"] * 1e-3) / 1e12
    gemm_ms = dur["gdn"] + dur["gate_up"] + dur["down"]
    achieved = prefill_flop / (gemm_ms * 1e-3) / 1e12
    sweep = None if args.no_decode_sweep else decode_sweep(torch, B, S)
    progress("decode sweep done")
    linear2 = linear_config(torch, B)
    quant = quantizer_rates(torch, B)
    progress("single linear layer and quantizer rates timed")
    fused_mlp = mlp_fused(torch, B, S)
    repairs = gdn_repairs(torch, B, S)
    recurrence = gdn_recurrence_run(torch, B, S)
    bf16_ctx = bf16_library_context(torch)
    progress("fused MLP, GDN repairs, the recurrence and the bf16 library context timed")
    traffic = measured_traffic()
    copy_probe(torch, args.copy_probe_mib)
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "hybrid-layer linear path: prefill M=4096 (GDN fused in-projection N=16480 K=5120 "
                               "with 6 per-module global scales + MLP gate_up N=34816 SiLU*mul, h quantize, down "
                               "K=17408) and decode M=1 (N=17408 K=5120)",
                   "prefill_tokens": 4096, "decode_tokens": 1, "weights": "NVFP4 packed, 16-element E4M3 scales",
                   "activations": "quantized per call (dynamic FP32 global scale)"},
        "roofline": {"bound": "mfma",
                     "kernel": "gemm_prefill_dma_kernel (3 GEMMs per step: gdn, gate_up, down; each a full-round "
                               "launch plus one for the partly filled last round: split-K pieces, "
                               "gemm_prefill_splitk_kernel, for gdn and down)",
                     "achieved": round(achieved, 2), "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_F16_TFLOPS, 4),
                     "traffic": None if traffic is None else int(sum(traffic.values()) / 3),
                     "traffic_per": "HBM bytes per GEMM (mean of the 3), FETCH_SIZE + WRITE_SIZE, copy-calibrated",
                     "algorithmic_bytes": int(sum(ALGO_BYTES.values()) / 3),
                     "fp4_peak_frac_context": round(achieved / PEAK_FP4_TFLOPS, 4)},
        "prefill_ms": {k: round(dur[k], 4) for k in ("prefill", "gdn", "gate_up", "down")},
        "prefill_ms_with_inner_events": round(prefill_instrumented_ms, 4),
        "decode": decode_summary(dur, sweep),
        "linear_M2048": linear2,
        "quantizer": quant,
        "mlp_fused_h_quantize": fused_mlp,
        "gdn_scale_repairs": repairs,
        "gdn_recurrence": recurrence,
        "bf16_torch_linear_context": bf16_ctx,
        "setup_s": round(S["setup_s"], 1),
    }
    if not args.no_cpu_baseline:
        progress("timing the CPU oracle")
        result["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
