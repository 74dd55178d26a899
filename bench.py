"""Benchmark of the Gated DeltaNet layer core on one MI355X.

One step = the prefill path of one layer over the 4096-token workload
(B=1, T=4096, 16 q/k heads, 32 v heads, d_k=d_v=128, bf16 in, fp32 state,
chunk 64): the causal conv1d+SiLU over the 8192 projected channels, then
the chunked prefill (phase 1 + phase 2) producing o and the final state.
`value` is tokens/s of that step.  Inputs are resident in HBM before timing
starts; 4 input/output buffer sets (~750 MB) are rotated so the 256 MB
Infinity Cache cannot serve a step from the previous one.

The roofline line is that of the chunked prefill itself, gdn_prefill_chunked
(prepare + scan) timed as one call on the q/k/v column blocks of the conv
output, against the layer's algorithmic bytes (HBM-bound) with its bf16
matrix-core fraction beside it.  The adversarial fp32 (8192 tokens) and
varlen bf16 (16 sequences) workloads get the same call timed on their own.

The decode path (conv step + recurrent step, B=64, fp32 32x128x128 states,
4 rotated state pools of 134 MB, 1000 steps) is measured in the same run and
reported under "decode", as two library calls and as the one fused call.
The timed loops run back to back with no event markers in them (a marker
leaves the GPU idle for a few microseconds between calls).  Per-call times
come from HIP events on the launch stream: each call alone, run back to
back under one event pair (the per-launch time the roofline uses), in
blocks of 10 launches for the spread (p10 / p50 / p90 of the block means),
and, separately, a marker after every call of a step.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2516.6      # dense bf16 matrix
FP32_PEAK_TFLOPS = 157.3       # fp32 matrix
METRIC = "GDN prefill tokens/s per layer (T=4096) + decode step HBM GB/s, % roofline"


def prefill_alg_bytes(T, hk, hv, dk, dv, n_seq=1, esize=2, state_in=False):
    """Algorithmic bytes of the prefill: q, k, v, o in the input dtype, g and
    beta in fp32, and the fp32 final state (+ the initial state if read)."""
    per_tok = (2 * hk * dk + 2 * hv * dv) * esize + 2 * hv * 4
    st = n_seq * hv * dk * dv * 4
    return T * per_tok + st * (2 if state_in else 1)


def prefill_alg_flops(T, hv, dk, dv, C=64):
    """Triangular-counted flops of the chunked algorithm: A = K K^T and P = Q K^T
    (lower triangles), the chunk inverse (C^3/6), W/U products, the three
    C x d_k x d_v state products and P U."""
    per_chunk = 2 * (C * (C - 1) / 2 * dk + C * (C + 1) / 2 * dk + C ** 3 / 6
                     + 2 * C * (C - 1) / 2 * dk + 3 * C * dk * dv + C * (C + 1) / 2 * dv)
    return per_chunk * (T / C) * hv


def prefill_alg_flops_varlen(lens, hv, dk, dv, C=64):
    """prefill_alg_flops summed over sequences chunked from their own starts,
    a partial last chunk of C' tokens counted at C'."""
    def chunk(c):
        return 2 * (c * (c - 1) / 2 * dk + c * (c + 1) / 2 * dk + c ** 3 / 6
                    + 2 * c * (c - 1) / 2 * dk + 3 * c * dk * dv + c * (c + 1) / 2 * dv)
    return sum((int(n) // C * chunk(C) + (chunk(int(n) % C) if int(n) % C else 0)) * hv for n in lens)


def percentiles(xs):
    """mean, p10, p50, p90 of a list of per-launch times (us)."""
    a = np.asarray(xs, dtype=np.float64)
    return {"mean": round(float(a.mean()), 2), "p10": round(float(np.percentile(a, 10)), 2),
            "p50": round(float(np.percentile(a, 50)), 2), "p90": round(float(np.percentile(a, 90)), 2),
            "blocks": int(a.size)}


def conv_prepare_alg_bytes(T, C, hv, esize=2, W=4):
    """Raw rows in, conv output (q | k | v) out, taps, and g, beta."""
    return T * C * esize * 2 + C * W * 4 + 2 * T * hv * 4


def decode_alg_bytes(B, hk, hv, dk, dv, esize=2):
    return 2 * B * hv * dk * dv * 4 + B * (2 * hk * dk + 2 * hv * dv) * esize + 2 * B * hv * 4


def gated_norm_alg_bytes(T, hv, dv, esize=2):
    """o and the gate z read, y written, and the fp32 weight."""
    return 3 * T * hv * dv * esize + dv * 4


def gating_alg_bytes(T, hv, esize=2):
    """a and b read, g and beta (fp32) written, and the two fp32 parameters."""
    return 2 * T * hv * esize + 2 * T * hv * 4 + 2 * hv * 4


def decode_conv_alg_bytes(B, hk, hv, dk, dv, W=4, esize=2):
    """The fused step: state read and written, the raw row and the conv
    window (read and written) in, o out, g and beta, and the conv taps."""
    cc = 2 * hk * dk + hv * dv
    return (2 * B * hv * dk * dv * 4 + B * cc * esize + 2 * B * (W - 1) * cc * esize + B * hv * dv * esize
            + 2 * B * hv * 4 + cc * W * 4)


KERNEL_SOURCES = {"conv_prepare": ["conv1d.hip", "conv_math.h", "prefill.hip"],
                  "scan_gated_norm": ["prefill.hip", "prefill_seg.hip"],
                  "prefill_chunked": ["prefill.hip", "prefill_seg.hip"],
                  "prefill_scan": ["prefill.hip", "prefill_seg.hip"], "decode_step": ["decode.hip", "conv_math.h"],
                  "conv_step": ["conv1d.hip", "conv_math.h"], "decode_conv_step": ["decode.hip", "conv_math.h"],
                  "gated_norm": ["gated_norm.hip"], "gating": ["gating.hip"]}
# The GPU kernels each library call launches on the 4096-token bf16 layer
# (conv_prepare: the convolution, then the chunk prepare; the scan call runs
# the segment-parallel carry: two passes and a combine; prefill_chunked is
# the prepare followed by the scan, the whole chunked prefill) and on the
# 64-sequence decode step (two calls, or the one fused call).
CALL_KERNELS = {"conv_prepare": ["k_conv1d", "k_prepare"],
                "prefill_chunked": ["k_prepare", "k_seg_pass1", "k_seg_combine", "k_seg_pass2"],
                "prefill_scan": ["k_seg_pass1", "k_seg_combine", "k_seg_pass2"],
                "scan_gated_norm": ["k_seg_pass1", "k_seg_combine", "k_seg_pass2"], "decode_step": ["k_decode"],
                "conv_step": ["k_conv_step"], "decode_conv_step": ["k_decode_conv"],
                "gated_norm": ["k_gated_norm"], "gating": ["k_gating"]}


def source_digest(kernel=None):
    """Hash of the sources a kernel is built from: its own .hip file and the
    shared device headers (all of csrc/ if kernel is None)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "linear_attention_delta_amd", "csrc")
    names = sorted(os.listdir(csrc)) if kernel is None else \
        sorted(KERNEL_SOURCES[kernel] + ["gdn_device.h", "gdn_internal.h"])
    for f in names:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def read_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary
    profiles/<kernel>.<workload>.counters.txt, if it was taken on the
    kernel's current sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"{kernel}.{workload}.counters.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_digest") != source_digest(kernel):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--blocks", type=int, default=20, help="blocks of back-to-back launches for the percentiles")
    ap.add_argument("--no-extra-workloads", action="store_true",
                    help="skip the adversarial fp32 and varlen throughput lines")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sets", type=int, default=4, help="rotated buffer sets (MALL control)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run 3 plain fp32 copies of 512 MiB (y = x * 1), so that a counter run can "
                         "scale FETCH_SIZE / WRITE_SIZE by what they read for a kernel of known traffic")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the layer shards by "
              "heads or sequences with no collective inside it); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from linear_attention_delta_amd import gdn, synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    if args.calibrate_copy:
        src = torch.ones(128 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    # ---------------------------------------------------------------- prefill
    inp = synth.prefill_4k_bf16()
    sh = inp.shape
    T = inp.total_tokens
    CC = sh.conv_channels
    a = sh.num_qk_heads * sh.head_dim_k
    nsets = max(1, args.sets)
    w = torch.from_numpy(inp.conv_w).to(dev)
    sets = []
    for i in range(nsets):
        x = torch.from_numpy(inp.x).to(torch.bfloat16).to(dev)
        y = torch.empty((T, CC), dtype=torch.bfloat16, device=dev)
        g = torch.from_numpy(inp.g).to(dev)
        beta = torch.from_numpy(inp.beta).to(dev)
        o = torch.empty((T, sh.num_v_heads, sh.head_dim_v), dtype=torch.bfloat16, device=dev)
        st = torch.empty((1, sh.num_v_heads, sh.head_dim_k, sh.head_dim_v), dtype=torch.float32, device=dev)
        sets.append(dict(x=x, y=y, g=g, beta=beta, o=o, st=st))
    # the gated norm's gate and weight (the step after the scan, timed on its own)
    zn, wn = synth.gate_inputs(5, T, sh.num_v_heads, sh.head_dim_v, "bf16")
    wn = torch.from_numpy(wn).to(dev)
    # and the gates' raw projections (the step before it)
    abn, A_log, dt_bias = synth.gating_inputs(6, T, sh.num_v_heads, "bf16")
    A_log, dt_bias = torch.from_numpy(A_log).to(dev), torch.from_numpy(dt_bias).to(dev)
    for s_ in sets:
        s_["z"] = torch.from_numpy(zn).to(torch.bfloat16).to(dev)
        s_["yn"] = torch.empty_like(s_["o"])
        s_["ab"] = torch.from_numpy(abn).to(torch.bfloat16).to(dev)
        s_["a_"], s_["b_"] = s_["ab"][:, :sh.num_v_heads], s_["ab"][:, sh.num_v_heads:]
        s_["gg"] = torch.empty_like(s_["g"])
        s_["bg"] = torch.empty_like(s_["beta"])
    # one bound problem (dims + workspace) serves every buffer set
    cp = gdn.ConvPrefill(sets[0]["x"], w, num_qk_heads=sh.num_qk_heads, num_v_heads=sh.num_v_heads,
                         head_dim_k=sh.head_dim_k, head_dim_v=sh.head_dim_v, seqlen=T, chunk_size=64)
    torch.cuda.synchronize()

    def step(s):
        cp.conv_prepare(s["x"], s["y"], s["g"], s["beta"])
        cp.scan(s["y"], s["g"], s["beta"], s["o"], None, s["st"])

    # Per-call figures: an event marker after each call.  A marker costs the
    # stream a few microseconds of idle GPU time between the calls, so the
    # timed loop below runs without any.
    def step_marked(s, ev):
        cp.conv_prepare(s["x"], s["y"], s["g"], s["beta"])
        ev[0].record(stream)
        cp.scan(s["y"], s["g"], s["beta"], s["o"], None, s["st"])
        ev[1].record(stream)

    # One call alone, n times back to back over the rotating buffer sets,
    # with one event pair around the run: its per-launch time.  Every set
    # holds the same input, so the workspace prepared for one serves all.
    def back_to_back(fn, n):
        r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        r0.record(stream)
        for i in range(n):
            fn(sets[i % nsets])
        r1.record(stream)
        torch.cuda.synchronize()
        return r0.elapsed_time(r1) * 1e3 / n

    # The same in `blocks` blocks of `per` launches, one event pair per block:
    # the mean per-launch time over all launches and the spread of the block
    # means (p10 / p50 / p90).
    def blocks_of(fn, per=10, blocks=None):
        nb_ = blocks or args.blocks
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(nb_)]
        torch.cuda.synchronize()
        for b in range(nb_):
            ev[b][0].record(stream)
            for i in range(per):
                fn(sets[(b * per + i) % nsets])
            ev[b][1].record(stream)
        torch.cuda.synchronize()
        per_launch = [e0.elapsed_time(e1) * 1e3 / per for e0, e1 in ev]
        return float(np.mean(per_launch)), percentiles(per_launch)

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    m0 = torch.cuda.Event(enable_timing=True)
    m0.record(stream)
    for i in range(args.steps):
        step_marked(sets[i % nsets], evs[i])
    torch.cuda.synchronize()
    prev = [m0] + [e[1] for e in evs[:-1]]
    k_cp_ev = float(np.mean([p.elapsed_time(e[0]) for p, e in zip(prev, evs)]) * 1e3)   # us
    k_scan_ev = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]) * 1e3)

    nb = max(args.steps, 20)
    k_cp = back_to_back(lambda s: cp.conv_prepare(s["x"], s["y"], s["g"], s["beta"]), nb)
    k_scan = back_to_back(lambda s: cp.scan(s["y"], s["g"], s["beta"], s["o"], None, s["st"]), nb)
    # the whole chunked prefill as one library call (gdn_prefill_chunked:
    # prepare + scan) on the q, k, v column blocks of each set's conv output
    pc = gdn.Prefill(*cp.views(sets[0]["y"]), seqlen=T, chunk_size=64)

    def prefill_call(s):
        q_, k_, v_ = cp.views(s["y"])
        pc(q_, k_, v_, s["g"], s["beta"], s["o"], None, s["st"])

    for i in range(nsets):
        prefill_call(sets[i])
    k_pc = back_to_back(prefill_call, nb)
    _, pct_pc = blocks_of(prefill_call)
    _, pct_cp = blocks_of(lambda s: cp.conv_prepare(s["x"], s["y"], s["g"], s["beta"]))
    _, pct_scan = blocks_of(lambda s: cp.scan(s["y"], s["g"], s["beta"], s["o"], None, s["st"]))
    _, pct_step = blocks_of(step)

    # The timed run comes after the per-call measurements above: the GPU's
    # clocks take some 25 ms of sustained load to settle, and a step measured
    # before that runs about 3 % slower.
    for i in range(args.warmup):
        step(sets[i % nsets])
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        step(sets[i % nsets])
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    gpu_ms = t_start.elapsed_time(t_end)
    ms_per_step = wall * 1e3 / args.steps
    tokens_per_s = T / (ms_per_step * 1e-3)

    norm = gdn.GatedNorm(sets[0]["o"], sets[0]["z"], wn, y=sets[0]["yn"])
    for i in range(nsets):  # its first launches, before the timed run
        norm(sets[i]["o"], sets[i]["z"], sets[i]["yn"])
    k_norm = back_to_back(lambda s: norm(s["o"], s["z"], s["yn"]), nb)
    B_norm = gated_norm_alg_bytes(T, sh.num_v_heads, sh.head_dim_v)
    hv_ = sh.num_v_heads
    gate = gdn.Gating(sets[0]["a_"], sets[0]["b_"], A_log, dt_bias)
    for i in range(nsets):
        gate(sets[i]["a_"], sets[i]["b_"], sets[i]["gg"], sets[i]["bg"])
    k_gate = back_to_back(lambda s: gate(s["a_"], s["b_"], s["gg"], s["bg"]), nb)
    B_gate = gating_alg_bytes(T, hv_)
    # the whole prefill from the raw projections in one call, the gates
    # computed in the prepare (against gating + conv_prepare + scan)
    for s_ in sets:
        s_["gates"] = gdn.gate_inputs(s_["a_"], s_["b_"], A_log, dt_bias)
    k_gated = back_to_back(lambda s: gdn.conv_prefill_gated(cp, s["x"], s["y"], s["gates"], s["o"],
                                                            state_out=s["st"]), nb)
    gating = {"gating_us": round(k_gate, 2), "prefill_conv_gated_us": round(k_gated, 2),
              "prefill_gating_then_calls_us": round(k_gate + k_cp + k_scan, 2),
              "roofline": {"bound": "hbm", "kernel": "gating", "gpu_kernels": CALL_KERNELS["gating"],
                           "achieved": round(B_gate / (k_gate * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(B_gate / (k_gate * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                           "traffic": read_traffic("gating", inp.name), "alg_bytes_per_launch": int(B_gate),
                           "avg_launch_us": round(k_gate, 2)}}
    # the carry with the norm fused into its output write (o never goes
    # through memory), against the carry followed by the norm
    for i in range(nsets):
        cp.scan_gated_norm(sets[i]["y"], sets[i]["g"], sets[i]["beta"], sets[i]["z"], wn, sets[i]["yn"], None,
                           sets[i]["st"])
    k_scan_norm = back_to_back(lambda s: cp.scan_gated_norm(s["y"], s["g"], s["beta"], s["z"], wn, s["yn"], None,
                                                            s["st"]), nb)
    gated_norm = {"gated_norm_us": round(k_norm, 2),
                  "scan_gated_norm_us": round(k_scan_norm, 2), "scan_then_gated_norm_us": round(k_scan + k_norm, 2),
                  "roofline": {"bound": "hbm", "kernel": "gated_norm", "gpu_kernels": CALL_KERNELS["gated_norm"],
                               "achieved": round(B_norm / (k_norm * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBS,
                               "unit": "GB/s", "frac": round(B_norm / (k_norm * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                               "traffic": read_traffic("gated_norm", inp.name), "alg_bytes_per_launch": int(B_norm),
                               "avg_launch_us": round(k_norm, 2)}}

    # warm figure: one buffer set, back to back (MALL may serve it)
    warm_evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(50)]
    for i in range(10):
        step(sets[0])
    w0 = torch.cuda.Event(enable_timing=True)
    w0.record(stream)
    for i in range(50):
        step_marked(sets[0], warm_evs[i])
    torch.cuda.synchronize()
    wprev = [w0] + [e[1] for e in warm_evs[:-1]]
    warm_cp = float(np.mean([p.elapsed_time(e[0]) for p, e in zip(wprev, warm_evs)]) * 1e3)
    warm_scan = float(np.mean([e[0].elapsed_time(e[1]) for e in warm_evs]) * 1e3)

    B_pre = prefill_alg_bytes(T, sh.num_qk_heads, sh.num_v_heads, sh.head_dim_k, sh.head_dim_v)
    F_pre = prefill_alg_flops(T, sh.num_v_heads, sh.head_dim_k, sh.head_dim_v)
    B_cp = conv_prepare_alg_bytes(T, CC, sh.num_v_heads)
    kernels = {"conv_prepare": float(k_cp), "prefill_scan": float(k_scan)}
    # The roofline is that of the chunked prefill, gdn_prefill_chunked timed
    # as one call: the layer's algorithmic bytes (q, k, v, o, g, beta and the
    # final state) and flops over its per-launch time.  Arithmetic intensity
    # 177 flop/B is below the chip's ridge (2516.6 TFLOP/s / 8 TB/s = 315), so
    # HBM bounds it; the bf16 matrix-core fraction is given beside.
    achieved = B_pre / (k_pc * 1e-6) / 1e9
    roofline = {"bound": "hbm", "kernel": "prefill_chunked", "gpu_kernels": CALL_KERNELS["prefill_chunked"],
                "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": read_traffic("prefill_chunked", inp.name),
                "alg_bytes_per_launch": int(B_pre), "alg_flops_per_launch": int(F_pre),
                "avg_launch_us": round(k_pc, 2), "launch_us_blocks": pct_pc,
                "tokens_per_s": round(T / (k_pc * 1e-6), 1),
                "mfma_bf16": {"achieved": round(F_pre / (k_pc * 1e-6) / 1e12, 2), "peak": BF16_PEAK_TFLOPS,
                              "unit": "TFLOP/s", "frac": round(F_pre / (k_pc * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4)}}
    step_us = kernels["conv_prepare"] + kernels["prefill_scan"]

    # ----------------------------------------------------------------- decode
    dinp = synth.decode_b64_bf16()
    dsh = dinp.shape
    Bd = dinp.batch
    npool = 4
    pools = [torch.from_numpy(dinp.state0).to(dev) for _ in range(npool)]
    cwins = [torch.from_numpy(dinp.conv_state0).to(torch.bfloat16).to(dev) for _ in range(npool)]
    xs = [torch.from_numpy(dinp.x[p]).to(torch.bfloat16).to(dev) for p in range(dinp.pool)]
    gs = [torch.from_numpy(dinp.g[p]).to(dev) for p in range(dinp.pool)]
    bs = [torch.from_numpy(dinp.beta[p]).to(dev) for p in range(dinp.pool)]
    wd = torch.from_numpy(dinp.conv_w).to(dev)
    yd = torch.empty((Bd, dsh.conv_channels), dtype=torch.bfloat16, device=dev)
    od = torch.empty((Bd, dsh.num_v_heads, dsh.head_dim_v), dtype=torch.bfloat16, device=dev)
    ad = dsh.num_qk_heads * dsh.head_dim_k
    qd = yd[:, :ad].view(Bd, dsh.num_qk_heads, dsh.head_dim_k)
    kd = yd[:, ad:2 * ad].view(Bd, dsh.num_qk_heads, dsh.head_dim_k)
    vd = yd[:, 2 * ad:].view(Bd, dsh.num_v_heads, dsh.head_dim_v)

    conv_d = gdn.Conv1d(xs[0], wd, seqlen=1, num_seqs=Bd)
    dec = gdn.Decode(qd, kd, vd, num_slots=Bd)

    def dstep(i, ev=None):
        p = i % dinp.pool
        pool = i % npool
        if ev is not None:
            ev[0].record(stream)
        conv_d(xs[p], yd, cwins[pool])
        if ev is not None:
            ev[1].record(stream)
        dec(qd, kd, vd, gs[p], bs[p], pools[pool], od)
        if ev is not None:
            ev[2].record(stream)

    for i in range(20):
        dstep(i)
    torch.cuda.synchronize()
    dw0 = time.perf_counter()
    for i in range(args.decode_steps):
        dstep(i)
    torch.cuda.synchronize()
    dwall = time.perf_counter() - dw0
    devs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.decode_steps)]
    for i in range(args.decode_steps):
        dstep(i, devs[i])
    torch.cuda.synchronize()
    d_conv = float(np.mean([e[0].elapsed_time(e[1]) for e in devs]) * 1e3)
    d_step_events = float(np.mean([e[1].elapsed_time(e[2]) for e in devs]) * 1e3)
    # the recurrent step alone, back to back over the rotating state pools,
    # with one event pair around the whole run: per-launch average without
    # the per-call event packets (they add ~3 us to each bracketed call)
    nrun = args.decode_steps
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    r0.record(stream)
    for i in range(nrun):
        p = i % dinp.pool
        dec(qd, kd, vd, gs[p], bs[p], pools[i % npool], od)
    r1.record(stream)
    torch.cuda.synchronize()
    d_step = r0.elapsed_time(r1) * 1e3 / nrun

    def decode_blocks(fn, per=10):
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.blocks)]
        torch.cuda.synchronize()
        for b in range(args.blocks):
            ev[b][0].record(stream)
            for i in range(per):
                fn(b * per + i)
            ev[b][1].record(stream)
        torch.cuda.synchronize()
        return percentiles([e0.elapsed_time(e1) * 1e3 / per for e0, e1 in ev])

    pct_dec = decode_blocks(lambda i: dec(qd, kd, vd, gs[i % dinp.pool], bs[i % dinp.pool], pools[i % npool], od))
    B_dec = decode_alg_bytes(Bd, dsh.num_qk_heads, dsh.num_v_heads, dsh.head_dim_k, dsh.head_dim_v)
    dec_gbs = B_dec / (d_step * 1e-6) / 1e9

    # the same step as one fused call (conv step + recurrent step in one
    # kernel): wall time of the marker-free loop, and the per-launch time
    # back to back under one event pair
    fused = gdn.DecodeConv(xs[0], wd, num_qk_heads=dsh.num_qk_heads, num_v_heads=dsh.num_v_heads,
                           head_dim_k=dsh.head_dim_k, head_dim_v=dsh.head_dim_v, num_slots=Bd)

    def fstep(i):
        p = i % dinp.pool
        fused(xs[p], gs[p], bs[p], pools[i % npool], cwins[i % npool], od)

    for i in range(20):
        fstep(i)
    torch.cuda.synchronize()
    fw0 = time.perf_counter()
    for i in range(args.decode_steps):
        fstep(i)
    torch.cuda.synchronize()
    fwall = time.perf_counter() - fw0
    r0.record(stream)
    for i in range(nrun):
        fstep(i)
    r1.record(stream)
    torch.cuda.synchronize()
    f_step = r0.elapsed_time(r1) * 1e3 / nrun
    pct_fused = decode_blocks(fstep)
    B_fused = decode_conv_alg_bytes(Bd, dsh.num_qk_heads, dsh.num_v_heads, dsh.head_dim_k, dsh.head_dim_v,
                                    W=dinp.conv_w.shape[1])
    fused_gbs = B_fused / (f_step * 1e-6) / 1e9
    decode = {"workload": dinp.name, "batch": Bd, "state_pools": npool, "steps": args.decode_steps,
              "decode_step_us": round(d_step, 2), "decode_step_us_per_call_events": round(d_step_events, 2),
              "conv_step_us": round(d_conv, 2),
              "ms_per_token_step_wall": round(dwall * 1e3 / args.decode_steps, 4),
              "tokens_per_s": round(Bd / (dwall / args.decode_steps), 1),
              "roofline": {"bound": "hbm", "kernel": "decode_step", "gpu_kernels": CALL_KERNELS["decode_step"],
                           "achieved": round(dec_gbs, 1),
                           "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                           "traffic": read_traffic("decode_step", dinp.name), "alg_bytes_per_launch": int(B_dec),
                           "avg_launch_us": round(d_step, 2), "launch_us_blocks": pct_dec},
              "fused_conv_step": {
                  "decode_conv_step_us": round(f_step, 2),
                  "ms_per_token_step_wall": round(fwall * 1e3 / args.decode_steps, 4),
                  "tokens_per_s": round(Bd / (fwall / args.decode_steps), 1),
                  "roofline": {"bound": "hbm", "kernel": "decode_conv_step",
                               "gpu_kernels": CALL_KERNELS["decode_conv_step"], "achieved": round(fused_gbs, 1),
                               "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(fused_gbs / HBM_PEAK_GBS, 4),
                               "traffic": read_traffic("decode_conv_step", dinp.name),
                               "alg_bytes_per_launch": int(B_fused), "avg_launch_us": round(f_step, 2),
                               "launch_us_blocks": pct_fused}}}

    # ------------------------------------- multi-layer decode, eager vs graph
    # A token's step through `layers` layers of the fused, gated decode step
    # (each layer its own taps, gates, state pool and window), issued call by
    # call from Python, and as one captured HIP graph replayed per token.
    def decode_graph_figures(batch, layers=8, tokens=50):
        hv, cc_ = dsh.num_v_heads, dsh.conv_channels
        r = np.random.default_rng(batch)
        ly = []
        for _ in range(layers):
            ly.append(dict(
                w=torch.from_numpy((0.5 * r.normal(size=(cc_, 4))).astype(np.float32)).to(dev),
                A=torch.from_numpy(r.uniform(-1, 1.5, size=hv).astype(np.float32)).to(dev),
                D=torch.from_numpy((0.5 * r.normal(size=hv)).astype(np.float32)).to(dev),
                S=torch.from_numpy((0.02 * r.normal(size=(batch, hv, dsh.head_dim_k, dsh.head_dim_v)))
                                   .astype(np.float32)).to(dev),
                W=torch.zeros((batch, 3, cc_), dtype=torch.bfloat16, device=dev),
                x=torch.from_numpy(r.normal(size=(batch, cc_)).astype(np.float32)).to(torch.bfloat16).to(dev),
                ab=torch.from_numpy(r.normal(size=(batch, 2 * hv)).astype(np.float32)).to(torch.bfloat16).to(dev),
                o=torch.empty((batch, hv, dsh.head_dim_v), dtype=torch.bfloat16, device=dev)))

        def bind():
            return ([gdn.DecodeConv(l_["x"], l_["w"], num_qk_heads=dsh.num_qk_heads, num_v_heads=hv,
                                    head_dim_k=dsh.head_dim_k, head_dim_v=dsh.head_dim_v, num_slots=batch)
                     for l_ in ly],
                    [gdn.gate_inputs(l_["ab"][:, :hv], l_["ab"][:, hv:], l_["A"], l_["D"]) for l_ in ly])

        def token(steps, gates):
            for i, l_ in enumerate(ly):
                gdn.decode_conv_gated_step(steps[i], l_["x"], gates[i], l_["S"], l_["W"], l_["o"])

        steps_e, gates_e = bind()
        for _ in range(5):
            token(steps_e, gates_e)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(tokens):
            token(steps_e, gates_e)
        torch.cuda.synchronize()
        eager = (time.perf_counter() - t0) / tokens
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            steps_w, gates_w = bind()
            token(steps_w, gates_w)
        stream.wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            steps_g, gates_g = bind()
            token(steps_g, gates_g)
        for _ in range(5):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(tokens):
            graph.replay()
        torch.cuda.synchronize()
        replay = (time.perf_counter() - t0) / tokens
        del graph, ly
        return {"batch": batch, "layers": layers, "tokens": tokens, "eager_us_per_token": round(eager * 1e6, 1),
                "graph_us_per_token": round(replay * 1e6, 1),
                "graph_tokens_per_s": round(batch / replay, 1)}

    decode["multilayer_graph"] = [decode_graph_figures(1), decode_graph_figures(Bd)]

    # ------------------------------- the adversarial and varlen prefill lines
    # gdn_prefill_chunked alone on the other two prefill workloads: 8192
    # tokens of repeated keys in fp32 (one sequence), and 16 packed bf16
    # sequences with initial states.  Their inputs (268 MB and 981 MB of
    # conv output) exceed the 256 MB Infinity Cache, so no rotation is needed.
    extra = None
    if not args.no_extra_workloads:
        extra = {}
        for key, make in (("adversarial_fp32", synth.adversarial_8k_fp32), ("varlen_bf16", synth.varlen_bf16)):
            winp = make()
            wsh = winp.shape
            tdt = torch.bfloat16 if winp.dtype == "bf16" else torch.float32
            esz = 2 if winp.dtype == "bf16" else 4
            Tw = winp.total_tokens
            xw = torch.from_numpy(winp.x).to(tdt).to(dev)
            cuw = None if winp.dense_T else torch.from_numpy(winp.cu_seqlens).to(dev)
            yw = gdn.conv1d(xw, torch.from_numpy(winp.conv_w).to(dev), cu_seqlens=cuw,
                            seqlen=winp.dense_T or None, num_seqs=winp.num_seqs)
            del xw
            aw = wsh.num_qk_heads * wsh.head_dim_k
            qw = yw[:, :aw].view(Tw, wsh.num_qk_heads, wsh.head_dim_k)
            kw = yw[:, aw:2 * aw].view(Tw, wsh.num_qk_heads, wsh.head_dim_k)
            vw = yw[:, 2 * aw:].view(Tw, wsh.num_v_heads, wsh.head_dim_v)
            gw, bw = torch.from_numpy(winp.g).to(dev), torch.from_numpy(winp.beta).to(dev)
            s0w = None if winp.state0 is None else torch.from_numpy(winp.state0).to(dev)
            ow = torch.empty((Tw, wsh.num_v_heads, wsh.head_dim_v), dtype=tdt, device=dev)
            stw = torch.empty((winp.num_seqs, wsh.num_v_heads, wsh.head_dim_k, wsh.head_dim_v), dtype=torch.float32,
                              device=dev)
            pw = gdn.Prefill(qw, kw, vw, cu_seqlens=cuw, seqlen=winp.dense_T or None, num_seqs=winp.num_seqs,
                             chunk_size=64)
            for _ in range(3):
                pw(qw, kw, vw, gw, bw, ow, s0w, stw)
            nw = 20
            r0.record(stream)
            for _ in range(nw):
                pw(qw, kw, vw, gw, bw, ow, s0w, stw)
            r1.record(stream)
            torch.cuda.synchronize()
            t_w = r0.elapsed_time(r1) * 1e3 / nw
            lens = np.diff(winp.cu_seqlens)
            Bw = prefill_alg_bytes(Tw, wsh.num_qk_heads, wsh.num_v_heads, wsh.head_dim_k, wsh.head_dim_v,
                                   n_seq=winp.num_seqs, esize=esz, state_in=s0w is not None)
            Fw = prefill_alg_flops_varlen(lens, wsh.num_v_heads, wsh.head_dim_k, wsh.head_dim_v)
            hbm = Bw / (t_w * 1e-6) / 1e9
            if winp.dtype == "f32":   # fp32 operands: the fp32 matrix rate bounds it (36.8 GFLOP vs 407 MB)
                rl = {"bound": "mfma", "achieved": round(Fw / (t_w * 1e-6) / 1e12, 2), "peak": FP32_PEAK_TFLOPS,
                      "unit": "TFLOP/s", "frac": round(Fw / (t_w * 1e-6) / 1e12 / FP32_PEAK_TFLOPS, 4),
                      "hbm_frac": round(hbm / HBM_PEAK_GBS, 4)}
            else:
                rl = {"bound": "hbm", "achieved": round(hbm, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                      "frac": round(hbm / HBM_PEAK_GBS, 4),
                      "mfma_bf16_frac": round(Fw / (t_w * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4)}
            rl.update({"kernel": "prefill_chunked", "traffic": read_traffic("prefill_chunked", winp.name),
                       "alg_bytes_per_launch": int(Bw), "alg_flops_per_launch": int(Fw),
                       "avg_launch_us": round(t_w, 2)})
            extra[key] = {"workload": winp.name, "tokens": Tw, "sequences": winp.num_seqs, "dtype": winp.dtype,
                          "prefill_chunked_us": round(t_w, 2), "tokens_per_s": round(Tw / (t_w * 1e-6), 1),
                          "roofline": rl}
            del yw, qw, kw, vw, ow, stw, pw, s0w, gw, bw
            torch.cuda.empty_cache()

    # ------------------------------------------------------------ CPU oracle
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        # the whole workload, repeated until about 10 s of CPU time have passed
        reps = 0
        t0 = time.perf_counter()
        while reps == 0 or (time.perf_counter() - t0 < 10.0 and reps < 50):
            y64, _ = oracle.conv1d(inp.x, inp.conv_w)
            qo, ko, vo = synth.split_qkv(y64, sh)
            _, _, nt = oracle.scan(qo, ko, vo, inp.g, inp.beta, n_threads=min(16, oracle.available_cores()),
                                   return_threads=True)
            reps += 1
        ct = time.perf_counter() - t0
        # and on one core: the whole workload once (the conv is single-threaded
        # in both figures)
        t1 = time.perf_counter()
        y64, _ = oracle.conv1d(inp.x, inp.conv_w)
        qo, ko, vo = synth.split_qkv(y64, sh)
        oracle.scan(qo, ko, vo, inp.g, inp.beta, n_threads=1)
        c1 = time.perf_counter() - t1
        cpu = {"value": round(reps * T / ct, 1), "unit": "tokens/s", "cores": int(nt), "kind": "oracle",
               "sample": f"the whole workload {reps} times: fp64 conv1d+SiLU over {T}x{CC} and the token-by-token "
                         f"scan of all {sh.num_v_heads} v-heads x {T} tokens, {ct:.2f} s on {cpu_model()} "
                         f"({oracle.available_cores()} cores in the affinity mask; the scan is threaded over "
                         f"(sequence, v-head) on at most 16, the box's CPU share for one GPU)",
               "one_core": {"value": round(T / c1, 1), "unit": "tokens/s", "cores": 1,
                            "sample": f"the whole workload once on one thread, {c1:.2f} s"}}

    out = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; Qwen3.5-4B-shaped GDN layer)",
        "config": {"workload": inp.name, "global_batch": 1, "seq_len": T, "qk_heads": sh.num_qk_heads,
                   "v_heads": sh.num_v_heads, "head_dim": sh.head_dim_k, "chunk": 64, "conv_width": 4,
                   "step": "conv1d+SiLU -> prefill prepare -> prefill scan (two library calls)",
                   "buffer_sets": nsets},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels_us": {k: round(v, 2) for k, v in kernels.items()},
        "kernels_us_blocks": {"conv_prepare": pct_cp, "prefill_scan": pct_scan, "step": pct_step},
        "kernels_us_per_call_events": {"conv_prepare": round(k_cp_ev, 2), "prefill_scan": round(k_scan_ev, 2)},
        "gpu_ms_per_step_events": round(gpu_ms / args.steps, 5),
        "prefill_chunked_us": round(k_pc, 2),
        "step_kernels": {"us": round(step_us, 2), "tokens_per_s": round(T / (step_us * 1e-6), 1),
                         "hbm_frac": round(B_pre / (step_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                         "mfma_frac_bf16": round(F_pre / (step_us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4),
                         "alg_bytes": int(B_pre), "alg_flops": int(F_pre)},
        "warm_single_set_us": {"conv_prepare": round(warm_cp, 2), "prefill_scan": round(warm_scan, 2)},
        "gated_norm": gated_norm,
        "gating": gating,
        "decode": decode,
        "prefill_workloads": extra,
        "source_digest": {k: source_digest(k) for k in KERNEL_SOURCES},
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
