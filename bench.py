"""Throughput of the Mamba-3 SSM recurrence on one MI355X, through the C ABI.

One step = one m3_prefill call over the SISO prefill workload (batch 4, 64
heads, P 64, N 128, 2048 tokens, chunk 64, bf16 I/O, fp32 state, B/C shared by
all heads). `value` is prefill tokens/s (mean over the timed calls; median,
p10 and p90 of the per-call event times are reported beside it). The same run
measures the decode step loop (batch 128, 64 heads, 1024 steps, R = 1 and
R = 4, with batch 64 and 256 beside it and a plain 1 GiB copy as the DRAM
reference), the MIMO R = 4 prefill and the long R = 4 prefill (32768 tokens)
+ 256 decode steps, each against the HBM and bf16-MFMA roofline with
algorithmic bytes / flops. The CPU oracle is timed on the host cores on a
bounded sample of the SISO, MIMO, long prefill and both decode workloads.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--quick] [--no-cpu]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prefill tokens/s + decode steps/s on 1 GPU; % of HBM / MFMA roofline"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s
FP32_VALU_PEAK_TFLOPS = 157.3  # MI355X fp32 vector (VALU), TFLOP/s
N_COPIES = 4                 # input copies rotated through so the 256 MB MALL cannot hold them

# HBM traffic per launch measured with rocprofv3 (FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0,
# KiB -> bytes; the factors come from a 1 GiB copy), valid only for the kernel
# sources it was taken on (sha256 prefix over the listed files, in order); the
# summaries with the commands are in profiles/. None until a kernel is profiled.
MEASURED_TRAFFIC = {
    "prefill1": ("f96f57ce3e0e1d1f", (2.0 * 39182.0 + 73728.0) * 1024),
    "prefill2": ("91c0da9e1364c8c6", (2.0 * 150050.3 + 270336.0) * 1024),
    "long": ("91c0da9e1364c8c6", (2.0 * 744735.6 + 1079920.3) * 1024),
    "decode1": ("0d01cb79fbad41c3", (2.0 * 133328.6 + 264563.3) * 1024),
    "decode4": ("0d01cb79fbad41c3", (2.0 * 137557.3 + 270875.6) * 1024),
}


def source_sha(files):
    """sha256 prefix over the concatenated kernel sources (the key of a measured traffic figure)."""
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "mamba_ssm_scan_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# kernel sources behind each timed workload (their sha256 prefix keys the traffic figures)
SOURCES = {
    "prefill1": ("m3_prefill_mfma.hip", "m3_mfma_common.h", "m3_device.h"),
    "prefill2": ("m3_prefill_ws4.hip", "m3_mfma_common.h", "m3_device.h"),
    "long": ("m3_prefill_ws4.hip", "m3_mfma_common.h", "m3_device.h"),
    "decode1": ("m3_decode.hip", "m3_device.h"),
    "decode4": ("m3_decode.hip", "m3_device.h"),
}


def measured_traffic(key):
    """Counter-measured bytes per launch, or None if the kernel source changed since (or never taken)."""
    if key not in MEASURED_TRAFFIC:
        return None
    sha, nbytes = MEASURED_TRAFFIC[key]
    try:
        cur = source_sha(SOURCES[key])
    except OSError:
        return None
    return nbytes if cur == sha else None


def prefill_bytes(b, L, H, G, P, N, R, io_bytes=2, h0=False, h_out=True):
    """Compulsory HBM bytes of one prefill: x, y, B, C (once per group), dt, lambda, h_out (+ h0)."""
    tok = b * L
    by = 2 * tok * H * R * P * io_bytes + 2 * tok * G * R * N * io_bytes + 2 * tok * H * 4
    by += H * (2 + N // 2) * 4
    if h_out:
        by += b * H * N * P * 4
    if h0:
        by += b * H * N * P * 4
    return by


def prefill_flops(b, L, H, P, N, R, Q):
    """Algorithmic flops: causal intra-chunk scores and masked product, inter-chunk output, state update."""
    full, last = divmod(L, Q)

    def chunk(q):
        return q * (q + 1) * R * R * (N + P) + 4 * q * R * N * P

    return b * H * (full * chunk(Q) + (chunk(last) if last else 0))


def decode_bytes(b, H, G, P, N, R, io_bytes=2):
    """Per step: state read + write, x_t, y_t, x_prev, x carry write, B_t, C_t, B_prev, B carry write, dt, lambda."""
    return b * H * N * P * 8 + 4 * b * H * R * P * io_bytes + 4 * b * G * R * N * io_bytes + 2 * b * H * 4


def _events():
    import torch
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def time_calls(run, steps, warmup):
    """`warmup` untimed calls of run(k), then two timed passes of `steps` calls each.

    Pass 1 (the throughput figure): the calls back to back between two HIP
    events, with the device synchronised on both sides; mean = elapsed / steps.
    Pass 2 (the spread): an event before the first call and after every call,
    giving per-call times (median, p10, p90). An event between two calls keeps
    the next launch from overlapping the previous one's tail, so pass 2's times
    carry that gap (a few microseconds) on top of pass 1's mean. All events are
    recorded on torch's current stream, the stream the library launches on.
    """
    import numpy as np
    import torch
    for k in range(warmup):
        run(k)
    torch.cuda.synchronize()
    e0, e1 = _events()
    e0.record()
    for k in range(steps):
        run(warmup + k)
    e1.record()
    torch.cuda.synchronize()
    mean = e0.elapsed_time(e1) / steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for k in range(steps):
        run(warmup + steps + k)
        ev[k + 1].record()
    torch.cuda.synchronize()
    per = np.array([ev[k].elapsed_time(ev[k + 1]) for k in range(steps)])
    p10, p50, p90 = np.percentile(per, [10, 50, 90])
    return {"mean": mean, "median": float(p50), "p10": float(p10), "p90": float(p90), "n": steps}


def _pct(t, scale=1.0, unit="ms"):
    """median / p10 / p90 of a time_calls result (its per-call pass), scaled (e.g. per step of a loop)."""
    return {f"median_{unit}": t["median"] * scale, f"p10_{unit}": t["p10"] * scale,
            f"p90_{unit}": t["p90"] * scale, "timed_calls": t["n"]}


def bench_prefill(wid, steps, warmup, log, special="", groups=1, dstate=None, rank=None, headdim=None):
    """special: "" (the workload), "real" (omega NULL: omega = 0), "euler" (lambda NULL: lambda = 1) or both;
    "raw": m3_prefill_fused on raw dt / lambda projections (softplus with a per-head bias, sigmoid in the kernels).

    groups: 1 (B, C shared by all heads, the primary reading) or H (one B, C per head).
    dstate / rank: the workload's shape with another state size or rank (R 8: the token-walk kernel;
    N 64 / 256: the chunked kernels, rows zero-padded / in two row passes).
    """
    import dataclasses
    import torch
    from mamba_ssm_scan_amd import binding, inputs
    w = inputs.WORKLOADS[wid]
    base = w.name
    if dstate is not None or rank is not None or headdim is not None:
        w = dataclasses.replace(w, dstate=dstate or w.dstate, rank=rank or w.rank, headdim=headdim or w.headdim)
    G = groups
    copies = [inputs.make_problem(batch=w.batch, seqlen=w.seqlen, heads=w.heads, groups=G, headdim=w.headdim,
                                  dstate=w.dstate, rank=w.rank, io_dtype=w.io_dtype, dist=w.dist, wid=wid,
                                  step=k, device="cuda") for k in range(N_COPIES)]
    y = torch.empty_like(copies[0]["x"])
    h = torch.empty((w.batch, w.heads, w.dstate, w.headdim), dtype=torch.float32, device="cuda")
    plan = binding.plan(binding.dims(w.batch, w.seqlen, w.heads, G, w.headdim, w.dstate), w.rank, w.chunk,
                        binding.M3_BF16)
    ws = torch.empty(max(plan.workspace_bytes, 256), dtype=torch.uint8, device="cuda")

    no_om, no_lam, raw = "real" in special, "euler" in special, "raw" in special
    if raw:  # raw projections of the step and the trapezoid weight
        for k, p in enumerate(copies):
            r = inputs.prologue_inputs(tokens=(w.batch, w.seqlen), heads=w.heads, groups=G, rank=w.rank,
                                       dstate=w.dstate, io_dtype=w.io_dtype, wid=400 + wid, step=k, device="cuda")
            p.update(dt=r["dt_raw"], lam=r["lambda_raw"], dt_bias=r["dt_bias"])

    def run(k):
        p = copies[k % N_COPIES]
        binding.prefill(p["x"], p["dt"], p["A"], None if no_om else p["omega"], None if no_lam else p["lam"],
                        p["B"], p["C"], p["D"], w.rank, w.chunk, y=y, h_out=h, workspace=ws, raw_steps=raw,
                        dt_bias=p.get("dt_bias"))

    t = time_calls(run, steps, warmup)
    ms = t["mean"]
    by = prefill_bytes(w.batch, w.seqlen, w.heads, G, w.headdim, w.dstate, w.rank)
    if no_lam:
        by -= w.batch * w.seqlen * w.heads * 4
    # algorithmic flops at the chunk the kernel walks (the plan's: at most 32 tokens at R 8)
    qk = -(-w.seqlen // plan.n_chunks) if plan.n_chunks else w.chunk
    fl = prefill_flops(w.batch, w.seqlen, w.heads, w.headdim, w.dstate, w.rank, qk)
    name = base + (f" ({special})" if special else "") + (f" G={G}" if G != 1 else "")
    if (w.dstate, w.rank, w.headdim) != (inputs.WORKLOADS[wid].dstate, inputs.WORKLOADS[wid].rank,
                                          inputs.WORKLOADS[wid].headdim):
        name += f" with N={w.dstate} R={w.rank} P={w.headdim}"
    r = {"workload": name, "ms_per_call": ms, "tokens_per_s": w.batch * w.seqlen / (ms * 1e-3),
         "hbm_gbs": by / (ms * 1e-3) / 1e9, "mfma_tflops": fl / (ms * 1e-3) / 1e12,
         "bytes": by, "flops": fl, "chunk": qk, "path": {binding.M3_PATH_MFMA: "mfma", binding.M3_PATH_SCAN: "scan"}.get(plan.path, "generic"),
         "segments": plan.segments, **_pct(t)}
    r["hbm_frac"] = r["hbm_gbs"] / HBM_PEAK_GBS
    r["mfma_frac"] = r["mfma_tflops"] / BF16_PEAK_TFLOPS
    log(f"prefill {name}: {ms * 1e3:.1f} us/call (median {t['median'] * 1e3:.1f}, p10 {t['p10'] * 1e3:.1f}, "
        f"p90 {t['p90'] * 1e3:.1f}), {r['tokens_per_s'] / 1e6:.1f} M tok/s, "
        f"{r['hbm_gbs']:.0f} GB/s ({100 * r['hbm_frac']:.1f}% HBM), {r['mfma_tflops']:.1f} TFLOP/s "
        f"({100 * r['mfma_frac']:.1f}% bf16 MFMA)")
    return r


def bench_decode(R, steps_total, reps, log, batch=None, wid=3, fused=False):
    """The decode loop: steps_total steps of m3_decode_step at batch b, timed per loop over all steps.

    fused: m3_decode_step_fused on raw projections (the input prologue in the step kernel) instead.
    """
    import torch
    from mamba_ssm_scan_amd import binding, inputs
    w = inputs.WORKLOADS[wid]
    b = w.batch if batch is None else batch
    di = inputs.decode_inputs(wid, steps_total, device="cuda", rank=R, batch=b)
    y = torch.empty_like(di["x"])
    st = binding.DecodeState(b, w.heads, 1, w.headdim, w.dstate, R, io_dtype=torch.bfloat16, h0=di["h0"])
    sh = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    A, om, D = di["A"].data_ptr(), di["omega"].data_ptr(), di["D"].data_ptr()
    if fused:  # raw B, C, dt, lambda for every step, and the prologue's weights
        raw = inputs.prologue_inputs(tokens=(steps_total, b), heads=w.heads, groups=1, rank=R, dstate=w.dstate,
                                     io_dtype="bf16", wid=320, device="cuda")
        di.update(B=raw["B_raw"], C=raw["C_raw"], dt=raw["dt_raw"], lam=raw["lambda_raw"])
        lib = binding.load()
        vp = ctypes.c_void_p
        wts = [vp(raw[k].data_ptr()) for k in ("B_weight", "B_bias", "C_weight", "C_bias")]
        dtb, eps = vp(raw["dt_bias"].data_ptr()), ctypes.c_float(1e-6)
    ptrs = [(di["x"][t].data_ptr(), di["dt"][t].data_ptr(), di["lam"][t].data_ptr(), di["B"][t].data_ptr(),
             di["C"][t].data_ptr(), y[t].data_ptr()) for t in range(steps_total)]

    def loop():
        if fused:
            for (xp, dp, lp, bp, cp, yp) in ptrs:
                binding.check(lib.m3_decode_step_fused(ctypes.byref(st._st), vp(xp), vp(dp), dtb, vp(A), vp(om),
                                                       vp(lp), vp(bp), vp(cp), *wts, eps, vp(D), R, vp(yp), sh))
            return
        for (xp, dp, lp, bp, cp, yp) in ptrs:
            st.step_raw(xp, dp, A, om, lp, bp, cp, D, yp, sh)

    # one call = one loop over all the steps (the first is the warm-up pass)
    t = time_calls(lambda k: loop(), reps, 1)
    ms_step = t["mean"] / steps_total
    by = decode_bytes(b, w.heads, 1, w.headdim, w.dstate, R)
    r = {"workload": f"decode_b{b}_h{w.heads}_p{w.headdim}_n{w.dstate}_r{R}_{steps_total}_steps"
                     + ("_fused_prologue" if fused else ""),
         "us_per_step": ms_step * 1e3, "steps_per_s": 1e3 / ms_step, "hbm_gbs": by / (ms_step * 1e-3) / 1e9,
         "bytes_per_step": by, **_pct(t, 1e3 / steps_total, "us_per_step")}
    r["timed_loops"] = r.pop("timed_calls")
    r["hbm_frac"] = r["hbm_gbs"] / HBM_PEAK_GBS
    # the rank-R contractions of a step (u_t = B_t x_t^T and y_t = h_t^T C_t, 2 N P R flops each per
    # head; the previous token's u is the last step's): what the MFMA decode kernel puts on the matrix
    # cores at R 2/4, against the bf16 peak -- tiny, the step is bound by the state stream
    fl = 4 * b * w.heads * w.dstate * w.headdim * R
    r["mfma_tflops"] = fl / (ms_step * 1e-3) / 1e12
    r["mfma_frac"] = r["mfma_tflops"] / BF16_PEAK_TFLOPS
    log(f"decode{' fused' if fused else ''} R={R} b={b}: {ms_step * 1e3:.1f} us/step (median {r['median_us_per_step']:.1f}, p10 "
        f"{r['p10_us_per_step']:.1f}, p90 {r['p90_us_per_step']:.1f} over {reps} loops of {steps_total}), "
        f"{r['steps_per_s']:.0f} steps/s, "
        f"{r['hbm_gbs']:.0f} GB/s ({100 * r['hbm_frac']:.1f}% HBM), rank contractions "
        f"{r['mfma_tflops']:.1f} TFLOP/s ({100 * r['mfma_frac']:.2f}% of bf16 MFMA peak)")
    return r


def bench_long(log, reps=20):
    """Workload 4: prefill of 32768 tokens (R = 4) then 256 decode steps, batch 1."""
    import torch
    from mamba_ssm_scan_amd import binding, inputs
    w = inputs.WORKLOADS[4]
    p = inputs.long_sequence(4, device="cuda")
    L = w.seqlen
    pre = inputs.slice_tokens(p, 0, L)
    y = torch.empty_like(pre["x"])
    h = torch.empty((1, w.heads, w.dstate, w.headdim), dtype=torch.float32, device="cuda")
    plan = binding.plan(binding.dims(1, L, w.heads, 1, w.headdim, w.dstate), w.rank, w.chunk, binding.M3_BF16)
    ws = torch.empty(max(plan.workspace_bytes, 256), dtype=torch.uint8, device="cuda")

    def pf():
        binding.prefill(pre["x"], pre["dt"], pre["A"], pre["omega"], pre["lam"], pre["B"], pre["C"], pre["D"],
                        w.rank, w.chunk, y=y, h_out=h, workspace=ws)

    tp = time_calls(lambda k: pf(), reps, 3)
    ms = tp["mean"]
    e0, e1 = _events()
    by = prefill_bytes(1, L, w.heads, 1, w.headdim, w.dstate, w.rank)
    fl = prefill_flops(1, L, w.heads, w.headdim, w.dstate, w.rank, w.chunk)
    # decode handoff: 256 steps from the prefill's final state
    st = binding.DecodeState(1, w.heads, 1, w.headdim, w.dstate, w.rank, io_dtype=torch.bfloat16, h0=h,
                             B_last=p["B"][:, L - 1].contiguous(), x_last=p["x"][:, L - 1].contiguous(), t0=L)
    steps = w.decode_steps
    xs = [p["x"][:, t].contiguous() for t in range(L, L + steps)]
    Bs = [p["B"][:, t].contiguous() for t in range(L, L + steps)]
    Cs = [p["C"][:, t].contiguous() for t in range(L, L + steps)]
    ds = [p["dt"][:, t].contiguous() for t in range(L, L + steps)]
    ls = [p["lam"][:, t].contiguous() for t in range(L, L + steps)]
    ys = [torch.empty_like(xs[0]) for _ in range(steps)]
    sh = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    e0.record()
    for k in range(steps):
        st.step_raw(xs[k].data_ptr(), ds[k].data_ptr(), p["A"].data_ptr(), p["omega"].data_ptr(), ls[k].data_ptr(),
                    Bs[k].data_ptr(), Cs[k].data_ptr(), p["D"].data_ptr(), ys[k].data_ptr(), sh)
    e1.record()
    torch.cuda.synchronize()
    dms = e0.elapsed_time(e1) / steps
    # the same 256 steps captured in one HIP graph: at batch 1 a step is a few
    # microseconds of GPU work and the launches from Python dominate; replaying
    # the captured loop (it continues from the state the eager loop left, which
    # changes nothing in the work) times the GPU side
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        shg = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for k in range(steps):
            st.step_raw(xs[k].data_ptr(), ds[k].data_ptr(), p["A"].data_ptr(), p["omega"].data_ptr(),
                        ls[k].data_ptr(), Bs[k].data_ptr(), Cs[k].data_ptr(), p["D"].data_ptr(), ys[k].data_ptr(),
                        shg)
    g.replay()
    torch.cuda.synchronize()
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    gms = e0.elapsed_time(e1) / steps
    r = {"workload": w.name, "prefill_ms": ms, "prefill_tokens_per_s": L / (ms * 1e-3),
         "prefill_hbm_gbs": by / (ms * 1e-3) / 1e9, "prefill_mfma_tflops": fl / (ms * 1e-3) / 1e12,
         "prefill_hbm_frac": by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "prefill_bytes": by, "prefill_flops": fl,
         "prefill_mfma_frac": fl / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, "segments": plan.segments,
         "prefill_timing": _pct(tp),
         "decode_us_per_step": dms * 1e3, "decode_steps_per_s": 1e3 / dms,
         "decode_graph_us_per_step": gms * 1e3, "decode_graph_steps_per_s": 1e3 / gms}
    log(f"long prefill {L} tokens R=4: {ms:.3f} ms, {r['prefill_tokens_per_s'] / 1e6:.1f} M tok/s "
        f"({100 * r['prefill_mfma_frac']:.1f}% MFMA, {100 * r['prefill_hbm_frac']:.1f}% HBM, "
        f"{plan.segments} segments); decode b=1: {dms * 1e3:.1f} us/step eager, {gms * 1e3:.1f} us/step "
        f"as a captured graph")
    return r


def backward_flops(b, L, H, P, N, R):
    """fp32 VALU flops of the sequential backward as built: per state entry and token, two forward
    passes (the checkpoint pass and the block recompute, 2R + 7 each) and the reverse step (12R + 18)."""
    return b * L * H * N * P * (2 * (2 * R + 7) + 12 * R + 18)


def bench_backward(wid, steps, warmup, log):
    """m3_prefill_backward on a prefill workload's inputs with a random dy (bf16) and dh_out."""
    import torch
    from mamba_ssm_scan_amd import binding, inputs
    w = inputs.WORKLOADS[wid]
    p = inputs.workload_prefill(wid, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(7)
    dy = torch.randn(p["x"].shape, generator=g, device="cuda").to(p["x"].dtype)
    dh = torch.randn((w.batch, w.heads, w.dstate, w.headdim), generator=g, device="cuda")
    need = binding.load().m3_prefill_backward_workspace_size(
        ctypes.byref(binding.dims(w.batch, w.seqlen, w.heads, 1, w.headdim, w.dstate)), w.rank)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")

    def run():
        binding.prefill_backward(p["x"], p["dt"], p["A"], p["omega"], p["lam"], p["B"], p["C"], p["D"], w.rank, dy,
                                 None, dh, workspace=ws)

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    e0, e1 = _events()
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    fl = backward_flops(w.batch, w.seqlen, w.heads, w.headdim, w.dstate, w.rank)
    r = {"workload": w.name + " backward", "ms_per_call": ms, "tokens_per_s": w.batch * w.seqlen / (ms * 1e-3),
         "valu_tflops": fl / (ms * 1e-3) / 1e12, "flops": fl, "workspace_bytes": need}
    r["valu_frac"] = r["valu_tflops"] / FP32_VALU_PEAK_TFLOPS
    log(f"backward {w.name}: {ms:.3f} ms/call, {r['tokens_per_s'] / 1e6:.2f} M tok/s, "
        f"{r['valu_tflops']:.1f} TFLOP/s fp32 VALU ({100 * r['valu_frac']:.1f}% of {FP32_VALU_PEAK_TFLOPS})")
    return r


def mixer_gemm_flops(T, d_model, H, G, P, N, R):
    """The block's projections: in (x, z, B, C, dt, lambda) and out, 2 flops per multiply-add."""
    HRP, GRN = H * R * P, G * R * N
    return 2 * T * d_model * (2 * HRP + 2 * GRN + 2 * H) + 2 * T * HRP * d_model


def bench_mixer(wid, steps, warmup, log, d_model=2048, decode_batch=128, decode_steps=64):
    """The mixer block (projections + prologue + recurrence + gate + output projection) on a
    prefill workload's token shape with d_model 2048 (H P = 4096 = 2 d_model, the Mamba-2
    expansion), then decode steps at batch 128 continuing from a prefill, eager and as a graph."""
    import torch
    from mamba_ssm_scan_amd import binding, inputs
    w = inputs.WORKLOADS[wid]
    b, L, H, P, N, R = w.batch, w.seqlen, w.heads, w.headdim, w.dstate, w.rank
    wt = inputs.mixer_inputs(batch=b, seqlen=L, d_model=d_model, heads=H, groups=1, headdim=P, dstate=N, rank=R,
                             wid=700, device="cuda")
    m = binding.Mixer(wt)
    u, out = wt["u"], torch.empty_like(wt["u"])
    for _ in range(warmup):
        m.prefill(u, chunk=w.chunk, out=out)
    torch.cuda.synchronize()
    e0, e1 = _events()
    e0.record()
    for _ in range(steps):
        m.prefill(u, chunk=w.chunk, out=out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    T = b * L
    fl = mixer_gemm_flops(T, d_model, H, 1, P, N, R) + prefill_flops(b, L, H, P, N, R, w.chunk)
    r = {"workload": f"mixer block d_model {d_model} on {w.name}", "ms_per_call": ms, "tokens_per_s": T / (ms * 1e-3),
         "tflops": fl / (ms * 1e-3) / 1e12, "flops": fl}
    r["mfma_frac"] = r["tflops"] / BF16_PEAK_TFLOPS
    log(f"mixer prefill {r['workload']}: {ms:.3f} ms/call, {r['tokens_per_s'] / 1e6:.1f} M tok/s, "
        f"{r['tflops']:.0f} TFLOP/s ({100 * r['mfma_frac']:.1f}% bf16 MFMA)")

    # decode: batch decode_batch sequences, a 64-token prefill, then steps
    bd = decode_batch
    wd = inputs.mixer_inputs(batch=bd, seqlen=64 + decode_steps, d_model=d_model, heads=H, groups=1, headdim=P,
                             dstate=N, rank=R, wid=701, device="cuda")
    md = binding.Mixer(wd)
    st = md.decode_state(bd)
    md.prefill(wd["u"][:, :64].contiguous(), chunk=w.chunk, state=st)
    us = [wd["u"][:, 64 + t].contiguous() for t in range(decode_steps)]
    outs = [torch.empty_like(us[0]) for _ in range(decode_steps)]
    for t in range(4):
        md.decode_step(st, us[t], outs[t])
    torch.cuda.synchronize()
    e0.record()
    for t in range(decode_steps):
        md.decode_step(st, us[t], outs[t])
    e1.record()
    torch.cuda.synchronize()
    dms = e0.elapsed_time(e1) / decode_steps
    # the same steps captured once
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        md.decode_step(st, us[0], outs[0])
        md.decode_step(st, us[1], outs[1])
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for t in range(decode_steps):
            md.decode_step(st, us[t], outs[t])
    g.replay()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(4):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    gms = e0.elapsed_time(e1) / (4 * decode_steps)
    r.update({"decode_batch": bd, "decode_ms_per_step": dms, "decode_graph_ms_per_step": gms,
              "decode_tokens_per_s": bd / (gms * 1e-3)})
    log(f"mixer decode step, batch {bd}: {dms * 1e3:.1f} us eager, {gms * 1e3:.1f} us as a captured graph "
        f"({r['decode_tokens_per_s'] / 1e6:.2f} M tok/s)")
    return r


def bench_prologue(log, steps=20, warmup=3, wid=2, tokens=None, copies=16):
    """m3_prologue (QK-norm + bias on B, C; softplus / sigmoid on dt, lambda) on a workload's raw projections.

    Inputs rotate through `copies` resident sets so the 256 MB MALL cannot hold
    them all; bytes = raw B, C, dt, lambda read + the four outputs written (+
    the small weight / bias arrays).
    """
    import torch
    from mamba_ssm_scan_amd import binding, inputs
    w = inputs.WORKLOADS[wid]
    tok = (w.batch, w.seqlen) if tokens is None else tuple(tokens)
    G, R, N, H = 1, w.rank, w.dstate, w.heads
    sets = [inputs.prologue_inputs(tokens=tok, heads=H, groups=G, rank=R, dstate=N, io_dtype=w.io_dtype, wid=300,
                                   step=k, device="cuda") for k in range(copies)]
    outs = [torch.empty_like(sets[0][k]) for k in ("B_raw", "C_raw", "dt_raw", "lambda_raw")]

    def run(k):
        p = sets[k % copies]
        binding.prologue(p["B_raw"], p["C_raw"], B_weight=p["B_weight"], B_bias=p["B_bias"], C_weight=p["C_weight"],
                         C_bias=p["C_bias"], eps=1e-6, dt_raw=p["dt_raw"], dt_bias=p["dt_bias"],
                         lambda_raw=p["lambda_raw"], B=outs[0], C=outs[1], dt=outs[2], lam=outs[3])

    # one call is a few microseconds of GPU work, less than the Python binding's
    # own overhead: the calls over all copies are captured in a HIP graph and
    # the graph is replayed, so the events time the GPU work
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for k in range(warmup):
            run(k)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for k in range(copies):
            run(k)
    g.replay()
    torch.cuda.synchronize()
    reps = max(2, steps // copies)
    e0, e1 = _events()
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (reps * copies)
    ntok = 1
    for v in tok:
        ntok *= v
    by = 2 * 2 * ntok * G * R * N * 2 + 2 * 2 * ntok * H * 4 + 4 * G * R * N * 4 + H * 4
    r = {"workload": f"prologue tokens={'x'.join(map(str, tok))} H={H} G={G} R={R} N={N} {w.io_dtype}",
         "ms_per_call": ms, "bytes": by, "hbm_gbs": by / (ms * 1e-3) / 1e9}
    r["hbm_frac"] = r["hbm_gbs"] / HBM_PEAK_GBS
    log(f"{r['workload']}: {ms * 1e3:.2f} us/call, {r['hbm_gbs']:.0f} GB/s ({100 * r['hbm_frac']:.1f}% HBM)")
    return r


def copy_probe(log, nbytes=1 << 30, reps=10):
    """A plain device-to-device copy of known size: the DRAM rate a streaming kernel can reach
    (2 GiB of traffic per call, 8x the 256 MB MALL), and the reference for the HBM byte counters."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    t = time_calls(lambda k: dst.copy_(src), reps, 3)
    gbs = 2 * nbytes / (t["median"] * 1e-3) / 1e9
    log(f"copy {nbytes >> 20} MiB: {t['median'] * 1e3:.1f} us (median of {reps}), {gbs:.0f} GB/s (read + write)")
    return {"bytes_moved": 2 * nbytes, "median_ms": t["median"], "gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS}


def _cpu_problem(p):
    import torch
    return {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in p.items()}


def _oracle_loop(subs, budget_s, max_s, threads):
    """oracle.scan over the sub-problems in order, cycling, until budget_s seconds of it.
    Returns (calls, list of the sub-problem indices run, seconds)."""
    import oracle
    done, secs, k = [], 0.0, 0
    while secs < budget_s and secs < max_s:
        i = k % len(subs)
        t0 = time.perf_counter()
        oracle.scan(subs[i], nthreads=threads)
        secs += time.perf_counter() - t0
        done.append(i)
        k += 1
    return done, secs


def cpu_baseline_prefill(log, wid, budget_s=8.0, max_s=30.0, block=None):
    """The oracle (fp64 C, OpenMP over the (batch, head) walks) on the host cores, on a bounded
    sample of a prefill workload: its heads in blocks (all batches, all tokens), in order and
    cycling from the first block if the whole workload takes less than budget_s; tokens/s is
    scaled by the fraction of the heads processed."""
    import oracle
    from mamba_ssm_scan_amd import inputs
    w = inputs.WORKLOADS[wid]
    threads = oracle.default_threads()
    if wid == 4:
        p = inputs.slice_tokens(inputs.long_sequence(4, device="cuda"), 0, w.seqlen)
    else:
        p = inputs.workload_prefill(wid, device="cuda")
    block = block or max(1, min(w.heads, (threads + w.batch - 1) // w.batch if wid == 4 else 8))
    subs = [_cpu_problem(inputs.select_heads(p, range(h0, min(w.heads, h0 + block))))
            for h0 in range(0, w.heads, block)]
    del p
    done, secs = _oracle_loop(subs, budget_s, max_s, threads)
    heads_done = sum(subs[i]["A"].shape[0] for i in done)
    tok_s = w.batch * w.seqlen * (heads_done / w.heads) / secs
    log(f"cpu oracle {w.name}: {heads_done} head-walks of {w.heads} x {w.batch} batches x {w.seqlen} tokens in "
        f"{secs:.1f} s on {threads} threads -> {tok_s:.0f} tokens/s")
    return {"value": tok_s, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{w.name}: {heads_done} (x {w.batch} batches) head walks of {w.seqlen} tokens "
                      f"(heads in blocks of {block}, cycling), fp64 sequential recurrence, {secs:.1f} s wall; "
                      f"tokens/s = batch*seqlen*heads_done/heads/seconds"}


def cpu_baseline_decode(log, R, steps=1024, budget_s=8.0, max_s=30.0, block=4):
    """The oracle on a bounded sample of the batch-128 decode loop: all 1024 steps of every head
    of `block` sequences at a time (the decode loop is the recurrence over the step axis, from
    h0 with zero carries), cycling over the blocks; steps/s is scaled from the fraction of the
    batch processed (steps / (seconds * batch / sequences done))."""
    import oracle
    from mamba_ssm_scan_amd import inputs
    w = inputs.WORKLOADS[3]
    threads = oracle.default_threads()
    di = inputs.decode_inputs(3, steps, device="cuda", rank=R)
    subs = []
    for b0 in range(0, w.batch, block):
        sl = slice(b0, b0 + block)
        # step-major [steps][b]... -> the prefill layout [b][steps]... (a transpose, no arithmetic)
        sub = {k: di[k][:, sl].transpose(0, 1).contiguous() for k in ("x", "B", "C", "dt", "lam")}
        sub.update(A=di["A"], omega=di["omega"], D=di["D"], h0=di["h0"][sl].contiguous())
        subs.append(_cpu_problem(sub))
        if len(subs) * block >= 32:  # the sample never needs more than 32 sequences
            break
    del di
    done, secs = _oracle_loop(subs, budget_s, max_s, threads)
    seqs = block * len(done)
    steps_s = steps / (secs * w.batch / seqs)
    log(f"cpu oracle decode R={R}: {seqs} sequences x {w.heads} heads x {steps} steps in {secs:.1f} s on "
        f"{threads} threads -> {steps_s:.2f} batch-{w.batch} steps/s")
    return {"value": steps_s, "unit": "steps/s", "cores": threads, "kind": "oracle",
            "sample": f"decode R {R}: {seqs} of {w.batch} sequences (blocks of {block}, all {w.heads} heads, "
                      f"all {steps} steps, cycling over the first 32), fp64 sequential recurrence, {secs:.1f} s "
                      f"wall; steps/s = steps / (seconds * {w.batch} / sequences done)"}


def roofline(bound, achieved, peak, unit, traffic, kernel, per_launch, **extra):
    """The bench line's roofline object for one workload's dominant kernel."""
    return {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit, "frac": achieved / peak,
            "traffic": traffic, "kernel": kernel, **per_launch, **extra}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--quick", action="store_true", help="headline only (for profiling runs)")
    ap.add_argument("--only", default="", help="comma list of prefill1,prefill2,decode1,decode4,long,copy,prologue, "
                                               "prefill1_real/_euler/_real_euler/_raw, prefill2_raw: run just these (profiling runs); "
                                               "copy = a 1 GiB device copy for counter scaling")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from mamba_ssm_scan_amd import binding
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    binding.load()
    log = lambda m: print(m, file=sys.stderr, flush=True)

    if args.only:
        for item in args.only.split(","):
            if item == "prefill1":
                bench_prefill(1, args.steps, args.warmup, log)
            elif item == "prefill2":
                bench_prefill(2, args.steps, args.warmup, log)
            elif item in ("prefill1_n256", "prefill1_n64", "prefill2_n64"):
                bench_prefill(int(item[7]), args.steps, args.warmup, log, dstate=int(item[10:]))
            elif item == "prefill2_r8":
                bench_prefill(2, args.steps, args.warmup, log, rank=8)
            elif item in ("prefill1_g64", "prefill2_g64"):
                bench_prefill(int(item[7]), args.steps, args.warmup, log, groups=64)
            elif item == "prefill2_raw":
                bench_prefill(2, args.steps, args.warmup, log, special="raw")
            elif item.startswith("prefill1_"):
                bench_prefill(1, args.steps, args.warmup, log, special=item[len("prefill1_"):])
            elif item in ("decode1", "decode4"):
                bench_decode(int(item[-1]), 1024, 1, log)
            elif item in ("decode1_fused", "decode4_fused"):
                bench_decode(int(item[6]), 1024, 1, log, fused=True)
            elif item.startswith("decode") and "_b" in item:  # decode1_b256: R 1 at batch 256, 256 steps
                bench_decode(int(item[6]), 256, 1, log, batch=int(item.split("_b")[1]))
            elif item == "long":
                bench_long(log)
            elif item == "copy":
                copy_probe(log)
            elif item in ("backward1", "backward2"):
                bench_backward(int(item[-1]), max(2, args.steps // 4), 1, log)
            elif item in ("mixer1", "mixer2"):
                bench_mixer(int(item[-1]), args.steps, args.warmup, log)
            elif item == "prologue":
                bench_prologue(log, args.steps, args.warmup)
            elif item == "prologue_decode":
                bench_prologue(log, args.steps, args.warmup, wid=3, tokens=(128,))
            else:
                raise SystemExit(f"unknown --only item {item!r}")
        return

    head = bench_prefill(1, args.steps, args.warmup, log)
    out = {
        "metric": METRIC, "value": head["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": head["ms_per_call"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": head["workload"], "batch": 4, "seqlen": 2048, "heads": 64, "groups": 1,
                   "headdim": 64, "dstate": 128, "rank": 1, "chunk": 64, "state_dtype": "f32",
                   "parallelism": "single-gpu"},
        "timing": {k: head[k] for k in ("median_ms", "p10_ms", "p90_ms", "timed_calls")},
        "roofline": roofline("hbm", head["hbm_gbs"], HBM_PEAK_GBS, "GB/s", measured_traffic("prefill1"),
                             "prefill_ws_r1_kernel", {"bytes_per_launch": head["bytes"]},
                             mfma={"achieved": head["mfma_tflops"], "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                   "frac": head["mfma_frac"], "flops_per_launch": head["flops"]}),
    }
    if not args.quick:
        # the batch-128 decode loop (1024 steps, 20 timed loops) at R 1 and R 4: HBM-bound
        kern = {1: "decode_rows_kernel", 4: "decode_mfma32_kernel"}
        out["decode"] = {}
        for R in (1, 4):
            d = bench_decode(R, 1024, 20, log)
            d["roofline"] = roofline("hbm", d["hbm_gbs"], HBM_PEAK_GBS, "GB/s", measured_traffic(f"decode{R}"),
                                     kern[R], {"bytes_per_launch": d["bytes_per_step"]})
            # the same loop on the raw projections, the input prologue in the step kernel
            d["fused_prologue"] = bench_decode(R, 1024, 5, log, fused=True)
            out["decode"][f"r{R}"] = d
        # the same step at batch 64 and 256 (state 128 / 512 MiB against the 256 MB MALL), and a
        # plain 1 GiB copy: the DRAM rate that bounds a stream larger than the MALL
        out["decode_batch_sweep"] = {f"r{R}_b{b}": bench_decode(R, 256, 5, log, batch=b)
                                     for R in (1, 4) for b in (64, 256)}
        out["dram_copy"] = copy_probe(log)
        # the MIMO R 4 prefill: at the ridge of the bf16 MFMA / HBM roofline
        p2 = bench_prefill(2, args.steps, args.warmup, log)
        p2["roofline"] = roofline("mfma", p2["mfma_tflops"], BF16_PEAK_TFLOPS, "TFLOP/s",
                                  measured_traffic("prefill2"), "prefill_ws4_kernel<4> (1 segment)",
                                  {"flops_per_launch": p2["flops"]},
                                  hbm={"achieved": p2["hbm_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                       "frac": p2["hbm_frac"], "bytes_per_launch": p2["bytes"]})
        out["prefill_mimo_r4"] = p2
        lg = bench_long(log)
        lg["roofline"] = roofline("mfma", lg["prefill_mfma_tflops"], BF16_PEAK_TFLOPS, "TFLOP/s",
                                  measured_traffic("long"), "prefill_ws4_kernel<4> (4 segments)",
                                  {"flops_per_launch": lg["prefill_flops"]},
                                  hbm={"achieved": lg["prefill_hbm_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                       "frac": lg["prefill_hbm_frac"], "bytes_per_launch": lg["prefill_bytes"]})
        out["long_prefill_decode"] = lg
        # the pages' special cases on the same workload: omega = 0 (no rotation), lambda = 1 (Euler)
        # dt and lambda from raw projections, mapped inside the prefill kernels (m3_prefill_fused)
        out["prefill_raw_steps"] = {"siso_r1": bench_prefill(1, args.steps, args.warmup, log, special="raw"),
                                    "mimo_r4": bench_prefill(2, args.steps, args.warmup, log, special="raw")}
        out["prefill_special_cases"] = {sp: bench_prefill(1, args.steps, args.warmup, log, special=sp)
                                        for sp in ("real", "euler", "real_euler")}
        # the secondary reading: one B, C per head (64x the B/C bytes)
        out["prefill_groups_eq_heads"] = {f"r{w}": bench_prefill(wid, args.steps, args.warmup, log, groups=64)
                                          for w, wid in ((1, 1), (4, 2))}
        # larger state / rank on the same token shapes (N 256: the chunked kernels in two row passes;
        # R 8: the token-walk kernel)
        out["prefill_larger_sizes"] = {"n256_r1": bench_prefill(1, 5, 1, log, dstate=256),
                                       "n128_r8": bench_prefill(2, 5, 1, log, rank=8)}
        # half the state (N 64) on the same token shapes (the chunked kernels, rows zero-padded)
        out["prefill_smaller_state"] = {f"n64_r{R}": bench_prefill(wid, args.steps, args.warmup, log, dstate=64)
                                        for R, wid in ((1, 1), (4, 2))}
        # the mixer block around the recurrence (d_model 2048), prefill and batch-128 decode
        out["mixer"] = {f"r{R}": bench_mixer(wid, max(3, args.steps // 4), 1, log) for R, wid in ((1, 1), (4, 2))}
        # the backward pass (training) on workloads 1 and 2
        out["backward"] = {f"r{R}": bench_backward(wid, 5, 1, log) for R, wid in ((1, 1), (4, 2))}
        # the input prologue on the R 4 prefill's raw projections and on one decode step's
        out["prologue"] = {"prefill_r4": bench_prologue(log, args.steps, args.warmup),
                           "decode_step_b128": bench_prologue(log, args.steps, args.warmup, wid=3, tokens=(128,))}
    if not args.no_cpu and not args.quick:
        # the oracle on the host cores, on a bounded sample of each workload, next to its GPU figure
        out["cpu_baseline"] = cpu_baseline_prefill(log, 1)
        out["prefill_mimo_r4"]["cpu_baseline"] = cpu_baseline_prefill(log, 2)
        out["long_prefill_decode"]["cpu_baseline"] = cpu_baseline_prefill(log, 4)
        for R in (1, 4):
            out["decode"][f"r{R}"]["cpu_baseline"] = cpu_baseline_decode(log, R)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
