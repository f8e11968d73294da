#!/usr/bin/env python3
"""Benchmark of the causal kernelized linear attention hot path on one MI355X.

One step = one la_forward_causal call over the whole batch of the headline
workload (elu+1 with per-head decay, B=2, H=16, N=32768, d_k=d_v=128, bf16
inputs, fp32 state): the segment-state pass, the segment scan and the chunked
output pass.  Inputs are seeded synthetic tensors already resident in HBM
when timing starts.

Printed last, on stdout: ONE compact JSON line with the headline throughput
(Mtokens/s, tokens = B*N), the roofline of its dominant kernel (algorithmic
bytes per launch over its mean device time, from HIP events the library
records around each of its launches on the launch stream), the whole step's
HBM fraction, the matrix-core rate, the decode step (256x32 head-states,
d=128, plain visiting order) against HBM, the throughput against sequence
length, short figures of the other workloads and the fp64 CPU oracle timed
on the host as a baseline.  Each line's full record goes to stderr as it is
measured (and to --detail FILE as one JSON document).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra]
                       [--no-cpu-baseline] [--only NAME] [--detail FILE]
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 matrix peak, TFLOP/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
KERNEL_SOURCES = ["la_forward.h", "la_output.h", "la_state.h", "la_decode.h", "la_device.h", "la_scan.hip", "la_internal.h",
                  "la_backward.h", "la_rf_grad.hip", "la_api.cpp"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "weight_sequence_mixing_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(workload, kernel):
    """Counter-measured HBM bytes per launch, if taken on the current kernels."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != source_hash():
        return None
    return t.get("per_launch_bytes", {}).get("%s/%s" % (workload, kernel))


class Ctx:
    def __init__(self, steps, warmup):
        import torch
        import weight_sequence_mixing_amd as la
        self.torch, self.la = torch, la
        self.dev = torch.device("cuda:0")
        self.steps, self.warmup = steps, warmup

    def clock_warmup(self, fn, seconds=0.5):
        """Run fn back to back for about `seconds` of wall time, so that the
        GPU's clocks have risen before a short workload is timed."""
        torch = self.torch
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            for _ in range(200):
                fn()
            torch.cuda.synchronize()

    def time_steps(self, fn, steps=None, warmup=None, clock_warmup=0.0):
        torch = self.torch
        steps = self.steps if steps is None else steps
        warmup = self.warmup if warmup is None else warmup
        if clock_warmup > 0:
            self.clock_warmup(fn, clock_warmup)
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    def kernel_times(self, fn, steps=None, launches_per_step=8):
        """Mean device ms per launch, by kernel id, from the library's event brackets."""
        la = self.la
        steps = self.steps if steps is None else steps
        self.torch.cuda.synchronize()
        la.la_profile_begin(steps * launches_per_step)
        for _ in range(steps):
            fn()
        rec = la.la_profile_end(steps * launches_per_step)
        out = {}
        for kid, ms in rec:
            out.setdefault(kid, []).append(ms)
        return {kid: (float(np.mean(v)), len(v) // steps) for kid, v in out.items()}


def roofline(achieved_gbs, traffic):
    return {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved_gbs / HBM_PEAK_GBS, 4), "traffic": traffic}


def causal_bytes(B, H, N, dk, dv, in_bytes, out_bytes):
    """Algorithmic bytes of the causal forward: q, k, v read once, y written once."""
    return B * H * N * ((2 * dk + dv) * in_bytes + dv * out_bytes)


def kernel_alg_bytes(kid, la, B, H, N, dk, dv, F, P, in_bytes=2, out_bytes=2):
    """Algorithmic bytes of one launch.  A map of F > 256 features runs each
    pass twice, over halves of F: the output launches also hand d_v + 1 fp32
    values per row from the first half to the second (the mean of the two
    launches is returned)."""
    ids = la.KERNEL_IDS
    rows = B * H * N
    split = F > 256
    F = F // 2 if split else F
    SZ = F * dv + F
    if kid == ids["fwd_causal"]:
        if split:
            return rows * ((2 * dk + dv) * in_bytes + (dv + 1) * 4 + dv * out_bytes / 2)
        return rows * ((2 * dk + dv) * in_bytes + dv * out_bytes)
    if kid == ids["fwd_local"]:
        return rows * (dk + dv) * in_bytes + P * B * H * SZ * 4
    if kid == ids["fwd_query"]:
        return rows * (dk * in_bytes + dv * out_bytes)
    if kid == ids["scan"]:
        return 2 * P * B * H * SZ * 4
    return None


def bench_causal(ctx, name, B, H, N, dk, dv, lam, phi, gen, steps=None, planned_P=None, warmup=None,
                 clock_warmup=0.0):
    """Time one causal workload; returns a result dict."""
    torch, la = ctx.torch, ctx.la
    q, k, v = gen
    y = torch.empty(B, H, N, dv, dtype=torch.bfloat16, device=ctx.dev)
    F = phi.F(dk)
    ws_n = la.la_workspace_size(B, H, N, dk, dv, phi=phi)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=ctx.dev)
    lam_l = list(map(float, lam))

    def step():
        la.la_forward_causal(q, k, v, y, phi=phi, lambda_h=lam_l, eps=1e-6, workspace=ws)

    ms = ctx.time_steps(step, steps=steps, warmup=warmup, clock_warmup=clock_warmup)
    kt = ctx.kernel_times(step, steps=steps)
    tokens = B * N
    P = planned_P if planned_P is not None else max(1, -(-512 // (B * H)))
    # dominant kernel by total device time per step
    dom = max(kt.items(), key=lambda kv: kv[1][0] * kv[1][1])[0]
    dom_ms = kt[dom][0]
    # segments actually used: infer from the workspace (states of P segments
    # of one half of F for F > 256, beside the rows handed between halves)
    if ws_n:
        Fh = F // 2 if F > 256 else F
        hand = B * H * N * (dv + 1) * 4 if F > 256 else 0
        P = max(1, int(round((ws_n - hand) / (B * H * (Fh * dv + Fh) * 4))))
    alg = kernel_alg_bytes(dom, la, B, H, N, dk, dv, F, P)
    achieved = alg / (dom_ms * 1e-3) / 1e9
    step_bytes = causal_bytes(B, H, N, dk, dv, 2, 2)
    flops_min = 4.0 * F * dv * B * H * N
    C = 64  # tokens per chunk of the bf16 causal output kernels (every score tile formed)
    flops_exec = flops_min + 2.0 * C * (F + dv) * B * H * N
    step_gbs = step_bytes / (ms * 1e-3) / 1e9
    res = {
        "workload": name, "ms_per_step": round(ms, 4), "Mtokens_per_s": round(tokens / (ms * 1e-3) / 1e6, 2),
        "head_tokens_per_s": round(B * H * N / (ms * 1e-3), 1),
        "step_alg_bytes": step_bytes, "step_GBps": round(step_gbs, 1),
        "step_hbm_frac": round(step_gbs / HBM_PEAK_GBS, 4),
        "recurrent_TFLOPs": round(flops_min / (ms * 1e-3) / 1e12, 2),
        "recurrent_mfma_frac": round(flops_min / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
        "executed_TFLOPs": round(flops_exec / (ms * 1e-3) / 1e12, 2),
        "executed_mfma_frac": round(flops_exec / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
        "segments": P,
        "kernels": {la.la_kernel_name(kid): {"mean_ms": round(t, 4), "launches_per_step": n}
                    for kid, (t, n) in kt.items()},
        "dominant_kernel": la.la_kernel_name(dom),
        "roofline": roofline(achieved, load_traffic(name, la.la_kernel_name(dom))),
        "roofline_alg_bytes_per_launch": alg,
        "dominant_mean_ms": round(dom_ms, 4),
    }
    return res


def device_normal(torch, gen, shape, scale, dev):
    return (torch.randn(shape, generator=gen, device=dev, dtype=torch.float32) * scale).to(torch.bfloat16)


def host_to_dev(ctx, inp, name):
    """Seeded host inputs (bf16 bit patterns) on the device."""
    return ctx.torch.from_numpy(inp[name + "_bits"].view(np.int16)).view(ctx.torch.bfloat16).to(ctx.dev)


def workload3_headline(ctx):
    """The headline: the seeded inputs of the per-head-decay workload (the
    same bytes the CPU baseline reads), timed for exactly --steps steps after
    --warmup steps and half a second of clock warm-up."""
    import seeded_inputs as si
    wl = si.workload(3)
    inp = si.make_inputs(wl)
    gen = tuple(host_to_dev(ctx, inp, n) for n in ("q", "k", "v"))
    res = bench_causal(ctx, wl.name, wl.B, wl.H, wl.N, wl.dk, wl.dv, inp["lam"], ctx.la.Phi(), gen,
                       clock_warmup=0.5)
    return wl, inp, res


# Timed steps of the secondary workloads: about 10-20 ms of device time each.
SECONDARY_STEPS = {"w2": 200, "w5": 25}


def workload2(ctx):
    import seeded_inputs as si
    wl = si.workload(2)
    inp = si.make_inputs(wl)
    gen = tuple(host_to_dev(ctx, inp, n) for n in ("q", "k", "v"))
    return bench_causal(ctx, wl.name, wl.B, wl.H, wl.N, wl.dk, wl.dv, inp["lam"], ctx.la.Phi(), gen,
                        steps=SECONDARY_STEPS["w2"], warmup=max(ctx.warmup, 5), clock_warmup=0.2)


def workload5(ctx, m=128):
    import seeded_inputs as si
    torch = ctx.torch
    wl = si.workload(5).with_(m=m)
    g = torch.Generator(device=ctx.dev)
    g.manual_seed(5)
    shape = (wl.B, wl.H, wl.N, wl.dk)
    gen = tuple(device_normal(torch, g, shape, wl.scale, ctx.dev) for _ in range(3))
    omega = torch.from_numpy(si.make_omega(wl.m, wl.dk, wl.index)).to(ctx.dev)
    phi = ctx.la.Phi("trig_rf", omega, wl.qk_scale)
    name = wl.name if m == 128 else wl.name.replace("m128", "m%d" % m)
    return bench_causal(ctx, name, wl.B, wl.H, wl.N, wl.dk, wl.dv, si.make_lambda(wl), phi, gen,
                        steps=SECONDARY_STEPS["w5"], warmup=max(ctx.warmup, 5))


def length_scaling(ctx, Ns=(1024, 2048, 4096, 8192, 16384, 32768, 65536, 131072)):
    """Throughput against sequence length at the headline's heads (B=2, H=16,
    d=128, per-head decay): one causal forward per step, about 10 ms of
    device time per point.  Device bytes = q, k, v, y and the workspace."""
    import seeded_inputs as si
    torch, la = ctx.torch, ctx.la
    wl = si.workload(3)
    lam = si.make_lambda(wl)
    g = torch.Generator(device=ctx.dev)
    out = []
    for N in Ns:
        g.manual_seed(N)
        shape = (wl.B, wl.H, N, wl.dk)
        gen = tuple(device_normal(torch, g, shape, wl.scale, ctx.dev) for _ in range(3))
        steps = max(5, int(10.0 / max(1e-3, 0.45 * N / 32768)))
        r = bench_causal(ctx, "scaling_N%d" % N, wl.B, wl.H, N, wl.dk, wl.dv, lam, la.Phi(), gen, steps=steps,
                         warmup=3)
        ws = la.la_workspace_size(wl.B, wl.H, N, wl.dk, wl.dv)
        out.append({"N": N, "ms": r["ms_per_step"], "Mtokens_per_s": r["Mtokens_per_s"],
                    "step_hbm_frac": r["step_hbm_frac"], "out_pass_frac": r["roofline"]["frac"],
                    "device_MB": round((r["step_alg_bytes"] + ws) / 1e6, 1)})
        log(json.dumps(out[-1]))
        del gen
        torch.cuda.empty_cache()
    return out


def feature_map_variant(ctx, base, phi, m=0, steps=20):
    """A feature-map variant at the shape of workload `base` (2 or 5): the same
    synthetic inputs and decay, another map (ReLU, a random-feature prefactor,
    another m)."""
    import seeded_inputs as si
    torch = ctx.torch
    wl = si.workload(base).with_(phi=phi, m=m)
    g = torch.Generator(device=ctx.dev)
    g.manual_seed(base)
    shape = (wl.B, wl.H, wl.N, wl.dk)
    gen = tuple(device_normal(torch, g, shape, wl.scale, ctx.dev) for _ in range(3))
    if wl.random_features:
        omega = torch.from_numpy(si.make_omega(wl.m, wl.dk, wl.index)).to(ctx.dev)
        phi_c = ctx.la.Phi(phi, omega, wl.qk_scale)
    else:
        phi_c = ctx.la.Phi(phi)
    name = "%s_causal_B%d_H%d_N%d_d%d_%s" % (phi.replace("_", "") + ("_m%d" % m if m else ""), wl.B, wl.H,
                                             wl.N, wl.dk, wl.dtype)
    res = bench_causal(ctx, name, wl.B, wl.H, wl.N, wl.dk, wl.dv, si.make_lambda(wl), phi_c, gen,
                       steps=steps, warmup=max(ctx.warmup, 5), planned_P=max(1, -(-512 // (wl.B * wl.H))))
    return res


# Feature-map variants measured beside the main workloads: (key, base shape, map, m, steps)
VARIANTS = (("relu_w2", 2, "relu", 0, 200), ("rf_softmax_w5", 5, "trig_rf_softmax", 128, 25),
            ("rf_m64_w5", 5, "trig_rf", 64, 25), ("rf_m32_w5", 5, "trig_rf", 32, 25))


def bench_call(ctx, name, step, tokens, kernel_bytes, steps, warmup, launches_per_step=8):
    """Time `step` (one call over the whole batch) and report its dominant
    kernel against HBM with the algorithmic bytes kernel_bytes[kernel id]."""
    la = ctx.la
    ms = ctx.time_steps(step, steps=steps, warmup=warmup)
    kt = ctx.kernel_times(step, steps=steps, launches_per_step=launches_per_step)
    dom = max(kt.items(), key=lambda kv: kv[1][0] * kv[1][1])[0]
    dom_ms = kt[dom][0]
    alg = kernel_bytes.get(dom)
    achieved = alg / (dom_ms * 1e-3) / 1e9 if alg else 0.0
    return {
        "workload": name, "ms_per_step": round(ms, 4), "Mtokens_per_s": round(tokens / (ms * 1e-3) / 1e6, 2),
        "kernels": {la.la_kernel_name(k): {"mean_ms": round(t, 4), "launches_per_step": n} for k, (t, n) in kt.items()},
        "dominant_kernel": la.la_kernel_name(dom),
        "roofline": roofline(achieved, load_traffic(name, la.la_kernel_name(dom))),
        "roofline_alg_bytes_per_launch": alg,
        "dominant_mean_ms": round(dom_ms, 4),
    }


def _w2_inputs(ctx, B, H, N, seed=2):
    import seeded_inputs as si
    wl = si.workload(2)
    g = ctx.torch.Generator(device=ctx.dev)
    g.manual_seed(seed)
    return wl, tuple(device_normal(ctx.torch, g, (B, H, N, wl.dk), wl.scale, ctx.dev) for _ in range(3))


def masked_w2(ctx, steps=200):
    """Causal forward at the headline shape over a padded batch: batch b keeps
    its first L_b keys (L_0 = N, the others uniform), the rest are masked."""
    import seeded_inputs as si
    torch, la = ctx.torch, ctx.la
    wl, (q, k, v) = _w2_inputs(ctx, 4, 8, 4096)
    B, H, N, d = wl.B, wl.H, wl.N, wl.dk
    mask = torch.from_numpy(si.make_key_padding_mask(B, N, "right", seed=2)).to(ctx.dev)
    y = torch.empty_like(q)
    ws = torch.empty(max(la.la_workspace_size(B, H, N, d, d), 1), dtype=torch.uint8, device=ctx.dev)
    P = max(1, -(-512 // (B * H)))
    ids = la.KERNEL_IDS
    SZ = d * d + d
    kb = {ids["fwd_causal"]: B * H * N * 4 * d * 2 + B * N,
          ids["fwd_local"]: B * H * N * 2 * d * 2 + B * N + P * B * H * SZ * 4,
          ids["scan"]: 2 * P * B * H * SZ * 4}

    def step():
        la.la_forward_causal_masked(q, k, v, y, mask, eps=wl.eps, workspace=ws)

    name = "elu1_causal_masked_right_B%d_H%d_N%d_d%d_bf16" % (B, H, N, d)
    return bench_call(ctx, name, step, B * N, kb, steps, max(ctx.warmup, 5))


def varlen_w2(ctx, steps=200):
    """Packed causal forward: 32 sequences of mixed lengths (log-uniform in
    [1, 4096], one of 4096) back to back in one row per head, 8 heads, d = 64."""
    import seeded_inputs as si
    torch, la = ctx.torch, ctx.la
    H, d = 8, 64
    L = si.make_varlen_lengths(32, 4096, seed=2)
    cu_np = si.cu_seqlens(L)
    T = int(cu_np[-1])
    wl, (q, k, v) = _w2_inputs(ctx, 1, H, T)
    q, k, v = q[0], k[0], v[0]
    cu = torch.from_numpy(cu_np).to(ctx.dev)
    y = torch.empty_like(q)
    mx = int(L.max())
    ws_n = la.la_workspace_size_varlen(len(L), H, T, mx, d, d)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=ctx.dev)
    SZ = d * d + d
    P = max(1, int(round(ws_n / (len(L) * H * SZ * 4)))) if ws_n else 1
    ids = la.KERNEL_IDS
    kb = {ids["fwd_causal"]: H * T * 4 * d * 2,
          ids["fwd_local"]: H * T * 2 * d * 2 + P * len(L) * H * SZ * 4,
          ids["scan"]: 2 * P * len(L) * H * SZ * 4}

    def step():
        la.la_forward_causal_varlen(q, k, v, y, cu, mx, eps=wl.eps, workspace=ws)

    name = "elu1_causal_varlen_S%d_T%d_H%d_d%d_bf16" % (len(L), T, H, d)
    res = bench_call(ctx, name, step, T, kb, steps, max(ctx.warmup, 5))
    res["sequences"] = int(len(L))
    res["max_seqlen"] = mx
    res["segments"] = P
    return res


def cross_w2(ctx, steps=200):
    """Cross attention at the headline batch: 1024 queries against 4096 keys
    and values per (batch, head), B = 4, H = 8, d = 64, keys right-padded."""
    import seeded_inputs as si
    torch, la = ctx.torch, ctx.la
    B, H, Nq, Nk, d = 4, 8, 1024, 4096, 64
    wl, (k, v, _) = _w2_inputs(ctx, B, H, Nk)
    _, (q, _, _) = _w2_inputs(ctx, B, H, Nq, seed=12)
    mask = torch.from_numpy(si.make_key_padding_mask(B, Nk, "right", seed=2)).to(ctx.dev)
    y = torch.empty_like(q)
    ws_n = la.la_workspace_size_cross(B, H, Nq, Nk, d, d)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=ctx.dev)
    SZ = d * d + d
    P = max(1, int(round(ws_n / (B * H * SZ * 4)))) if ws_n else 1
    ids = la.KERNEL_IDS
    kb = {ids["fwd_local"]: B * H * Nk * 2 * d * 2 + B * Nk + P * B * H * SZ * 4,
          ids["fwd_query"]: B * H * Nq * 2 * d * 2,
          ids["scan"]: (P + 1) * B * H * SZ * 4}

    def step():
        la.la_forward_cross(q, k, v, y, mask, eps=wl.eps, workspace=ws)

    name = "elu1_cross_masked_B%d_H%d_Nq%d_Nk%d_d%d_bf16" % (B, H, Nq, Nk, d)
    res = bench_call(ctx, name, step, B * Nq, kb, steps, max(ctx.warmup, 5))
    res["key_Mtokens_per_s"] = round(B * Nk / (res["ms_per_step"] * 1e-3) / 1e6, 2)
    res["segments"] = P
    return res


def cross_backward_w2(ctx, steps=100):
    """Backward of the cross-attention line (1024 queries against 4096
    right-padded keys per (batch, head), B = 4, H = 8, d = 64 bf16): one
    la_backward_cross call -- the keys' state sums and their reduction, the
    query sweep (dq and the adjoint's segment sums), the adjoint reduction,
    the key sweep (dk, dv)."""
    import seeded_inputs as si
    torch, la = ctx.torch, ctx.la
    B, H, Nq, Nk, d = 4, 8, 1024, 4096, 64
    wl, (k, v, _) = _w2_inputs(ctx, B, H, Nk)
    _, (q, _, _) = _w2_inputs(ctx, B, H, Nq, seed=12)
    mask = torch.from_numpy(si.make_key_padding_mask(B, Nk, "right", seed=2)).to(ctx.dev)
    g = torch.Generator(device=ctx.dev)
    g.manual_seed(23)
    dy = device_normal(torch, g, (B, H, Nq, d), 0.5, ctx.dev)
    y = torch.empty_like(q)
    la.la_forward_cross(q, k, v, y, mask, eps=wl.eps)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(la.la_workspace_size_backward_cross(B, H, Nq, Nk, d, d), dtype=torch.uint8, device=ctx.dev)
    SZ = d * d + d
    P = max(1, -(-512 // (B * H)))  # segments of every pass at this shape (>= P chunks each way)
    ids = la.KERNEL_IDS
    kb = {ids["fwd_local"]: B * H * Nk * 2 * d * 2 + B * Nk + P * B * H * SZ * 4,
          ids["bwd_ncq"]: B * H * Nq * 4 * d * 2 + 2 * P * B * H * SZ * 4,
          ids["bwd_nckv"]: B * H * Nk * 4 * d * 2 + B * Nk + P * B * H * SZ * 4,
          ids["scan"]: (P + 1) * B * H * SZ * 4}

    def step():
        la.la_backward_cross(q, k, v, y, dy, dq, dk, dv, mask, eps=wl.eps, workspace=ws)

    name = "elu1_cross_backward_masked_B%d_H%d_Nq%d_Nk%d_d%d_bf16" % (B, H, Nq, Nk, d)
    res = bench_call(ctx, name, step, B * Nq, kb, steps, max(ctx.warmup, 5))
    res["key_Mtokens_per_s"] = round(B * Nk / (res["ms_per_step"] * 1e-3) / 1e6, 2)
    res["segments"] = P
    return res


def backward_w2(ctx, steps=100, with_dlam=False):
    """Backward of the headline forward (B=4 H=8 N=4096 d=64 bf16, lambda = 1):
    one la_backward_causal call -- forward segment states and scan, the dq
    sweep, the adjoint segment sums and reverse scan, the dk/dv sweep (and,
    with_dlam, the lambda gradient: dS/dlambda carried in the dq sweep and
    the reduction over segments and batch)."""
    torch, la = ctx.torch, ctx.la
    B, H, N, d = 4, 8, 4096, 64
    wl, (q, k, v) = _w2_inputs(ctx, B, H, N)
    g = torch.Generator(device=ctx.dev)
    g.manual_seed(22)
    dy = device_normal(torch, g, (B, H, N, d), 0.5, ctx.dev)
    y = torch.empty_like(q)
    la.la_forward_causal(q, k, v, y, eps=wl.eps)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_n = la.la_workspace_size_backward(B, H, N, d, d)
    ws = torch.empty(ws_n, dtype=torch.uint8, device=ctx.dev)
    SZ = d * d + d
    P = max(1, -(-512 // (B * H)))
    rows = B * H * N
    ids = la.KERNEL_IDS
    kb = {ids["bwd_q"]: rows * (5 * d * 2 + d * 2 + 8) + P * B * H * SZ * 4,
          ids["bwd_rlocal"]: rows * (2 * d * 2 + 8) + P * B * H * SZ * 4,
          ids["bwd_kv"]: rows * (4 * d * 2 + 8 + 2 * d * 2) + P * B * H * SZ * 4,
          ids["fwd_local"]: rows * 2 * d * 2 + P * B * H * SZ * 4,
          ids["scan"]: 2 * P * B * H * SZ * 4}

    dlam = torch.empty(H, device=ctx.dev) if with_dlam else None

    def step():
        la.la_backward_causal(q, k, v, y, dy, dq, dk, dv, eps=wl.eps, dlambda=dlam, workspace=ws)

    name = "elu1_backward%s_B%d_H%d_N%d_d%d_bf16" % ("_dlam" if with_dlam else "", B, H, N, d)
    res = bench_call(ctx, name, step, B * N, kb, steps, max(ctx.warmup, 5), launches_per_step=8)
    res["segments"] = P
    return res


def rf_backward_w5(ctx, steps=5):
    """Backward of workload 5 (B=1 H=16 N=65536, m=128 random features, d=64
    bf16, lambda = 1): one la_backward_causal call -- phi(q) and phi(k), the
    backward sweeps on them at F = 256 with the identity map (d phi in bf16),
    and the vector-Jacobian products through omega to dq and dk."""
    import seeded_inputs as si
    torch, la = ctx.torch, ctx.la
    wl = si.workload(5)
    B, H, N, d, m = wl.B, wl.H, wl.N, wl.dk, wl.m
    F = 2 * m
    g = torch.Generator(device=ctx.dev)
    g.manual_seed(5)
    q, k, v = (device_normal(torch, g, (B, H, N, d), wl.scale, ctx.dev) for _ in range(3))
    omega = torch.from_numpy(si.make_omega(m, d, wl.index)).to(ctx.dev)
    phi = la.Phi("trig_rf", omega, wl.qk_scale)
    g.manual_seed(25)
    dy = device_normal(torch, g, (B, H, N, d), 0.5, ctx.dev)
    y = torch.empty_like(q)
    la.la_forward_causal(q, k, v, y, phi=phi, eps=wl.eps)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(la.la_workspace_size_backward(B, H, N, d, d, phi=phi), dtype=torch.uint8, device=ctx.dev)
    SZ = F * d + F
    P = max(1, -(-512 // (B * H)))
    rows = B * H * N
    ids = la.KERNEL_IDS
    # per launch: the feature pass and the gradient pass each cover q or k
    kb = {ids["rf_features"]: rows * (d * 2 + F * 2),
          ids["rf_vjp"]: rows * (d * 2 + F * 2 + d * 2),
          ids["bwd_q"]: rows * (2 * F * 2 + 3 * d * 2 + F * 2 + 8) + P * B * H * SZ * 4,
          ids["bwd_rlocal"]: rows * (F * 2 + d * 2 + 8) + P * B * H * SZ * 4,
          ids["bwd_kv"]: rows * (2 * F * 2 + 2 * d * 2 + 8 + F * 2 + d * 2) + P * B * H * SZ * 4,
          ids["fwd_local"]: rows * (F * 2 + d * 2) + P * B * H * SZ * 4,
          ids["scan"]: 2 * P * B * H * SZ * 4}

    def step():
        la.la_backward_causal(q, k, v, y, dy, dq, dk, dv, phi=phi, eps=wl.eps, workspace=ws)

    name = "trigrf_m%d_backward_B%d_H%d_N%d_d%d_bf16" % (m, B, H, N, d)
    res = bench_call(ctx, name, step, B * N, kb, steps, max(ctx.warmup, 3), launches_per_step=12)
    res["segments"] = P
    return res


def noncausal(ctx, B, H, N, d, steps=100):
    """Non-causal forward (every query against the whole sequence, no decay):
    the state sums over segments of the sequence, their reduction, the query
    pass.  Bytes: the state sums read k, v and write P partial states; the
    query pass reads q and the state and writes y."""
    torch, la = ctx.torch, ctx.la
    g = torch.Generator(device=ctx.dev)
    g.manual_seed(31)
    q, k, v = (device_normal(torch, g, (B, H, N, d), 0.5, ctx.dev) for _ in range(3))
    y = torch.empty_like(q)
    ws_n = la.la_workspace_size(B, H, N, d, d, causal=False)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=ctx.dev)
    SZ = d * d + d
    P = max(1, int(round(ws_n / (B * H * SZ * 4)))) if ws_n else 1
    ids = la.KERNEL_IDS
    kb = {ids["fwd_local"]: B * H * N * 2 * d * 2 + P * B * H * SZ * 4,
          ids["fwd_query"]: B * H * N * 2 * d * 2 + B * H * SZ * 4,
          ids["scan"]: (P + 1) * B * H * SZ * 4}

    def step():
        la.la_forward_noncausal(q, k, v, y, eps=1e-6, workspace=ws)

    name = "elu1_noncausal_B%d_H%d_N%d_d%d_bf16" % (B, H, N, d)
    res = bench_call(ctx, name, step, B * N, kb, steps, max(ctx.warmup, 5))
    res["segments"] = P
    return res


# Mask / cross / packed / non-causal / backward lines measured beside the
# main workloads
SHAPE_VARIANTS = (("masked_w2", masked_w2), ("varlen_w2", varlen_w2), ("cross_w2", cross_w2),
                  ("noncausal_w2", lambda c: noncausal(c, 4, 8, 4096, 64)),
                  ("noncausal_w3", lambda c: noncausal(c, 2, 16, 32768, 128, steps=50)),
                  ("backward_w2", backward_w2), ("backward_dlam_w2", lambda c: backward_w2(c, with_dlam=True)),
                  ("cross_backward_w2", cross_backward_w2), ("rf_backward_w5", rf_backward_w5))


def workload4_decode(ctx, steps=1024):
    """Decode: prefix of 512 tokens through the causal forward, then `steps`
    single-token steps timed back to back (head-states visited in plain
    ascending order on every step).  Bytes per step: the state read and
    written once, plus q, k, v, y."""
    import seeded_inputs as si
    torch, la = ctx.torch, ctx.la
    wl = si.workload(4)
    B, H, d = wl.B, wl.H, wl.dk
    F = wl.F
    g = torch.Generator(device=ctx.dev)
    g.manual_seed(4)
    lam = list(map(float, si.make_lambda(wl)))
    pq, pk, pv = (device_normal(torch, g, (B, H, wl.N, d), wl.scale, ctx.dev) for _ in range(3))
    S = torch.empty(B, H, F, d, dtype=torch.float32, device=ctx.dev)
    z = torch.empty(B, H, F, dtype=torch.float32, device=ctx.dev)
    yp = torch.empty_like(pq)
    la.la_forward_causal(pq, pk, pv, yp, lambda_h=lam, eps=wl.eps, S_out=S, z_out=z)
    del pq, pk, pv, yp
    sq, sk, sv = (device_normal(torch, g, (steps, B, H, 1, d), wl.scale, ctx.dev) for _ in range(3))
    y = torch.empty(B, H, 1, d, dtype=torch.bfloat16, device=ctx.dev)
    counter = [0]

    def step():
        i = counter[0] % steps
        counter[0] += 1
        la.la_decode_step(sq[i], sk[i], sv[i], y, S, z, lambda_h=lam, eps=wl.eps)

    ms = ctx.time_steps(step, steps=steps, warmup=8)
    kt = ctx.kernel_times(step, steps=min(steps, 256), launches_per_step=1)
    dec_ms = kt[la.KERNEL_IDS["decode"]][0]
    state_bytes = 2 * B * H * (F * d + F) * 4
    io_bytes = B * H * (3 * d * 2 + d * 2)
    per_step = state_bytes + io_bytes
    achieved = per_step / (dec_ms * 1e-3) / 1e9
    return {
        "workload": wl.name, "ms_per_step": round(ms, 4), "steps_timed": steps, "order": "plain",
        "state_GBps": round(per_step / (ms * 1e-3) / 1e9, 1),
        "hbm_frac": round(per_step / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "Mtokens_per_s": round(B / (ms * 1e-3) / 1e6, 4),
        "head_tokens_per_s": round(B * H / (ms * 1e-3), 1),
        "alg_bytes_per_step": per_step,
        "kernels": {la.la_kernel_name(k): {"mean_ms": round(t, 4), "launches_per_step": n} for k, (t, n) in kt.items()},
        "dominant_kernel": la.la_kernel_name(la.KERNEL_IDS["decode"]),
        "roofline": roofline(achieved, load_traffic(wl.name, la.la_kernel_name(la.KERNEL_IDS["decode"]))),
        "dominant_mean_ms": round(dec_ms, 4),
    }


def workload4_multi(ctx, k_tok=4, calls=256):
    """Fused multi-token decode at the decode workload's shape: the same
    512-token prefix, then `calls` calls of la_decode_step with k_tok new tokens
    per head-state (the state read once, kept on chip across the tokens, written
    once).  Bytes per call: the state read and written once, plus k_tok tokens of
    q, k, v, y."""
    import seeded_inputs as si
    torch, la = ctx.torch, ctx.la
    wl = si.workload(4)
    B, H, d = wl.B, wl.H, wl.dk
    F = wl.F
    g = torch.Generator(device=ctx.dev)
    g.manual_seed(4)
    lam = list(map(float, si.make_lambda(wl)))
    pq, pk, pv = (device_normal(torch, g, (B, H, wl.N, d), wl.scale, ctx.dev) for _ in range(3))
    S = torch.empty(B, H, F, d, dtype=torch.float32, device=ctx.dev)
    z = torch.empty(B, H, F, dtype=torch.float32, device=ctx.dev)
    yp = torch.empty_like(pq)
    la.la_forward_causal(pq, pk, pv, yp, lambda_h=lam, eps=wl.eps, S_out=S, z_out=z)
    del pq, pk, pv, yp
    nbuf = 16
    sq, sk, sv = (device_normal(torch, g, (nbuf, B, H, k_tok, d), wl.scale, ctx.dev) for _ in range(3))
    y = torch.empty(B, H, k_tok, d, dtype=torch.bfloat16, device=ctx.dev)
    counter = [0]

    def call():
        i = counter[0] % nbuf
        counter[0] += 1
        la.la_decode_step(sq[i], sk[i], sv[i], y, S, z, lambda_h=lam, eps=wl.eps)

    ms = ctx.time_steps(call, steps=calls, warmup=8)
    kt = ctx.kernel_times(call, steps=min(calls, 128), launches_per_step=4)
    dom = max(kt.items(), key=lambda kv: kv[1][0] * kv[1][1])[0]
    dom_ms = kt[dom][0]
    state_bytes = 2 * B * H * (F * d + F) * 4
    io_bytes = B * H * k_tok * (3 * d * 2 + d * 2)
    per_call = state_bytes + io_bytes
    name = "elu1_decode_multi%d_B%d_H%d_d%d_prefix%d_bf16" % (k_tok, B, H, d, wl.N)
    return {
        "workload": name, "ms_per_call": round(ms, 4), "tokens_per_call": k_tok, "calls_timed": calls,
        "state_GBps": round(per_call / (ms * 1e-3) / 1e9, 1),
        "Mtokens_per_s": round(B * k_tok / (ms * 1e-3) / 1e6, 4),
        "head_tokens_per_s": round(B * H * k_tok / (ms * 1e-3), 1),
        "alg_bytes_per_call": per_call,
        "kernels": {la.la_kernel_name(k): {"mean_ms": round(t, 4), "launches_per_step": n} for k, (t, n) in kt.items()},
        "dominant_kernel": la.la_kernel_name(dom),
        "roofline": roofline(per_call / (dom_ms * 1e-3) / 1e9, load_traffic(name, la.la_kernel_name(dom))),
        "dominant_mean_ms": round(dom_ms, 4),
    }


def state_copy(ctx, B=256, H=32, F=128, D=128, steps=50):
    """Reference stream: the library's state copy (la_forward_causal with N=0
    and S_in -> S_out) over a decode-sized fp32 state; bytes = read + write."""
    torch, la = ctx.torch, ctx.la
    S_in = torch.randn(B, H, F, D, device=ctx.dev)
    z_in = torch.rand(B, H, F, device=ctx.dev)
    S_out, z_out = torch.empty_like(S_in), torch.empty_like(z_in)
    q = torch.empty(B, H, 0, D, dtype=torch.bfloat16, device=ctx.dev)
    y = torch.empty_like(q)

    def step():
        la.la_forward_causal(q, q, q, y, S_in=S_in, z_in=z_in, S_out=S_out, z_out=z_out)

    ms = ctx.time_steps(step, steps=steps, warmup=5)
    kt = ctx.kernel_times(step, steps=steps, launches_per_step=2)
    assert torch.equal(S_out, S_in) and torch.equal(z_out, z_in)
    cid = la.KERNEL_IDS["copy"]
    dev_ms = kt[cid][0] * kt[cid][1]
    nbytes = 2 * 4 * (B * H * F * D + B * H * F)
    return {"workload": "state copy fp32 %dx%dx%dx%d" % (B, H, F, D), "bytes_per_step": nbytes,
            "ms_per_step": round(ms, 4), "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "device_GBps": round(nbytes / (dev_ms * 1e-3) / 1e9, 1),
            "hbm_frac": round(nbytes / (dev_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


# ---- HBM traffic from rocprofv3 counter runs -------------------------------
# rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) runs of `bench.py --only TAG`
# write <dir>/<counter>_<tag>/**/*_counter_collection.csv.  The counters are
# scaled by what they read for the library's state copy, whose bytes are known.
COUNTER_TAGS = {"copy": None, "w2": 2, "w3": 3, "w4": 4, "w5": 5,
                "backward_w2": "elu1_backward_B4_H8_N4096_d64_bf16",
                "rf_backward_w5": "trigrf_m128_backward_B1_H16_N65536_d64_bf16",
                "w5m256": "trigrf_m256_causal_B1_H16_N65536_d64_bf16"}


def _kernel_label(mangled):
    if "la_copy_kernel" in mangled:
        return "la_copy_kernel"
    if "la_bwd_q_kernel" in mangled:
        # the last bool template argument: the non-causal variant
        if re.search(r"Lb1EE+vNS_7BwdArgsE", mangled) or mangled.split(">(")[0].rstrip().endswith("true"):
            return "la_bwd_q_kernel (non-causal)"
        return "la_bwd_q_kernel"
    if "la_bwd_kv_kernel" in mangled:
        # the mode is the last int template argument
        if "EEEvNS_7BwdArgsE" in mangled:
            mode = mangled.split("EEEvNS_7BwdArgsE")[0].rsplit("ELi", 1)[-1]
        else:
            ints = [x.strip() for x in mangled.split(">(")[0].split(",") if x.strip().lstrip("-").isdigit()]
            mode = ints[-1] if ints else ""
        return {"1": "la_bwd_kv_kernel (adjoint segment)", "2": "la_bwd_kv_kernel (dk dv)",
                "4": "la_bwd_kv_kernel (non-causal dk dv)"}.get(mode, "la_bwd_kv_kernel")
    if "la_decode_kernel" in mangled:
        return "la_decode_kernel"
    # fp32 (vector ALU) and bf16 (matrix-core) instances
    if "la_rf_features" in mangled:
        return "la_rf_features_kernel"
    if "la_rf_vjp" in mangled:
        return "la_rf_vjp_kernel"
    if "la_scan_kernel" in mangled:
        return "la_scan_kernel"
    if "la_out_kernel" in mangled:
        return "causal output pass"
    if "la_state_kernel" in mangled:
        return "segment state pass"
    if "la_fwd_kernel" in mangled:
        # the mode is the last int template argument (a bool, the output type,
        # follows it), mangled (...ELi1ELb0EEEvNS_7FwdArgsE) or demangled
        # (..., 4, 1, false>(la::FwdArgs))
        if "EEEvNS_7FwdArgsE" in mangled:
            mode = mangled.split("EEEvNS_7FwdArgsE")[0].rsplit("ELi", 1)[-1].split("E")[0]
        else:
            args = [x.strip() for x in mangled.split(">(")[0].split(",")]
            ints = [x for x in args if x.lstrip("-").isdigit()]
            mode = ints[-1] if ints else ""
        return {"0": "segment state pass", "1": "causal output pass",
                "2": "non-causal output pass"}.get(mode, "la_fwd_kernel")
    return None


def _counter_means(root, counter, tag):
    import csv
    import glob
    vals = {}
    for path in glob.glob(os.path.join(root, "%s_%s" % (counter.lower(), tag), "**", "*_counter_collection.csv"),
                          recursive=True):
        with open(path) as fh:
            for row in csv.DictReader(fh):
                if row["Counter_Name"] != counter:
                    continue
                label = _kernel_label(row["Kernel_Name"])
                if label:
                    vals.setdefault(label, []).append(float(row["Counter_Value"]))
    return vals


def traffic_from(root):
    """Write profiles/traffic_counters.json from counter runs under `root`."""
    import seeded_inputs as si
    fetch = {t: _counter_means(root, "FETCH_SIZE", t) for t in COUNTER_TAGS}
    write = {t: _counter_means(root, "WRITE_SIZE", t) for t in COUNTER_TAGS}
    # calibration: the largest copy dispatch moves the fp32 state 256x32x128x128
    state_bytes = 4 * 256 * 32 * 128 * 128
    f_copy = max(fetch["copy"]["la_copy_kernel"]) * 1024.0
    w_copy = max(write["copy"]["la_copy_kernel"]) * 1024.0
    cal = {"read_factor": state_bytes / f_copy, "write_factor": state_bytes / w_copy,
           "copy_fetch_KiB": f_copy / 1024, "copy_write_KiB": w_copy / 1024, "copy_bytes_each_way": state_bytes}
    out = {"source_hash": source_hash(), "calibration": cal, "per_launch_bytes": {}, "raw_KiB": {}}
    for tag, idx in COUNTER_TAGS.items():
        if idx is None:
            continue
        name = idx if isinstance(idx, str) else si.workload(idx).name
        for label in sorted(set(fetch[tag]) & set(write[tag])):
            fr = float(np.mean(fetch[tag][label]))
            wr = float(np.mean(write[tag][label]))
            key = "%s/%s" % (name, label)
            out["per_launch_bytes"][key] = int(fr * 1024 * cal["read_factor"] + wr * 1024 * cal["write_factor"])
            out["raw_KiB"][key] = {"FETCH_SIZE": fr, "WRITE_SIZE": wr}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(out, fh, indent=1, sort_keys=True)
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, inp, min_seconds=10.0, max_passes=400):
    """The fp64 oracle, as it stands, on the host cores granted to this
    process: whole passes over the headline workload, repeated until at least
    `min_seconds` of CPU work."""
    import oracle
    threads = oracle.default_threads()
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count() or 1
    passes, t0 = 0, time.perf_counter()
    while True:
        oracle.causal(inp["q"], inp["k"], inp["v"], inp["lam"], wl.eps, threads=threads)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or passes >= max_passes:
            break
    return {"value": round(passes * wl.B * wl.N / dt / 1e6, 5), "unit": "Mtokens/s", "cores": threads,
            "kind": "oracle", "cpu": cpu_model(), "affinity_cores": affinity,
            "sample": "%d whole passes over the workload (B=%d H=%d N=%d d=%d, fp64 per-token recurrence) "
                      "in %.2f s" % (passes, wl.B, wl.H, wl.N, wl.dk, dt)}


def compact(r):
    """Short figures of a secondary line for the printed JSON line."""
    out = {"ms": r.get("ms_per_step", r.get("ms_per_call"))}
    if "Mtokens_per_s" in r:
        out["Mtok_s"] = r["Mtokens_per_s"]
    if "roofline" in r:
        out["frac"] = r["roofline"]["frac"]
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-extra", action="store_true", help="skip the secondary workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--detail", metavar="FILE", help="write every line's full record to FILE (JSON)")
    ap.add_argument("--only", choices=["w2", "w3", "w4", "w4multi", "w5", "w5m256", "copy", "scaling"] +
                    [v[0] for v in VARIANTS] +
                    [v[0] for v in SHAPE_VARIANTS],
                    help="run one workload (profiling)")
    ap.add_argument("--traffic-from", metavar="DIR",
                    help="host only: turn rocprofv3 FETCH_SIZE/WRITE_SIZE runs under DIR into "
                         "profiles/traffic_counters.json and exit")
    args = ap.parse_args()
    if args.traffic_from:
        print(json.dumps(traffic_from(args.traffic_from), indent=1))
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        log("bench.py measures one GPU: the library has no multi-GPU path "
            "(the heads are independent, so each GPU would run its own share).")
        sys.exit(2)

    ctx = Ctx(args.steps, args.warmup)
    if args.only:
        fns = {"w2": workload2, "w3": lambda c: workload3_headline(c)[2], "w4": workload4_decode, "w5": workload5,
               "w5m256": lambda c: workload5(c, m=256),
               "copy": state_copy, "w4multi": workload4_multi, "scaling": length_scaling}
        for key, base, phi, m, steps in VARIANTS:
            fns[key] = (lambda c, b=base, p=phi, mm=m, st=steps: feature_map_variant(c, b, p, mm, st))
        fns.update(dict(SHAPE_VARIANTS))
        fn = fns[args.only]
        log("running", args.only)
        print(json.dumps({"only": args.only, "result": fn(ctx)}), flush=True)
        return

    # the headline first (after its own clock warm-up), then the decode line
    log("workload 3 (headline) ...")
    wl, inp, res = workload3_headline(ctx)
    log(json.dumps(res))
    ctx.torch.cuda.empty_cache()
    log("decode_w4 ...")
    dec = workload4_decode(ctx)
    log(json.dumps(dec))
    ctx.torch.cuda.empty_cache()
    log("state copy ...")
    cp = state_copy(ctx)
    log(json.dumps(cp))
    detail = {"headline": res, "decode_w4": dec, "state_copy": cp}
    scaling, extra = None, {}
    if not args.no_extra:
        log("length scaling ...")
        scaling = length_scaling(ctx)
        detail["length_scaling"] = scaling
        for key, fn in (("w2", workload2), ("decode_multi4_w4", workload4_multi),
                        ("decode_multi16_w4", lambda c: workload4_multi(c, 16, 64)), ("w5", workload5),
                        ("rf_m256_w5", lambda c: workload5(c, m=256))):
            log(key, "...")
            extra[key] = fn(ctx)
            log(json.dumps(extra[key]))
            ctx.torch.cuda.empty_cache()
        for key, base, phi, m, steps in VARIANTS:
            log(key, "...")
            extra[key] = feature_map_variant(ctx, base, phi, m, steps)
            log(json.dumps(extra[key]))
            ctx.torch.cuda.empty_cache()
        for key, fn in SHAPE_VARIANTS:
            log(key, "...")
            extra[key] = fn(ctx)
            log(json.dumps(extra[key]))
            ctx.torch.cuda.empty_cache()
        detail["secondary"] = extra
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        cpu = cpu_baseline(wl, inp)
        detail["cpu_baseline"] = cpu
    if args.detail:
        with open(args.detail, "w") as fh:
            json.dump(detail, fh, indent=1)
    step_bytes = res["step_alg_bytes"]
    line = {
        "metric": "causal linear-attn fwd Mtokens/s + MFMA util; decode-step state GB/s vs HBM",
        "value": res["Mtokens_per_s"],
        "unit": "Mtokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1)*0.5, rounded to bf16)",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "N": wl.N, "d_k": wl.dk, "d_v": wl.dv,
                   "phi": wl.phi, "lambda": "per head U[0.9,0.999]", "eps": wl.eps, "state": "fp32",
                   "segments": res["segments"]},
        "roofline": res["roofline"],
        "dominant_kernel": res["dominant_kernel"],
        "step_roofline": {"bound": "hbm", "achieved": res["step_GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": res["step_hbm_frac"], "alg_bytes": step_bytes},
        "mfma": {"recurrent_TFLOPs": res["recurrent_TFLOPs"], "recurrent_frac": res["recurrent_mfma_frac"],
                 "executed_TFLOPs": res["executed_TFLOPs"], "executed_frac": res["executed_mfma_frac"],
                 "peak_TFLOPs": BF16_PEAK_TFLOPS},
        "decode": {"workload": dec["workload"], "ms_per_step": dec["ms_per_step"], "state_GBps": dec["state_GBps"],
                   "hbm_frac": dec["hbm_frac"], "kernel_frac": dec["roofline"]["frac"], "order": "plain",
                   "copy_GBps": cp["device_GBps"]},
        "cpu_baseline": cpu,
    }
    if scaling:
        line["length_scaling"] = [[p["N"], p["Mtokens_per_s"]] for p in scaling]
    if extra:
        line["secondary"] = {k: compact(v) for k, v in extra.items()}
    sys.stderr.flush()
    print(json.dumps(line, separators=(",", ":")), flush=True)


if __name__ == "__main__":
    main()
