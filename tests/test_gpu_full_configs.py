"""Parity at the workloads' full sizes, in the launch configuration the bench
times, against the fp64 oracle.

- Long causal forwards: every head of the per-head-decay workload (B=2, H=16,
  N=32768, d=128) and of the random-feature workload (B=1, H=16, N=65536,
  d=64, m=128).
- The decode workload as configured: 256 sequences x 32 heads, d=128, a
  512-token prefix through la_forward_causal (S_out, z_out), then 1024
  single-token la_decode_step calls at lambda = 0.999.  y at every step and
  the final S, z are compared on 256 sampled head-states (the oracle runs
  their whole 1536-token trajectories); for every head-state the 1024 steps
  are also compared with one la_forward_causal call over the same tokens from
  the same prefix state (decode = forward row by row, a property that holds
  at any size).

Metric: per row (b,h,i) max_c |y - y_ref| / max_c |y_ref|; the bar is 2e-2 for
bf16 inputs with an fp32 state.  Each test prints its per-configuration
figures (max row error, where it occurs) so that the log records them.
"""
import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
import weight_sequence_mixing_amd as la
from gpu_util import DEV, TOL, check_kappa_rows, oracle_causal, rel_err, row_errors, run_causal

pytestmark = pytest.mark.gpu


def _report(tag, err_rows):
    """Print the max row error and its (b,h,i), and where the 99.9% quantile sits."""
    flat = int(np.argmax(err_rows))
    idx = np.unravel_index(flat, err_rows.shape)
    print("%s: max row err %.3e at %s, 99.9%% quantile %.3e, rows %d"
          % (tag, float(err_rows.reshape(-1)[flat]), tuple(int(i) for i in idx),
             float(np.quantile(err_rows, 0.999)), err_rows.size), flush=True)


def test_workload3_full_every_head():
    wl = si.workload(3)
    inp = si.make_inputs(wl)
    y = run_causal(wl, inp)
    ref = oracle_causal(wl, inp)
    err = row_errors(y, ref)
    _report(wl.name, err)
    per_head = err.reshape(wl.B * wl.H, -1).max(axis=1)
    print("per-(b,h) max:", " ".join("%.2e" % e for e in per_head), flush=True)
    assert np.isfinite(err).all()
    assert float(err.max()) < TOL["bf16"], float(err.max())
    rel_err(y, ref)  # parity log


def test_workload5_full_every_head():
    wl = si.workload(5)
    inp = si.make_inputs(wl)
    y = run_causal(wl, inp)
    ref, kap = oracle_causal(wl, inp, want_kappa=True)
    err = row_errors(y, ref)
    _report(wl.name, err)
    print("largest kappa %.1f; per-head max:" % float(kap.max()),
          " ".join("%.2e" % e for e in err.reshape(wl.H, -1).max(axis=1)), flush=True)
    assert np.isfinite(err).all()
    check_kappa_rows(y, ref, kap, "bf16")


def test_workload5_m256_full_sampled_heads():
    # the m sweep's last point at workload 5's size (two halves of 128
    # directions); all 16 heads run, four are compared (every row of each)
    wl = si.workload(5).with_(m=256)
    inp = si.make_inputs(wl)
    y = run_causal(wl, inp).float().cpu().numpy()
    heads = [0, 5, 10, 15]
    sub = dict(inp, q=inp["q"][:, heads], k=inp["k"][:, heads], v=inp["v"][:, heads], lam=inp["lam"][heads])
    ref, kap = oracle_causal(wl, sub, want_kappa=True)
    err = row_errors(y[:, heads], ref)
    _report(wl.name + "_m256_heads0-5-10-15", err)
    assert np.isfinite(err).all()
    check_kappa_rows(y[:, heads], ref, kap, "bf16")


def _bits_to_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def test_workload4_full_trajectory():
    wl = si.workload(4)
    B, H, d, F, Np, T = wl.B, wl.H, wl.dk, wl.F, wl.N, wl.steps
    threads = oracle.default_threads()
    lam = list(map(float, si.make_lambda(wl)))
    # 256 sampled head-states, the first and the last among them
    rng = np.random.default_rng(404)
    flat = np.unique(np.concatenate([[0, B * H - 1], rng.choice(B * H, size=254, replace=False)]))[:256]
    if flat.size < 256:
        extra = np.setdiff1d(np.arange(B * H), flat)[: 256 - flat.size]
        flat = np.sort(np.concatenate([flat, extra]))
    sb, sh = flat // H, flat % H
    ns = flat.size

    # prefix: drawn in blocks of batch rows straight to the device; the
    # sampled head-states' values kept on the host for the oracle
    dev = {n: torch.empty(B, H, Np, d, dtype=torch.bfloat16, device=DEV) for n in ("q", "k", "v")}
    host = {n: np.empty((ns, Np + T, d), dtype=np.float32) for n in ("q", "k", "v")}
    RB = 16
    for b0 in range(0, B, RB):
        blk = si.make_decode_prefix(wl, B=RB, threads=threads, values=False, b0=b0)
        sel = np.nonzero((sb >= b0) & (sb < b0 + RB))[0]
        for n in ("q", "k", "v"):
            dev[n][b0:b0 + RB].copy_(_bits_to_dev(blk[n + "_bits"]))
            host[n][sel, :Np] = si.bf16_bits_to_f32(blk[n + "_bits"][sb[sel] - b0, sh[sel]])
    S = torch.full((B, H, F, d), float("nan"), dtype=torch.float32, device=DEV)
    z = torch.full((B, H, F), float("nan"), dtype=torch.float32, device=DEV)
    yp = torch.empty(B, H, Np, d, dtype=torch.bfloat16, device=DEV)
    la.la_forward_causal(dev["q"], dev["k"], dev["v"], yp, lambda_h=lam, eps=wl.eps, S_out=S, z_out=z)
    S0, z0 = S.clone(), z.clone()
    del dev

    # 1024 decode steps, inputs drawn in blocks of steps; the same tokens also
    # laid out as [B,H,T,d] for the forward over them
    ys = torch.empty(T, B, H, 1, d, dtype=torch.bfloat16, device=DEV)
    seq = {n: torch.empty(B, H, T, d, dtype=torch.bfloat16, device=DEV) for n in ("q", "k", "v")}
    TB = 64
    for t0 in range(0, T, TB):
        blk = si.make_decode_steps(wl, t0, t0 + TB, threads=threads)
        st = {n: _bits_to_dev(blk[n + "_bits"]) for n in ("q", "k", "v")}
        for i in range(TB):
            la.la_decode_step(st["q"][i], st["k"][i], st["v"][i], ys[t0 + i], S, z, lambda_h=lam, eps=wl.eps)
        for n in ("q", "k", "v"):
            seq[n][:, :, t0:t0 + TB].copy_(st[n][:, :, :, 0].permute(1, 2, 0, 3))
            host[n][:, Np + t0:Np + t0 + TB] = si.bf16_bits_to_f32(blk[n + "_bits"][:, sb, sh, 0]).transpose(1, 0, 2)
    torch.cuda.synchronize()

    # the oracle over the sampled head-states' whole trajectories (each one
    # a "head" of its own with lambda = 0.999)
    ref, Sr, zr = oracle.causal(host["q"][None], host["k"][None], host["v"][None], [lam[0]] * ns, wl.eps,
                                want_state=True, threads=threads)
    ref, Sr, zr = ref[0], Sr[0], zr[0]
    y_pre = yp[sb, sh].float().cpu().numpy()                          # [ns, Np, d]
    y_dec = ys[:, sb, sh, 0].float().cpu().numpy().transpose(1, 0, 2)  # [ns, T, d]
    err_pre = row_errors(y_pre, ref[:, :Np])
    err_dec = row_errors(y_dec, ref[:, Np:])
    _report("prefix (la_forward_causal)", err_pre)
    _report("decode steps 1..1024", err_dec)
    for t in (1, 2, 512, 1024):
        print("step %4d: max row err over the sampled head-states %.3e" % (t, float(err_dec[:, t - 1].max())))
    assert np.isfinite(err_dec).all() and np.isfinite(err_pre).all()
    assert float(err_pre.max()) < TOL["bf16"], float(err_pre.max())
    assert float(err_dec.max()) < TOL["bf16"], float(err_dec.max())

    # final state of the sampled head-states: per feature row of S, relative
    # to that row's largest entry; z elementwise (elu+1 keeps it positive)
    Sg = S[sb, sh].cpu().numpy().astype(np.float64)
    zg = z[sb, sh].cpu().numpy().astype(np.float64)
    s_err = np.max(np.abs(Sg - Sr), axis=-1) / np.max(np.abs(Sr), axis=-1)
    z_err = np.abs(zg - zr) / np.abs(zr)
    print("final S: max row err %.3e; final z: max rel err %.3e" % (float(s_err.max()), float(z_err.max())))
    assert float(s_err.max()) < TOL["bf16"] and float(z_err.max()) < TOL["bf16"]

    # every head-state: the steps equal one forward over the same tokens from
    # the same prefix state
    yf = torch.empty(B, H, T, d, dtype=torch.bfloat16, device=DEV)
    Sf, zf = torch.empty_like(S), torch.empty_like(z)
    la.la_forward_causal(seq["q"], seq["k"], seq["v"], yf, lambda_h=lam, eps=wl.eps, S_in=S0, z_in=z0,
                         S_out=Sf, z_out=zf)
    torch.cuda.synchronize()
    yd = ys[:, :, :, 0].permute(1, 2, 0, 3).float()
    num = (yd - yf.float()).abs().amax(dim=-1)
    den = yf.float().abs().amax(dim=-1).clamp_min(1e-30)
    diff = float((num / den).max())
    s_diff = float(((S - Sf).abs().amax(dim=-1) / Sf.abs().amax(dim=-1)).max())
    print("all %d head-states: decode vs forward max row diff %.3e, final S diff %.3e" % (B * H, diff, s_diff))
    assert diff < TOL["bf16"] and s_diff < TOL["bf16"]
