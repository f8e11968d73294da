"""Helpers for the GPU parity tests: seeded inputs to device tensors, calls
through the C ABI binding, and the oracle comparison metric."""
import json
import os

import numpy as np
import torch

import oracle
import seeded_inputs as si
import weight_sequence_mixing_amd as la

TOL = {"f32": 1e-4, "bf16": 2e-2}
DEV = torch.device("cuda:0")


def to_dev(inp, name, dtype):
    if dtype == "bf16":
        return torch.from_numpy(inp[name + "_bits"].view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(inp[name])).to(DEV)


def tdtype(dtype):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def phi_for(wl, omega_np):
    if wl.random_features:
        return la.Phi(wl.phi, torch.from_numpy(np.ascontiguousarray(omega_np)).to(DEV), wl.qk_scale)
    return la.Phi(wl.phi)


def run_causal(wl, inp, lam=None, out_f32=False, S_in=None, z_in=None, want_state=False, eps=None):
    q, k, v = (to_dev(inp, n, wl.dtype) for n in ("q", "k", "v"))
    B, H, N, _ = q.shape
    ydt = torch.float32 if out_f32 else tdtype(wl.dtype)
    y = torch.full((B, H, N, wl.dv), float("nan"), dtype=ydt, device=DEV)
    phi = phi_for(wl, inp.get("omega"))
    F = wl.F
    S_out = z_out = None
    if want_state:
        S_out = torch.full((B, H, F, wl.dv), float("nan"), dtype=torch.float32, device=DEV)
        z_out = torch.full((B, H, F), float("nan"), dtype=torch.float32, device=DEV)
    lam = inp["lam"] if lam is None else lam
    la.la_forward_causal(q, k, v, y, phi=phi, lambda_h=list(map(float, lam)),
                         eps=wl.eps if eps is None else eps, S_in=S_in, z_in=z_in, S_out=S_out, z_out=z_out)
    torch.cuda.synchronize()
    if want_state:
        return y, S_out, z_out
    return y


def oracle_causal(wl, inp, lam=None, heads=None, **kw):
    q, k, v = inp["q"], inp["k"], inp["v"]
    lam = inp["lam"] if lam is None else lam
    if heads is not None:
        b, h = heads
        q, k, v = q[b][:, h], k[b][:, h], v[b][:, h]
        lam = np.asarray(lam)[h]
    return oracle.causal(q, k, v, lam, kw.pop("eps", wl.eps), wl.phi, inp.get("omega"), wl.qk_scale, **kw)


def rel_err(y_gpu, y_ref):
    y = y_gpu.float().cpu().numpy() if isinstance(y_gpu, torch.Tensor) else y_gpu
    err = oracle.rowwise_rel_err(y, y_ref)
    _record(err)
    return err


def row_errors(y_gpu, y_ref):
    """Per-row errors max_c |y - y_ref| / max_c |y_ref|, shape [B,H,N]."""
    y = y_gpu.float().cpu().numpy() if isinstance(y_gpu, torch.Tensor) else np.asarray(y_gpu)
    num = np.max(np.abs(y - y_ref), axis=-1)
    den = np.max(np.abs(y_ref), axis=-1)
    return num / np.where(den == 0, 1.0, den)


def _record(err, **extra):
    """Append the error to $LA_PARITY_LOG (one JSON line per comparison)."""
    path = os.environ.get("LA_PARITY_LOG")
    if not path:
        return
    test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
    with open(path, "a") as fh:
        fh.write(json.dumps(dict({"test": test, "max_row_rel_err": err}, **extra)) + "\n")


def inputs(index, **over):
    wl = si.workload(index)
    sizes = {k: over.pop(k) for k in ("B", "H", "N") if k in over}
    if over:
        wl = wl.with_(**over)
    return wl, si.make_inputs(wl, **sizes)


# Rows of sign-indefinite features whose denominator nearly cancels carry a
# rounding error that grows with their condition factor kappa_r; they are
# held to tol * max(1, kappa_r).  Rows with kappa_r at most KAPPA_FLAT are held
# to the flat bar.  A row whose scaled bound reaches 1 is not checked by it at
# all (the metric is relative to the row), so the share of such rows is
# recorded and must stay a minority.
KAPPA_FLAT = {"bf16": 10.0, "f32": 1e3}


def check_kappa_rows(y, ref, kap, dtype):
    err = row_errors(y, ref)
    tol = TOL[dtype]
    bound = tol * np.maximum(1.0, kap)
    worst = int(np.argmax(err / bound))
    assert np.all(err <= bound), (float(err.reshape(-1)[worst]), float(kap.reshape(-1)[worst]))
    flat = kap <= KAPPA_FLAT[dtype]
    assert flat.sum() > 0
    flat_max = float(err[flat].max())
    unchecked = int((bound >= 1.0).sum())
    stats = {"rows": int(err.size), "rows_flat_bar": int(flat.sum()), "rows_bound_ge_1": unchecked,
             "max_err_flat_rows": flat_max, "max_kappa": float(kap.max())}
    print("kappa rows:", json.dumps(stats), flush=True)
    _record(float(err.max()), kappa=stats)
    assert flat_max < tol, (flat_max, KAPPA_FLAT[dtype])
    assert unchecked < 0.5 * err.size, stats
    return stats
