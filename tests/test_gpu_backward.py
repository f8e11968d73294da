"""GPU parity of the backward (la_backward_causal) against the fp64 oracle's
gradients, through the C ABI.

y is the product forward's own output for the same inputs.  Gradient rows are
sums of terms that cancel: the gradient of a normalised weighted mean is
centred (phi(q_i) . d phi(q_i) = 0 exactly, and the first token's dq vanishes
but for eps), so a row's rounding error scales with its terms, not with its
own size.  The bar is therefore normwise per (batch, head): the largest error
over the head's gradient rows against the head's largest entry, within the
tolerance; rows of at least a tenth of that largest entry are also held to
the tolerance of their own size; and every row to tol * max(1, kappa_r),
kappa_r the oracle's ratio of the row's absolute terms to the row."""
import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
import weight_sequence_mixing_amd as la
from gpu_util import DEV, row_errors, tdtype, to_dev, _record

pytestmark = pytest.mark.gpu


# Gradient tolerance: fp32 as the forward; bf16 twice the forward's, since
# every gradient row is formed from bf16-rounded operands of both sweeps and
# then cancels by kappa (median 20-250 for dq rows).
TOL_BWD = {"f32": 1e-4, "bf16": 4e-2}


def head_scale(ref):
    """Per (batch, head): the head's largest |entry|, but at least a tenth of
    the tensor's (a head whose gradient vanishes up to eps -- lambda = 0,
    where each output is its own token's value -- is measured on the
    tensor's scale)."""
    s = np.abs(ref).reshape(ref.shape[0], ref.shape[1], -1).max(-1)
    return np.maximum(s, 0.1 * np.abs(ref).max())


def _check(name, got, ref, kappa, dtype, normwise=True):
    tol = TOL_BWD[dtype]
    err = row_errors(got, ref)
    if kappa is not None:
        # every row within tol * kappa_r (rounding error against the row's terms)
        bound = tol * np.maximum(1.0, kappa)
        worst = int(np.argmax(err / bound))
        assert np.all(err <= bound), (name, float(err.reshape(-1)[worst]), float(kappa.reshape(-1)[worst]))
    # normwise per head within tol, and rows of at least a tenth of their
    # head's scale within tol of their own size
    scale = head_scale(ref)
    he = np.abs(got - ref).reshape(got.shape[0], got.shape[1], -1).max(-1) / scale
    big = np.abs(ref).max(-1) >= 0.1 * scale[..., None]
    _record(float(he.max()))
    print("%s head-normwise %.3e  large-row %.3e  kappa median %.1f" % (
        name, he.max(), err[big].max(), float(np.median(kappa)) if kappa is not None else float("nan")))
    if not normwise:
        return  # every row cancels (the rows are no scale): the kappa bound alone
    assert float(he.max()) < tol, (name, float(he.max()))
    assert float(err[big].max()) < tol, (name, float(err[big].max()))


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def _grad_out(wl, B, H, N, seed):
    """dy ~ 0.5 N(0,1), rounded to the input type."""
    g = (np.random.default_rng(seed).standard_normal((B, H, N, wl.dv)) * 0.5).astype(np.float32)
    if wl.dtype == "bf16":
        bits, g = si.round_to_bf16(g)
        return g, torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    return g, _dev(g)


def run_backward(wl, B, H, N, lam, mask=None, state=False, dsout=False, seed=0):
    inp = si.make_inputs(wl, B=B, H=H, N=N)
    q, k, v = (to_dev(inp, n, wl.dtype) for n in ("q", "k", "v"))
    g_np, g = _grad_out(wl, B, H, N, seed + 1)
    rng = np.random.default_rng(seed + 2)
    F = wl.F
    S0 = z0 = dSo = dzo = None
    if state:
        S0 = (rng.standard_normal((B, H, F, wl.dv)) * 0.1).astype(np.float32)
        z0 = (rng.random((B, H, F)) + 0.5).astype(np.float32)
    if dsout:
        dSo = (rng.standard_normal((B, H, F, wl.dv)) * 0.01).astype(np.float32)
        dzo = (rng.standard_normal((B, H, F)) * 0.01).astype(np.float32)
    m = None if mask is None else si.make_key_padding_mask(B, N, mask, seed=seed + 3)
    mt = None if m is None else _dev(m)
    t = {n: (None if a is None else _dev(a)) for n, a in (("S0", S0), ("z0", z0), ("dSo", dSo), ("dzo", dzo))}
    phi = la.Phi(wl.phi)
    y = torch.empty(B, H, N, wl.dv, dtype=tdtype(wl.dtype), device=DEV)
    if mt is None:
        la.la_forward_causal(q, k, v, y, phi=phi, lambda_h=lam, eps=wl.eps, S_in=t["S0"], z_in=t["z0"])
    else:
        la.la_forward_causal_masked(q, k, v, y, mt, phi=phi, lambda_h=lam, eps=wl.eps, S_in=t["S0"], z_in=t["z0"])
    dq, dk, dv = torch.full_like(q, float("nan")), torch.full_like(k, float("nan")), torch.full_like(v, float("nan"))
    dSi = torch.full((B, H, F, wl.dv), float("nan"), device=DEV)
    dzi = torch.full((B, H, F), float("nan"), device=DEV)
    with_dlam = not (wl.dtype == "f32" and wl.dk == 128 and wl.dv == 128)
    dlam = torch.full((H,), float("nan"), device=DEV) if with_dlam else None
    la.la_backward_causal(q, k, v, y, g, dq, dk, dv, phi=phi, lambda_h=lam, eps=wl.eps, key_padding_mask=mt,
                          S_in=t["S0"], z_in=t["z0"], dS_out=t["dSo"], dz_out=t["dzo"], dS_in=dSi, dz_in=dzi,
                          dlambda=dlam)
    torch.cuda.synchronize()
    ref = oracle.backward(inp["q"], inp["k"], inp["v"], g_np, lam, wl.eps, wl.phi, None, 1.0, S0, z0, dSo, dzo,
                          key_padding_mask=m, want_kappa=True)
    got = {"dq": dq.float().cpu().numpy(), "dk": dk.float().cpu().numpy(), "dv": dv.float().cpu().numpy(),
           "dS0": dSi.cpu().numpy(), "dz0": dzi.cpu().numpy()}
    if with_dlam:
        got["dlam"] = dlam.cpu().numpy()
    return got, ref


def check_all(wl, got, ref):
    for n in ("dq", "dk", "dv"):
        _check(n, got[n], ref[n], ref["kappa_" + n], wl.dtype)
    tol = TOL_BWD[wl.dtype]
    for n in ("dS0", "dz0"):
        err = oracle.rowwise_rel_err(got[n], ref[n])
        _record(err)
        assert err < tol, (n, err)
    if "dlam" in got:
        # normwise over the heads: each head's dlambda sums O(N^2) pair terms
        # of both signs, so its rounding error follows the terms, whose size
        # is alike across heads, not the (possibly small) sum
        r = ref["dlam"].sum(0)
        err = float(np.abs(got["dlam"] - r).max() / np.abs(r).max())
        print("dlam normwise %.3e" % err, got["dlam"], r)
        _record(err)
        assert err < tol, ("dlam", got["dlam"], r)


CASES = [
    # workload, overrides, B, H, N, lambda per head, mask, initial state, final-state gradient
    (2, {}, 2, 2, 300, [0.9, 1.0], None, False, False),
    (2, {}, 2, 2, 777, [0.95, 1.0], None, True, True),
    (2, {}, 1, 2, 8200, [0.99, 1.0], None, True, True),            # many segments: both scans
    (1, {}, 1, 2, 257, [0.0, 0.95], None, True, False),             # fp32, lambda = 0
    (1, {"dk": 128, "dv": 128}, 1, 2, 300, [0.95, 1.0], "right", False, True),
    (3, {"phi": "relu", "lam": "one"}, 1, 2, 400, [0.9, 0.99], "random", False, False),  # d = 128
    (2, {"dv": 128}, 1, 3, 500, [0.9, 0.95, 1.0], None, True, False),
    (1, {"dk": 128, "dv": 64}, 2, 1, 333, [0.97], "random", True, True),
]


@pytest.mark.parametrize("wi,over,B,H,N,lam,mask,state,dsout", CASES)
def test_backward_parity(wi, over, B, H, N, lam, mask, state, dsout):
    wl = si.workload(wi).with_(**over)
    got, ref = run_backward(wl, B, H, N, lam, mask, state, dsout, seed=wi * 100 + N)
    check_all(wl, got, ref)


def test_backward_padded_keys_get_zero():
    wl = si.workload(2)
    B, H, N = 2, 2, 200
    got, ref = run_backward(wl, B, H, N, [0.9, 1.0], mask="random", seed=5)
    m = si.make_key_padding_mask(B, N, "random", seed=8)
    padded = np.broadcast_to(m[:, None, :], (B, H, N))
    assert float(np.abs(got["dk"][padded]).max()) == 0.0
    assert float(np.abs(got["dv"][padded]).max()) == 0.0


def test_backward_without_tokens_copies_state_gradient():
    B, H, d = 2, 3, 64
    q = torch.empty(B, H, 0, d, dtype=torch.bfloat16, device=DEV)
    dSo = torch.randn(B, H, d, d, device=DEV)
    dzo = torch.randn(B, H, d, device=DEV)
    dSi, dzi = torch.empty_like(dSo), torch.empty_like(dzo)
    la.la_backward_causal(q, q, q, q, q, q, q, q, dS_out=dSo, dz_out=dzo, dS_in=dSi, dz_in=dzi)
    torch.cuda.synchronize()
    assert torch.equal(dSi, dSo) and torch.equal(dzi, dzo)


def test_backward_full_size_headline_shape():
    # B=4 H=8 N=4096 d=64 bf16, lambda = 1: the benchmarked configuration
    wl = si.workload(2)
    got, ref = run_backward(wl, wl.B, wl.H, wl.N, [1.0] * wl.H, seed=42)
    check_all(wl, got, ref)


# ---------------------------------------------------------------------------
# Non-causal / cross form (la_backward_cross): the same bar as the causal
# form, with the oracle's kappa for this form.  With a single key the output
# is that key's value whatever q and k are (but for eps), so every dq and dk
# row cancels to the eps term: those rows are held to the kappa bound only.

def run_cross_backward(wl, B, H, Nq, Nk, mask=None, seed=0, self_attention=False):
    qi = si.make_inputs(wl, B=B, H=H, N=Nq)
    kv = qi if self_attention else si.make_kv(wl, Nk, B=B, H=H, seed=seed)
    q, k, v = to_dev(qi, "q", wl.dtype), to_dev(kv, "k", wl.dtype), to_dev(kv, "v", wl.dtype)
    g_np, g = _grad_out(wl, B, H, Nq, seed + 1)
    m = None if mask is None else si.make_key_padding_mask(B, Nk, mask, seed=seed + 3)
    mt = None if m is None else _dev(m)
    phi = la.Phi(wl.phi)
    y = torch.empty(B, H, Nq, wl.dv, dtype=tdtype(wl.dtype), device=DEV)
    if self_attention:
        la.la_forward_noncausal(q, k, v, y, phi=phi, eps=wl.eps)
    else:
        la.la_forward_cross(q, k, v, y, mt, phi=phi, eps=wl.eps)
    dq, dk, dv = torch.full_like(q, float("nan")), torch.full_like(k, float("nan")), torch.full_like(v, float("nan"))
    la.la_backward_cross(q, k, v, y, g, dq, dk, dv, mt, phi=phi, eps=wl.eps)
    torch.cuda.synchronize()
    ref = oracle.cross_backward(qi["q"], kv["k"], kv["v"], g_np, wl.eps, wl.phi, key_padding_mask=m,
                                want_kappa=True)
    got = {"dq": dq.float().cpu().numpy(), "dk": dk.float().cpu().numpy(), "dv": dv.float().cpu().numpy()}
    return got, ref, m


CROSS_CASES = [
    # workload, overrides, B, H, Nq, Nk, mask
    (2, {}, 2, 2, 300, 777, None),
    (2, {"phi": "relu"}, 2, 2, 1000, 513, "right"),
    (1, {}, 2, 1, 257, 100, "random"),                  # fp32
    (1, {"dk": 128, "dv": 128}, 1, 2, 64, 3000, None),  # many key segments
    (2, {"dv": 128}, 1, 2, 5000, 200, "random"),        # many query segments: the adjoint reduction
    (3, {"phi": "relu", "lam": "one"}, 1, 2, 33, 1, None),  # d = 128, one key
    (2, {}, 1, 1, 1, 40, "random"),                     # one query
]


@pytest.mark.parametrize("wi,over,B,H,Nq,Nk,mask", CROSS_CASES)
def test_cross_backward_parity(wi, over, B, H, Nq, Nk, mask):
    wl = si.workload(wi).with_(**over)
    got, ref, m = run_cross_backward(wl, B, H, Nq, Nk, mask, seed=wi * 100 + Nq)
    for n in ("dq", "dk", "dv"):
        _check(n, got[n], ref[n], ref["kappa_" + n], wl.dtype, normwise=Nk > 1 or n == "dv")
    if m is not None:
        padded = np.broadcast_to(m[:, None, :], (B, H, Nk))
        assert float(np.abs(got["dk"][padded]).max(initial=0.0)) == 0.0
        assert float(np.abs(got["dv"][padded]).max(initial=0.0)) == 0.0


def test_noncausal_self_attention_backward():
    # la_forward_noncausal's gradients: the same rows for keys and queries
    wl = si.workload(2).with_(dk=128, dv=128)
    got, ref, _ = run_cross_backward(wl, 1, 2, 4096, 4096, seed=7, self_attention=True)
    for n in ("dq", "dk", "dv"):
        _check(n, got[n], ref[n], ref["kappa_" + n], wl.dtype)


def test_cross_backward_all_keys_padded_gives_zero():
    # no key kept: S = z = 0, so y = 0 and every gradient vanishes
    wl = si.workload(2)
    got, _, _ = run_cross_backward(wl, 2, 2, 100, 70, mask="all", seed=3)
    for n in ("dq", "dk", "dv"):
        assert float(np.abs(got[n]).max()) == 0.0, n


def test_cross_backward_full_size():
    # B=4 H=8, 1024 queries against 4096 right-padded keys, d=64 bf16: the
    # benchmarked cross-attention shape
    wl = si.workload(2)
    got, ref, _ = run_cross_backward(wl, 4, 8, 1024, 4096, mask="right", seed=11)
    for n in ("dq", "dk", "dv"):
        _check(n, got[n], ref[n], ref["kappa_" + n], wl.dtype)
