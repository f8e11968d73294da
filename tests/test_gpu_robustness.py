"""Numerical robustness on the GPU (the debugging list of "Attention is also an
FFN" sec. 5.1: NaN, state blow-up, the feature map's sign, the normaliser and
eps):

- a NaN or an infinity in one input element stays in its own (batch, head)
  row: every other row of the output, and of the final state, is bit for bit
  what it is without it, and so are the rows of its own head that precede
  the chunk holding it (causal forward, decode step);
- features that all but vanish (elu+1 of inputs near -11.5 and -20, so that
  phi(q).z is near or far below eps): the outputs stay finite and match the
  oracle, i.e. eps enters the denominator the same way on both sides;
- the fp32 decode step (plain single-token update and the lambda^-e-scaled
  multi-token update) against the oracle at the fp32 bar, 1e-4.
"""
import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
import weight_sequence_mixing_amd as la
from gpu_util import DEV, TOL, inputs, oracle_causal, rel_err, row_errors, run_causal, to_dev

pytestmark = pytest.mark.gpu

# the kernels never carry a state across more than 64 tokens inside a chunk,
# so rows before the largest multiple of 64 at or below the poisoned token
# cannot see it
CHUNK_BOUND = 64


def _poison(inp, name, b, h, i, c, value):
    out = dict(inp)
    f = inp[name].copy()
    f[b, h, i, c] = value
    out[name] = f
    if name + "_bits" in inp:
        bits = inp[name + "_bits"].copy()
        bits[b, h, i, c] = si.bf16_bits_rne(np.array([value], dtype=np.float32))[0]
        out[name + "_bits"] = bits
    return out


@pytest.mark.parametrize("name", ["q", "k", "v"])
@pytest.mark.parametrize("value", [float("nan"), float("inf"), float("-inf")])
def test_nonfinite_input_stays_in_its_row(name, value):
    wl, inp = inputs(2, B=2, H=3, N=700)
    lam = [1.0, 0.97, 0.9]
    b, h, i = 1, 2, 300
    bad = _poison(inp, name, b, h, i, 5, value)
    y0, S0, z0 = run_causal(wl, inp, lam=lam, want_state=True)
    y1, S1, z1 = run_causal(wl, bad, lam=lam, want_state=True)
    keep = torch.ones(2, 3, dtype=torch.bool)
    keep[b, h] = False
    assert torch.equal(y1[keep], y0[keep])
    assert torch.equal(S1[keep], S0[keep]) and torch.equal(z1[keep], z0[keep])
    before = (i // CHUNK_BOUND) * CHUNK_BOUND
    assert torch.equal(y1[b, h, :before], y0[b, h, :before])
    if value == float("-inf") and name in ("q", "k"):
        # elu+1 maps -inf to the feature 0: a finite input to the method
        ref = oracle_causal(wl, bad, lam=lam)
        assert rel_err(y1, ref) < TOL["bf16"]
    else:
        # the poisoned row itself is not finite (the value reaches it)
        assert not torch.isfinite(y1[b, h, i].float()).all()


@pytest.mark.parametrize("name", ["q", "k", "v"])
def test_nonfinite_decode_input_stays_in_its_head_state(name):
    wl = si.workload(4)
    B, H = 4, 8
    pre = si.make_decode_prefix(wl, B=B, H=H, N=64)
    lam = list(map(float, si.make_lambda(wl, H=H)))
    q, k, v = (to_dev(pre, n, wl.dtype) for n in ("q", "k", "v"))
    S = torch.empty(B, H, wl.F, wl.dv, device=DEV)
    z = torch.empty(B, H, wl.F, device=DEV)
    la.la_forward_causal(q, k, v, torch.empty_like(q), lambda_h=lam, eps=wl.eps, S_out=S, z_out=z)
    st = si.make_decode_step(wl, 0, B=B, H=H)
    outs = []
    for poisoned in (False, True):
        s = _poison(st, name, 2, 5, 0, 7, float("nan")) if poisoned else st
        Sx, zx = S.clone(), z.clone()
        y = torch.empty(B, H, 1, wl.dv, dtype=torch.bfloat16, device=DEV)
        la.la_decode_step(*(to_dev(s, n, wl.dtype) for n in ("q", "k", "v")), y, Sx, zx, lambda_h=lam, eps=wl.eps)
        torch.cuda.synchronize()
        outs.append((y, Sx, zx))
    keep = torch.ones(B, H, dtype=torch.bool)
    keep[2, 5] = False
    for a, c in zip(outs[0], outs[1]):
        assert torch.equal(a[keep], c[keep])
    assert not torch.isfinite(outs[1][0][2, 5].float()).all()


@pytest.mark.parametrize("shift", [-11.5, -20.0])
def test_vanishing_features_normaliser_near_eps(shift):
    wl, inp = inputs(2, B=1, H=2, N=300)
    moved = dict(inp)
    for n in ("q", "k"):
        bits, vals = si.round_to_bf16(inp[n] + np.float32(shift))
        moved[n], moved[n + "_bits"] = vals, bits
    lam = [1.0, 0.95]
    y = run_causal(wl, moved, lam=lam)
    assert torch.isfinite(y.float()).all()
    ref = oracle_causal(wl, moved, lam=lam)
    # phi(q).z against eps: ~1 at -11.5, ~1e-8 at -20 (then y is num / eps)
    pq = oracle.phi_map(moved["q"][0, 0, -1])
    z = oracle.phi_map(moved["k"][0, 0]).sum(axis=0)
    print("shift %.1f: phi(q_last).z = %.3e, eps = %.0e" % (shift, float(pq @ z), wl.eps))
    err = rel_err(y, ref)
    assert err < TOL["bf16"], err


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("ntok", [1, 12])
def test_decode_fp32_inputs(d, ntok):
    wl = si.workload(1).with_(dk=d, dv=d)  # fp32 N(0,1)
    B, H, T = 2, 3, 24
    lam = [0.3, 0.97, 1.0]
    pre = si.make_inputs(wl, B=B, H=H, N=40)
    _, S0, z0 = oracle.causal(pre["q"], pre["k"], pre["v"], lam, wl.eps, want_state=True)
    S0, z0 = S0.astype(np.float32), z0.astype(np.float32)
    st = si.make_inputs(wl, seed=77, B=B, H=H, N=T)
    S = torch.from_numpy(S0).to(DEV)
    z = torch.from_numpy(z0).to(DEV)
    ys = []
    for c in range(T // ntok):
        part = {n: np.ascontiguousarray(st[n][:, :, c * ntok:(c + 1) * ntok]) for n in ("q", "k", "v")}
        y = torch.empty(B, H, ntok, d, dtype=torch.float32, device=DEV)
        la.la_decode_step(*(torch.from_numpy(part[n]).to(DEV) for n in ("q", "k", "v")), y, S, z,
                          lambda_h=lam, eps=wl.eps)
        ys.append(y)
    torch.cuda.synchronize()
    ref, Sr, zr = oracle.causal(st["q"], st["k"], st["v"], lam, wl.eps, S0=S0, z0=z0, want_state=True)
    err = rel_err(torch.cat(ys, dim=2), ref)
    s_err = float((np.abs(S.cpu().numpy() - Sr).max(axis=-1) / np.abs(Sr).max(axis=-1)).max())
    z_err = float((np.abs(z.cpu().numpy() - zr) / np.abs(zr)).max())
    print("d=%d ntok=%d: y %.2e, S %.2e, z %.2e" % (d, ntok, err, s_err, z_err))
    assert err < TOL["f32"] and s_err < TOL["f32"] and z_err < TOL["f32"], (err, s_err, z_err)
