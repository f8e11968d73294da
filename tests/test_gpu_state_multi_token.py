"""GPU parity of the identity-initialised state and of multi-token decode
(several tokens per call through la_forward_causal, carrying the fp32 state in
place between calls) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
import weight_sequence_mixing_amd as la
from gpu_util import DEV, TOL, rel_err, tdtype, to_dev

pytestmark = pytest.mark.gpu


def _identity(B, H, F, dv, alpha):
    S0 = np.broadcast_to(alpha * np.eye(F, dv), (B, H, F, dv)).copy()
    z0 = np.zeros((B, H, F))
    z0[..., :min(F, dv)] = alpha
    return S0, z0


@pytest.mark.parametrize("F,dv,alpha", [(64, 128, 0.5), (128, 64, 1.0), (64, 64, -2.0)])
def test_init_state_identity_exact(F, dv, alpha):
    B, H = 3, 5
    S = torch.full((B, H, F, dv), float("nan"), device=DEV)
    z = torch.full((B, H, F), float("nan"), device=DEV)
    la.la_init_state_identity(S, z, alpha)
    torch.cuda.synchronize()
    S0, z0 = _identity(B, H, F, dv, alpha)
    assert np.array_equal(S.cpu().numpy(), S0.astype(np.float32))
    assert np.array_equal(z.cpu().numpy(), z0.astype(np.float32))


@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 64)])
def test_forward_from_identity_state_in_place(dk, dv):
    wl = si.workload(3).with_(dk=dk, dv=dv)
    inp = si.make_inputs(wl, B=2, H=2, N=333)
    B, H, N = 2, 2, 333
    S = torch.empty(B, H, wl.F, dv, device=DEV)
    z = torch.empty(B, H, wl.F, device=DEV)
    la.la_init_state_identity(S, z, 0.5)
    q, k, v = (to_dev(inp, n, wl.dtype) for n in ("q", "k", "v"))
    y = torch.empty(B, H, N, dv, dtype=tdtype(wl.dtype), device=DEV)
    la.la_forward_causal(q, k, v, y, lambda_h=list(map(float, inp["lam"])), eps=wl.eps,
                         S_in=S, z_in=z, S_out=S, z_out=z)
    torch.cuda.synchronize()
    S0, z0 = _identity(B, H, wl.F, dv, 0.5)
    ref, Sr, zr = oracle.causal(inp["q"], inp["k"], inp["v"], inp["lam"], wl.eps, S0=S0, z0=z0, want_state=True)
    assert rel_err(y, ref) < TOL["bf16"]
    np.testing.assert_allclose(z.cpu().numpy(), zr, rtol=2e-2)
    np.testing.assert_allclose(S.cpu().numpy(), Sr, rtol=2e-2, atol=2e-2 * np.abs(Sr).max())


@pytest.mark.parametrize("k_tok", [1, 5, 32, 40])
def test_multi_token_decode_in_place(k_tok):
    # decode workload (lambda = 0.999, d = 128) at reduced B, H: a 96-token
    # prefix, then 4 calls of k_tok tokens each with S_in = S_out, z_in = z_out
    wl = si.workload(4).with_(N=96)
    B, H, calls = 2, 4, 4
    pre = si.make_decode_prefix(wl, B=B, H=H)
    lam = list(map(float, si.make_lambda(wl, H=H)))
    S = torch.empty(B, H, wl.F, wl.dv, device=DEV)
    z = torch.empty(B, H, wl.F, device=DEV)
    q, k, v = (to_dev(pre, n, wl.dtype) for n in ("q", "k", "v"))
    yp = torch.empty(B, H, wl.N, wl.dv, dtype=tdtype(wl.dtype), device=DEV)
    la.la_forward_causal(q, k, v, yp, lambda_h=lam, eps=wl.eps, S_out=S, z_out=z)
    rng = np.random.default_rng(k_tok)
    chunks, ys = [], []
    for c in range(calls):
        blk = {}
        for n, d in (("q", wl.dk), ("k", wl.dk), ("v", wl.dv)):
            bits, vals = si.round_to_bf16((rng.standard_normal((B, H, k_tok, d)) * wl.scale).astype(np.float32))
            blk[n], blk[n + "_bits"] = vals, bits
        chunks.append(blk)
        qs, ks, vs = (to_dev(blk, n, wl.dtype) for n in ("q", "k", "v"))
        y = torch.empty(B, H, k_tok, wl.dv, dtype=tdtype(wl.dtype), device=DEV)
        la.la_forward_causal(qs, ks, vs, y, lambda_h=lam, eps=wl.eps, S_in=S, z_in=z, S_out=S, z_out=z)
        ys.append(y)
    torch.cuda.synchronize()
    cat = {n: np.concatenate([pre[n]] + [c[n] for c in chunks], axis=2) for n in ("q", "k", "v")}
    ref, Sr, zr = oracle.causal(cat["q"], cat["k"], cat["v"], np.array(lam), wl.eps, want_state=True)
    assert rel_err(torch.cat(ys, dim=2), ref[:, :, wl.N:]) < TOL["bf16"]
    np.testing.assert_allclose(z.cpu().numpy(), zr, rtol=2e-2)
    np.testing.assert_allclose(S.cpu().numpy(), Sr, rtol=2e-2, atol=2e-2 * np.abs(Sr).max())


@pytest.mark.parametrize("phi,m,dk,k_tok", [("elu1", 0, 128, 3), ("elu1", 0, 128, 16), ("elu1", 0, 64, 64),
                                            ("relu", 0, 128, 5), ("trig_rf", 32, 64, 7),
                                            ("elu1", 0, 128, 10), ("elu1", 0, 128, 11), ("elu1", 0, 64, 9),
                                            ("relu", 0, 64, 10), ("trig_rf", 32, 64, 20)])
def test_decode_step_multi_token(phi, m, dk, k_tok):
    # la_decode_step with k_tok tokens per head-state per call (state held on
    # chip across them), three calls after a 96-token prefix; with bf16
    # inputs and an elementwise map, calls from 10 tokens (11 at d = 128) run
    # the causal forward's kernels from S back into S, shorter ones and the
    # random features the decode kernel: both sides of each threshold
    wl = si.workload(4).with_(N=96, phi=phi, m=m, dk=dk, dv=dk)
    B, H, calls = 2, 4, 3
    omega = si.make_omega(m, dk, 4) if m else None
    phi_c = la.Phi(phi, torch.from_numpy(omega).to(DEV), wl.qk_scale) if m else la.Phi(phi)
    pre = si.make_decode_prefix(wl, B=B, H=H)
    lam = list(map(float, si.make_lambda(wl, H=H)))
    S = torch.empty(B, H, wl.F, wl.dv, device=DEV)
    z = torch.empty(B, H, wl.F, device=DEV)
    q, k, v = (to_dev(pre, n, wl.dtype) for n in ("q", "k", "v"))
    yp = torch.empty(B, H, wl.N, wl.dv, dtype=tdtype(wl.dtype), device=DEV)
    la.la_forward_causal(q, k, v, yp, phi=phi_c, lambda_h=lam, eps=wl.eps, S_out=S, z_out=z)
    rng = np.random.default_rng(100 + k_tok)
    chunks, ys = [], []
    for c in range(calls):
        blk = {}
        for n, d in (("q", wl.dk), ("k", wl.dk), ("v", wl.dv)):
            bits, vals = si.round_to_bf16((rng.standard_normal((B, H, k_tok, d)) * wl.scale).astype(np.float32))
            blk[n], blk[n + "_bits"] = vals, bits
        chunks.append(blk)
        qs, ks, vs = (to_dev(blk, n, wl.dtype) for n in ("q", "k", "v"))
        y = torch.empty(B, H, k_tok, wl.dv, dtype=tdtype(wl.dtype), device=DEV)
        la.la_decode_step(qs, ks, vs, y, S, z, phi=phi_c, lambda_h=lam, eps=wl.eps)
        ys.append(y)
    torch.cuda.synchronize()
    cat = {n: np.concatenate([pre[n]] + [c[n] for c in chunks], axis=2) for n in ("q", "k", "v")}
    ref, Sr, zr, kap = oracle.causal(cat["q"], cat["k"], cat["v"], np.array(lam), wl.eps, phi, omega, wl.qk_scale,
                                     want_state=True, want_kappa=True)
    y = torch.cat(ys, dim=2)
    err = oracle.rowwise_rel_err(y.float().cpu().numpy(), ref[:, :, wl.N:]) if not m else None
    if m:
        from gpu_util import row_errors
        e = row_errors(y, ref[:, :, wl.N:])
        assert np.all(e <= TOL["bf16"] * np.maximum(1.0, kap[:, :, wl.N:]))
    else:
        assert err < TOL["bf16"], err
    np.testing.assert_allclose(S.cpu().numpy(), Sr, rtol=2e-2, atol=2e-2 * np.abs(Sr).max())


@pytest.mark.parametrize("lam", [[0.3, 0.5, 0.97, 1.0], [0.0, 1e-4, 0.3, 1.0]])
def test_decode_step_multi_token_decay_range(lam):
    # 12 tokens per call over the whole decay range: small lambda (the state
    # forgets within a few tokens), lambda = 0 (0^0 = 1: the state is the last
    # key's term alone) and lambda = 1
    wl = si.workload(4).with_(N=96)
    B, H, calls, k_tok = 2, 4, 3, 12
    pre = si.make_decode_prefix(wl, B=B, H=H)
    S = torch.empty(B, H, wl.F, wl.dv, device=DEV)
    z = torch.empty(B, H, wl.F, device=DEV)
    q, k, v = (to_dev(pre, n, wl.dtype) for n in ("q", "k", "v"))
    yp = torch.empty(B, H, wl.N, wl.dv, dtype=tdtype(wl.dtype), device=DEV)
    la.la_forward_causal(q, k, v, yp, lambda_h=lam, eps=wl.eps, S_out=S, z_out=z)
    rng = np.random.default_rng(77)
    chunks, ys = [], []
    for c in range(calls):
        blk = {}
        for n, d in (("q", wl.dk), ("k", wl.dk), ("v", wl.dv)):
            bits, vals = si.round_to_bf16((rng.standard_normal((B, H, k_tok, d)) * wl.scale).astype(np.float32))
            blk[n], blk[n + "_bits"] = vals, bits
        chunks.append(blk)
        qs, ks, vs = (to_dev(blk, n, wl.dtype) for n in ("q", "k", "v"))
        y = torch.empty(B, H, k_tok, wl.dv, dtype=tdtype(wl.dtype), device=DEV)
        la.la_decode_step(qs, ks, vs, y, S, z, lambda_h=lam, eps=wl.eps)
        ys.append(y)
    torch.cuda.synchronize()
    cat = {n: np.concatenate([pre[n]] + [c[n] for c in chunks], axis=2) for n in ("q", "k", "v")}
    ref, Sr, zr = oracle.causal(cat["q"], cat["k"], cat["v"], np.array(lam), wl.eps, want_state=True)
    err = oracle.rowwise_rel_err(torch.cat(ys, dim=2).float().cpu().numpy(), ref[:, :, wl.N:])
    assert err < TOL["bf16"], err
    np.testing.assert_allclose(z.cpu().numpy(), zr, rtol=2e-2, atol=1e-6)
    np.testing.assert_allclose(S.cpu().numpy(), Sr, rtol=2e-2, atol=2e-2 * np.abs(Sr).max())


def test_decode_step_many_head_states_multi_token():
    # more head-states than one grid dimension takes (B*H = 70400 > 65535): a
    # 12-token call, which with fewer head-states would run the causal
    # forward's kernels, stays on the decode kernel; sampled head-states
    # against the oracle from an identity initial state
    B, H, d, n = 1100, 64, 64, 12
    g = torch.Generator(device=DEV)
    g.manual_seed(7)
    q, k, v = (torch.randn(B, H, n, d, generator=g, device=DEV).mul_(0.5).to(torch.bfloat16) for _ in range(3))
    S = torch.empty(B, H, d, d, device=DEV)
    z = torch.empty(B, H, d, device=DEV)
    la.la_init_state_identity(S, z, 0.5)
    y = torch.empty_like(q)
    lam = 0.97
    la.la_decode_step(q, k, v, y, S, z, lambda_h=[lam] * H, eps=1e-6)
    torch.cuda.synchronize()
    S0, z0 = _identity(1, 1, d, d, 0.5)
    for b, h in ((0, 0), (B - 1, H - 1), (550, 31), (1023, 1)):
        one = lambda t: t[b, h].float().cpu().numpy()[None, None]
        ref, Sr, zr = oracle.causal(one(q), one(k), one(v), np.array([lam]), 1e-6, S0=S0, z0=z0, want_state=True)
        assert oracle.rowwise_rel_err(y[b, h].float().cpu().numpy()[None, None], ref) < TOL["bf16"], (b, h)
        np.testing.assert_allclose(S[b, h].cpu().numpy(), Sr[0, 0], rtol=2e-2, atol=2e-2 * np.abs(Sr).max())
        np.testing.assert_allclose(z[b, h].cpu().numpy(), zr[0, 0], rtol=2e-2, atol=2e-2 * np.abs(zr).max())
