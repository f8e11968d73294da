"""GPU parity of the feature-map variants against the fp64 oracle: ReLU, the
two other random-feature prefactors (1/sqrt(m) and exp(+|x'|^2/2)/sqrt(m)),
random directions drawn without orthogonalisation, and the m sweep -- for the
causal forward, the non-causal forward and the decode step."""
import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
import weight_sequence_mixing_amd as la
from gpu_util import DEV, TOL, check_kappa_rows, oracle_causal, phi_for, rel_err, run_causal, tdtype, to_dev

pytestmark = pytest.mark.gpu


def _check_rows(y, ref, kap, dtype):
    """Every row within tol * max(1, kappa_r); well-conditioned rows within tol;
    the rows a scaled bound leaves unchecked are a minority."""
    check_kappa_rows(y, ref, kap, dtype)


@pytest.mark.parametrize("dk,dv,dtype,N", [(64, 64, "bf16", 1000), (128, 128, "bf16", 777),
                                           (64, 128, "f32", 300), (128, 64, "f32", 257)])
def test_relu_causal(dk, dv, dtype, N):
    wl = si.workload(3).with_(phi="relu", dk=dk, dv=dv, dtype=dtype, scale=0.5 if dtype == "bf16" else 1.0)
    inp = si.make_inputs(wl, B=2, H=3, N=N)
    lam = [0.9, 0.99, 1.0]
    y, S, z = run_causal(wl, inp, lam=lam, want_state=True)
    ref, Sr, zr = oracle_causal(wl, inp, lam=lam, want_state=True)
    err = rel_err(y, ref)
    assert err < TOL[dtype], err
    np.testing.assert_allclose(z.cpu().numpy(), zr, rtol=TOL[dtype], atol=TOL[dtype] * np.abs(zr).max())
    np.testing.assert_allclose(S.cpu().numpy(), Sr, rtol=TOL[dtype], atol=TOL[dtype] * np.abs(Sr).max())


def test_relu_all_zero_queries_give_zero():
    # a query with no positive component has no features: numerator 0, output 0
    wl = si.workload(2).with_(phi="relu")
    inp = si.make_inputs(wl, B=1, H=2, N=300)
    bits = inp["q_bits"].copy()
    f = inp["q"].copy()
    nb, nv = si.round_to_bf16(-np.abs(f[:, :, 5:40]) - 0.01)
    bits[:, :, 5:40] = nb
    f[:, :, 5:40] = nv
    inp = dict(inp, q=f, q_bits=bits)
    y = run_causal(wl, inp, lam=[1.0, 0.9])
    assert float(y[:, :, 5:40].float().abs().max()) == 0.0
    err = rel_err(y, oracle_causal(wl, inp, lam=[1.0, 0.9]))
    assert err < TOL["bf16"], err


@pytest.mark.parametrize("phi", ["trig_rf_plain", "trig_rf_softmax"])
@pytest.mark.parametrize("m", [32, 64, 128])
def test_random_feature_prefactors_causal(phi, m):
    wl = si.workload(5).with_(phi=phi, m=m)
    inp = si.make_inputs(wl, B=1, H=2, N=333)
    lam = [0.97, 1.0]
    y = run_causal(wl, inp, lam=lam)
    ref, kap = oracle_causal(wl, inp, lam=lam, want_kappa=True)
    _check_rows(y, ref, kap, "bf16")


@pytest.mark.parametrize("m,dk,dv", [(32, 128, 128), (64, 128, 64), (128, 64, 128), (64, 64, 128)])
def test_random_features_head_sizes(m, dk, dv, monkeypatch):
    # random features beyond d_k = d_v = 64: four k blocks of omega per
    # feature tile, eight value tiles per wave in the segment states, two
    # waves per omega row block for m <= 64; three segments of six 64-token
    # chunks, the last one ragged
    monkeypatch.setenv("LA_SEGMENTS", "3")
    wl = si.workload(5).with_(m=m, dk=dk, dv=dv)
    inp = si.make_inputs(wl, B=1, H=2, N=1100)
    lam = [0.98, 1.0]
    y, S, z = run_causal(wl, inp, lam=lam, want_state=True)
    ref, Sr, zr, kap = oracle_causal(wl, inp, lam=lam, want_state=True, want_kappa=True)
    _check_rows(y, ref, kap, "bf16")
    np.testing.assert_allclose(z.cpu().numpy(), zr, rtol=TOL["bf16"], atol=TOL["bf16"] * np.abs(zr).max())
    np.testing.assert_allclose(S.cpu().numpy(), Sr, rtol=TOL["bf16"], atol=TOL["bf16"] * np.abs(Sr).max())


@pytest.mark.parametrize("m", [32, 64, 128, 256])
@pytest.mark.parametrize("lam", [[0.5, 0.0, 0.3, 1.0], [0.71, 0.75, 1.0, 0.999]], ids=["small", "edge"])
def test_random_features_decay_range(m, lam, monkeypatch):
    # the causal output pass stages the values with their key weights only
    # where every head has lambda = 1 or lambda >= 2^-1/2; "small" takes the
    # other form (lambda = 0 among the heads), "edge" the weighted one near
    # its limit, where a chunk's weights span lambda^63 ~ 2^-31; four
    # segments of 64-token chunks, the last one ragged
    monkeypatch.setenv("LA_SEGMENTS", "4")
    wl = si.workload(5).with_(m=m)
    inp = si.make_inputs(wl, B=1, H=4, N=1500)
    y, S, z = run_causal(wl, inp, lam=lam, want_state=True)
    ref, Sr, zr, kap = oracle_causal(wl, inp, lam=lam, want_state=True, want_kappa=True)
    _check_rows(y, ref, kap, "bf16")
    np.testing.assert_allclose(z.cpu().numpy(), zr, rtol=TOL["bf16"], atol=TOL["bf16"] * np.abs(zr).max())
    np.testing.assert_allclose(S.cpu().numpy(), Sr, rtol=TOL["bf16"], atol=TOL["bf16"] * np.abs(Sr).max())


@pytest.mark.parametrize("phi", ["trig_rf", "trig_rf_softmax"])
def test_random_features_gaussian_omega(phi):
    # rows of omega drawn independently from N(0, I), no orthogonal blocks
    wl = si.workload(5).with_(phi=phi, m=64, omega="gaussian")
    inp = si.make_inputs(wl, B=1, H=2, N=500)
    lam = [1.0, 0.95]
    y = run_causal(wl, inp, lam=lam)
    ref, kap = oracle_causal(wl, inp, lam=lam, want_kappa=True)
    _check_rows(y, ref, kap, "bf16")


def test_random_feature_prefactor_fp32():
    wl = si.workload(1).with_(phi="trig_rf_softmax", m=32, scale=0.35)
    inp = si.make_inputs(wl, B=1, H=2, N=200)
    y = run_causal(wl, inp, lam=[0.95, 1.0])
    ref, kap = oracle_causal(wl, inp, lam=[0.95, 1.0], want_kappa=True)
    _check_rows(y, ref, kap, "f32")


@pytest.mark.parametrize("phi,m", [("relu", 0), ("trig_rf_softmax", 64), ("trig_rf_plain", 32)])
def test_feature_map_noncausal(phi, m):
    wl = (si.workload(2) if phi == "relu" else si.workload(5)).with_(phi=phi, m=m)
    inp = si.make_inputs(wl, B=2, H=2, N=555)
    q, k, v = (to_dev(inp, n, wl.dtype) for n in ("q", "k", "v"))
    B, H, N, _ = q.shape
    y = torch.empty(B, H, N, wl.dv, dtype=tdtype(wl.dtype), device=DEV)
    la.la_forward_noncausal(q, k, v, y, phi=phi_for(wl, inp["omega"]), eps=wl.eps)
    torch.cuda.synchronize()
    ref = oracle.noncausal(inp["q"], inp["k"], inp["v"], wl.eps, wl.phi, inp["omega"], wl.qk_scale)
    # condition factor of each row's denominator phi(q_i) . sum_j phi(k_j) + eps:
    # sign-indefinite random features can cancel (1 for non-negative features)
    pq = oracle.phi_map(inp["q"], wl.phi, inp["omega"], wl.qk_scale)
    pk = oracle.phi_map(inp["k"], wl.phi, inp["omega"], wl.qk_scale)
    den = np.einsum("bhnf,bhf->bhn", pq, pk.sum(axis=2)) + wl.eps
    kap = np.einsum("bhnf,bhf->bhn", np.abs(pq), np.abs(pk).sum(axis=2)) / np.abs(den)
    if phi == "relu":
        assert float(kap.max()) <= 1.0 + 1e-9
    _check_rows(y, ref, kap, wl.dtype)


@pytest.mark.parametrize("phi,m,dk", [("relu", 0, 128), ("trig_rf_softmax", 32, 64)])
def test_feature_map_decode_matches_forward_trajectory(phi, m, dk):
    # prefix through the causal forward (S_out, z_out), then single-token steps;
    # the outputs equal the oracle's causal pass over prefix + steps
    wl = si.workload(4).with_(phi=phi, m=m, dk=dk, dv=dk, N=96)
    B, H, steps = 2, 4, 8
    omega = si.make_omega(m, dk, 4) if m else None
    phi_c = phi_for(wl, omega)
    pre = si.make_decode_prefix(wl, B=B, H=H)
    lam = si.make_lambda(wl, H=H)
    q, k, v = (to_dev(pre, n, wl.dtype) for n in ("q", "k", "v"))
    S = torch.empty(B, H, wl.F, wl.dv, dtype=torch.float32, device=DEV)
    z = torch.empty(B, H, wl.F, dtype=torch.float32, device=DEV)
    yp = torch.empty(B, H, wl.N, wl.dv, dtype=tdtype(wl.dtype), device=DEV)
    la.la_forward_causal(q, k, v, yp, phi=phi_c, lambda_h=list(map(float, lam)), eps=wl.eps, S_out=S, z_out=z)
    ys, step_inp = [], []
    for t in range(steps):
        st = si.make_decode_step(wl, t, B=B, H=H)
        step_inp.append(st)
        qs, ks, vs = (to_dev(st, n, wl.dtype) for n in ("q", "k", "v"))
        y = torch.empty(B, H, 1, wl.dv, dtype=tdtype(wl.dtype), device=DEV)
        la.la_decode_step(qs, ks, vs, y, S, z, phi=phi_c, lambda_h=list(map(float, lam)), eps=wl.eps)
        ys.append(y)
    torch.cuda.synchronize()
    y = torch.cat(ys, dim=2)
    cat = {n: np.concatenate([pre[n]] + [s[n] for s in step_inp], axis=2) for n in ("q", "k", "v")}
    ref, kap = oracle.causal(cat["q"], cat["k"], cat["v"], lam, wl.eps, phi, omega, wl.qk_scale,
                             want_kappa=True)
    _check_rows(y, ref[:, :, wl.N:], kap[:, :, wl.N:], "bf16")


@pytest.mark.parametrize("phi,dv,N,out_f32", [("trig_rf", 64, 700, False), ("trig_rf_softmax", 64, 333, False),
                                             ("trig_rf", 64, 4133, True)])
def test_random_features_m256_causal(phi, dv, N, out_f32):
    # m = 256 (F = 512) runs as two halves of 128 directions; the second adds
    # the first's numerators and denominators.  Several segments at N = 4133.
    wl = si.workload(5).with_(phi=phi, m=256, dv=dv)
    inp = si.make_inputs(wl, B=1, H=2, N=N)
    lam = [0.97, 1.0]
    y, S, z = run_causal(wl, inp, lam=lam, out_f32=out_f32, want_state=True)
    ref, kap = oracle_causal(wl, inp, lam=lam, want_kappa=True)
    _check_rows(y, ref, kap, "bf16")
    _, Sr, zr = oracle_causal(wl, inp, lam=lam, want_state=True)
    np.testing.assert_allclose(z.cpu().numpy(), zr, rtol=TOL["bf16"], atol=TOL["bf16"] * np.abs(zr).max())
    np.testing.assert_allclose(S.cpu().numpy(), Sr, rtol=TOL["bf16"], atol=TOL["bf16"] * np.abs(Sr).max())


def test_random_features_m256_state_in_and_varlen():
    # carried-in state (both halves read their rows of S_in, z_in) and packed
    # sequences (the stored numerators are indexed by packed row)
    wl = si.workload(5).with_(m=256)
    inp = si.make_inputs(wl, B=1, H=2, N=600)
    lam = [0.99, 0.9]
    cut = lambda sl: {n: (np.ascontiguousarray(x[:, :, sl]) if n in ("q", "k", "v", "q_bits", "k_bits", "v_bits")
                          else x) for n, x in inp.items()}
    _, S0, z0 = run_causal(wl, cut(slice(0, 200)), lam=lam, want_state=True)
    rest = cut(slice(200, None))
    y = run_causal(wl, rest, lam=lam, S_in=S0, z_in=z0)
    ref, kap = oracle_causal(wl, inp, lam=lam, want_kappa=True)
    _check_rows(y, ref[:, :, 200:], kap[:, :, 200:], "bf16")
    # packed: two sequences of 250 and 350 tokens in head rows of 600
    q, k, v = (to_dev(inp, n, "bf16")[0] for n in ("q", "k", "v"))
    cu = torch.tensor([0, 250, 600], dtype=torch.int32, device=DEV)
    yv = torch.empty(2, 600, wl.dv, dtype=torch.bfloat16, device=DEV)
    la.la_forward_causal_varlen(q, k, v, yv, cu, 350, phi=phi_for(wl, inp["omega"]), lambda_h=lam, eps=wl.eps)
    torch.cuda.synchronize()
    for s0, s1 in ((0, 250), (250, 600)):
        part = {n: inp[n][:, :, s0:s1] for n in ("q", "k", "v")}
        refp, kapp = oracle.causal(part["q"], part["k"], part["v"], np.asarray(lam), wl.eps, wl.phi, inp["omega"],
                                   wl.qk_scale, want_kappa=True)
        _check_rows(yv[None, :, s0:s1], refp, kapp, "bf16")
