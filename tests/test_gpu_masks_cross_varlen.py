"""GPU parity of the key padding mask, cross attention (N_q != N_k) and packed
variable-length causal forwards against the fp64 oracle, through the C ABI.

Sizes span several chunks and segments with ragged tails; every case is
seeded.  Masks are padded batches (right padding) and independent random
padding; packed batches mix empty, short and long sequences."""
import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
import weight_sequence_mixing_amd as la
from gpu_util import DEV, TOL, phi_for, rel_err, row_errors, tdtype, to_dev

pytestmark = pytest.mark.gpu


def _dev_mask(mask):
    return torch.from_numpy(np.ascontiguousarray(mask)).to(DEV)


def _check_rows(y, ref, kap, dtype):
    """Every row within tol * max(1, kappa_r) (kappa_r: cancellation factor of
    the row's normaliser, 1 for positive features)."""
    err = row_errors(y, ref)
    bound = TOL[dtype] * np.maximum(1.0, kap)
    worst = int(np.argmax(err / bound))
    assert np.all(err <= bound), (float(err.reshape(-1)[worst]), float(kap.reshape(-1)[worst]))


def _kappa_cross(wl, q, k, omega, mask):
    """|phi(q)|^T sum_j |phi(k_j)| / |phi(q)^T z + eps| over the kept keys."""
    pq = oracle.phi_map(q, wl.phi, omega, wl.qk_scale)
    pk = oracle.phi_map(k, wl.phi, omega, wl.qk_scale)
    keep = np.ones(k.shape[:1] + k.shape[2:3]) if mask is None else (~mask).astype(float)
    pk = pk * keep[:, None, :, None]
    den = np.einsum("bhnf,bhf->bhn", pq, pk.sum(2)) + wl.eps
    return np.einsum("bhnf,bhf->bhn", np.abs(pq), np.abs(pk).sum(2)) / np.abs(den)


# ------------------------------------------------------------------ cross attention
CROSS = [
    # workload, overrides, B, H, Nq, Nk, mask kind
    (2, {}, 2, 4, 100, 1000, None),
    (2, {}, 2, 4, 1000, 37, "right"),
    (2, {}, 1, 2, 777, 9000, "random"),        # the keys split into many segments
    (3, {"lam": "one"}, 2, 3, 300, 513, "random"),       # d = 128
    (1, {"phi": "relu"}, 2, 2, 65, 200, "right"),        # fp32
    (5, {"m": 64}, 1, 4, 257, 1500, "random"),           # random features
]


@pytest.mark.parametrize("wi,over,B,H,Nq,Nk,kind", CROSS)
def test_cross_parity(wi, over, B, H, Nq, Nk, kind):
    wl = si.workload(wi).with_(**over)
    inp = si.make_inputs(wl, B=B, H=H, N=Nq)
    kv = si.make_kv(wl, Nk, B=B, H=H)
    mask = None if kind is None else si.make_key_padding_mask(B, Nk, kind, seed=wi)
    q = to_dev(inp, "q", wl.dtype)
    k, v = to_dev(kv, "k", wl.dtype), to_dev(kv, "v", wl.dtype)
    y = torch.full((B, H, Nq, wl.dv), float("nan"), dtype=tdtype(wl.dtype), device=DEV)
    la.la_forward_cross(q, k, v, y, None if mask is None else _dev_mask(mask), phi=phi_for(wl, inp.get("omega")),
                        eps=wl.eps)
    torch.cuda.synchronize()
    ref = oracle.cross(inp["q"], kv["k"], kv["v"], wl.eps, wl.phi, inp.get("omega"), wl.qk_scale,
                       key_padding_mask=mask)
    if wl.random_features:
        _check_rows(y, ref, _kappa_cross(wl, inp["q"], kv["k"], inp.get("omega"), mask), wl.dtype)
    else:
        err = rel_err(y, ref)
        assert err < TOL[wl.dtype], err


def test_cross_same_length_equals_noncausal():
    # N_q == N_k without a mask runs the same launches as the non-causal form
    wl = si.workload(2)
    inp = si.make_inputs(wl, B=2, H=4, N=1500)
    q, k, v = (to_dev(inp, n, "bf16") for n in ("q", "k", "v"))
    y1 = torch.empty(2, 4, 1500, 64, dtype=torch.bfloat16, device=DEV)
    y2 = torch.empty_like(y1)
    la.la_forward_cross(q, k, v, y1)
    la.la_forward_noncausal(q, k, v, y2)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_cross_mask_equals_dropped_keys():
    # a padding mask gives the result of the kept keys alone (to rounding)
    wl = si.workload(1)
    inp = si.make_inputs(wl, B=1, H=2, N=90)
    kv = si.make_kv(wl, 300, B=1, H=2)
    mask = si.make_key_padding_mask(1, 300, "random", seed=9, p=0.5)
    keep = ~mask[0]
    q = to_dev(inp, "q", "f32")
    k, v = to_dev(kv, "k", "f32"), to_dev(kv, "v", "f32")
    y1 = torch.empty(1, 2, 90, 64, device=DEV)
    y2 = torch.empty_like(y1)
    la.la_forward_cross(q, k, v, y1, _dev_mask(mask))
    kk = torch.from_numpy(np.ascontiguousarray(kv["k"][:, :, keep])).to(DEV)
    vv = torch.from_numpy(np.ascontiguousarray(kv["v"][:, :, keep])).to(DEV)
    la.la_forward_cross(q, kk, vv, y2)
    torch.cuda.synchronize()
    err = oracle.rowwise_rel_err(y1.cpu().numpy(), y2.cpu().numpy().astype(np.float64))
    assert err < TOL["f32"], err


# ------------------------------------------------------------- masked causal forward
MASKED = [
    # workload, overrides, B, H, N, mask kind, initial state
    (2, {}, 2, 4, 1000, "right", False),
    (2, {}, 2, 4, 777, "random", True),
    (2, {}, 1, 2, 8200, "random", True),      # many segments: mask across the scan
    (3, {}, 2, 3, 600, "right", True),        # d = 128, per-head decay
    (1, {}, 2, 2, 300, "random", False),      # fp32
    (1, {"phi": "relu"}, 1, 2, 257, "random", True),
    (5, {"m": 64}, 1, 4, 700, "random", False),
    (5, {"m": 128}, 1, 2, 1500, "random", True),   # F = 256: features in the output kernel
    (5, {"m": 256}, 1, 2, 900, "right", True),     # two halves of 128 directions
]


def _state_in(wl, B, H, seed):
    rng = np.random.default_rng(seed)
    F = wl.F
    S0 = rng.standard_normal((B, H, F, wl.dv)).astype(np.float32) * 0.1
    z0 = (rng.random((B, H, F)).astype(np.float32) + 0.5) if not wl.random_features else \
        rng.standard_normal((B, H, F)).astype(np.float32) * 0.01
    return S0, z0


@pytest.mark.parametrize("wi,over,B,H,N,kind,with_state", MASKED)
def test_causal_masked_parity(wi, over, B, H, N, kind, with_state):
    wl = si.workload(wi).with_(**over)
    inp = si.make_inputs(wl, B=B, H=H, N=N)
    lam = [0.9 + 0.1 * h / max(1, H - 1) for h in range(H)]  # decay from 0.9 to 1.0 over the heads
    mask = si.make_key_padding_mask(B, N, kind, seed=wi + N)
    q, k, v = (to_dev(inp, n, wl.dtype) for n in ("q", "k", "v"))
    F = wl.F
    S0 = z0 = S_in = z_in = None
    if with_state:
        S0, z0 = _state_in(wl, B, H, wi)
        S_in, z_in = torch.from_numpy(S0).to(DEV), torch.from_numpy(z0).to(DEV)
    y = torch.full((B, H, N, wl.dv), float("nan"), dtype=tdtype(wl.dtype), device=DEV)
    S = torch.full((B, H, F, wl.dv), float("nan"), device=DEV)
    z = torch.full((B, H, F), float("nan"), device=DEV)
    la.la_forward_causal_masked(q, k, v, y, _dev_mask(mask), phi=phi_for(wl, inp.get("omega")), lambda_h=lam,
                                eps=wl.eps, S_in=S_in, z_in=z_in, S_out=S, z_out=z)
    torch.cuda.synchronize()
    ref, Sr, zr, kap = oracle.causal(inp["q"], inp["k"], inp["v"], lam, wl.eps, wl.phi, inp.get("omega"),
                                     wl.qk_scale, S0=S0, z0=z0, want_state=True, want_kappa=True,
                                     key_padding_mask=mask)
    if wl.random_features:
        _check_rows(y, ref, kap, wl.dtype)
    else:
        err = rel_err(y, ref)
        assert err < TOL[wl.dtype], err
    tol = TOL[wl.dtype]
    np.testing.assert_allclose(S.cpu().numpy(), Sr, rtol=tol, atol=tol * np.abs(Sr).max())
    np.testing.assert_allclose(z.cpu().numpy(), zr, rtol=tol, atol=tol * np.abs(zr).max())


@pytest.mark.parametrize("wi,over,kind", [(3, {}, "random"), (5, {"m": 64}, "random"),
                                         (2, {"phi": "relu", "dk": 128, "dv": 128}, "right")])
def test_causal_masked_multichunk_segments(wi, over, kind, monkeypatch):
    # three segments of several 64-token chunks each and no final state asked
    # for, so the segment-state pass leaves out each row's last segment
    monkeypatch.setenv("LA_SEGMENTS", "3")
    wl = si.workload(wi).with_(**over)
    B, H, N = 2, 2, 1500
    inp = si.make_inputs(wl, B=B, H=H, N=N)
    lam = [0.95, 1.0]
    mask = si.make_key_padding_mask(B, N, kind, seed=wi + N + 1)
    q, k, v = (to_dev(inp, n, wl.dtype) for n in ("q", "k", "v"))
    y = torch.full((B, H, N, wl.dv), float("nan"), dtype=tdtype(wl.dtype), device=DEV)
    la.la_forward_causal_masked(q, k, v, y, _dev_mask(mask), phi=phi_for(wl, inp.get("omega")), lambda_h=lam,
                                eps=wl.eps)
    torch.cuda.synchronize()
    ref, kap = oracle.causal(inp["q"], inp["k"], inp["v"], lam, wl.eps, wl.phi, inp.get("omega"), wl.qk_scale,
                             want_kappa=True, key_padding_mask=mask)
    if wl.random_features:
        _check_rows(y, ref, kap, wl.dtype)
    else:
        err = rel_err(y, ref)
        assert err < TOL[wl.dtype], err


def test_causal_mask_all_padded_and_none():
    wl = si.workload(2)
    B, H, N = 2, 2, 300
    inp = si.make_inputs(wl, B=B, H=H, N=N)
    q, k, v = (to_dev(inp, n, "bf16") for n in ("q", "k", "v"))
    lam = [0.95, 1.0]
    y = torch.empty(B, H, N, 64, dtype=torch.bfloat16, device=DEV)
    S = torch.empty(B, H, 64, 64, device=DEV)
    z = torch.empty(B, H, 64, device=DEV)
    # every key padded from a zero state: nothing enters, outputs and state are 0
    la.la_forward_causal_masked(q, k, v, y, _dev_mask(si.make_key_padding_mask(B, N, "all")), lambda_h=lam,
                                S_out=S, z_out=z)
    torch.cuda.synchronize()
    assert float(y.float().abs().max()) == 0.0
    assert float(S.abs().max()) == 0.0 and float(z.abs().max()) == 0.0
    # no key padded: the same bits as the unmasked forward
    y2 = torch.empty_like(y)
    la.la_forward_causal_masked(q, k, v, y, _dev_mask(si.make_key_padding_mask(B, N, "none")), lambda_h=lam)
    la.la_forward_causal(q, k, v, y2, lambda_h=lam)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)


# ------------------------------------------------------ packed variable-length causal
VARLEN = [
    # workload, overrides, H, lengths (n_seq, max_len, empty), max_seqlen hint, initial state
    (2, {}, 4, (12, 900, 2), "exact", False),
    (2, {}, 2, (5, 9000, 1), "exact", True),     # long sequences: many segments each
    (2, {}, 2, (7, 3000, 0), "zero", True),      # hint 0: one segment per sequence
    (2, {}, 2, (5, 9000, 0), "half", False),     # understated hint: the last segment takes the rest
    (2, {}, 4, (64, 2000, 8), "exact", True),    # many sequences, several empty
    (3, {}, 3, (6, 700, 1), "exact", True),      # d = 128, per-head decay
    (1, {}, 2, (9, 300, 2), "exact", False),     # fp32
    (5, {"m": 64}, 2, (6, 1200, 1), "exact", False),
    (5, {"m": 256}, 2, (5, 1500, 1), "exact", True),
]


@pytest.mark.parametrize("wi,over,H,lens,hint,with_state", VARLEN)
def test_causal_varlen_parity(wi, over, H, lens, hint, with_state):
    wl = si.workload(wi).with_(**over)
    n_seq, max_len, empty = lens
    L = si.make_varlen_lengths(n_seq, max_len, seed=wi + max_len, empty=empty)
    cu = si.cu_seqlens(L)
    T = int(cu[-1]) + 5  # a few tokens after the last sequence belong to none
    inp = si.pack_heads(wl, T, H=H)
    if wl.random_features:
        inp["omega"] = si.make_omega(wl.m, wl.dk, wl.index, orthogonal=wl.omega == "orthogonal")
    lam = [0.9 + 0.099 * h / max(1, H - 1) for h in range(H)]
    q, k, v = (to_dev(inp, n, wl.dtype)[0].contiguous() for n in ("q", "k", "v"))
    F = wl.F
    S0 = z0 = S_in = z_in = None
    if with_state:
        S0, z0 = _state_in(wl, n_seq, H, wi + 1)
        S_in, z_in = torch.from_numpy(S0).to(DEV), torch.from_numpy(z0).to(DEV)
    y = torch.full((H, T, wl.dv), float("nan"), dtype=tdtype(wl.dtype), device=DEV)
    S = torch.full((n_seq, H, F, wl.dv), float("nan"), device=DEV)
    z = torch.full((n_seq, H, F), float("nan"), device=DEV)
    mx = {"exact": int(L.max()), "half": int(L.max()) // 2, "zero": 0}[hint]
    la.la_forward_causal_varlen(q, k, v, y, torch.from_numpy(cu).to(DEV), mx, phi=phi_for(wl, inp.get("omega")),
                                lambda_h=lam, eps=wl.eps, S_in=S_in, z_in=z_in, S_out=S, z_out=z)
    torch.cuda.synchronize()
    ref, Sr, zr = oracle.causal_varlen(inp["q"], inp["k"], inp["v"], cu, lam, wl.eps, wl.phi, inp.get("omega"),
                                       wl.qk_scale, S0=S0, z0=z0)
    yv = y[:, :cu[-1]].float().cpu().numpy()[None]
    # rows after the last sequence are never written
    assert bool(torch.isnan(y[:, cu[-1]:].float()).all())
    if wl.random_features:
        kap = np.concatenate([oracle.causal(inp["q"][:, :, a:b], inp["k"][:, :, a:b], inp["v"][:, :, a:b], lam,
                                            wl.eps, wl.phi, inp["omega"], wl.qk_scale, want_kappa=True)[1]
                              for a, b in zip(cu[:-1], cu[1:]) if b > a], axis=2)
        _check_rows(yv, ref[:, :, :cu[-1]], kap, wl.dtype)
    else:
        err = rel_err(yv, ref[:, :, :cu[-1]])
        assert err < TOL[wl.dtype], err
    tol = TOL[wl.dtype]
    np.testing.assert_allclose(S.cpu().numpy(), Sr, rtol=tol, atol=tol * np.abs(Sr).max())
    np.testing.assert_allclose(z.cpu().numpy(), zr, rtol=tol, atol=tol * np.abs(zr).max())


# ------------------------------------------- the benchmarked configurations, full size
def test_full_size_masked_headline_shape():
    # B=4 H=8 N=4096 d=64 bf16 with a right-padded batch, the benchmark's launch plan
    wl = si.workload(2)
    inp = si.make_inputs(wl)
    mask = si.make_key_padding_mask(wl.B, wl.N, "right", seed=2)
    q, k, v = (to_dev(inp, n, "bf16") for n in ("q", "k", "v"))
    y = torch.empty(wl.B, wl.H, wl.N, wl.dv, dtype=torch.bfloat16, device=DEV)
    la.la_forward_causal_masked(q, k, v, y, _dev_mask(mask), eps=wl.eps)
    torch.cuda.synchronize()
    ref = oracle.causal(inp["q"], inp["k"], inp["v"], None, wl.eps, key_padding_mask=mask)
    err = rel_err(y, ref)
    assert err < TOL["bf16"], err


def test_full_size_varlen_32_sequences():
    # 32 packed sequences (log-uniform lengths up to 4096), 8 heads, d = 64
    wl = si.workload(2)
    L = si.make_varlen_lengths(32, 4096, seed=2)
    cu = si.cu_seqlens(L)
    T = int(cu[-1])
    inp = si.pack_heads(wl, T, H=8)
    q, k, v = (to_dev(inp, n, "bf16")[0].contiguous() for n in ("q", "k", "v"))
    y = torch.empty(8, T, 64, dtype=torch.bfloat16, device=DEV)
    S = torch.empty(32, 8, 64, 64, device=DEV)
    z = torch.empty(32, 8, 64, device=DEV)
    la.la_forward_causal_varlen(q, k, v, y, torch.from_numpy(cu).to(DEV), int(L.max()), eps=wl.eps,
                                S_out=S, z_out=z)
    torch.cuda.synchronize()
    ref, Sr, zr = oracle.causal_varlen(inp["q"], inp["k"], inp["v"], cu, None, wl.eps)
    err = rel_err(y[None], ref)
    assert err < TOL["bf16"], err
    np.testing.assert_allclose(z.cpu().numpy(), zr, rtol=TOL["bf16"])


def test_full_size_cross_1024_by_4096():
    # B=4 H=8, 1024 queries against 4096 right-padded keys, d = 64
    wl = si.workload(2)
    inp = si.make_inputs(wl, N=1024)
    kv = si.make_kv(wl, 4096)
    mask = si.make_key_padding_mask(wl.B, 4096, "right", seed=2)
    q = to_dev(inp, "q", "bf16")
    k, v = to_dev(kv, "k", "bf16"), to_dev(kv, "v", "bf16")
    y = torch.empty(wl.B, wl.H, 1024, 64, dtype=torch.bfloat16, device=DEV)
    la.la_forward_cross(q, k, v, y, _dev_mask(mask), eps=wl.eps)
    torch.cuda.synchronize()
    ref = oracle.cross(inp["q"], kv["k"], kv["v"], wl.eps, key_padding_mask=mask)
    err = rel_err(y, ref)
    assert err < TOL["bf16"], err
