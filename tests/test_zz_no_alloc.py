"""la_forward_causal_noalloc (the causal forward without a workspace: the
segment states live in the library's static device scratch) against
la_forward_causal with a workspace, through the C ABI.

Two calls in a row, the second on a smaller input: the scratch keeps the
first call's contents, and the second must not depend on them.  Where the
segment count is the same the two entry points run the same kernels on the
same plan, so the outputs and final states are bit for bit equal; both are
also held to the oracle.  With more segments forced than the scratch holds,
the static variant runs fewer segments: equal to the oracle within the bar.
"""
import numpy as np
import pytest
import torch

import weight_sequence_mixing_amd as la
from gpu_util import DEV, TOL, check_kappa_rows, inputs, oracle_causal, phi_for, rel_err, to_dev

pytestmark = pytest.mark.gpu


def _both(wl, inp):
    q, k, v = (to_dev(inp, n, wl.dtype) for n in ("q", "k", "v"))
    B, H, N, _ = q.shape
    lam = list(map(float, inp["lam"]))
    phi = phi_for(wl, inp.get("omega"))
    outs = []
    for fn in (la.la_forward_causal, la.la_forward_causal_noalloc):
        y = torch.full((B, H, N, wl.dv), float("nan"), dtype=torch.bfloat16, device=DEV)
        S = torch.full((B, H, wl.F, wl.dv), float("nan"), device=DEV)
        z = torch.full((B, H, wl.F), float("nan"), device=DEV)
        fn(q, k, v, y, phi=phi, lambda_h=lam, eps=wl.eps, S_out=S, z_out=z)
        torch.cuda.synchronize()
        outs.append((y, S, z))
    return outs


def test_noalloc_two_calls_match_workspace_entry_point():
    for over in (dict(B=2, H=16, N=4096), dict(B=1, H=3, N=777)):
        wl, inp = inputs(3, **over)
        (y0, S0, z0), (y1, S1, z1) = _both(wl, inp)
        print("B=%d H=%d N=%d: noalloc equal %s" % (over["B"], over["H"], over["N"], torch.equal(y0, y1)))
        assert torch.equal(y1, y0) and torch.equal(S1, S0) and torch.equal(z1, z0)
        ref = oracle_causal(wl, inp)
        assert rel_err(y1, ref) < TOL["bf16"]


def test_noalloc_caps_segments_to_its_scratch(monkeypatch):
    # 64 forced segments of 32 heads of 128 x 129 fp32 states need 135 MB:
    # the static variant runs the 31 that fit
    monkeypatch.setenv("LA_SEGMENTS", "64")
    wl, inp = inputs(3, B=2, H=16, N=8192)
    (y0, S0, z0), (y1, S1, z1) = _both(wl, inp)
    ref, Sr, zr = oracle_causal(wl, inp, want_state=True)
    e0, e1 = rel_err(y0, ref), rel_err(y1, ref)
    print("forced 64 segments: workspace %.2e, static scratch %.2e" % (e0, e1))
    assert e0 < TOL["bf16"] and e1 < TOL["bf16"]
    s_err = float((np.abs(S1.cpu().numpy() - Sr).max(axis=-1) / np.abs(Sr).max(axis=-1)).max())
    assert s_err < TOL["bf16"]


def test_noalloc_random_features():
    # m = 128 (features inside the output kernel) and m = 256 (the numerators
    # and denominators handed between halves sit in the static scratch too),
    # two calls in a row each, the second smaller
    for m in (128, 256):
        for over in (dict(B=1, H=4, N=3000), dict(B=1, H=2, N=555)):
            wl, inp = inputs(5, m=m, **over)
            (y0, S0, z0), (y1, S1, z1) = _both(wl, inp)
            assert torch.equal(y1, y0) and torch.equal(S1, S0) and torch.equal(z1, z0), (m, over)
            ref, kap = oracle_causal(wl, inp, want_kappa=True)
            check_kappa_rows(y1, ref, kap, "bf16")
