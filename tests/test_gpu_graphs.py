"""HIP graph capture of the library's entry points.

Every call launches kernels only (state fills and copies included, no memset
nodes), so a sequence of calls can be recorded once on a stream and replayed.
Each test records a sequence into a graph, replays it several times with
eager work and synchronisations between the replays, and requires every
replay to reproduce the eager results bit for bit (the kernels are
deterministic: no atomics, fixed reduction orders)."""
import numpy as np
import pytest
import torch

import seeded_inputs as si
import weight_sequence_mixing_amd as la
from gpu_util import DEV, to_dev

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _ws(n):
    return torch.empty(max(int(n), 1), dtype=torch.uint8, device=DEV)


def _replay_and_compare(graph, outputs, eager, scramble):
    for rep in range(REPLAYS):
        scramble()  # overwrite the outputs eagerly, so a replay must rewrite them
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, t in outputs.items():
            assert torch.equal(t, eager[name]), (rep, name)
        # unrelated eager work between replays
        torch.randn(1 << 16, device=DEV).sum().item()


def test_graph_forward_decode_backward():
    wl = si.workload(2)
    B, H, N, d = 2, 4, 1000, 64
    inp = si.make_inputs(wl, B=B, H=H, N=N)
    q, k, v = (to_dev(inp, n, "bf16") for n in ("q", "k", "v"))
    lam = [0.9, 0.95, 0.99, 1.0]
    steps = si.make_decode_step(si.workload(4).with_(dk=d, dv=d), 0, B=B, H=H)
    sq, sk, sv = (torch.from_numpy(steps[n + "_bits"].view(np.int16)).view(torch.bfloat16).to(DEV)
                  for n in ("q", "k", "v"))
    g = torch.randn(B, H, N, d, device=DEV).to(torch.bfloat16)
    y = torch.empty(B, H, N, d, dtype=torch.bfloat16, device=DEV)
    S = torch.empty(B, H, d, d, device=DEV)
    z = torch.empty(B, H, d, device=DEV)
    yd = torch.empty(B, H, 1, d, dtype=torch.bfloat16, device=DEV)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dlam = torch.empty(H, device=DEV)
    wsf = _ws(la.la_workspace_size(B, H, N, d, d))
    wsb = _ws(la.la_workspace_size_backward(B, H, N, d, d))

    def run():
        la.la_init_state(S, z)
        la.la_forward_causal(q, k, v, y, lambda_h=lam, S_in=S, z_in=z, S_out=S, z_out=z, workspace=wsf)
        la.la_decode_step(sq, sk, sv, yd, S, z, lambda_h=lam)
        la.la_backward_causal(q, k, v, y, g, dq, dk, dv, lambda_h=lam, dlambda=dlam, workspace=wsb)

    run()
    torch.cuda.synchronize()
    outs = {"y": y, "S": S, "z": z, "yd": yd, "dq": dq, "dk": dk, "dv": dv, "dlam": dlam}
    eager = {n: t.clone() for n, t in outs.items()}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            run()
    torch.cuda.synchronize()

    def scramble():
        for t in outs.values():
            t.fill_(float("nan"))

    _replay_and_compare(graph, outs, eager, scramble)


def test_graph_varlen_and_cross():  # cross attention forward and backward
    wl = si.workload(2)
    H, d = 4, 64
    L = si.make_varlen_lengths(9, 700, seed=4, empty=1)
    cu = si.cu_seqlens(L)
    T = int(cu[-1])
    inp = si.pack_heads(wl, T, H=H)
    q, k, v = (to_dev(inp, n, "bf16")[0].contiguous() for n in ("q", "k", "v"))
    cu_t = torch.from_numpy(cu).to(DEV)
    y = torch.empty(H, T, d, dtype=torch.bfloat16, device=DEV)
    Sf = torch.empty(len(L), H, d, d, device=DEV)
    zf = torch.empty(len(L), H, d, device=DEV)
    mx = int(L.max())
    wsv = _ws(la.la_workspace_size_varlen(len(L), H, T, mx, d, d))
    # cross attention: 2 x 4 heads, 300 queries against 1200 right-padded keys
    B, Nq, Nk = 2, 300, 1200
    cq = to_dev(si.make_inputs(wl, B=B, H=H, N=Nq), "q", "bf16")
    kv = si.make_kv(wl, Nk, B=B, H=H)
    ck, cv = to_dev(kv, "k", "bf16"), to_dev(kv, "v", "bf16")
    mask = torch.from_numpy(si.make_key_padding_mask(B, Nk, "right", seed=4)).to(DEV)
    yc = torch.empty(B, H, Nq, d, dtype=torch.bfloat16, device=DEV)
    wsc = _ws(la.la_workspace_size_cross(B, H, Nq, Nk, d, d))
    gc = torch.randn(B, H, Nq, d, device=DEV).to(torch.bfloat16)
    dqc, dkc, dvc = torch.empty_like(cq), torch.empty_like(ck), torch.empty_like(cv)
    wscb = _ws(la.la_workspace_size_backward_cross(B, H, Nq, Nk, d, d))

    def run():
        la.la_forward_causal_varlen(q, k, v, y, cu_t, mx, lambda_h=[0.9, 0.95, 0.99, 1.0], S_out=Sf, z_out=zf,
                                    workspace=wsv)
        la.la_forward_cross(cq, ck, cv, yc, mask, workspace=wsc)
        la.la_backward_cross(cq, ck, cv, yc, gc, dqc, dkc, dvc, mask, workspace=wscb)

    y.fill_(0.0)  # rows after the last sequence are never written: same value in every run
    run()
    torch.cuda.synchronize()
    outs = {"y": y, "S": Sf, "z": zf, "yc": yc, "dqc": dqc, "dkc": dkc, "dvc": dvc}
    eager = {n: t.clone() for n, t in outs.items()}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            run()
    torch.cuda.synchronize()

    def scramble():
        y[:, :T].fill_(float("nan"))  # only the rows the call writes
        for t in (Sf, zf, yc, dqc, dkc, dvc):
            t.fill_(float("nan"))

    _replay_and_compare(graph, outs, eager, scramble)


def test_graph_random_feature_forward_and_backward():
    # m = 64 random features (F = 128), d = 64 bf16: forward, causal backward
    # with a padded batch (feature pass, identity-map sweeps, vector-Jacobian
    # products) and the cross backward
    from gpu_util import phi_for
    wl = si.workload(5).with_(m=64)
    B, H, N, d = 2, 2, 700, 64
    inp = si.make_inputs(wl, B=B, H=H, N=N)
    q, k, v = (to_dev(inp, n, "bf16") for n in ("q", "k", "v"))
    phi = phi_for(wl, inp["omega"])
    lam = [0.97, 1.0]
    mask = torch.from_numpy(si.make_key_padding_mask(B, N, "random", seed=6)).to(DEV)
    g = torch.randn(B, H, N, d, device=DEV).to(torch.bfloat16)
    y = torch.empty(B, H, N, d, dtype=torch.bfloat16, device=DEV)
    yc = torch.empty_like(y)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dqc, dkc, dvc = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    wsf = _ws(la.la_workspace_size(B, H, N, d, d, phi=phi))
    wsb = _ws(la.la_workspace_size_backward(B, H, N, d, d, phi=phi))
    wsc = _ws(la.la_workspace_size_cross(B, H, N, N, d, d, phi=phi))
    wscb = _ws(la.la_workspace_size_backward_cross(B, H, N, N, d, d, phi=phi))

    def run():
        la.la_forward_causal_masked(q, k, v, y, mask, phi=phi, lambda_h=lam, workspace=wsf)
        la.la_backward_causal(q, k, v, y, g, dq, dk, dv, phi=phi, lambda_h=lam, key_padding_mask=mask,
                              workspace=wsb)
        la.la_forward_cross(q, k, v, yc, mask, phi=phi, workspace=wsc)
        la.la_backward_cross(q, k, v, yc, g, dqc, dkc, dvc, mask, phi=phi, workspace=wscb)

    run()
    torch.cuda.synchronize()
    outs = {"y": y, "dq": dq, "dk": dk, "dv": dv, "yc": yc, "dqc": dqc, "dkc": dkc, "dvc": dvc}
    eager = {n: t.clone() for n, t in outs.items()}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            run()
    torch.cuda.synchronize()

    def scramble():
        for t in outs.values():
            t.fill_(float("nan"))

    _replay_and_compare(graph, outs, eager, scramble)
