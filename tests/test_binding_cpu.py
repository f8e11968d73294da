"""The Python binding rejects malformed tensor arguments before anything
reaches the library: wrong shapes, dtypes, lengths and devices raise
ValueError (a smaller k or S would otherwise let the kernels run past the
buffer).  CPU tensors only: every check runs before the device check, and the
device check itself is the last case."""
import pytest
import torch

import weight_sequence_mixing_amd as la

B, H, N, D = 2, 3, 40, 64


def t(*shape, dtype=torch.bfloat16):
    return torch.zeros(*shape, dtype=dtype)


def qkvy(dtype=torch.bfloat16):
    return t(B, H, N, D, dtype=dtype), t(B, H, N, D, dtype=dtype), t(B, H, N, D, dtype=dtype), t(B, H, N, D, dtype=dtype)


@pytest.fixture(scope="module", autouse=True)
def lib():
    return la.load_library()


def raises(match, fn, *a, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*a, **kw)


def test_forward_shapes_and_dtypes():
    q, k, v, y = qkvy()
    raises("k must have shape", la.la_forward_causal, q, t(B, H, N - 1, D), v, y)
    raises("v must have shape", la.la_forward_causal, q, k, t(B, H, N - 2, D), y)
    raises("v must be", la.la_forward_causal, q, k, v.float(), y)
    raises("y must have shape", la.la_forward_causal, q, k, v, t(B, H, N + 1, D))
    raises("q must be", la.la_forward_causal, t(B, H, D), k, v, y)
    raises("q must be", la.la_forward_causal, q.half(), k.half(), v.half(), y.half())
    raises("k must be", la.la_forward_noncausal, q, k.float(), v, y)


def test_state_arguments():
    q, k, v, y = qkvy()
    S, z = t(B, H, D, D, dtype=torch.float32), t(B, H, D, dtype=torch.float32)
    raises("S_out must have shape", la.la_forward_causal, q, k, v, y, S_out=t(B, H, D - 16, D, dtype=torch.float32),
           z_out=z)
    raises("z_in must have shape", la.la_forward_causal, q, k, v, y, S_in=S, z_in=t(B, H, D + 1, dtype=torch.float32))
    raises("S_in must be", la.la_forward_causal, q, k, v, y, S_in=S.bfloat16(), z_in=z)
    raises("given together", la.la_forward_causal, q, k, v, y, S_out=S)
    one = t(B, H, 1, D)
    raises("S must have shape", la.la_decode_step, one, one.clone(), one.clone(), one.clone(),
           t(B, H + 1, D, D, dtype=torch.float32), z)
    raises("S must be", la.la_init_state, t(B, H, D), z)
    raises("z must have shape", la.la_init_state, S, t(B, H, D + 4, dtype=torch.float32))


def test_lambda_length_must_equal_heads():
    q, k, v, y = qkvy()
    raises("one value per head", la.la_forward_causal, q, k, v, y, lambda_h=[0.9] * (H - 1))
    raises("one value per head", la.la_forward_causal, q, k, v, y, lambda_h=[0.9] * (H + 1))


def test_random_feature_directions():
    q, k, v, y = qkvy()
    raises("need omega", la.la_forward_causal, q, k, v, y, phi=la.Phi("trig_rf", None, 0.5))
    # omega must be [m, d_k]; a wrong d_k is caught before the device check
    raises(r"omega must be \[m, d_k=64\]", la.la_forward_causal, q, k, v, y,
           phi=la.Phi("trig_rf", torch.zeros(32, 128), 0.5))


def test_masks_and_packed_offsets():
    q, k, v, y = qkvy()
    raises("key_padding_mask must be", la.la_forward_causal_masked, q, k, v, y, torch.zeros(B, N + 1, dtype=torch.bool))
    raises("key_padding_mask must be bool", la.la_forward_causal_masked, q, k, v, y, torch.zeros(B, N))
    raises("key_padding_mask must be", la.la_forward_cross, q, k, v, y, torch.zeros(B + 1, N, dtype=torch.bool))
    raises("cu_seqlens must be", la.la_forward_causal_varlen, q[0], k[0], v[0], y[0],
           torch.tensor([0, 5, N], dtype=torch.int64), N)
    raises("v must have shape", la.la_forward_causal_varlen, q[0], k[0], v[0, :, :-1].contiguous(), y[0],
           torch.tensor([0, 5, N], dtype=torch.int32), N)


def test_cross_key_length():
    q, _, _, y = qkvy()
    k, v = t(B, H, 2 * N, D), t(B, H, 2 * N - 1, D)
    raises("v must have shape", la.la_forward_cross, q, k, v, y)


def test_backward_gradients():
    q, k, v, y = qkvy()
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    raises("dy must have shape", la.la_backward_causal, q, k, v, y, t(B, H, N - 1, D), dq, dk, dv)
    raises("dk must have shape", la.la_backward_causal, q, k, v, y, y, dq, t(B, H, N, 2 * D), dv)
    raises("dv must be", la.la_backward_causal, q, k, v, y, y, dq, dk, dv.float())
    raises("dlambda must have shape", la.la_backward_causal, q, k, v, y, y, dq, dk, dv,
           dlambda=torch.zeros(H + 1))
    raises("input type", la.la_backward_causal, q, k, v, y.float(), y.float(), dq, dk, dv)


def test_cpu_tensors_are_rejected_last():
    q, k, v, y = qkvy()
    raises("GPU device", la.la_forward_causal, q, k, v, y)
    one = t(B, H, 1, D)
    raises("GPU device", la.la_decode_step, one, one.clone(), one.clone(), one.clone(),
           t(B, H, D, D, dtype=torch.float32), t(B, H, D, dtype=torch.float32))


def test_package_exports_every_entry_point():
    for name in la.EXPORTS:
        if name.startswith("la_") and name not in ("la_status_string", "la_last_error"):
            assert hasattr(la, name), name
