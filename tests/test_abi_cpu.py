"""The C-ABI library on the host: it loads, exports every declared symbol, and
rejects malformed calls during host-side validation (nothing is enqueued, so
no GPU is needed)."""
import ctypes
import os
import re

import pytest

import weight_sequence_mixing_amd as la
from weight_sequence_mixing_amd.binding import LaPhiC, LaShapeC

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation fails first


@pytest.fixture(scope="module")
def lib():
    return la.load_library()


def _declared():
    with open(os.path.join(ROOT, "include", "la.h")) as fh:
        text = fh.read()
    return sorted(set(re.findall(r"^\s*(?:la_status|size_t|const char\*)\s+(la_\w+)\s*\(", text, re.M)))


def test_profile_hooks_host_side(lib):
    # ending without a begin is rejected on the host (creating events needs a GPU)
    with pytest.raises(la.LaError):
        la.la_profile_end()
    with pytest.raises(la.LaError):
        la.la_profile_begin(0)
    assert la.la_kernel_name(1) == "causal output pass"
    assert la.la_kernel_name(4) == "la_decode_kernel"


def test_header_declarations_are_exported(lib):
    names = _declared()
    assert set(names) == set(la.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code, name in enumerate(["LA_OK", "LA_ERR_INVALID_ARGUMENT", "LA_ERR_UNSUPPORTED",
                                 "LA_ERR_WORKSPACE", "LA_ERR_HIP"]):
        assert la.la_status_string(code) == name


def _shape(B=1, H=2, N=64, dk=64, dv=64, it=la.LA_BF16, ot=None):
    return LaShapeC(B, H, N, dk, dv, it, it if ot is None else ot)


ELU = LaPhiC(la.LA_PHI_ELU1, 0, None, 1.0)


GAP = 1 << 32


def _causal(lib, shape, phi=ELU, lam=None, eps=1e-6, q=FAKE, k=FAKE + GAP, v=FAKE + 2 * GAP,
            y=FAKE + 3 * GAP, S_in=None, z_in=None, S_out=None, z_out=None, ws=None, ws_bytes=0):
    lam_arr = None
    if lam is not None:
        lam_arr = (ctypes.c_float * len(lam))(*lam)
    return lib.la_forward_causal(q, k, v, y, ctypes.byref(shape), ctypes.byref(phi),
                                 ctypes.cast(lam_arr, ctypes.c_void_p) if lam_arr else None, eps,
                                 S_in, z_in, S_out, z_out, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(shape=_shape(dk=96)), la.binding.LA_ERR_UNSUPPORTED),
    (dict(shape=_shape(dv=32)), la.binding.LA_ERR_UNSUPPORTED),
    (dict(shape=_shape(B=0)), la.binding.LA_ERR_INVALID_ARGUMENT),
    (dict(shape=_shape(N=-1)), la.binding.LA_ERR_INVALID_ARGUMENT),
    (dict(shape=_shape(H=300)), la.binding.LA_ERR_UNSUPPORTED),
    (dict(shape=_shape(it=7)), la.binding.LA_ERR_INVALID_ARGUMENT),
    (dict(shape=_shape(it=la.LA_F32, ot=la.LA_BF16)), la.binding.LA_ERR_UNSUPPORTED),
    (dict(shape=_shape(), lam=[1.5, 1.0]), la.binding.LA_ERR_INVALID_ARGUMENT),
    (dict(shape=_shape(), lam=[-0.1, 1.0]), la.binding.LA_ERR_INVALID_ARGUMENT),
    (dict(shape=_shape(), lam=[float("nan"), 1.0]), la.binding.LA_ERR_INVALID_ARGUMENT),
    (dict(shape=_shape(), eps=-1.0), la.binding.LA_ERR_INVALID_ARGUMENT),
    (dict(shape=_shape(), eps=float("inf")), la.binding.LA_ERR_INVALID_ARGUMENT),
    (dict(shape=_shape(), S_in=FAKE), la.binding.LA_ERR_INVALID_ARGUMENT),
    (dict(shape=_shape(), S_out=FAKE, z_out=None), la.binding.LA_ERR_INVALID_ARGUMENT),
    (dict(shape=_shape(), q=None), la.binding.LA_ERR_INVALID_ARGUMENT),
    (dict(shape=_shape(), q=FAKE + 8), la.binding.LA_ERR_INVALID_ARGUMENT),
    (dict(shape=_shape(), y=FAKE), la.binding.LA_ERR_INVALID_ARGUMENT),          # y aliases q
    (dict(shape=_shape(), phi=LaPhiC(la.LA_PHI_ELU1, 4, None, 1.0)), la.binding.LA_ERR_INVALID_ARGUMENT),
    (dict(shape=_shape(), phi=LaPhiC(la.LA_PHI_TRIG_RF, 64, None, 0.35)), la.binding.LA_ERR_INVALID_ARGUMENT),
    (dict(shape=_shape(), phi=LaPhiC(la.LA_PHI_TRIG_RF, 48, FAKE, 0.35)), la.binding.LA_ERR_UNSUPPORTED),
    (dict(shape=_shape(dk=128), phi=LaPhiC(la.LA_PHI_TRIG_RF, 128, FAKE, 0.35)), la.binding.LA_ERR_UNSUPPORTED),
    (dict(shape=_shape(), phi=LaPhiC(9, 0, None, 1.0)), la.binding.LA_ERR_INVALID_ARGUMENT),
    (dict(shape=_shape(), phi=LaPhiC(la.LA_PHI_RELU, 4, None, 1.0)), la.binding.LA_ERR_INVALID_ARGUMENT),
    (dict(shape=_shape(), phi=LaPhiC(la.LA_PHI_RELU, 0, None, 0.5)), la.binding.LA_ERR_INVALID_ARGUMENT),
    (dict(shape=_shape(), phi=LaPhiC(la.LA_PHI_TRIG_RF_SOFTMAX, 64, None, 0.35)), la.binding.LA_ERR_INVALID_ARGUMENT),
    (dict(shape=_shape(), phi=LaPhiC(la.LA_PHI_TRIG_RF_PLAIN, 48, FAKE, 0.35)), la.binding.LA_ERR_UNSUPPORTED),
    (dict(shape=_shape(), phi=LaPhiC(la.LA_PHI_TRIG_RF_PLAIN, 64, FAKE, 0.0)), la.binding.LA_ERR_INVALID_ARGUMENT),
    (dict(shape=_shape(B=4, H=8, N=4096)), la.binding.LA_ERR_WORKSPACE),        # needs a workspace
    (dict(shape=_shape(B=4, H=8, N=4096), ws=FAKE + 5 * (1 << 32), ws_bytes=16), la.binding.LA_ERR_WORKSPACE),
])
def test_causal_validation(lib, kw, status):
    st = _causal(lib, **kw)
    assert st == status, (st, la.la_last_error())
    assert la.la_last_error()


def test_workspace_size_queries(lib):
    s = _shape(B=4, H=8, N=4096)
    assert lib.la_workspace_size(ctypes.byref(s), ctypes.byref(ELU), 1) > 0
    assert lib.la_workspace_size(ctypes.byref(s), ctypes.byref(ELU), 0) > 0
    bad = _shape(dk=96)
    assert lib.la_workspace_size(ctypes.byref(bad), ctypes.byref(ELU), 1) == 0
    # a long single head splits into segments: the workspace holds their states
    one = _shape(B=1, H=1, N=1 << 16, dk=128, dv=128)
    ws = lib.la_workspace_size(ctypes.byref(one), ctypes.byref(ELU), 1)
    assert ws >= 2 * (128 * 128 + 128) * 4


def test_noncausal_and_decode_validation(lib):
    s = _shape(N=0)
    st = lib.la_forward_noncausal(FAKE, FAKE + 0x100000, FAKE + 0x200000, FAKE + 0x300000, ctypes.byref(s),
                                  ctypes.byref(ELU), 1e-6, None, 0, None)
    assert st == la.binding.LA_ERR_INVALID_ARGUMENT
    for n in (0, la.binding.LA_DECODE_MAX_TOKENS + 1):  # tokens per call outside [1, 64]
        s = _shape(N=n)
        st = lib.la_decode_step(FAKE, FAKE + 0x100000, FAKE + 0x200000, FAKE + 0x300000, FAKE + 0x400000,
                                FAKE + 0x500000, ctypes.byref(s), ctypes.byref(ELU), None, 1e-6, None)
        assert st == la.binding.LA_ERR_INVALID_ARGUMENT
    s = _shape(N=1)
    st = lib.la_decode_step(FAKE, FAKE + 0x100000, FAKE + 0x200000, FAKE + 0x300000, None,
                            FAKE + 0x500000, ctypes.byref(s), ctypes.byref(ELU), None, 1e-6, None)
    assert st == la.binding.LA_ERR_INVALID_ARGUMENT
    st = lib.la_init_state(FAKE, FAKE, 0, 1, 64, 64, None)
    assert st == la.binding.LA_ERR_INVALID_ARGUMENT


def test_masked_cross_varlen_validation(lib):
    """Argument errors of the mask, cross-attention and packed entry points are
    caught on the host (no launch)."""
    E = la.binding.LA_ERR_INVALID_ARGUMENT
    s = _shape()
    q, k, v, y = FAKE, FAKE + 0x100000, FAKE + 0x200000, FAKE + 0x300000
    # masked causal without a mask
    st = lib.la_forward_causal_masked(q, k, v, y, ctypes.byref(s), ctypes.byref(ELU), None, 1e-6, None,
                                      None, None, None, None, None, 0, None)
    assert st == E and "key_padding_mask" in la.la_last_error()
    # cross: no keys; y overlapping the (longer) key rows
    st = lib.la_forward_cross(q, k, v, y, ctypes.byref(s), 0, None, ctypes.byref(ELU), 1e-6, None, 0, None)
    assert st == E and "n_kv" in la.la_last_error()
    st = lib.la_forward_cross(q, k, v, k + 64 * 64 * 2 * 2 * 4, ctypes.byref(s), 1024, None, ctypes.byref(ELU),
                              1e-6, None, 0, None)
    assert st == E and "alias" in la.la_last_error()
    # packed sequences: no offsets, misaligned offsets, max_seqlen beyond T
    sv = _shape(B=3, H=2, N=100)
    for cu, mx in ((None, 50), (FAKE + 2, 50), (FAKE, 101), (FAKE, -1)):
        st = lib.la_forward_causal_varlen(q, k, v, y, cu, mx, ctypes.byref(sv), ctypes.byref(ELU), None, 1e-6,
                                          None, None, None, None, None, 0, None)
        assert st == E, (cu, mx, st)
    # y overlapping q's H x T rows
    st = lib.la_forward_causal_varlen(q, k, v, q + 2 * 100 * 64, FAKE, 50, ctypes.byref(sv), ctypes.byref(ELU),
                                      None, 1e-6, None, None, None, None, None, 0, None)
    assert st == E and "alias" in la.la_last_error()


def test_cross_and_varlen_workspace_queries(lib):
    s = _shape(B=1, H=1, N=64, dk=128, dv=128)
    # sized by the key count, not the query count
    small = lib.la_workspace_size_cross(ctypes.byref(s), 64, ctypes.byref(ELU))
    big = lib.la_workspace_size_cross(ctypes.byref(s), 1 << 16, ctypes.byref(ELU))
    assert big >= 2 * (128 * 128 + 128) * 4 and big > small
    assert lib.la_workspace_size_cross(ctypes.byref(s), 0, ctypes.byref(ELU)) == 0
    # packed: sized by the longest sequence; many head-sequences need no segments
    sv = _shape(B=2, H=1, N=1 << 16, dk=128, dv=128)
    assert lib.la_workspace_size_varlen(ctypes.byref(sv), 1 << 15, ctypes.byref(ELU)) >= 2 * (128 * 128 + 128) * 4
    assert lib.la_workspace_size_varlen(ctypes.byref(sv), (1 << 16) + 1, ctypes.byref(ELU)) == 0
    # many head-sequences: one segment each, so only the table of work items
    # (one int32 per sequence) remains
    wide = _shape(B=64, H=16, N=1 << 16)
    assert 64 * 4 <= lib.la_workspace_size_varlen(ctypes.byref(wide), 1024, ctypes.byref(ELU)) <= 1024


def test_backward_validation(lib):
    """Argument errors of la_backward_causal are caught on the host (no launch)."""
    E, U = la.binding.LA_ERR_INVALID_ARGUMENT, la.binding.LA_ERR_UNSUPPORTED
    s = _shape()
    P = [FAKE + i * 0x100000 for i in range(8)]  # q k v y dy dq dk dv

    def call(shape=s, phi=ELU, ptrs=P, S_in=None, z_in=None, dS_out=None, dz_out=None, dS_in=None,
             dz_in=None, dlam=None, ws=None, ws_bytes=0):
        return lib.la_backward_causal(*ptrs, ctypes.byref(shape), ctypes.byref(phi), None, 1e-6, None, S_in, z_in,
                                      dS_out, dz_out, dS_in, dz_in, dlam, ws, ws_bytes, None)

    RF = LaPhiC(la.LA_PHI_TRIG_RF, 64, FAKE, 0.35)
    assert call(phi=RF) == la.binding.LA_ERR_WORKSPACE                       # random features: supported
    assert call(shape=_shape(it=la.LA_F32, ot=la.LA_F32), phi=LaPhiC(la.LA_PHI_TRIG_RF, 128, FAKE, 0.35)) == U
    assert call(shape=_shape(ot=la.LA_F32)) == U                             # y in another type
    assert call(S_in=FAKE) == E                                              # S_in without z_in
    assert call(dS_in=FAKE) == E
    assert call(ptrs=P[:5] + [P[0]] + P[6:]) == E                           # dq aliases q
    assert call(ptrs=P[:6] + [P[5]] + P[7:]) == E                           # dk overlaps dq
    assert call() == la.binding.LA_ERR_WORKSPACE                            # no workspace
    big = _shape(it=la.LA_F32, dk=128, dv=128)
    assert call(shape=big, dlam=FAKE) == U                                   # no lambda gradient for fp32 d=128
    n = lib.la_workspace_size_backward(ctypes.byref(s), ctypes.byref(ELU))
    assert n >= 2 * 4 * s.B * s.H * s.N                                      # 8 bytes per token at least
    # random features add phi(q), phi(k), d phi(q), d phi(k) (input type, bf16
    # here) for every token: F = 2m = 128 values each
    nrf = lib.la_workspace_size_backward(ctypes.byref(s), ctypes.byref(RF))
    rows = s.B * s.H * s.N
    assert nrf >= n + rows * 128 * (2 + 2 + 2 + 2)
    ws_rf = FAKE
    assert call(phi=RF, ws=ws_rf, ws_bytes=nrf - 1) == la.binding.LA_ERR_WORKSPACE


def test_cross_backward_validation(lib):
    """Argument errors of la_backward_cross are caught on the host (no launch)."""
    E, U, W = la.binding.LA_ERR_INVALID_ARGUMENT, la.binding.LA_ERR_UNSUPPORTED, la.binding.LA_ERR_WORKSPACE
    s = _shape(N=64)
    P = [FAKE + i * 0x100000 for i in range(8)]  # q k v y dy dq dk dv
    RF = LaPhiC(la.LA_PHI_TRIG_RF, 64, FAKE, 0.35)

    def call(shape=s, n_kv=100, phi=ELU, ptrs=P, eps=1e-6, ws=None, ws_bytes=0):
        return lib.la_backward_cross(*ptrs, ctypes.byref(shape), n_kv, None, ctypes.byref(phi), eps, ws, ws_bytes,
                                     None)

    assert call(phi=RF) == W                                    # random features: supported
    assert call(shape=_shape(ot=la.LA_F32)) == U                # y in another type
    assert call(shape=_shape(N=0)) == E                         # no queries
    assert call(n_kv=0) == E                                    # no keys
    assert call(eps=-1.0) == E
    assert call(ptrs=P[:5] + [P[0]] + P[6:]) == E              # dq aliases q
    assert call(ptrs=P[:6] + [P[5] + 64] + P[7:]) == E         # dk overlaps dq
    # dv runs over n_kv rows: with 4096 keys it reaches into the next buffer (dy)
    assert call(n_kv=4096, ptrs=P[:7] + [P[4] - 0x40000]) == E
    assert call() == W                                          # no workspace
    n = lib.la_workspace_size_backward_cross(ctypes.byref(s), 100, ctypes.byref(ELU))
    assert n > 0 and call(ws=FAKE, ws_bytes=n - 1) == W
    # random features add phi and d phi of the 64 queries and 100 keys (F = 128)
    nrf = lib.la_workspace_size_backward_cross(ctypes.byref(s), 100, ctypes.byref(RF))
    assert nrf >= s.B * s.H * (64 + 100) * 128 * (2 + 4)
    assert call(phi=RF, ws=FAKE, ws_bytes=nrf - 1) == W
    assert lib.la_workspace_size_backward_cross(ctypes.byref(s), 0, ctypes.byref(ELU)) == 0
    assert lib.la_workspace_size_backward_cross(ctypes.byref(_shape(N=0)), 100, ctypes.byref(ELU)) == 0
    # segment states for the keys' and the queries' splits: grows with both lengths
    big_k = lib.la_workspace_size_backward_cross(ctypes.byref(s), 1 << 16, ctypes.byref(ELU))
    big_q = lib.la_workspace_size_backward_cross(ctypes.byref(_shape(N=1 << 16)), 100, ctypes.byref(ELU))
    assert big_k > n and big_q > n


def test_noalloc_forward_host_validation(lib, monkeypatch):
    """The static-scratch forward validates like la_forward_causal, and a
    window carry larger than its scratch is refused on the host."""
    def call(shape, lam=None, eps=1e-6):
        lam_arr = (ctypes.c_float * len(lam))(*lam) if lam else None
        return lib.la_forward_causal_noalloc(FAKE, FAKE + GAP, FAKE + 2 * GAP, FAKE + 3 * GAP, ctypes.byref(shape),
                                             ctypes.byref(ELU), ctypes.cast(lam_arr, ctypes.c_void_p) if lam else None,
                                             eps, None, None, None, None, None)
    assert call(_shape(dk=96)) == la.binding.LA_ERR_UNSUPPORTED
    assert call(_shape(), lam=[1.5, 1.0]) == la.binding.LA_ERR_INVALID_ARGUMENT
    assert call(_shape(), eps=float("nan")) == la.binding.LA_ERR_INVALID_ARGUMENT
    # 1024 heads of a 128 x 129 fp32 state: one carry slot is 67.6 MB > 64 MiB
    monkeypatch.setenv("LA_WINDOWS", "2")
    st = call(_shape(B=4, H=256, N=256, dk=128, dv=128))
    assert st == la.binding.LA_ERR_WORKSPACE, la.la_last_error()
    assert "static scratch" in la.la_last_error()


def test_random_features_m256_scope(lib):
    """m = 256 (F = 512) runs the causal forward as two halves of 256 features:
    its workspace holds one half's segment states plus one float per output
    element and per row for the numerators and denominators handed from the
    first half to the second.  Every other entry point, and fp32 inputs or
    heads other than d_k = d_v = 64, refuse it on the host."""
    rf256 = LaPhiC(la.LA_PHI_TRIG_RF, 256, FAKE, 0.125)
    rf128 = LaPhiC(la.LA_PHI_TRIG_RF, 128, FAKE, 0.125)
    s = _shape(B=1, H=2, N=4096)
    ws256 = lib.la_workspace_size(ctypes.byref(s), ctypes.byref(rf256), 1)
    ws128 = lib.la_workspace_size(ctypes.byref(s), ctypes.byref(rf128), 1)
    assert ws256 >= ws128 + 2 * 4096 * (64 + 1) * 4
    sv = _shape(B=2, H=2, N=4096)
    assert lib.la_workspace_size_varlen(ctypes.byref(sv), 2048, ctypes.byref(rf256)) >= 2 * 4096 * (64 + 1) * 4
    assert lib.la_workspace_size(ctypes.byref(s), ctypes.byref(rf256), 0) == 0          # non-causal
    assert lib.la_workspace_size(ctypes.byref(_shape(dk=128, dv=128)), ctypes.byref(rf256), 1) == 0
    assert lib.la_workspace_size(ctypes.byref(_shape(dv=128)), ctypes.byref(rf256), 1) == 0
    assert lib.la_workspace_size(ctypes.byref(_shape(it=la.LA_F32)), ctypes.byref(rf256), 1) == 0
    U = la.binding.LA_ERR_UNSUPPORTED
    s1 = _shape(N=1)
    st = lib.la_decode_step(FAKE, FAKE + 0x100000, FAKE + 0x200000, FAKE + 0x300000, FAKE + 0x400000,
                            FAKE + 0x500000, ctypes.byref(s1), ctypes.byref(rf256), None, 1e-6, None)
    assert st == U
    st = lib.la_forward_noncausal(FAKE, FAKE + 0x100000, FAKE + 0x200000, FAKE + 0x300000, ctypes.byref(s),
                                  ctypes.byref(rf256), 1e-6, None, 0, None)
    assert st == U
