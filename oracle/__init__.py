"""fp64 CPU oracle for causal kernelized linear attention (fast-weight form).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
CPU-baseline leg of the benchmark.  The product path never imports it.

The arithmetic lives in ``la_oracle.c`` (plain C, double precision, one token
at a time).  This module compiles it with gcc, loads it with ctypes and splits
independent (batch, head) rows over a thread pool (ctypes releases the GIL
during the foreign call, so the C loops run in parallel).

All public functions take numpy arrays in the [B, H, N, d] layout (any float
dtype; values are widened exactly to float64) and return float64 arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "la_oracle.c")
_LIB = os.path.join(_HERE, "liborc.so")
PHI_KINDS = {"elu1": 0, "trig_rf": 1, "relu": 2, "trig_rf_plain": 3, "trig_rf_softmax": 4}
# feature maps with F = d_k (the others are random features with F = 2m)
ELEMENTWISE = ("elu1", "relu")

_lib = None


def build(force: bool = True) -> str:
    """Compile la_oracle.c into liborc.so (plain gcc, -O2, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # (re)build when the library is missing or older than its source
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build(force=True)
    lib = ctypes.CDLL(_LIB)
    P = ctypes.POINTER(ctypes.c_double)
    L, I, D = ctypes.c_long, ctypes.c_int, ctypes.c_double
    lib.orc_phi.argtypes = [I, P, I, I, P, D, P]
    lib.orc_phi.restype = None
    U = ctypes.POINTER(ctypes.c_ubyte)
    lib.orc_causal.argtypes = [P, P, P, L, L, I, I, I, I, P, D, P, D, U, P, P, P, P, P, P]
    lib.orc_causal.restype = None
    lib.orc_noncausal.argtypes = [P, P, P, L, L, I, I, I, I, P, D, D, P]
    lib.orc_noncausal.restype = None
    lib.orc_cross.argtypes = [P, P, P, L, L, L, I, I, I, I, P, D, D, U, P]
    lib.orc_cross.restype = None
    lib.orc_phi_vjp.argtypes = [I, P, I, I, P, D, P, P]
    lib.orc_phi_vjp.restype = None
    lib.orc_backward.argtypes = [P, P, P, P, L, L, I, I, I, I, P, D, P, D, U, P, P, P, P,
                                 P, P, P, P, P, P, P, P, P]
    lib.orc_backward.restype = None
    lib.orc_cross_backward.argtypes = [P, P, P, P, L, L, L, I, I, I, I, P, D, D, U, P, P, P, P, P, P]
    lib.orc_cross_backward.restype = None
    lib.orc_decode_step.argtypes = [P, P, P, L, I, I, I, I, P, D, P, D, P, P, P]
    lib.orc_decode_step.restype = None
    _lib = lib
    return lib


def _f64(a):
    return None if a is None else np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a, offset_elems=0):
    if a is None:
        return None
    base = a.ctypes.data + 8 * int(offset_elems)
    return ctypes.cast(base, ctypes.POINTER(ctypes.c_double))


def _mask_rows(mask, B, H, N):
    """Key padding mask [B, N] (True / nonzero = the key is ignored) expanded
    to one uint8 row per (batch, head), or None."""
    if mask is None:
        return None
    mask = np.asarray(mask).astype(bool)
    assert mask.shape == (B, N), "key padding mask must be [B, N_keys]"
    return np.ascontiguousarray(np.repeat(mask, H, axis=0).astype(np.uint8))


def _uptr(a, offset=0):
    if a is None:
        return None
    return ctypes.cast(a.ctypes.data + int(offset), ctypes.POINTER(ctypes.c_ubyte))


def default_threads() -> int:
    """Host cores this process may use: its affinity set, capped by the CPU
    share the environment grants through OMP_NUM_THREADS when that is set."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    share = os.environ.get("OMP_NUM_THREADS", "")
    if share.isdigit() and int(share) > 0:
        n = min(n, int(share))
    return max(1, n)


def feature_dim(phi: str, dk: int, omega) -> int:
    return dk if phi in ELEMENTWISE else 2 * int(np.asarray(omega).shape[0])


def phi_map(x, phi: str = "elu1", omega=None, scale: float = 1.0):
    """Feature map applied to the last axis of x; returns float64 [..., F]."""
    lib = _load()
    x = _f64(x)
    dk = x.shape[-1]
    om = _f64(omega)
    m = 0 if om is None else om.shape[0]
    F = feature_dim(phi, dk, om)
    flat = x.reshape(-1, dk)
    out = np.empty((flat.shape[0], F), dtype=np.float64)
    for r in range(flat.shape[0]):
        lib.orc_phi(PHI_KINDS[phi], _ptr(flat, r * dk), dk, m, _ptr(om), float(scale),
                    _ptr(out, r * F))
    return out.reshape(x.shape[:-1] + (F,))


def _lam_rows(lam, B, H):
    if lam is None:
        lam = np.ones(H)
    lam = np.asarray(lam, dtype=np.float64).reshape(-1)
    if lam.size == 1:
        lam = np.full(H, lam[0])
    assert lam.size == H, "lambda must have one value per head"
    return np.ascontiguousarray(np.tile(lam, B))


def _split(nbh, threads):
    threads = max(1, min(threads, nbh))
    edges = np.linspace(0, nbh, threads + 1).astype(int)
    return [(int(a), int(b)) for a, b in zip(edges[:-1], edges[1:]) if b > a]


def causal(q, k, v, lam=None, eps=1e-6, phi="elu1", omega=None, scale=1.0,
           S0=None, z0=None, want_state=False, want_kappa=False, threads=None,
           key_padding_mask=None):
    """Causal forward, per (b,h) one token at a time (update, then query).

    q, k: [B,H,N,dk]; v: [B,H,N,dv]; lam: [H] (None = 1); S0: [B,H,F,dv],
    z0: [B,H,F] or None (zero state); key_padding_mask: [B,N] bool (True =
    the key adds no term) or None.  Returns y [B,H,N,dv] and, if asked, the
    final (S, z) and the cancellation factor kappa [B,H,N].
    """
    lib = _load()
    q, k, v, om = _f64(q), _f64(k), _f64(v), _f64(omega)
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    m = 0 if om is None else om.shape[0]
    F = feature_dim(phi, dk, om)
    nbh = B * H
    lam_r = _lam_rows(lam, B, H)
    S0, z0 = _f64(S0), _f64(z0)
    y = np.empty((B, H, N, dv), dtype=np.float64)
    S = np.empty((B, H, F, dv), dtype=np.float64) if want_state else None
    z = np.empty((B, H, F), dtype=np.float64) if want_state else None
    kap = np.empty((B, H, N), dtype=np.float64) if want_kappa else None
    kpm = _mask_rows(key_padding_mask, B, H, N)

    def run(rng):
        a, b = rng
        lib.orc_causal(_ptr(q, a * N * dk), _ptr(k, a * N * dk), _ptr(v, a * N * dv),
                       b - a, N, dk, dv, PHI_KINDS[phi], m, _ptr(om), float(scale),
                       _ptr(lam_r, a), float(eps), _uptr(kpm, a * N),
                       _ptr(S0, a * F * dv), _ptr(z0, a * F),
                       _ptr(y, a * N * dv), _ptr(S, a * F * dv), _ptr(z, a * F),
                       _ptr(kap, a * N))

    parts = _split(nbh, threads or default_threads())
    if len(parts) == 1:
        run(parts[0])
    else:
        with ThreadPoolExecutor(len(parts)) as ex:
            list(ex.map(run, parts))
    out = [y]
    if want_state:
        out += [S, z]
    if want_kappa:
        out.append(kap)
    return out[0] if len(out) == 1 else tuple(out)


def noncausal(q, k, v, eps=1e-6, phi="elu1", omega=None, scale=1.0, threads=None):
    """Non-causal forward: one state summed over the whole sequence, no decay."""
    lib = _load()
    q, k, v, om = _f64(q), _f64(k), _f64(v), _f64(omega)
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    m = 0 if om is None else om.shape[0]
    y = np.empty((B, H, N, dv), dtype=np.float64)

    def run(rng):
        a, b = rng
        lib.orc_noncausal(_ptr(q, a * N * dk), _ptr(k, a * N * dk), _ptr(v, a * N * dv),
                          b - a, N, dk, dv, PHI_KINDS[phi], m, _ptr(om), float(scale),
                          float(eps), _ptr(y, a * N * dv))

    parts = _split(B * H, threads or default_threads())
    if len(parts) == 1:
        run(parts[0])
    else:
        with ThreadPoolExecutor(len(parts)) as ex:
            list(ex.map(run, parts))
    return y


def cross(q, k, v, eps=1e-6, phi="elu1", omega=None, scale=1.0, key_padding_mask=None,
          threads=None):
    """Non-causal cross attention: q [B,H,Nq,dk] against k [B,H,Nk,dk] and
    v [B,H,Nk,dv]; key_padding_mask [B,Nk] bool (True = the key is ignored)
    or None.  Returns y [B,H,Nq,dv]."""
    lib = _load()
    q, k, v, om = _f64(q), _f64(k), _f64(v), _f64(omega)
    B, H, Nq, dk = q.shape
    Nk = k.shape[2]
    dv = v.shape[-1]
    assert k.shape == (B, H, Nk, dk) and v.shape[:3] == (B, H, Nk)
    m = 0 if om is None else om.shape[0]
    kpm = _mask_rows(key_padding_mask, B, H, Nk)
    y = np.empty((B, H, Nq, dv), dtype=np.float64)

    def run(rng):
        a, b = rng
        lib.orc_cross(_ptr(q, a * Nq * dk), _ptr(k, a * Nk * dk), _ptr(v, a * Nk * dv),
                      b - a, Nq, Nk, dk, dv, PHI_KINDS[phi], m, _ptr(om), float(scale),
                      float(eps), _uptr(kpm, a * Nk), _ptr(y, a * Nq * dv))

    parts = _split(B * H, threads or default_threads())
    if len(parts) == 1:
        run(parts[0])
    else:
        with ThreadPoolExecutor(len(parts)) as ex:
            list(ex.map(run, parts))
    return y


def causal_varlen(q, k, v, cu_seqlens, lam=None, eps=1e-6, phi="elu1", omega=None,
                  scale=1.0, S0=None, z0=None, threads=None):
    """Causal forward over packed sequences of different lengths.

    q, k: [1,H,T,dk], v: [1,H,T,dv]: sequence b holds tokens
    cu_seqlens[b] .. cu_seqlens[b+1]-1 of every head's row; S0 [B,H,F,dv],
    z0 [B,H,F] (None = zero) are the sequences' initial states.  Each sequence
    is its own causal problem: this calls causal() on each slice.  Returns
    y [1,H,T,dv] (tokens outside every sequence are 0) and the final S, z
    [B,H,F,dv], [B,H,F].
    """
    q, k, v, om = _f64(q), _f64(k), _f64(v), _f64(omega)
    _, H, T, dk = q.shape
    dv = v.shape[-1]
    cu = [int(c) for c in np.asarray(cu_seqlens).reshape(-1)]
    B = len(cu) - 1
    assert cu[0] == 0 and all(b >= a for a, b in zip(cu[:-1], cu[1:])) and cu[-1] <= T
    F = feature_dim(phi, dk, om)
    y = np.zeros((1, H, T, dv), dtype=np.float64)
    S = np.empty((B, H, F, dv), dtype=np.float64)
    z = np.empty((B, H, F), dtype=np.float64)
    S0, z0 = _f64(S0), _f64(z0)
    for b in range(B):
        s0 = None if S0 is None else S0[b:b + 1]
        zz0 = None if z0 is None else z0[b:b + 1]
        lo, hi = cu[b], cu[b + 1]
        if hi == lo:
            S[b] = 0.0 if s0 is None else s0[0]
            z[b] = 0.0 if zz0 is None else zz0[0]
            continue
        yb, Sb, zb = causal(q[:, :, lo:hi], k[:, :, lo:hi], v[:, :, lo:hi], lam=lam, eps=eps,
                            phi=phi, omega=om, scale=scale, S0=s0, z0=zz0, want_state=True,
                            threads=threads)
        y[:, :, lo:hi] = yb
        S[b], z[b] = Sb[0], zb[0]
    return y, S, z


def backward(q, k, v, gy, lam=None, eps=1e-6, phi="elu1", omega=None, scale=1.0, S0=None, z0=None,
             dS_out=None, dz_out=None, key_padding_mask=None, threads=None, want_kappa=False):
    """Gradients of the causal forward for the loss sum(gy * y) +
    <dS_out, S_final> + <dz_out, z_final>.

    Returns a dict: dq, dk [B,H,N,dk], dv [B,H,N,dv], dS0 [B,H,F,dv],
    dz0 [B,H,F] (gradient of the initial state) and dlam [B,H] (per row;
    a per-head parameter's gradient is its sum over B); with want_kappa
    (elementwise feature maps) also the rows' cancellation factors
    kappa_dq, kappa_dk, kappa_dv [B,H,N].
    """
    lib = _load()
    q, k, v, gy, om = _f64(q), _f64(k), _f64(v), _f64(gy), _f64(omega)
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    m = 0 if om is None else om.shape[0]
    F = feature_dim(phi, dk, om)
    lam_r = _lam_rows(lam, B, H)
    S0, z0, dS_out, dz_out = _f64(S0), _f64(z0), _f64(dS_out), _f64(dz_out)
    kpm = _mask_rows(key_padding_mask, B, H, N)
    out = {"dq": np.empty((B, H, N, dk)), "dk": np.empty((B, H, N, dk)), "dv": np.empty((B, H, N, dv)),
           "dS0": np.empty((B, H, F, dv)), "dz0": np.empty((B, H, F)), "dlam": np.empty((B, H))}
    if want_kappa:
        for name in ("kappa_dq", "kappa_dk", "kappa_dv"):
            out[name] = np.empty((B, H, N))

    def run(rng):
        a, b = rng
        lib.orc_backward(_ptr(q, a * N * dk), _ptr(k, a * N * dk), _ptr(v, a * N * dv), _ptr(gy, a * N * dv),
                         b - a, N, dk, dv, PHI_KINDS[phi], m, _ptr(om), float(scale), _ptr(lam_r, a),
                         float(eps), _uptr(kpm, a * N), _ptr(S0, a * F * dv), _ptr(z0, a * F),
                         _ptr(dS_out, a * F * dv), _ptr(dz_out, a * F),
                         _ptr(out["dq"], a * N * dk), _ptr(out["dk"], a * N * dk), _ptr(out["dv"], a * N * dv),
                         _ptr(out["dS0"], a * F * dv), _ptr(out["dz0"], a * F), _ptr(out["dlam"], a),
                         _ptr(out.get("kappa_dq"), a * N), _ptr(out.get("kappa_dk"), a * N),
                         _ptr(out.get("kappa_dv"), a * N))

    parts = _split(B * H, threads or default_threads())
    if len(parts) == 1:
        run(parts[0])
    else:
        with ThreadPoolExecutor(len(parts)) as ex:
            list(ex.map(run, parts))
    return out


def cross_backward(q, k, v, gy, eps=1e-6, phi="elu1", omega=None, scale=1.0, key_padding_mask=None,
                   threads=None, want_kappa=False):
    """Gradients of cross() (non-causal; Nq may differ from Nk) for the loss
    sum(gy * y).  Returns a dict: dq [B,H,Nq,dk], dk [B,H,Nk,dk], dv [B,H,Nk,dv];
    with want_kappa (elementwise feature maps) also the rows' cancellation
    factors kappa_dq [B,H,Nq], kappa_dk, kappa_dv [B,H,Nk] (as backward())."""
    lib = _load()
    q, k, v, gy, om = _f64(q), _f64(k), _f64(v), _f64(gy), _f64(omega)
    B, H, Nq, dk = q.shape
    Nk = k.shape[2]
    dv = v.shape[-1]
    m = 0 if om is None else om.shape[0]
    kpm = _mask_rows(key_padding_mask, B, H, Nk)
    out = {"dq": np.empty((B, H, Nq, dk)), "dk": np.empty((B, H, Nk, dk)), "dv": np.empty((B, H, Nk, dv))}
    if want_kappa:
        out["kappa_dq"] = np.empty((B, H, Nq))
        out["kappa_dk"] = np.empty((B, H, Nk))
        out["kappa_dv"] = np.empty((B, H, Nk))

    def run(rng):
        a, b = rng
        lib.orc_cross_backward(_ptr(q, a * Nq * dk), _ptr(k, a * Nk * dk), _ptr(v, a * Nk * dv),
                               _ptr(gy, a * Nq * dv), b - a, Nq, Nk, dk, dv, PHI_KINDS[phi], m, _ptr(om),
                               float(scale), float(eps), _uptr(kpm, a * Nk), _ptr(out["dq"], a * Nq * dk),
                               _ptr(out["dk"], a * Nk * dk), _ptr(out["dv"], a * Nk * dv),
                               _ptr(out.get("kappa_dq"), a * Nq), _ptr(out.get("kappa_dk"), a * Nk),
                               _ptr(out.get("kappa_dv"), a * Nk))

    parts = _split(B * H, threads or default_threads())
    if len(parts) == 1:
        run(parts[0])
    else:
        with ThreadPoolExecutor(len(parts)) as ex:
            list(ex.map(run, parts))
    return out


def phi_vjp(x, dp, phi="elu1", omega=None, scale=1.0):
    """J_phi(x)^T dp over the last axis (x [..., dk], dp [..., F])."""
    lib = _load()
    x, dp, om = _f64(x), _f64(dp), _f64(omega)
    dk = x.shape[-1]
    m = 0 if om is None else om.shape[0]
    F = dp.shape[-1]
    fx, fd = x.reshape(-1, dk), dp.reshape(-1, F)
    out = np.empty_like(fx)
    for r in range(fx.shape[0]):
        lib.orc_phi_vjp(PHI_KINDS[phi], _ptr(fx, r * dk), dk, m, _ptr(om), float(scale), _ptr(fd, r * F),
                        _ptr(out, r * dk))
    return out.reshape(x.shape)


def decode_step(q, k, v, S, z, lam=None, eps=1e-6, phi="elu1", omega=None, scale=1.0,
                threads=None):
    """One decode step.  q,k: [B,H,1,dk] (or [B,H,dk]); v: [B,H,1,dv];
    S [B,H,F,dv], z [B,H,F].  Returns (y [B,H,1,dv], S_new, z_new); the inputs
    are not modified."""
    lib = _load()
    q, k, v, om = _f64(q), _f64(k), _f64(v), _f64(omega)
    B, H = q.shape[0], q.shape[1]
    dk, dv = q.shape[-1], v.shape[-1]
    m = 0 if om is None else om.shape[0]
    F = feature_dim(phi, dk, om)
    S = np.array(S, dtype=np.float64, copy=True, order="C")
    z = np.array(z, dtype=np.float64, copy=True, order="C")
    y = np.empty((B, H, 1, dv), dtype=np.float64)
    lam_r = _lam_rows(lam, B, H)

    def run(rng):
        a, b = rng
        lib.orc_decode_step(_ptr(q, a * dk), _ptr(k, a * dk), _ptr(v, a * dv), b - a, dk,
                            dv, PHI_KINDS[phi], m, _ptr(om), float(scale), _ptr(lam_r, a),
                            float(eps), _ptr(S, a * F * dv), _ptr(z, a * F),
                            _ptr(y, a * dv))

    parts = _split(B * H, threads or default_threads())
    if len(parts) == 1:
        run(parts[0])
    else:
        with ThreadPoolExecutor(len(parts)) as ex:
            list(ex.map(run, parts))
    return y, S, z


def rowwise_rel_err(y, y_ref):
    """max over rows r=(b,h,i) of max_c |y - y_ref| / max_c |y_ref|.

    Elementwise relative error is unusable here (outputs cross zero), so each
    row is normalised by its own largest reference magnitude.
    """
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    num = np.max(np.abs(y - y_ref), axis=-1)
    den = np.max(np.abs(y_ref), axis=-1)
    den = np.where(den == 0, 1.0, den)
    r = num / den
    return float(np.max(r)) if r.size else 0.0
