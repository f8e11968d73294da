"""Thin ctypes binding of liblinattn (include/la.h), same names as the C ABI.

Argument marshalling only: torch tensors supply device pointers, shapes and
the current HIP stream; every step of the computation runs in the library's
HIP kernels.  There is no fallback: if the library is missing or fails to
load, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblinattn.so")

LA_OK, LA_ERR_INVALID_ARGUMENT, LA_ERR_UNSUPPORTED, LA_ERR_WORKSPACE, LA_ERR_HIP = range(5)
LA_F32, LA_BF16 = 0, 1
LA_DECODE_MAX_TOKENS = 64  # include/la.h
LA_PHI_ELU1, LA_PHI_TRIG_RF, LA_PHI_RELU, LA_PHI_TRIG_RF_PLAIN, LA_PHI_TRIG_RF_SOFTMAX = 0, 1, 2, 3, 4
PHI_KINDS = {"elu1": LA_PHI_ELU1, "trig_rf": LA_PHI_TRIG_RF, "relu": LA_PHI_RELU,
             "trig_rf_plain": LA_PHI_TRIG_RF_PLAIN, "trig_rf_softmax": LA_PHI_TRIG_RF_SOFTMAX}
ELEMENTWISE = ("elu1", "relu")
LA_MAX_HEADS = 256

# names declared in include/la.h
EXPORTS = ("la_init_state", "la_init_state_identity", "la_workspace_size", "la_forward_causal",
           "la_forward_causal_noalloc", "la_forward_noncausal",
           "la_forward_causal_masked", "la_workspace_size_varlen", "la_forward_causal_varlen",
           "la_workspace_size_cross", "la_forward_cross", "la_workspace_size_backward", "la_backward_causal",
           "la_workspace_size_backward_cross", "la_backward_cross",
           "la_decode_step", "la_status_string", "la_last_error", "la_profile_begin", "la_profile_end",
           "la_kernel_name")
KERNEL_IDS = {"fwd_local": 0, "fwd_causal": 1, "fwd_query": 2, "scan": 3, "decode": 4, "fill": 5, "copy": 6,
              "bwd_q": 7, "bwd_rlocal": 8, "bwd_kv": 9, "bwd_dlam": 10, "varlen_items": 11, "bwd_ncq": 12,
              "bwd_nckv": 13, "rf_features": 14, "rf_vjp": 15}


class LaPhiC(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("m", ctypes.c_int32),
                ("omega", ctypes.c_void_p), ("qk_scale", ctypes.c_float)]


class LaShapeC(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("H", ctypes.c_int64), ("N", ctypes.c_int64),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32)]


class LaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__("%s: %s" % (_status_name(status), detail))
        self.status = status


_lib = None


def _status_name(s):
    return {0: "LA_OK", 1: "LA_ERR_INVALID_ARGUMENT", 2: "LA_ERR_UNSUPPORTED",
            3: "LA_ERR_WORKSPACE", 4: "LA_ERR_HIP"}.get(int(s), "LA_ERR_UNKNOWN")


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load liblinattn.so (after torch, so both share torch's HIP runtime)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError("liblinattn.so is not built (%s); run __graft_entry__.build() or "
                           "python -m weight_sequence_mixing_amd.build" % p)
    lib = ctypes.CDLL(p)
    vp, sz, f, i32, i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_float, ctypes.c_int32, ctypes.c_int64
    SP, PP = ctypes.POINTER(LaShapeC), ctypes.POINTER(LaPhiC)
    lib.la_init_state.argtypes = [vp, vp, i64, i64, i32, i32, vp]
    lib.la_init_state.restype = ctypes.c_int
    lib.la_init_state_identity.argtypes = [vp, vp, i64, i64, i32, i32, f, vp]
    lib.la_init_state_identity.restype = ctypes.c_int
    lib.la_workspace_size.argtypes = [SP, PP, i32]
    lib.la_workspace_size.restype = sz
    lib.la_forward_causal.argtypes = [vp, vp, vp, vp, SP, PP, vp, f, vp, vp, vp, vp, vp, sz, vp]
    lib.la_forward_causal.restype = ctypes.c_int
    lib.la_forward_causal_noalloc.argtypes = [vp, vp, vp, vp, SP, PP, vp, f, vp, vp, vp, vp, vp]
    lib.la_forward_causal_noalloc.restype = ctypes.c_int
    lib.la_forward_noncausal.argtypes = [vp, vp, vp, vp, SP, PP, f, vp, sz, vp]
    lib.la_forward_noncausal.restype = ctypes.c_int
    lib.la_forward_causal_masked.argtypes = [vp, vp, vp, vp, SP, PP, vp, f, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.la_forward_causal_masked.restype = ctypes.c_int
    lib.la_workspace_size_varlen.argtypes = [SP, i64, PP]
    lib.la_workspace_size_varlen.restype = sz
    lib.la_forward_causal_varlen.argtypes = [vp, vp, vp, vp, vp, i64, SP, PP, vp, f, vp, vp, vp, vp, vp, sz, vp]
    lib.la_forward_causal_varlen.restype = ctypes.c_int
    lib.la_workspace_size_cross.argtypes = [SP, i64, PP]
    lib.la_workspace_size_cross.restype = sz
    lib.la_forward_cross.argtypes = [vp, vp, vp, vp, SP, i64, vp, PP, f, vp, sz, vp]
    lib.la_forward_cross.restype = ctypes.c_int
    lib.la_workspace_size_backward.argtypes = [SP, PP]
    lib.la_workspace_size_backward.restype = sz
    lib.la_backward_causal.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, SP, PP, vp, f, vp, vp, vp, vp, vp, vp,
                                       vp, vp, vp, sz, vp]
    lib.la_backward_causal.restype = ctypes.c_int
    lib.la_workspace_size_backward_cross.argtypes = [SP, i64, PP]
    lib.la_workspace_size_backward_cross.restype = sz
    lib.la_backward_cross.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, SP, i64, vp, PP, f, vp, sz, vp]
    lib.la_backward_cross.restype = ctypes.c_int
    lib.la_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, SP, PP, vp, f, vp]
    lib.la_decode_step.restype = ctypes.c_int
    lib.la_status_string.argtypes = [ctypes.c_int]
    lib.la_status_string.restype = ctypes.c_char_p
    lib.la_last_error.argtypes = []
    lib.la_last_error.restype = ctypes.c_char_p
    lib.la_profile_begin.argtypes = [i32]
    lib.la_profile_begin.restype = ctypes.c_int
    lib.la_profile_end.argtypes = [vp, vp, i32, vp]
    lib.la_profile_end.restype = ctypes.c_int
    lib.la_kernel_name.argtypes = [i32]
    lib.la_kernel_name.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def _check(status: int):
    if status != LA_OK:
        raise LaError(status, _lib.la_last_error().decode())


@dataclass
class Phi:
    """Feature map: 'elu1' (elu(x)+1), 'relu' (max(x, 0)), or cos/sin random
    features with the prefactor exp(-|x'|^2/2)/sqrt(m) ('trig_rf'), 1/sqrt(m)
    ('trig_rf_plain') or exp(+|x'|^2/2)/sqrt(m) ('trig_rf_softmax').

    For random features, omega is a device fp32 tensor [m, d_k] and qk_scale the
    factor applied to q and k before the map (typically d_k ** -0.25)."""
    kind: str = "elu1"
    omega: Optional[torch.Tensor] = None
    qk_scale: float = 1.0

    def c(self) -> LaPhiC:
        if self.kind not in PHI_KINDS:
            raise ValueError("unknown feature map %r" % (self.kind,))
        code = PHI_KINDS[self.kind]
        if self.kind in ELEMENTWISE:
            return LaPhiC(code, 0, None, 1.0)
        om = self.omega
        if om is None:
            return LaPhiC(code, 0, None, float(self.qk_scale))
        if om.dtype != torch.float32 or not om.is_contiguous():
            raise ValueError("omega must be a contiguous float32 tensor")
        return LaPhiC(code, int(om.shape[0]), om.data_ptr(), float(self.qk_scale))

    def F(self, d_k: int) -> int:
        return d_k if self.kind in ELEMENTWISE else 2 * int(self.omega.shape[0])


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return LA_BF16
    if t.dtype == torch.float32:
        return LA_F32
    raise ValueError("unsupported dtype %s" % t.dtype)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


# ---- argument checks: shapes, dtypes and devices of every tensor argument
# (the library sees raw pointers and trusts the sizes it is given)
def _one_device(*ts) -> torch.device:
    devs = {t.device for t in ts if t is not None}
    if len(devs) != 1:
        raise ValueError("all tensors must be on one device (got %s)" % sorted(map(str, devs)))
    dev = devs.pop()
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device (got %s)" % dev)
    return dev


def _expect(t, name, shape, dtypes):
    """t must have exactly `shape` and one of `dtypes` (None: not given)."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s (got %s)" % (name, tuple(shape), tuple(t.shape)))
    if t.dtype not in dtypes:
        raise ValueError("%s must be %s (got %s)" % (name, " or ".join(map(str, dtypes)), t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


_IO = (torch.bfloat16, torch.float32)
_F32 = (torch.float32,)


def _qkvy(q, k, v, y, n_kv=None):
    """q [B,H,N,d_k], k [B,H,M,d_k], v [B,H,M,d_v], y [B,H,N,d_v] (M = N
    unless n_kv is given); returns (B, H, N, d_k, d_v)."""
    if q.dim() != 4:
        raise ValueError("q must be [B,H,N,d_k] (got %s)" % (tuple(q.shape),))
    B, H, N, dk = q.shape
    M = N if n_kv is None else n_kv
    if v.dim() != 4:
        raise ValueError("v must be [B,H,N,d_v] (got %s)" % (tuple(v.shape),))
    dv = v.shape[-1]
    _expect(q, "q", (B, H, N, dk), _IO)
    _expect(k, "k", (B, H, M, dk), (q.dtype,))
    _expect(v, "v", (B, H, M, dv), (q.dtype,))
    _expect(y, "y", (B, H, N, dv), (q.dtype, torch.float32))
    return B, H, N, dk, dv


def _state(S, z, B, H, F, dv, sname="S", zname="z"):
    if (S is None) != (z is None):
        raise ValueError("%s and %s must be given together" % (sname, zname))
    _expect(S, sname, (B, H, F, dv), _F32)
    _expect(z, zname, (B, H, F), _F32)


def _shape(q: torch.Tensor, v: torch.Tensor, y: torch.Tensor) -> LaShapeC:
    B, H, N, dk = q.shape
    return LaShapeC(B, H, N, dk, v.shape[-1], _dt(q), _dt(y))


def _phi_checked(phi: Optional["Phi"], d_k: int) -> "Phi":
    phi = phi or Phi()
    if phi.kind not in PHI_KINDS:
        raise ValueError("unknown feature map %r" % (phi.kind,))
    if phi.kind not in ELEMENTWISE:
        om = phi.omega
        if om is None:
            raise ValueError("random features need omega [m, d_k]")
        if om.dim() != 2 or om.shape[1] != d_k:
            raise ValueError("omega must be [m, d_k=%d] (got %s)" % (d_k, tuple(om.shape)))
    return phi


def _omega(phi: "Phi"):
    return None if phi.kind in ELEMENTWISE else phi.omega


def _mask(mask, B, M):
    if mask is None:
        return
    if mask.dtype not in (torch.bool, torch.uint8):
        raise ValueError("key_padding_mask must be bool or uint8")
    if tuple(mask.shape) != (B, M):
        raise ValueError("key_padding_mask must be [B, N_keys] = %s (got %s)" % ((B, M), tuple(mask.shape)))


def _lam(lambda_h, H):
    if lambda_h is None:
        return None, None
    if isinstance(lambda_h, torch.Tensor):
        lambda_h = lambda_h.detach().to("cpu", torch.float32).reshape(-1).tolist()
    vals = [float(x) for x in lambda_h]
    if len(vals) != H:
        raise ValueError("lambda_h needs one value per head: %d given for H=%d" % (len(vals), H))
    arr = (ctypes.c_float * H)(*vals)
    return arr, ctypes.cast(arr, ctypes.c_void_p)


def la_status_string(status: int) -> str:
    return load_library().la_status_string(int(status)).decode()


def la_last_error() -> str:
    return load_library().la_last_error().decode()


def la_profile_begin(max_launches: int) -> None:
    """Start bracketing every library launch on this thread with HIP events."""
    load_library()
    _check(_lib.la_profile_begin(int(max_launches)))


def la_profile_end(capacity: int = 100000):
    """Stop recording; returns a list of (kernel_id, milliseconds) in launch order."""
    load_library()
    ids = (ctypes.c_int32 * capacity)()
    ms = (ctypes.c_float * capacity)()
    n = ctypes.c_int32(0)
    _check(_lib.la_profile_end(ctypes.cast(ids, ctypes.c_void_p), ctypes.cast(ms, ctypes.c_void_p),
                               capacity, ctypes.cast(ctypes.pointer(n), ctypes.c_void_p)))
    return [(int(ids[i]), float(ms[i])) for i in range(n.value)]


def la_kernel_name(kernel_id: int) -> str:
    return load_library().la_kernel_name(int(kernel_id)).decode()


def _state_shape(S, z):
    if S.dim() != 4:
        raise ValueError("S must be [B,H,F,d_v] (got %s)" % (tuple(S.shape),))
    B, H, F, dv = S.shape
    _state(S, z, B, H, F, dv)
    _one_device(S, z)
    return B, H, F, dv


def la_init_state(S: torch.Tensor, z: torch.Tensor, stream=None) -> None:
    """S [B,H,F,d_v] = 0, z [B,H,F] = 0 (fp32 device tensors)."""
    load_library()
    B, H, F, dv = _state_shape(S, z)
    _check(_lib.la_init_state(_ptr(S), _ptr(z), B, H, F, dv, _stream(stream)))


def la_init_state_identity(S: torch.Tensor, z: torch.Tensor, alpha: float = 1.0, stream=None) -> None:
    """S [B,H,F,d_v] = alpha * I (rectangular), z [B,H,F] = alpha on the first
    min(F, d_v) features, 0 elsewhere (fp32 device tensors)."""
    load_library()
    B, H, F, dv = _state_shape(S, z)
    _check(_lib.la_init_state_identity(_ptr(S), _ptr(z), B, H, F, dv, float(alpha), _stream(stream)))


def la_workspace_size(B, H, N, d_k, d_v, in_dtype=LA_BF16, out_dtype=None, phi: Optional[Phi] = None,
                      causal: bool = True) -> int:
    load_library()
    phi = phi or Phi()
    shape = LaShapeC(B, H, N, d_k, d_v, in_dtype, in_dtype if out_dtype is None else out_dtype)
    pc = phi.c()
    return int(_lib.la_workspace_size(ctypes.byref(shape), ctypes.byref(pc), 1 if causal else 0))


def _alloc_ws(need: int, workspace, device, stream=None):
    """The caller's workspace, or a new one.  A new block is marked as used on
    the launch stream, so that the caching allocator does not hand it out
    again before the kernels enqueued there have finished."""
    if workspace is None:
        if need == 0:
            return None, 0
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
        if stream is not None:
            s = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(int(stream), device=device)
            workspace.record_stream(s)
    elif not workspace.is_contiguous() or workspace.device != device:
        raise ValueError("workspace must be a contiguous tensor on %s" % device)
    return workspace, workspace.numel() * workspace.element_size()


def _workspace(shape: LaShapeC, pc: LaPhiC, causal: bool, workspace, device, stream=None):
    need = int(_lib.la_workspace_size(ctypes.byref(shape), ctypes.byref(pc), 1 if causal else 0))
    return _alloc_ws(need, workspace, device, stream)


def _causal_args(q, k, v, y, phi, S_in, z_in, S_out, z_out, mask=None):
    """Checks of the causal forwards' tensors; returns (device, phi, shape, LaPhiC)."""
    B, H, N, dk, dv = _qkvy(q, k, v, y)
    phi = _phi_checked(phi, dk)
    F = phi.F(dk)
    _state(S_in, z_in, B, H, F, dv, "S_in", "z_in")
    _state(S_out, z_out, B, H, F, dv, "S_out", "z_out")
    _mask(mask, B, N)
    dev = _one_device(q, k, v, y, S_in, z_in, S_out, z_out, mask, _omega(phi))
    return dev, phi, _shape(q, v, y), phi.c()


def la_forward_causal(q, k, v, y, phi: Optional[Phi] = None, lambda_h=None, eps: float = 1e-6,
                      S_in=None, z_in=None, S_out=None, z_out=None, workspace=None, stream=None):
    """Causal forward; writes y [B,H,N,d_v] (and S_out, z_out when given)."""
    load_library()
    lam_keep, lam_ptr = _lam(lambda_h, q.shape[1])
    dev, phi, shape, pc = _causal_args(q, k, v, y, phi, S_in, z_in, S_out, z_out)
    ws, ws_bytes = _workspace(shape, pc, True, workspace, dev, stream)
    _check(_lib.la_forward_causal(_ptr(q), _ptr(k), _ptr(v), _ptr(y), ctypes.byref(shape), ctypes.byref(pc),
                                  lam_ptr, float(eps), _ptr(S_in), _ptr(z_in), _ptr(S_out), _ptr(z_out),
                                  _ptr(ws), ws_bytes, _stream(stream)))
    del lam_keep
    return y


LA_NOALLOC_SCRATCH_BYTES = 64 << 20  # include/la.h


def la_forward_causal_noalloc(q, k, v, y, phi: Optional[Phi] = None, lambda_h=None, eps: float = 1e-6,
                              S_in=None, z_in=None, S_out=None, z_out=None, stream=None):
    """la_forward_causal without a workspace: the library's static device
    scratch holds the segment states (nothing is allocated by the call)."""
    load_library()
    lam_keep, lam_ptr = _lam(lambda_h, q.shape[1])
    dev, phi, shape, pc = _causal_args(q, k, v, y, phi, S_in, z_in, S_out, z_out)
    _check(_lib.la_forward_causal_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(y), ctypes.byref(shape), ctypes.byref(pc),
                                          lam_ptr, float(eps), _ptr(S_in), _ptr(z_in), _ptr(S_out), _ptr(z_out),
                                          _stream(stream)))
    del lam_keep
    return y


def la_forward_noncausal(q, k, v, y, phi: Optional[Phi] = None, eps: float = 1e-6, workspace=None, stream=None):
    """Non-causal forward; writes y [B,H,N,d_v]."""
    load_library()
    dev, phi, shape, pc = _causal_args(q, k, v, y, phi, None, None, None, None)
    ws, ws_bytes = _workspace(shape, pc, False, workspace, dev, stream)
    _check(_lib.la_forward_noncausal(_ptr(q), _ptr(k), _ptr(v), _ptr(y), ctypes.byref(shape), ctypes.byref(pc),
                                     float(eps), _ptr(ws), ws_bytes, _stream(stream)))
    return y


def _mask_ptr(mask: Optional[torch.Tensor]):
    if mask is None:
        return None
    if mask.dtype not in (torch.bool, torch.uint8):
        raise ValueError("key_padding_mask must be bool or uint8")
    return _ptr(mask)  # bool is stored as one byte per element, 0 or 1


def la_forward_causal_masked(q, k, v, y, key_padding_mask, phi: Optional[Phi] = None, lambda_h=None,
                             eps: float = 1e-6, S_in=None, z_in=None, S_out=None, z_out=None, workspace=None,
                             stream=None):
    """Causal forward with a key padding mask [B,N] (bool / uint8 on the device,
    True = the key adds nothing)."""
    load_library()
    if key_padding_mask is None:
        raise ValueError("key_padding_mask is required")
    lam_keep, lam_ptr = _lam(lambda_h, q.shape[1])
    dev, phi, shape, pc = _causal_args(q, k, v, y, phi, S_in, z_in, S_out, z_out, key_padding_mask)
    ws, ws_bytes = _workspace(shape, pc, True, workspace, dev, stream)
    _check(_lib.la_forward_causal_masked(_ptr(q), _ptr(k), _ptr(v), _ptr(y), ctypes.byref(shape),
                                         ctypes.byref(pc), lam_ptr, float(eps), _mask_ptr(key_padding_mask),
                                         _ptr(S_in), _ptr(z_in), _ptr(S_out), _ptr(z_out), _ptr(ws), ws_bytes,
                                         _stream(stream)))
    del lam_keep
    return y


def la_workspace_size_varlen(B, H, T, max_seqlen, d_k, d_v, in_dtype=LA_BF16, out_dtype=None,
                             phi: Optional[Phi] = None) -> int:
    load_library()
    phi = phi or Phi()
    shape = LaShapeC(B, H, T, d_k, d_v, in_dtype, in_dtype if out_dtype is None else out_dtype)
    pc = phi.c()
    return int(_lib.la_workspace_size_varlen(ctypes.byref(shape), int(max_seqlen), ctypes.byref(pc)))


def la_forward_causal_varlen(q, k, v, y, cu_seqlens, max_seqlen: int, phi: Optional[Phi] = None, lambda_h=None,
                             eps: float = 1e-6, S_in=None, z_in=None, S_out=None, z_out=None, workspace=None,
                             stream=None):
    """Causal forward over packed sequences: q, k [H,T,d_k], v, y [H,T,d_v];
    cu_seqlens: int32 device tensor [B+1]; states [B,H,F,d_v] / [B,H,F]."""
    load_library()
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be an int32 tensor [B+1] with B >= 1")
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("packed q, k, v, y must be [H,T,d]")
    H, T, dk = q.shape
    dv = v.shape[-1]
    B = cu_seqlens.numel() - 1
    _expect(q, "q", (H, T, dk), _IO)
    _expect(k, "k", (H, T, dk), (q.dtype,))
    _expect(v, "v", (H, T, dv), (q.dtype,))
    _expect(y, "y", (H, T, dv), (q.dtype, torch.float32))
    phi = _phi_checked(phi, dk)
    F = phi.F(dk)
    _state(S_in, z_in, B, H, F, dv, "S_in", "z_in")
    _state(S_out, z_out, B, H, F, dv, "S_out", "z_out")
    lam_keep, lam_ptr = _lam(lambda_h, H)
    dev = _one_device(q, k, v, y, cu_seqlens, S_in, z_in, S_out, z_out, _omega(phi))
    shape = LaShapeC(B, H, T, dk, dv, _dt(q), _dt(y))
    pc = phi.c()
    need = int(_lib.la_workspace_size_varlen(ctypes.byref(shape), int(max_seqlen), ctypes.byref(pc)))
    ws, ws_bytes = _alloc_ws(need, workspace, dev, stream)
    _check(_lib.la_forward_causal_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(y), _ptr(cu_seqlens), int(max_seqlen),
                                         ctypes.byref(shape), ctypes.byref(pc), lam_ptr, float(eps), _ptr(S_in),
                                         _ptr(z_in), _ptr(S_out), _ptr(z_out), _ptr(ws), ws_bytes,
                                         _stream(stream)))
    del lam_keep
    return y


def la_workspace_size_cross(B, H, N, n_kv, d_k, d_v, in_dtype=LA_BF16, out_dtype=None,
                            phi: Optional[Phi] = None) -> int:
    load_library()
    phi = phi or Phi()
    shape = LaShapeC(B, H, N, d_k, d_v, in_dtype, in_dtype if out_dtype is None else out_dtype)
    pc = phi.c()
    return int(_lib.la_workspace_size_cross(ctypes.byref(shape), int(n_kv), ctypes.byref(pc)))


def _cross_args(q, k, v, y, phi, mask):
    if k.dim() != 4:
        raise ValueError("k must be [B,H,M,d_k] (got %s)" % (tuple(k.shape),))
    n_kv = int(k.shape[2])
    B, H, N, dk, dv = _qkvy(q, k, v, y, n_kv)
    phi = _phi_checked(phi, dk)
    _mask(mask, B, n_kv)
    return phi, n_kv


def la_forward_cross(q, k, v, y, key_padding_mask=None, phi: Optional[Phi] = None, eps: float = 1e-6,
                     workspace=None, stream=None):
    """Non-causal cross attention: q [B,H,N,d_k] against k [B,H,M,d_k] and
    v [B,H,M,d_v]; optional key_padding_mask [B,M]; writes y [B,H,N,d_v]."""
    load_library()
    phi, n_kv = _cross_args(q, k, v, y, phi, key_padding_mask)
    dev = _one_device(q, k, v, y, key_padding_mask, _omega(phi))
    shape = _shape(q, v, y)
    pc = phi.c()
    need = int(_lib.la_workspace_size_cross(ctypes.byref(shape), n_kv, ctypes.byref(pc)))
    ws, ws_bytes = _alloc_ws(need, workspace, dev, stream)
    _check(_lib.la_forward_cross(_ptr(q), _ptr(k), _ptr(v), _ptr(y), ctypes.byref(shape), n_kv,
                                 _mask_ptr(key_padding_mask), ctypes.byref(pc), float(eps), _ptr(ws), ws_bytes,
                                 _stream(stream)))
    return y


def la_workspace_size_backward(B, H, N, d_k, d_v, in_dtype=LA_BF16, phi: Optional[Phi] = None) -> int:
    load_library()
    phi = phi or Phi()
    shape = LaShapeC(B, H, N, d_k, d_v, in_dtype, in_dtype)
    pc = phi.c()
    return int(_lib.la_workspace_size_backward(ctypes.byref(shape), ctypes.byref(pc)))


def _grads(q, k, v, y, dy, dq, dk, dv):
    """dy like y (input type); dq, dk, dv like q, k, v."""
    if y.dtype != q.dtype:
        raise ValueError("the backward takes y in the input type (got %s for %s inputs)" % (y.dtype, q.dtype))
    _expect(dy, "dy", tuple(y.shape), (q.dtype,))
    _expect(dq, "dq", tuple(q.shape), (q.dtype,))
    _expect(dk, "dk", tuple(k.shape), (q.dtype,))
    _expect(dv, "dv", tuple(v.shape), (q.dtype,))


def la_backward_causal(q, k, v, y, dy, dq, dk, dv, phi: Optional[Phi] = None, lambda_h=None, eps: float = 1e-6,
                       key_padding_mask=None, S_in=None, z_in=None, dS_out=None, dz_out=None, dS_in=None,
                       dz_in=None, dlambda=None, workspace=None, stream=None):
    """Gradients of la_forward_causal: writes dq, dk, dv (and dS_in, dz_in,
    dlambda [H] fp32 when given)."""
    load_library()
    if q.dim() != 4:
        raise ValueError("q must be [B,H,N,d_k] (got %s)" % (tuple(q.shape),))
    B, H, N, dk_ = q.shape
    _grads(q, k, v, y, dy, dq, dk, dv)
    phi_c = _phi_checked(phi, dk_)
    F, dv_ = phi_c.F(dk_), v.shape[-1]
    _state(dS_out, dz_out, B, H, F, dv_, "dS_out", "dz_out")
    _state(dS_in, dz_in, B, H, F, dv_, "dS_in", "dz_in")
    _expect(dlambda, "dlambda", (H,), _F32)
    lam_keep, lam_ptr = _lam(lambda_h, H)
    dev, phi, shape, pc = _causal_args(q, k, v, y, phi, S_in, z_in, None, None, key_padding_mask)
    _one_device(q, dy, dq, dk, dv, dS_out, dz_out, dS_in, dz_in, dlambda)
    need = int(_lib.la_workspace_size_backward(ctypes.byref(shape), ctypes.byref(pc)))
    ws, ws_bytes = _alloc_ws(need, workspace, dev, stream)
    _check(_lib.la_backward_causal(_ptr(q), _ptr(k), _ptr(v), _ptr(y), _ptr(dy), _ptr(dq), _ptr(dk), _ptr(dv),
                                   ctypes.byref(shape), ctypes.byref(pc), lam_ptr, float(eps),
                                   _mask_ptr(key_padding_mask), _ptr(S_in), _ptr(z_in), _ptr(dS_out),
                                   _ptr(dz_out), _ptr(dS_in), _ptr(dz_in), _ptr(dlambda), _ptr(ws), ws_bytes,
                                   _stream(stream)))
    del lam_keep
    return dq, dk, dv


def la_workspace_size_backward_cross(B, H, N, n_kv, d_k, d_v, in_dtype=LA_BF16, phi: Optional[Phi] = None) -> int:
    load_library()
    phi = phi or Phi()
    shape = LaShapeC(B, H, N, d_k, d_v, in_dtype, in_dtype)
    pc = phi.c()
    return int(_lib.la_workspace_size_backward_cross(ctypes.byref(shape), int(n_kv), ctypes.byref(pc)))


def la_backward_cross(q, k, v, y, dy, dq, dk, dv, key_padding_mask=None, phi: Optional[Phi] = None,
                      eps: float = 1e-6, workspace=None, stream=None):
    """Gradients of la_forward_cross (q, y, dy, dq: [B,H,N,*]; k, v, dk, dv:
    [B,H,M,*]): writes dq, dk, dv."""
    load_library()
    phi, n_kv = _cross_args(q, k, v, y, phi, key_padding_mask)
    _grads(q, k, v, y, dy, dq, dk, dv)
    dev = _one_device(q, k, v, y, dy, dq, dk, dv, key_padding_mask, _omega(phi))
    shape = _shape(q, v, y)
    pc = phi.c()
    need = int(_lib.la_workspace_size_backward_cross(ctypes.byref(shape), n_kv, ctypes.byref(pc)))
    ws, ws_bytes = _alloc_ws(need, workspace, dev, stream)
    _check(_lib.la_backward_cross(_ptr(q), _ptr(k), _ptr(v), _ptr(y), _ptr(dy), _ptr(dq), _ptr(dk), _ptr(dv),
                                  ctypes.byref(shape), n_kv, _mask_ptr(key_padding_mask), ctypes.byref(pc),
                                  float(eps), _ptr(ws), ws_bytes, _stream(stream)))
    return dq, dk, dv


def la_decode_step(q, k, v, y, S, z, phi: Optional[Phi] = None, lambda_h=None, eps: float = 1e-6, stream=None):
    """Decode steps on [B,H,N,d] inputs (N tokens per head-state, in order, N <= 64);
    updates S [B,H,F,d_v] and z [B,H,F] in place."""
    load_library()
    if S is None or z is None:
        raise ValueError("S and z are required")
    if q.dim() == 4 and v.dim() == 4:
        B, H, _, dk_ = q.shape
        _state(S, z, B, H, _phi_checked(phi, dk_).F(dk_), v.shape[-1])
    lam_keep, lam_ptr = _lam(lambda_h, q.shape[1])
    dev, phi, shape, pc = _causal_args(q, k, v, y, phi, S, z, None, None)
    _check(_lib.la_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(y), _ptr(S), _ptr(z), ctypes.byref(shape),
                               ctypes.byref(pc), lam_ptr, float(eps), _stream(stream)))
    del lam_keep
    return y


def rf_scale(d_k: int) -> float:
    return float(d_k) ** -0.25 if d_k > 0 else 1.0

