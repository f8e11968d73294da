"""Seeded synthetic inputs for the linear-attention workloads.

This module is shared by the CPU oracle tests and the GPU path.  It holds no
arithmetic of the method itself: only random draws, round-to-nearest-even
conversion to bfloat16, and shape bookkeeping.  Every array it returns is a
plain numpy array; the same bytes are handed to both sides.

Workloads (synthetic stand-ins; the pages measure on no public benchmark):

  1  causal, elu+1, lambda=1, eps=1e-6: B=1 H=1 N=256 d=64, fp32 N(0,1)
  2  causal, elu+1, lambda=1: B=4 H=8 N=4096 d=64, bf16 0.5*N(0,1)
  3  causal, elu+1, per-head lambda ~ U[0.9,0.999]: B=2 H=16 N=32768 d=128, bf16
  4  decode: 256 sequences x 32 heads, d=128, 512-token prefix then 1024
     single-token steps, lambda=0.999, bf16 0.5*N(0,1)
  5  causal, trigonometric random features m=128 (F=256): B=1 H=16 N=65536
     d=64, q/k scaled by d^-1/4 inside the feature map, bf16 0.5*N(0,1)

Each workload index is also its seed.  Independent sub-streams (q, k, v,
lambda, omega, prefix, steps) are spawned from numpy's SeedSequence so that
changing one tensor's size never changes another tensor's values.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "workload", "bf16_bits_rne", "bf16_bits_to_f32",
    "round_to_bf16", "make_qkv", "make_lambda", "make_omega", "make_inputs",
    "make_decode_step", "make_decode_steps", "make_decode_prefix", "make_kv", "make_key_padding_mask",
    "make_varlen_lengths", "cu_seqlens", "pack_heads",
]

# appended streams keep the earlier ones' values (child i of the seed's spawn)
STREAMS = ("q", "k", "v", "lam", "omega", "prefix", "steps", "mask", "lens", "kv")


# --------------------------------------------------------------------------
# bfloat16 rounding (explicit bit operations, independent of any torch version)
# --------------------------------------------------------------------------
def bf16_bits_rne(x) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest, ties to even.

    NaN inputs map to a quiet NaN; infinities are preserved; values that
    round past the largest finite bf16 become infinity (IEEE behaviour).
    The sum u + 0x7FFF + lsb stays below 2^32 for every non-NaN pattern u,
    so the arithmetic runs in place on 32-bit words.
    """
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = a.view(np.uint32)
    r = np.right_shift(u, np.uint32(16))
    np.bitwise_and(r, np.uint32(1), out=r)
    r += np.uint32(0x7FFF)
    r += u
    r >>= np.uint32(16)
    out = r.astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16)
    return out


def bf16_bits_to_f32(bits) -> np.ndarray:
    """bf16 bit patterns -> the exactly equal fp32 values."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32)


def round_to_bf16(x):
    """Return (bits uint16, values float32) of x rounded to bf16 (RNE)."""
    bits = bf16_bits_rne(x)
    return bits, bf16_bits_to_f32(bits)


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    kind: str            # "causal" | "decode"
    B: int
    H: int
    N: int               # sequence length (decode: prefix length)
    dk: int
    dv: int
    dtype: str           # "f32" | "bf16"
    scale: float         # standard deviation of q, k, v
    phi: str             # "elu1" | "relu" | "trig_rf" | "trig_rf_plain" | "trig_rf_softmax"
    m: int = 0           # random features (F = 2m) for the trig_rf kinds
    lam: str = "one"     # "one" | "per_head" | "const"
    lam_value: float = 1.0
    lam_lo: float = 0.9
    lam_hi: float = 0.999
    eps: float = 1e-6
    steps: int = 0       # decode steps after the prefix
    omega: str = "orthogonal"  # random directions: "orthogonal" blocks or plain "gaussian"

    @property
    def random_features(self) -> bool:
        return self.phi.startswith("trig_rf")

    @property
    def F(self) -> int:
        return 2 * self.m if self.random_features else self.dk

    @property
    def qk_scale(self) -> float:
        return float(self.dk) ** -0.25 if self.random_features else 1.0

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    1: Workload(1, "elu1_causal_B1_H1_N256_d64_f32", "causal", 1, 1, 256, 64, 64,
                "f32", 1.0, "elu1"),
    2: Workload(2, "elu1_causal_B4_H8_N4096_d64_bf16", "causal", 4, 8, 4096, 64, 64,
                "bf16", 0.5, "elu1"),
    3: Workload(3, "elu1_decay_causal_B2_H16_N32768_d128_bf16", "causal", 2, 16, 32768,
                128, 128, "bf16", 0.5, "elu1", lam="per_head"),
    4: Workload(4, "elu1_decode_B256_H32_d128_prefix512_steps1024_bf16", "decode", 256,
                32, 512, 128, 128, "bf16", 0.5, "elu1", lam="const", lam_value=0.999,
                steps=1024),
    5: Workload(5, "trigrf_m128_causal_B1_H16_N65536_d64_bf16", "causal", 1, 16, 65536,
                64, 64, "bf16", 0.5, "trig_rf", m=128),
}


def workload(index: int) -> Workload:
    return WORKLOADS[index]


def _streams(seed: int) -> dict:
    children = np.random.SeedSequence(seed).spawn(len(STREAMS))
    return {name: child for name, child in zip(STREAMS, children)}


def _rng(seed: int, stream: str, *extra: int) -> np.random.Generator:
    ss = _streams(seed)[stream]
    if extra:
        ss = np.random.SeedSequence(entropy=ss.entropy, spawn_key=ss.spawn_key + tuple(extra))
    return np.random.Generator(np.random.PCG64(ss))


def _normal(rng, shape, scale, dtype, values=True):
    """scale * N(0,1) in fp32, then (bf16) rounded: (bits or None, values or None)."""
    x = rng.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    if dtype == "bf16":
        bits = bf16_bits_rne(x)
        return bits, (bf16_bits_to_f32(bits) if values else None)
    return None, x


def make_qkv(wl: Workload, seed: Optional[int] = None, B=None, H=None, N=None):
    """q, k, v of shape [B,H,N,d] for a workload (sizes may be overridden).

    Returns a dict with float32 'q','k','v' (exact values) and, for bf16
    workloads, the uint16 bit patterns 'q_bits','k_bits','v_bits'.
    """
    seed = wl.index if seed is None else seed
    B = wl.B if B is None else B
    H = wl.H if H is None else H
    N = wl.N if N is None else N
    out = {}
    for name, d in (("q", wl.dk), ("k", wl.dk), ("v", wl.dv)):
        bits, vals = _normal(_rng(seed, name), (B, H, N, d), wl.scale, wl.dtype)
        out[name] = vals
        if bits is not None:
            out[name + "_bits"] = bits
    return out


def make_lambda(wl: Workload, seed: Optional[int] = None, H=None) -> np.ndarray:
    """Per-head decay as float32 [H]."""
    seed = wl.index if seed is None else seed
    H = wl.H if H is None else H
    if wl.lam == "one":
        return np.ones(H, dtype=np.float32)
    if wl.lam == "const":
        return np.full(H, wl.lam_value, dtype=np.float32)
    rng = _rng(seed, "lam")
    return rng.uniform(wl.lam_lo, wl.lam_hi, size=H).astype(np.float32)


def make_omega(m: int, dk: int, seed: int, orthogonal: bool = True) -> np.ndarray:
    """Random-feature directions omega [m, dk] float32.

    orthogonal=False: rows drawn independently from N(0, I).

    Rows are drawn from N(0, I) and orthogonalised in independent blocks of
    dk rows: each block is the Q factor of a dk x dk Gaussian matrix
    (sign-fixed by the diagonal of R so the factorisation is unique), and each
    row is then rescaled to the norm of a fresh N(0, I_dk) draw, so that rows
    keep the marginal distribution of N(0, I) while being exactly orthogonal
    within a block.
    """
    rng = _rng(seed, "omega")
    if not orthogonal:
        return np.ascontiguousarray(rng.standard_normal((m, dk)), dtype=np.float32)
    blocks = []
    remaining = m
    while remaining > 0:
        g = rng.standard_normal((dk, dk))
        qm, rm = np.linalg.qr(g)
        qm = qm * np.sign(np.diag(rm))[None, :]
        rows = qm.T                                   # orthonormal rows
        norms = np.linalg.norm(rng.standard_normal((dk, dk)), axis=1)
        blocks.append(rows * norms[:, None])
        remaining -= dk
    return np.ascontiguousarray(np.concatenate(blocks, axis=0)[:m], dtype=np.float32)


def make_inputs(wl: Workload, seed: Optional[int] = None, B=None, H=None, N=None):
    """Everything a forward call needs: q, k, v, lambda [H], omega or None."""
    seed = wl.index if seed is None else seed
    d = make_qkv(wl, seed, B, H, N)
    d["lam"] = make_lambda(wl, seed, H)
    d["omega"] = (make_omega(wl.m, wl.dk, seed, orthogonal=wl.omega == "orthogonal")
                  if wl.random_features else None)
    return d


def _pool_map(fn, items, threads):
    """Map fn over items on `threads` threads (numpy's generators release the
    GIL while they fill arrays, so independent streams draw in parallel)."""
    items = list(items)
    if threads <= 1 or len(items) <= 1:
        return [fn(i) for i in items]
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(min(threads, len(items))) as ex:
        return list(ex.map(fn, items))


def make_decode_prefix(wl: Workload, seed: Optional[int] = None, B=None, H=None, N=None,
                       threads: int = 1, values: bool = True, b0: int = 0):
    """The prefix tokens that initialise the decode state: [B,H,N,d], batch
    rows b0 .. b0+B-1 of the workload.

    Each (tensor, batch row) pair draws from a sub-stream of its own, so a
    smaller B keeps the first rows' values, any block of rows can be drawn on
    its own and rows can be drawn on several threads.  values=False returns
    only the bf16 bit patterns."""
    seed = wl.index if seed is None else seed
    B = wl.B if B is None else B
    H = wl.H if H is None else H
    N = wl.N if N is None else N
    out = {}
    for j, (name, d) in enumerate((("q", wl.dk), ("k", wl.dk), ("v", wl.dv))):
        rows = _pool_map(lambda b: _normal(_rng(seed, "prefix", j, b), (1, H, N, d), wl.scale, wl.dtype,
                                           values=values or wl.dtype != "bf16"),
                         range(b0, b0 + B), threads)
        if wl.dtype == "bf16":
            out[name + "_bits"] = np.concatenate([r[0] for r in rows], axis=0)
            if values:
                out[name] = bf16_bits_to_f32(out[name + "_bits"])
        else:
            out[name] = np.concatenate([r[1] for r in rows], axis=0)
    return out


def make_decode_step(wl: Workload, step: int, seed: Optional[int] = None, B=None, H=None, values: bool = True):
    """Single-token inputs of one decode step, [B,H,1,d]; regenerated from
    (seed, step) so that no trajectory needs to be stored.  values=False
    returns only the bf16 bit patterns of bf16 workloads."""
    seed = wl.index if seed is None else seed
    B = wl.B if B is None else B
    H = wl.H if H is None else H
    out = {}
    for j, (name, d) in enumerate((("q", wl.dk), ("k", wl.dk), ("v", wl.dv))):
        bits, vals = _normal(_rng(seed, "steps", step, j), (B, H, 1, d), wl.scale, wl.dtype,
                             values=values or wl.dtype != "bf16")
        if vals is not None:
            out[name] = vals
        if bits is not None:
            out[name + "_bits"] = bits
    return out


def make_decode_steps(wl: Workload, t0: int, t1: int, seed: Optional[int] = None, B=None, H=None,
                      threads: int = 1):
    """Steps t0..t1-1 of make_decode_step stacked on a leading axis:
    [t1-t0, B, H, 1, d] per tensor, bf16 bit patterns ('q_bits', ...) for
    bf16 workloads, float32 values ('q', ...) otherwise.  The same values as
    make_decode_step, drawn on `threads` threads."""
    bf = wl.dtype == "bf16"
    key = "_bits" if bf else ""
    first = make_decode_step(wl, t0, seed, B, H, values=not bf)
    out = {n + key: np.empty((t1 - t0,) + first[n + key].shape, dtype=first[n + key].dtype) for n in ("q", "k", "v")}

    def fill(t):
        st = first if t == t0 else make_decode_step(wl, t, seed, B, H, values=not bf)
        for n in ("q", "k", "v"):
            out[n + key][t - t0] = st[n + key]

    _pool_map(fill, range(t0, t1), threads)
    return out


# --------------------------------------------------------------------------
# masks, cross attention and packed sequences
# --------------------------------------------------------------------------
def make_kv(wl: Workload, n_kv: int, seed: Optional[int] = None, B=None, H=None):
    """Keys and values of their own length n_kv (cross attention): 'k', 'v'
    [B,H,n_kv,d] (and '_bits' for bf16), from a stream of their own."""
    seed = wl.index if seed is None else seed
    B = wl.B if B is None else B
    H = wl.H if H is None else H
    out = {}
    for i, (name, d) in enumerate((("k", wl.dk), ("v", wl.dv))):
        bits, vals = _normal(_rng(seed, "kv", i), (B, H, n_kv, d), wl.scale, wl.dtype)
        out[name] = vals
        if bits is not None:
            out[name + "_bits"] = bits
    return out


def make_key_padding_mask(B: int, N: int, kind: str = "right", seed: int = 0, p: float = 0.25) -> np.ndarray:
    """Key padding mask [B,N] bool, True = padded (ignored) key.

    kind "right": a padded batch -- batch b keeps its first L_b keys, L_0 = N
    and the others uniform in [1, N]; "random": each key padded independently
    with probability p; "none" / "all": no key / every key padded."""
    if kind == "none":
        return np.zeros((B, N), dtype=bool)
    if kind == "all":
        return np.ones((B, N), dtype=bool)
    rng = _rng(seed, "mask")
    if kind == "random":
        return rng.random((B, N)) < p
    if kind == "right":
        lens = rng.integers(1, N + 1, size=B)
        lens[0] = N
        return np.arange(N)[None, :] >= lens[:, None]
    raise ValueError(kind)


def make_varlen_lengths(n_seq: int, max_len: int, seed: int = 0, empty: int = 0) -> np.ndarray:
    """Lengths of n_seq packed sequences: log-uniform in [1, max_len] (many
    short, some long), one of exactly max_len, and `empty` zero-length ones
    placed at random positions."""
    rng = _rng(seed, "lens")
    lens = np.exp(rng.uniform(0.0, np.log(max_len), size=n_seq)).astype(np.int64)
    lens = np.clip(lens, 1, max_len)
    lens[rng.integers(n_seq)] = max_len
    if empty:
        lens[rng.choice(n_seq, size=empty, replace=False)] = 0
    return lens


def cu_seqlens(lengths) -> np.ndarray:
    """Offsets [n_seq + 1] int32 of sequences packed back to back."""
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int32)


def pack_heads(wl: Workload, T: int, seed: Optional[int] = None, H=None):
    """q, k, v for T packed tokens per head: [1,H,T,d] (the packed layout is
    one row of T tokens per head)."""
    return make_qkv(wl, seed=seed, B=1, H=H, N=T)
