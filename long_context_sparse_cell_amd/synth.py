"""Seeded synthetic inputs for the FS-L attention workloads.

This module is the only code shared by the oracle side and the HIP side. It
draws q/k/v tensors and plants the structure the workloads call for (norm
outliers, needles, probe queries); it computes none of the method's
arithmetic. Every tensor is returned as float32 holding values that are
exactly representable in the workload dtype (bf16 values are rounded to
nearest-even once, after planting), so both sides read identical numbers.

Workloads follow the FreeSolo pages: window w=512, cells of s=32 tokens,
P=64 high-norm cells plus W=8 recent cells, top K=4 cells, query blocks of
B=128 ("FreeSolo" digest, section on the core method; ai.info summary,
"Methodology in Plain English"), routing scalars sigma_h=4, lambda_h=1 (ai.info
summary, training paragraph). The planted needles stand in for the RULER
single/multi-needle retrieval tasks the pages evaluate on; they are vectors in
key space, not text.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"


@dataclasses.dataclass(frozen=True)
class Shape:
    """Sizes and method parameters of one workload (all plain integers)."""

    name: str
    H: int
    N: int
    d: int
    dtype: str
    seed: int
    w: int = 512
    s: int = 32
    P: int = 64
    W: int = 8
    K: int = 4
    B: int = 128
    rope_base: float = 10000.0
    rms_eps: float = 1e-6
    rho: float = 1.0
    # decode workloads only
    n_seq: int = 0
    prefix: int = 0
    steps: int = 0
    kind: str = "fwd"

    def replace(self, **kw) -> "Shape":
        return dataclasses.replace(self, **kw)


# The five workloads: four forward shapes and one streaming-decode shape.
CONFIGS: Dict[str, Shape] = {
    "fwd_f32_n4096": Shape("fwd_f32_h1_n4096_d64", H=1, N=4096, d=64, dtype=F32, seed=1),
    "fwd_bf16_n16384": Shape("fwd_bf16_h16_n16384_d64", H=16, N=16384, d=64, dtype=BF16, seed=2),
    "fwd_bf16_n65536": Shape("fwd_bf16_h16_n65536_d64", H=16, N=65536, d=64, dtype=BF16, seed=3),
    "fwd_bf16_n262144": Shape("fwd_bf16_h8_n262144_d128", H=8, N=262144, d=128, dtype=BF16, seed=4),
    "decode_64seq": Shape("decode_bf16_64seq_h16_d64_prefix131072", H=16, N=131072 + 256, d=64,
                dtype=BF16, seed=5, n_seq=64, prefix=131072, steps=256, kind="decode"),
}


# ----------------------------------------------------------------------------
# bf16 helpers (storage format only)
# ----------------------------------------------------------------------------

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16, nearest-even; return the uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_values(bits: np.ndarray) -> np.ndarray:
    """Float32 values of bfloat16 bit patterns (exact)."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 data to the workload dtype; result is float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == F32:
        return x
    if dtype == BF16:
        return bf16_values(bf16_bits(x))
    raise ValueError(f"unknown dtype {dtype!r}")


# ----------------------------------------------------------------------------
# per-head scalars
# ----------------------------------------------------------------------------

def head_scalars(H: int, sigma: float = 4.0, lam: float = 1.0):
    """sigma_h, lambda_h (fixed routing scalars) and a stand-in gamma_h.

    No trained mixing coefficient exists, so gamma_h spreads over [0.25, 1]
    across heads; distinct values make a head mix-up visible.
    """
    sig = np.full(H, sigma, dtype=np.float32)
    lamb = np.full(H, lam, dtype=np.float32)
    gam = (0.25 + 0.75 * np.arange(H, dtype=np.float64) / max(H - 1, 1)).astype(np.float32)
    return sig, lamb, gam


@dataclasses.dataclass
class Inputs:
    shape: Shape
    q: np.ndarray  # [H][N][d] float32, values exact in shape.dtype
    k: np.ndarray
    v: np.ndarray
    sigma: np.ndarray  # [H] float32
    lam: np.ndarray
    gamma: np.ndarray
    needles: List[List[int]] = dataclasses.field(default_factory=list)  # per head: token positions
    probes: List[List[int]] = dataclasses.field(default_factory=list)   # per head: probe query rows (aligned with needles)


def _normal(rng, shape):
    return rng.standard_normal(size=shape, dtype=np.float32)


def _unit(x: np.ndarray) -> np.ndarray:
    x64 = x.astype(np.float64)
    return (x64 / np.linalg.norm(x64)).astype(np.float32)


def eligible_token_limit(N: int, w: int, s: int, B: int) -> int:
    """Tokens below this position lie in complete cells eligible for the last block.

    Structure helper for planting needles where the last query block can reach
    them (the first query of the block sees cells wholly before its window).
    """
    t0 = ((N - 1) // B) * B
    nb = max(0, (t0 - w + 1) // s)
    return nb * s


def random_inputs(shape: Shape, seed: Optional[int] = None, q_scale: float = 1.0) -> Inputs:
    """q, k, v ~ N(0, 1), no planted structure."""
    rng = np.random.default_rng(shape.seed if seed is None else seed)
    dims = (shape.H, shape.N, shape.d)
    q = _normal(rng, dims) * np.float32(q_scale)
    k = _normal(rng, dims)
    v = _normal(rng, dims)
    sig, lamb, gam = head_scalars(shape.H)
    return Inputs(shape, to_dtype(q, shape.dtype), to_dtype(k, shape.dtype),
                  to_dtype(v, shape.dtype), sig, lamb, gam)


def _plant_equal_norm_needles(rng, q, k, h, n_needles, cell_limit, s, forbid_cells, N):
    """Needles of equal norm (4x the largest key norm of the head) in distinct cells."""
    C_lim = cell_limit // s
    allowed = np.setdiff1d(np.arange(C_lim), np.asarray(sorted(forbid_cells), dtype=np.int64))
    cells = rng.choice(allowed, size=n_needles, replace=False)
    kmax = float(np.max(np.linalg.norm(k[h].astype(np.float64), axis=1)))
    pos, probes = [], []
    for m, c in enumerate(cells):
        p = int(c) * s + int(rng.integers(0, s))
        k[h, p] = (_unit(k[h, p]).astype(np.float64) * 4.0 * kmax).astype(np.float32)
        row = N - 1 - m
        q[h, row] = _unit(k[h, p])
        pos.append(p)
        probes.append(row)
    return pos, probes


def make_inputs(shape: Shape) -> Inputs:
    """The seeded inputs of one forward workload (see CONFIGS)."""
    H, N, d, s = shape.H, shape.N, shape.d, shape.s
    rng = np.random.default_rng(shape.seed)
    dims = (H, N, d)
    limit = eligible_token_limit(N, shape.w, s, shape.B)
    needles: List[List[int]] = []
    probes: List[List[int]] = []
    if shape.seed == 1:
        # one needle: a key beyond the first 512 tokens scaled by 4, copied (unit) into the last query
        q = _normal(rng, dims); k = _normal(rng, dims); v = _normal(rng, dims)
        for h in range(H):
            p = int(rng.integers(512, limit))
            k[h, p] *= np.float32(4.0)
            q[h, N - 1] = _unit(k[h, p])
            needles.append([p]); probes.append([N - 1])
    elif shape.seed == 2:
        # 5% of cells get one token key scaled by 3; 4 equal-norm needles per head
        q = _normal(rng, dims); k = _normal(rng, dims); v = _normal(rng, dims)
        C = N // s
        n_out = int(round(0.05 * C))
        for h in range(H):
            cells = rng.choice(C, size=n_out, replace=False)
            for c in cells:
                t = int(c) * s + int(rng.integers(0, s))
                k[h, t] *= np.float32(3.0)
            pos, pr = _plant_equal_norm_needles(rng, q, k, h, 4, limit, s, set(int(c) for c in cells), N)
            needles.append(pos); probes.append(pr)
    elif shape.seed == 3:
        # k: log-normal norm times a uniform direction; 8 equal-norm needles per head
        q = _normal(rng, dims)
        g = _normal(rng, dims).astype(np.float64)
        rho = rng.lognormal(mean=0.0, sigma=0.5, size=(H, N, 1))
        k = (g / np.linalg.norm(g, axis=2, keepdims=True) * rho).astype(np.float32)
        del g
        v = _normal(rng, dims)
        for h in range(H):
            pos, pr = _plant_equal_norm_needles(rng, q, k, h, 8, limit, s, set(), N)
            needles.append(pos); probes.append(pr)
    elif shape.seed == 4:
        # one needle per head scaled by 4; the whole last block of queries probes it
        q = _normal(rng, dims); k = _normal(rng, dims); v = _normal(rng, dims)
        for h in range(H):
            p = int(rng.integers(0, limit))
            k[h, p] *= np.float32(4.0)
            u = _unit(k[h, p])
            last0 = ((N - 1) // shape.B) * shape.B
            q[h, last0:N] = u
            needles.append([p]); probes.append(list(range(last0, N)))
    else:
        return random_inputs(shape)
    sig, lamb, gam = head_scalars(H)
    return Inputs(shape, to_dtype(q, shape.dtype), to_dtype(k, shape.dtype),
                  to_dtype(v, shape.dtype), sig, lamb, gam, needles, probes)


@dataclasses.dataclass
class DecodeSeq:
    """One sequence of the decode workload: a prefix and the streamed steps."""

    k_prefix: np.ndarray  # [H][prefix][d]
    v_prefix: np.ndarray
    q_steps: np.ndarray   # [steps][H][d]
    k_steps: np.ndarray
    v_steps: np.ndarray


def decode_sequence(shape: Shape, r: int, prefix: Optional[int] = None,
                    steps: Optional[int] = None) -> DecodeSeq:
    """Sequence r of a decode workload, from its own sub-stream of the seed."""
    prefix = shape.prefix if prefix is None else prefix
    steps = shape.steps if steps is None else steps
    rng = np.random.default_rng([shape.seed, r])
    H, d = shape.H, shape.d
    kp = to_dtype(_normal(rng, (H, prefix, d)), shape.dtype)
    vp = to_dtype(_normal(rng, (H, prefix, d)), shape.dtype)
    qs = to_dtype(_normal(rng, (steps, H, d)), shape.dtype)
    ks = to_dtype(_normal(rng, (steps, H, d)), shape.dtype)
    vs = to_dtype(_normal(rng, (steps, H, d)), shape.dtype)
    return DecodeSeq(kp, vp, qs, ks, vs)


def full_sequence(seq: DecodeSeq):
    """k, v of prefix + steps as [H][T][d], and q as [H][T][d] (prefix rows zero)."""
    H, prefix, d = seq.k_prefix.shape
    steps = seq.q_steps.shape[0]
    T = prefix + steps
    k = np.empty((H, T, d), np.float32)
    v = np.empty((H, T, d), np.float32)
    q = np.zeros((H, T, d), np.float32)
    k[:, :prefix] = seq.k_prefix
    v[:, :prefix] = seq.v_prefix
    k[:, prefix:] = seq.k_steps.transpose(1, 0, 2)
    v[:, prefix:] = seq.v_steps.transpose(1, 0, 2)
    q[:, prefix:] = seq.q_steps.transpose(1, 0, 2)
    return q, k, v
