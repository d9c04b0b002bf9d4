"""Python face of the plain CPU oracle (fsl_oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module; the product path never does. It builds
the C oracle with gcc (fp64 arithmetic, no fast-math, no contraction) and wraps
each step of the method for the pins, plus a whole-forward driver.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fsl_oracle.c")
_LIB = os.path.join(_HERE, "libfsl_oracle.so")


def build(force: bool = True) -> str:
    """Compile the oracle into oracle/libfsl_oracle.so and return its path."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-ffp-contract=off", "-fno-fast-math", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


class Head(ctypes.Structure):
    _fields_ = [
        ("N", ctypes.c_int64), ("d", ctypes.c_int32), ("w", ctypes.c_int32),
        ("s", ctypes.c_int32), ("P", ctypes.c_int32), ("W", ctypes.c_int32),
        ("K", ctypes.c_int32), ("B", ctypes.c_int32), ("pad_", ctypes.c_int32),
        ("scale", ctypes.c_double), ("rho", ctypes.c_double),
        ("rope_base", ctypes.c_double), ("rms_eps", ctypes.c_double),
        ("sigma", ctypes.c_double), ("lam", ctypes.c_double), ("gamma", ctypes.c_double),
    ]


class FsbParams(ctypes.Structure):
    _fields_ = [("proj", ctypes.c_void_p), ("tau", ctypes.c_double), ("beam", ctypes.c_int32),
                ("pad_", ctypes.c_int32)]


_lib = None


def lib():
    """The loaded oracle. FSL_ORACLE_LIB names another build of fsl_oracle.c
    (the mutation test loads deliberately broken copies this way)."""
    global _lib
    if _lib is None:
        path = os.environ.get("FSL_ORACLE_LIB")
        if not path:
            path = _LIB
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
        L = ctypes.CDLL(path)
        P = ctypes.POINTER
        f32p, f64p, i32p, i64p = P(ctypes.c_float), P(ctypes.c_double), P(ctypes.c_int32), P(ctypes.c_int64)
        hp = P(Head)
        L.orc_num_cells.restype = ctypes.c_int64; L.orc_num_cells.argtypes = [hp]
        L.orc_num_blocks.restype = ctypes.c_int64; L.orc_num_blocks.argtypes = [hp]
        L.orc_eligible.restype = ctypes.c_int64; L.orc_eligible.argtypes = [ctypes.c_int64, hp]
        L.orc_cell_stats.restype = None; L.orc_cell_stats.argtypes = [f32p, hp, f32p, f32p]
        L.orc_pool.restype = ctypes.c_int32; L.orc_pool.argtypes = [f32p, ctypes.c_int64, hp, i32p]
        L.orc_cell_score.restype = ctypes.c_double
        L.orc_cell_score.argtypes = [f32p, ctypes.c_int64, f32p, ctypes.c_float, ctypes.c_int64, hp]
        L.orc_select.restype = ctypes.c_int32
        L.orc_select.argtypes = [f32p, ctypes.c_int64, f32p, f32p, i32p, ctypes.c_int32, hp, i32p, f64p]
        L.orc_rope.restype = None; L.orc_rope.argtypes = [f32p, ctypes.c_int64, hp, f64p]
        L.orc_window.restype = None; L.orc_window.argtypes = [f64p, f64p, f32p, ctypes.c_int64, hp, f64p]
        L.orc_readout.restype = None; L.orc_readout.argtypes = [f32p, f32p, f32p, i32p, ctypes.c_int32, hp, f64p]
        L.orc_mix.restype = None; L.orc_mix.argtypes = [f64p, f64p, hp, f64p]
        L.orc_backward_head.restype = ctypes.c_int
        L.orc_backward_head.argtypes = [f32p, f32p, f32p, f32p, i32p, hp, f64p, f64p, f64p, f64p]
        u32p = P(ctypes.c_uint32)
        L.orc_fsb_code.restype = ctypes.c_uint32; L.orc_fsb_code.argtypes = [f32p, f32p, ctypes.c_int]
        L.orc_fsb_select.restype = ctypes.c_int
        L.orc_fsb_select.argtypes = [f32p, f32p, hp, P(FsbParams), i64p, ctypes.c_int64, i32p, f64p]
        L.orc_forward_rows_sel.restype = ctypes.c_int
        L.orc_forward_rows_sel.argtypes = [f32p, f32p, f32p, hp, i64p, ctypes.c_int64, i32p, f64p, f64p, f64p]
        L.orc_fsb_tree_dump.restype = None
        L.orc_fsb_tree_dump.argtypes = [i32p, ctypes.c_int64, ctypes.c_int, u32p, f32p, f32p, hp, i32p, f32p, f64p,
                                        f32p, i64p]
        L.orc_fsb_tree_bounds.restype = None
        L.orc_fsb_tree_bounds.argtypes = [i32p, ctypes.c_int64, ctypes.c_int, u32p, f32p, f32p, hp, f32p,
                                          ctypes.c_int64, f64p]
        L.orc_forward_head.restype = ctypes.c_int
        L.orc_forward_head.argtypes = [f32p, f32p, f32p, hp, i64p, ctypes.c_int64, f64p, f64p, f64p,
                                       i32p, f64p, i32p, ctypes.c_int32, f32p, f32p, ctypes.c_int]
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray], ctype):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def head(N, d, w=512, s=32, P=64, W=8, K=4, B=128, scale=None, rho=1.0, rope_base=10000.0,
         rms_eps=1e-6, sigma=4.0, lam=1.0, gamma=1.0) -> Head:
    """Parameters of one head. scale defaults to 1/sqrt(d)."""
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    return Head(N=N, d=d, w=w, s=s, P=P, W=W, K=K, B=B, pad_=0, scale=float(scale), rho=float(rho),
                rope_base=float(rope_base), rms_eps=float(rms_eps), sigma=float(sigma),
                lam=float(lam), gamma=float(gamma))


def head_from_shape(shape, h: int, sigma, lam, gamma, N: Optional[int] = None, scale=None) -> Head:
    """Head parameters of head h of a workload (scale as a float32 value, like the GPU's)."""
    sc = np.float32(1.0 / np.sqrt(shape.d)) if scale is None else np.float32(scale)
    return head(N=shape.N if N is None else N, d=shape.d, w=shape.w, s=shape.s, P=shape.P, W=shape.W,
                K=shape.K, B=shape.B, scale=float(sc), rho=float(np.float32(shape.rho)),
                rope_base=float(np.float32(shape.rope_base)), rms_eps=float(np.float32(shape.rms_eps)),
                sigma=float(np.float32(sigma[h])), lam=float(np.float32(lam[h])),
                gamma=float(np.float32(gamma[h])))


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


# ---------------------------------------------------------------------------
# single steps

def num_cells(p: Head) -> int:
    return int(lib().orc_num_cells(ctypes.byref(p)))


def num_blocks(p: Head) -> int:
    return int(lib().orc_num_blocks(ctypes.byref(p)))


def eligible(b: int, p: Head) -> int:
    return int(lib().orc_eligible(b, ctypes.byref(p)))


def cell_stats(k: np.ndarray, p: Head):
    k = _f32(k)
    C = num_cells(p)
    kbar = np.zeros((max(C, 1), p.d), np.float32)
    amax = np.zeros(max(C, 1), np.float32)
    lib().orc_cell_stats(_p(k, ctypes.c_float), ctypes.byref(p), _p(kbar, ctypes.c_float), _p(amax, ctypes.c_float))
    return kbar[:C], amax[:C]


def pool(amax: np.ndarray, b: int, p: Head) -> np.ndarray:
    amax = _f32(amax)
    cap = max(num_cells(p), 1) if p.P < 0 else max(p.P + p.W, 1)
    out = np.full(cap, -1, np.int32)
    n = lib().orc_pool(_p(amax, ctypes.c_float), b, ctypes.byref(p), _p(out, ctypes.c_int32))
    return out[:n].copy()


def cell_score(q_i, i, kbar_c, a_c, c, p: Head) -> float:
    q_i = _f32(q_i); kbar_c = _f32(kbar_c)
    return float(lib().orc_cell_score(_p(q_i, ctypes.c_float), i, _p(kbar_c, ctypes.c_float),
                                      float(a_c), c, ctypes.byref(p)))


def select(q_i, i, kbar, amax, pool_ids, p: Head):
    q_i = _f32(q_i); kbar = _f32(kbar); amax = _f32(amax)
    pool_ids = np.ascontiguousarray(pool_ids, dtype=np.int32)
    sel = np.full(p.K, -1, np.int32)
    margin = np.zeros(1, np.float64)
    n = lib().orc_select(_p(q_i, ctypes.c_float), i, _p(kbar, ctypes.c_float), _p(amax, ctypes.c_float),
                         _p(pool_ids, ctypes.c_int32), len(pool_ids), ctypes.byref(p),
                         _p(sel, ctypes.c_int32), _p(margin, ctypes.c_double))
    return sel, int(n), float(margin[0])


def rope(x, t, p: Head) -> np.ndarray:
    x = _f32(x)
    out = np.zeros(p.d, np.float64)
    lib().orc_rope(_p(x, ctypes.c_float), t, ctypes.byref(p), _p(out, ctypes.c_double))
    return out


def window(qrot, krot, v, i, p: Head) -> np.ndarray:
    qrot = np.ascontiguousarray(qrot, np.float64); krot = np.ascontiguousarray(krot, np.float64)
    v = _f32(v)
    o = np.zeros(p.d, np.float64)
    lib().orc_window(_p(qrot, ctypes.c_double), _p(krot, ctypes.c_double), _p(v, ctypes.c_float), i,
                     ctypes.byref(p), _p(o, ctypes.c_double))
    return o


def readout(q_i, k, v, sel, p: Head) -> np.ndarray:
    q_i = _f32(q_i); k = _f32(k); v = _f32(v)
    sel = np.ascontiguousarray([c for c in sel if c >= 0], dtype=np.int32)
    o = np.zeros(p.d, np.float64)
    lib().orc_readout(_p(q_i, ctypes.c_float), _p(k, ctypes.c_float), _p(v, ctypes.c_float),
                      _p(sel, ctypes.c_int32), len(sel), ctypes.byref(p), _p(o, ctypes.c_double))
    return o


def mix(o_win, o_long, p: Head) -> np.ndarray:
    a = np.ascontiguousarray(o_win, np.float64); b = np.ascontiguousarray(o_long, np.float64)
    out = np.zeros(p.d, np.float64)
    lib().orc_mix(_p(a, ctypes.c_double), _p(b, ctypes.c_double), ctypes.byref(p), _p(out, ctypes.c_double))
    return out


# ---------------------------------------------------------------------------
# whole forward

def forward_head(q, k, v, p: Head, rows: Optional[Sequence[int]] = None, want_pool: bool = False,
                 want_stats: bool = False, nthreads: int = 0):
    """Forward of one head ([N][d] arrays) at the given query rows (default: all)."""
    q = _f32(q); k = _f32(k); v = _f32(v)
    N, d = p.N, p.d
    assert q.shape == (N, d) and k.shape == (N, d) and v.shape == (N, d)
    rows = np.arange(N, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    R = len(rows)
    out = np.zeros((R, d), np.float64); ow = np.zeros((R, d), np.float64); ol = np.zeros((R, d), np.float64)
    sel = np.full((R, p.K), -1, np.int32); margin = np.zeros(R, np.float64)
    C = num_cells(p); nblk = num_blocks(p)
    cap = (max(C, 1) if p.P < 0 else p.P + p.W)
    pool_out = np.full((nblk, max(cap, 1)), -1, np.int32) if want_pool else None
    kbar = np.zeros((max(C, 1), d), np.float32) if want_stats else None
    amax = np.zeros(max(C, 1), np.float32) if want_stats else None
    rc = lib().orc_forward_head(_p(q, ctypes.c_float), _p(k, ctypes.c_float), _p(v, ctypes.c_float),
                                ctypes.byref(p), _p(rows, ctypes.c_int64), R,
                                _p(out, ctypes.c_double), _p(ow, ctypes.c_double), _p(ol, ctypes.c_double),
                                _p(sel, ctypes.c_int32), _p(margin, ctypes.c_double),
                                _p(pool_out, ctypes.c_int32), max(cap, 1),
                                _p(kbar, ctypes.c_float), _p(amax, ctypes.c_float), nthreads)
    if rc != 0:
        raise ValueError(f"oracle rejected the parameters (code {rc})")
    res = dict(rows=rows, out=out, o_win=ow, o_long=ol, sel=sel, margin=margin)
    if want_pool:
        res["pool"] = pool_out[:, :cap] if cap > 0 else pool_out[:, :0]
    if want_stats:
        res["kbar"] = kbar[:C]; res["amax"] = amax[:C]
    return res


def forward(inputs, rows: Optional[Sequence[int]] = None, heads: Optional[Sequence[int]] = None,
            want_pool: bool = False, want_stats: bool = False, nthreads: int = 0, **overrides):
    """Forward of a synth.Inputs workload; returns a list of per-head results."""
    shape = inputs.shape
    heads = range(shape.H) if heads is None else heads
    res = []
    for h in heads:
        p = head_from_shape(shape, h, inputs.sigma, inputs.lam, inputs.gamma)
        for key, val in overrides.items():
            setattr(p, key, val)
        res.append(forward_head(inputs.q[h], inputs.k[h], inputs.v[h], p, rows, want_pool,
                                want_stats, nthreads))
    return res


# ---------------------------------------------------------------------------
# backward (training): gradients with the forward's selection held fixed

def backward_head(q, k, v, dout, sel, p: Head):
    """dq, dk, dv ([N][d] fp64) and dgamma of one head, for upstream gradient dout [N][d] and the
    forward's selection sel [N][K] (held fixed: the hard indices receive no gradient)."""
    q = _f32(q); k = _f32(k); v = _f32(v); dout = _f32(dout)
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    N, d = p.N, p.d
    assert q.shape == (N, d) and k.shape == (N, d) and v.shape == (N, d) and dout.shape == (N, d)
    assert sel.shape == (N, p.K)
    dq = np.zeros((N, d), np.float64); dk = np.zeros((N, d), np.float64); dv = np.zeros((N, d), np.float64)
    dg = np.zeros(1, np.float64)
    rc = lib().orc_backward_head(_p(q, ctypes.c_float), _p(k, ctypes.c_float), _p(v, ctypes.c_float),
                                 _p(dout, ctypes.c_float), _p(sel, ctypes.c_int32), ctypes.byref(p),
                                 _p(dq, ctypes.c_double), _p(dk, ctypes.c_double), _p(dv, ctypes.c_double),
                                 _p(dg, ctypes.c_double))
    if rc != 0:
        raise ValueError(f"oracle rejected the parameters (code {rc})")
    return dict(dq=dq, dk=dk, dv=dv, dgamma=float(dg[0]))


def backward(inputs, dout, sels, heads=None, workers: int = 0, **overrides):
    """Backward of a synth.Inputs workload: one result per head, heads run in parallel threads
    (the oracle call releases the GIL); sels[h] is head h's forward selection [N][K]."""
    from concurrent.futures import ThreadPoolExecutor
    shape = inputs.shape
    heads = list(range(shape.H)) if heads is None else list(heads)

    def one(h):
        p = head_from_shape(shape, h, inputs.sigma, inputs.lam, inputs.gamma)
        for key, val in overrides.items():
            setattr(p, key, val)
        return backward_head(inputs.q[h], inputs.k[h], inputs.v[h], dout[h], sels[h], p)

    n = workers or min(len(heads), len(os.sched_getaffinity(0)), 16)
    with ThreadPoolExecutor(max_workers=max(1, n)) as ex:
        return list(ex.map(one, heads))


# ---------------------------------------------------------------------------
# FS-B (beam search over two causal forests)

def fsb_code(x, proj) -> int:
    x = _f32(x); proj = _f32(proj)
    return int(lib().orc_fsb_code(_p(x, ctypes.c_float), _p(proj, ctypes.c_float), x.shape[-1]))


def fsb_select(q, k, p: Head, proj, tau: float, beam: int = 16, rows: Optional[Sequence[int]] = None):
    """FS-B selections of one head at the given rows (default all): sel [R][K] and the rerank
    log-sum-exp of each selected cell [R][K] (NaN for padding)."""
    q = _f32(q); k = _f32(k); proj = _f32(proj)
    assert proj.shape == (32, p.d)
    rows = np.arange(p.N, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    R = len(rows)
    sel = np.full((R, p.K), -1, np.int32)
    lse = np.zeros((R, p.K), np.float64)
    fb = FsbParams(proj=proj.ctypes.data, tau=float(tau), beam=int(beam), pad_=0)
    rc = lib().orc_fsb_select(_p(q, ctypes.c_float), _p(k, ctypes.c_float), ctypes.byref(p), ctypes.byref(fb),
                              _p(rows, ctypes.c_int64), R, _p(sel, ctypes.c_int32), _p(lse, ctypes.c_double))
    if rc != 0:
        raise ValueError(f"oracle rejected the parameters (code {rc})")
    return sel, lse


def forward_rows_sel(q, k, v, p: Head, rows, sel):
    """Forward outputs (out, o_win, o_long) at the given rows for a given selection [R][K]."""
    q = _f32(q); k = _f32(k); v = _f32(v)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    R, d = len(rows), p.d
    out = np.zeros((R, d)); ow = np.zeros((R, d)); ol = np.zeros((R, d))
    rc = lib().orc_forward_rows_sel(_p(q, ctypes.c_float), _p(k, ctypes.c_float), _p(v, ctypes.c_float),
                                    ctypes.byref(p), _p(rows, ctypes.c_int64), R, _p(sel, ctypes.c_int32),
                                    _p(out, ctypes.c_double), _p(ow, ctypes.c_double), _p(ol, ctypes.c_double))
    if rc != 0:
        raise ValueError(f"oracle rejected the parameters (code {rc})")
    return out, ow, ol


def fsb_tree(list_cells, a: int, k: int, codes, kbar, amax, p: Head):
    """One segment tree of a list: leaf cells [L], mu [2L][d], rad, amax, pmin [2L] (heap order, index 0 unused)."""
    lst = np.ascontiguousarray(list_cells, dtype=np.int32)
    codes = np.ascontiguousarray(codes, dtype=np.uint32)
    kbar = _f32(kbar); amax = _f32(amax)
    L = 1 << k
    cell = np.zeros(L, np.int32); mu = np.zeros((2 * L, p.d), np.float32); rad = np.zeros(2 * L)
    am = np.zeros(2 * L, np.float32); pmin = np.zeros(2 * L, np.int64)
    lib().orc_fsb_tree_dump(_p(lst, ctypes.c_int32), a, k, _p(codes, ctypes.c_uint32), _p(kbar, ctypes.c_float),
                            _p(amax, ctypes.c_float), ctypes.byref(p), _p(cell, ctypes.c_int32),
                            _p(mu, ctypes.c_float), _p(rad, ctypes.c_double), _p(am, ctypes.c_float),
                            _p(pmin, ctypes.c_int64))
    return dict(cell=cell, mu=mu, rad=rad, amax=am, pmin=pmin)


def fsb_tree_bounds(list_cells, a: int, k: int, codes, kbar, amax, p: Head, q_i, i: int):
    """Upper bound of every node of one segment tree for query q_i at position i ([2L], index 0 unused)."""
    lst = np.ascontiguousarray(list_cells, dtype=np.int32)
    codes = np.ascontiguousarray(codes, dtype=np.uint32)
    kbar = _f32(kbar); amax = _f32(amax); q_i = _f32(q_i)
    ub = np.zeros(2 << k)
    lib().orc_fsb_tree_bounds(_p(lst, ctypes.c_int32), a, k, _p(codes, ctypes.c_uint32), _p(kbar, ctypes.c_float),
                              _p(amax, ctypes.c_float), ctypes.byref(p), _p(q_i, ctypes.c_float), i,
                              _p(ub, ctypes.c_double))
    return ub
