"""Thin Python binding of the FS-L HIP library (libfsl.so, include/fsl.h).

Argument marshalling only: every step of the computation runs in the
library's HIP kernels. torch supplies device memory and the current stream.
If the library has not been built this module raises on first use; there is
no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfsl.so")

FSL_OK, FSL_E_INVAL, FSL_E_UNSUPPORTED, FSL_E_WORKSPACE, FSL_E_STATE, FSL_E_HIP = 0, -1, -2, -3, -4, -5
FSL_F32, FSL_BF16 = 0, 1


class FSLError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {strerror(code)} (status {code})")


class Params(ctypes.Structure):
    _fields_ = [
        ("N", ctypes.c_int64), ("H", ctypes.c_int32), ("d", ctypes.c_int32), ("w", ctypes.c_int32),
        ("s", ctypes.c_int32), ("P", ctypes.c_int32), ("W", ctypes.c_int32), ("K", ctypes.c_int32),
        ("B", ctypes.c_int32), ("dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
        ("scale", ctypes.c_float), ("rho", ctypes.c_float), ("rope_base", ctypes.c_float),
        ("rms_eps", ctypes.c_float), ("sigma", ctypes.c_void_p), ("lam", ctypes.c_void_p),
        ("gamma", ctypes.c_void_p),
    ]


class WorkspaceLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("kbar", "amax", "pool", "sel", "rope", "scan_a", "scan_i", "o_win", "rope_abs", "kt", "vt",
                                      "fixups", "khi", "klo", "kcf", "total")]


_lib = None


def lib():
    """The loaded library; raises if libfsl.so has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"FS-L HIP library not built: {LIB_PATH} is missing "
                               "(run __graft_entry__.build() or long_context_sparse_cell_amd/build.py)")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        pp = ctypes.POINTER(Params)
        L.fsl_version.restype = i32; L.fsl_version.argtypes = []
        L.fsl_strerror.restype = ctypes.c_char_p; L.fsl_strerror.argtypes = [i32]
        L.fsl_check_params.restype = i32; L.fsl_check_params.argtypes = [pp]
        L.fsl_workspace_bytes.restype = sz; L.fsl_workspace_bytes.argtypes = [pp]
        L.fsl_workspace_views.restype = i32; L.fsl_workspace_views.argtypes = [pp, ctypes.POINTER(WorkspaceLayout)]
        L.fsl_cell_stats.restype = i32; L.fsl_cell_stats.argtypes = [vp, vp, vp, pp, vp]
        L.fsl_prune_select.restype = i32
        L.fsl_prune_select.argtypes = [vp, vp, vp, vp, vp, pp, vp, sz, vp]
        L.fsl_attn_fwd.restype = i32
        L.fsl_attn_fwd.argtypes = [vp, vp, vp, vp, pp, vp, sz, vp, vp, vp, vp]
        L.fsl_attn_fwd_timed.restype = i32
        L.fsl_attn_fwd_timed.argtypes = [vp, vp, vp, vp, pp, vp, sz, vp, vp]
        i64 = ctypes.c_int64
        L.fsl_decode_state_bytes.restype = sz; L.fsl_decode_state_bytes.argtypes = [pp, ctypes.c_int32]
        L.fsl_decode_init.restype = i32; L.fsl_decode_init.argtypes = [vp, sz, ctypes.c_int32, pp, vp]
        L.fsl_decode_prefill_workspace_bytes.restype = sz
        L.fsl_decode_prefill_workspace_bytes.argtypes = [pp, i64]
        L.fsl_decode_prefill.restype = i32
        L.fsl_decode_prefill.argtypes = [vp, sz, ctypes.c_int32, vp, vp, i64, pp, vp, sz, vp]
        L.fsl_decode_append.restype = i32
        L.fsl_decode_append.argtypes = [vp, sz, ctypes.c_int32, ctypes.c_int32, vp, vp, i64, pp, vp]
        L.fsl_decode_step.restype = i32
        L.fsl_decode_step.argtypes = [vp, sz, vp, vp, vp, vp, ctypes.c_int32, pp, vp, vp]
        L.fsl_decode_validate.restype = i32
        L.fsl_decode_validate.argtypes = [vp, sz, pp, ctypes.c_int32]
        _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().fsl_strerror(code).decode()


def _check(code: int, where: str):
    if code != FSL_OK:
        raise FSLError(code, where)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the FS-L library must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return FSL_F32
    if t == torch.bfloat16:
        return FSL_BF16
    raise ValueError(f"unsupported dtype {t}")


def make_params(N, H, d, dtype, sigma: torch.Tensor, lam: torch.Tensor, gamma: torch.Tensor, w=512, s=32,
                P=64, W=8, K=4, B=128, out_dtype=None, scale=0.0, rho=1.0, rope_base=10000.0,
                rms_eps=1e-6) -> Params:
    """Parameter block; sigma/lam/gamma are device float32 tensors of shape [H], referenced by the block."""
    dt = dtype_code(dtype) if isinstance(dtype, torch.dtype) else int(dtype)
    odt = dt if out_dtype is None else (dtype_code(out_dtype) if isinstance(out_dtype, torch.dtype) else int(out_dtype))
    for t in (sigma, lam, gamma):
        assert t.dtype == torch.float32 and t.is_contiguous() and t.numel() >= H
    prm = Params(N=N, H=H, d=d, w=w, s=s, P=P, W=W, K=K, B=B, dtype=dt, out_dtype=odt, scale=scale, rho=rho,
                 rope_base=rope_base, rms_eps=rms_eps, sigma=sigma.data_ptr(), lam=lam.data_ptr(),
                 gamma=gamma.data_ptr())
    prm._keep = (sigma, lam, gamma)  # the struct holds raw device pointers: keep the tensors alive with it
    return prm


def check_params(p: Params) -> int:
    return int(lib().fsl_check_params(ctypes.byref(p)))


def workspace_bytes(p: Params) -> int:
    return int(lib().fsl_workspace_bytes(ctypes.byref(p)))


def workspace_layout(p: Params) -> WorkspaceLayout:
    L = WorkspaceLayout()
    _check(lib().fsl_workspace_views(ctypes.byref(p), ctypes.byref(L)), "fsl_workspace_views")
    return L


def new_workspace(p: Params, device="cuda") -> torch.Tensor:
    n = workspace_bytes(p)
    if n == 0:
        _check(check_params(p), "fsl_workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def cell_stats(k: torch.Tensor, p: Params, kbar: Optional[torch.Tensor] = None,
               amax: Optional[torch.Tensor] = None, stream=None):
    C = p.N // p.s
    if kbar is None:
        kbar = torch.empty((p.H, C, p.d), dtype=torch.float32, device=k.device)
    if amax is None:
        amax = torch.empty((p.H, C), dtype=torch.float32, device=k.device)
    _check(lib().fsl_cell_stats(_ptr(k), _ptr(kbar), _ptr(amax), ctypes.byref(p), _stream(stream)),
           "fsl_cell_stats")
    return kbar, amax


def prune_select(q: torch.Tensor, kbar: torch.Tensor, amax: torch.Tensor, p: Params,
                 ws: Optional[torch.Tensor] = None, stream=None):
    """Pools and per-query selections; without pruning (P = -1) no pool is formed and None is returned for it."""
    nblk = (p.N + p.B - 1) // p.B
    pool = torch.empty((p.H, nblk, p.P + p.W), dtype=torch.int32, device=q.device) if p.P >= 0 else None
    sel = torch.empty((p.H, p.N, p.K), dtype=torch.int32, device=q.device)
    ws = new_workspace(p, q.device) if ws is None else ws
    _check(lib().fsl_prune_select(_ptr(q), _ptr(kbar), _ptr(amax), _ptr(pool), _ptr(sel), ctypes.byref(p),
                                  _ptr(ws), ws.numel(), _stream(stream)), "fsl_prune_select")
    return pool, sel


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, p: Params, out: Optional[torch.Tensor] = None,
             ws: Optional[torch.Tensor] = None, sel_out: Optional[torch.Tensor] = None,
             o_win_out: Optional[torch.Tensor] = None, o_long_out: Optional[torch.Tensor] = None, stream=None):
    """FS-L forward. q, k, v: [H][N][d] device tensors (float32 or bfloat16)."""
    if out is None:
        odt = torch.float32 if p.out_dtype == FSL_F32 else torch.bfloat16
        out = torch.empty(q.shape, dtype=odt, device=q.device)
    ws = new_workspace(p, q.device) if ws is None else ws
    _check(lib().fsl_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), ctypes.byref(p), _ptr(ws), ws.numel(),
                              _ptr(sel_out), _ptr(o_win_out), _ptr(o_long_out), _stream(stream)), "fsl_attn_fwd")
    return out


NUM_STAGES = 6
STAGES = ("cell_stats", "prune", "select", "kv_prep", "window", "readout_mix")


def attn_fwd_timed(q, k, v, p: Params, out: torch.Tensor, ws: torch.Tensor, events, stream=None):
    """fsl_attn_fwd recording NUM_STAGES + 1 hipEvent_t handles (a ctypes array) between its stages."""
    _check(lib().fsl_attn_fwd_timed(_ptr(q), _ptr(k), _ptr(v), _ptr(out), ctypes.byref(p), _ptr(ws), ws.numel(),
                                    events, _stream(stream)), "fsl_attn_fwd_timed")
    return out


def workspace_views(ws: torch.Tensor, p: Params):
    """Named tensor views (kbar, amax, pool, sel) into a forward workspace."""
    L = workspace_layout(p)
    C = p.N // p.s
    nblk = (p.N + p.B - 1) // p.B

    def view(off, n, dt, shape):
        esz = torch.tensor([], dtype=dt).element_size()
        return ws[off: off + n * esz].view(dt).view(shape)

    return dict(
        kbar=view(L.kbar, p.H * C * p.d, torch.float32, (p.H, C, p.d)),
        amax=view(L.amax, p.H * C, torch.float32, (p.H, C)),
        pool=view(L.pool, p.H * nblk * max(p.P + p.W, 0), torch.int32, (p.H, nblk, max(p.P + p.W, 0))) if p.P >= 0
        else None,
        sel=view(L.sel, p.H * p.N * p.K, torch.int32, (p.H, p.N, p.K)),
    )


# ---------------------------------------------------------------------------
# streaming decode

class DecodeState:
    """A device state buffer for n_seq sequences (see fsl_decode_* in include/fsl.h)."""

    def __init__(self, p: Params, n_seq: int, device="cuda", stream=None):
        self.p = p
        self.n_seq = n_seq
        n = int(lib().fsl_decode_state_bytes(ctypes.byref(p), n_seq))
        if n == 0:
            _check(FSL_E_INVAL if n_seq < 1 else check_params(p), "fsl_decode_state_bytes")
        self.buf = torch.empty(n, dtype=torch.uint8, device=device)
        _check(lib().fsl_decode_init(_ptr(self.buf), n, n_seq, ctypes.byref(p), _stream(stream)), "fsl_decode_init")

    @property
    def nbytes(self) -> int:
        return self.buf.numel()

    def prefill(self, seq: int, k_prefix: torch.Tensor, v_prefix: torch.Tensor, ws: Optional[torch.Tensor] = None,
                stream=None):
        L = k_prefix.shape[1]
        need = int(lib().fsl_decode_prefill_workspace_bytes(ctypes.byref(self.p), L))
        if ws is None or ws.numel() < need:
            ws = torch.empty(max(need, 1), dtype=torch.uint8, device=self.buf.device)
        _check(lib().fsl_decode_prefill(_ptr(self.buf), self.nbytes, seq, _ptr(k_prefix), _ptr(v_prefix), L,
                                        ctypes.byref(self.p), _ptr(ws), ws.numel(), _stream(stream)),
               "fsl_decode_prefill")
        return ws

    def append(self, seq: int, k: torch.Tensor, v: torch.Tensor, stream=None):
        """Append tokens without queries (streamed prefill): k, v [H][len][d] for sequence seq, or
        [n][H][len][d] for sequences seq .. seq + n - 1."""
        n = 1 if k.dim() == 3 else int(k.shape[0])
        L = int(k.shape[-2])
        _check(lib().fsl_decode_append(_ptr(self.buf), self.nbytes, seq, n, _ptr(k), _ptr(v), L,
                                       ctypes.byref(self.p), _stream(stream)), "fsl_decode_append")

    def step(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: Optional[torch.Tensor] = None,
             sel_out: Optional[torch.Tensor] = None, stream=None):
        if out is None:
            odt = torch.float32 if self.p.out_dtype == FSL_F32 else torch.bfloat16
            out = torch.empty(q.shape, dtype=odt, device=q.device)
        _check(lib().fsl_decode_step(_ptr(self.buf), self.nbytes, _ptr(q), _ptr(k), _ptr(v), _ptr(out), self.n_seq,
                                     ctypes.byref(self.p), _ptr(sel_out), _stream(stream)), "fsl_decode_step")
        return out

    def validate(self) -> int:
        return int(lib().fsl_decode_validate(_ptr(self.buf), self.nbytes, ctypes.byref(self.p), self.n_seq))
