"""Thin Python binding of the FS-L HIP library (libfsl.so, include/fsl.h).

Argument marshalling only: every step of the computation runs in the
library's HIP kernels. torch supplies device memory and the current stream.
If the library has not been built this module raises on first use; there is
no fallback.
"""
from __future__ import annotations

import ctypes
import os
from contextlib import nullcontext as _nullcontext
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


class FsbParams(ctypes.Structure):
    _fields_ = [("beam", ctypes.c_int32), ("reserved", ctypes.c_int32), ("tau", ctypes.c_void_p),
                ("proj", ctypes.c_void_p)]


class WorkspaceLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("kbar", "amax", "pool", "sel", "rope", "scan_a", "scan_i", "o_win", "rope_abs", "kt", "vt",
                 "plan", "part", "plse", "fixups", "khi", "klo", "kcf", "status", "total")]


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
        L.fsl_attn_bwd_workspace_bytes.restype = sz; L.fsl_attn_bwd_workspace_bytes.argtypes = [pp]
        L.fsl_attn_bwd.restype = i32
        L.fsl_attn_bwd.argtypes = [vp, vp, vp, vp, pp, vp, sz, vp, sz, vp, vp, vp, vp, vp]
        fp = ctypes.POINTER(FsbParams)
        L.fsl_fsb_workspace_bytes.restype = sz; L.fsl_fsb_workspace_bytes.argtypes = [pp]
        L.fsl_fsb_select.restype = i32; L.fsl_fsb_select.argtypes = [vp, vp, pp, fp, vp, vp, sz, vp]
        L.fsl_attn_fwd_fsb.restype = i32; L.fsl_attn_fwd_fsb.argtypes = [vp, vp, vp, vp, pp, fp, vp, sz, vp, vp]
        L.fsl_attn_fwd_noalloc.restype = i32
        L.fsl_attn_fwd_noalloc.argtypes = [vp, vp, vp, vp, pp, vp, vp, vp, vp]
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


def _torch_dtype(code: int) -> torch.dtype:
    return torch.float32 if code == FSL_F32 else torch.bfloat16


def _expect(t: Optional[torch.Tensor], name: str, shape, dtype: torch.dtype, optional=False):
    """Reject a tensor whose shape or dtype does not match what the library will read or
    write through its pointer: a mismatch would become an out-of-bounds access on the
    device, so it is caught here, before any launch (devices are checked by _on_gpu)."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name}: a tensor is required")
    shape = tuple(int(x) for x in shape)
    if tuple(t.shape) != shape:
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {shape}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: tensors passed to the FS-L library must be contiguous")


def _on_gpu(**named):
    """Every given tensor (None entries skipped) must be GPU memory on one device; returns it."""
    dev = None
    for name, t in named.items():
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError(f"{name}: tensor on {t.device}, the library needs GPU memory")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name}: tensor on {t.device}, other operands on {dev}")
    return dev


def _expect_ws(ws: torch.Tensor, need: int, device, name="ws"):
    if ws.dtype != torch.uint8 or ws.dim() != 1:
        raise ValueError(f"{name}: a 1-D uint8 tensor is expected, got {ws.dtype} with shape {tuple(ws.shape)}")
    if ws.numel() < need:
        raise ValueError(f"{name}: {ws.numel()} bytes, the call needs {need}")
    if ws.device.type != "cuda" or ws.device != device:
        raise ValueError(f"{name}: tensor on {ws.device}, other operands on {device}")


def _empty(shape, dtype, device, stream):
    """A new tensor from torch's caching allocator, associated with the stream the library
    launches on, so that its memory is not handed to other work while the kernels still
    use it."""
    if stream is None:
        return torch.empty(shape, dtype=dtype, device=device)
    with torch.cuda.stream(stream):
        return torch.empty(shape, dtype=dtype, device=device)


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


def new_workspace(p: Params, device="cuda", stream=None) -> torch.Tensor:
    n = workspace_bytes(p)
    if n == 0:
        _check(check_params(p), "fsl_workspace_bytes")
    return _empty(n, torch.uint8, device, stream)


def _qkv_shape(p: Params):
    return (p.H, p.N, p.d)


def cell_stats(k: torch.Tensor, p: Params, kbar: Optional[torch.Tensor] = None,
               amax: Optional[torch.Tensor] = None, stream=None):
    C = p.N // p.s
    _expect(k, "k", _qkv_shape(p), _torch_dtype(p.dtype))
    _expect(kbar, "kbar", (p.H, C, p.d), torch.float32, optional=True)
    _expect(amax, "amax", (p.H, C), torch.float32, optional=True)
    dev = _on_gpu(k=k, kbar=kbar, amax=amax)
    if kbar is None:
        kbar = _empty((p.H, C, p.d), torch.float32, dev, stream)
    if amax is None:
        amax = _empty((p.H, C), torch.float32, dev, stream)
    _check(lib().fsl_cell_stats(_ptr(k), _ptr(kbar), _ptr(amax), ctypes.byref(p), _stream(stream)),
           "fsl_cell_stats")
    return kbar, amax


def prune_select(q: torch.Tensor, kbar: torch.Tensor, amax: torch.Tensor, p: Params,
                 ws: Optional[torch.Tensor] = None, pool: Optional[torch.Tensor] = None,
                 sel: Optional[torch.Tensor] = None, stream=None):
    """Pools and per-query selections; without pruning (P = -1) no pool is formed and None is returned for it."""
    C = p.N // p.s
    nblk = (p.N + p.B - 1) // p.B
    _expect(q, "q", _qkv_shape(p), _torch_dtype(p.dtype))
    _expect(kbar, "kbar", (p.H, C, p.d), torch.float32)
    _expect(amax, "amax", (p.H, C), torch.float32)
    if p.P < 0:
        pool = None
    _expect(pool, "pool", (p.H, nblk, p.P + p.W), torch.int32, optional=True)
    _expect(sel, "sel", (p.H, p.N, p.K), torch.int32, optional=True)
    dev = _on_gpu(q=q, kbar=kbar, amax=amax, pool=pool, sel=sel, ws=ws)
    if p.P >= 0 and pool is None:
        pool = _empty((p.H, nblk, p.P + p.W), torch.int32, dev, stream)
    if sel is None:
        sel = _empty((p.H, p.N, p.K), torch.int32, dev, stream)
    ws = new_workspace(p, dev, stream) if ws is None else ws
    _expect_ws(ws, workspace_bytes(p), dev)
    _check(lib().fsl_prune_select(_ptr(q), _ptr(kbar), _ptr(amax), _ptr(pool), _ptr(sel), ctypes.byref(p),
                                  _ptr(ws), ws.numel(), _stream(stream)), "fsl_prune_select")
    return pool, sel


def _check_fwd_operands(q, k, v, out, p: Params, sel_out=None, o_win_out=None, o_long_out=None, ws=None):
    shp = _qkv_shape(p)
    _expect(q, "q", shp, _torch_dtype(p.dtype))
    _expect(k, "k", shp, _torch_dtype(p.dtype))
    _expect(v, "v", shp, _torch_dtype(p.dtype))
    _expect(out, "out", shp, _torch_dtype(p.out_dtype), optional=True)
    _expect(sel_out, "sel_out", (p.H, p.N, p.K), torch.int32, optional=True)
    _expect(o_win_out, "o_win_out", shp, torch.float32, optional=True)
    _expect(o_long_out, "o_long_out", shp, torch.float32, optional=True)
    return _on_gpu(q=q, k=k, v=v, out=out, sel_out=sel_out, o_win_out=o_win_out, o_long_out=o_long_out, ws=ws)


FSL_STATUS_F16_RANGE = 1


def range_status(ws: torch.Tensor, p: Params) -> int:
    """The status word a forward left in its workspace (FSL_STATUS_* bits); waits for the stream."""
    L = workspace_layout(p)
    return int(ws[L.status: L.status + 4].view(torch.int32).item())


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, p: Params, out: Optional[torch.Tensor] = None,
             ws: Optional[torch.Tensor] = None, sel_out: Optional[torch.Tensor] = None,
             o_win_out: Optional[torch.Tensor] = None, o_long_out: Optional[torch.Tensor] = None, stream=None,
             check_range: bool = False):
    """FS-L forward. q, k, v: [H][N][d] device tensors (float32 or bfloat16).

    check_range: after the call, read the workspace's status word and raise ValueError if a bf16
    input (or a rotated key) was outside fp16's finite range, which both attention branches need."""
    dev = _check_fwd_operands(q, k, v, out, p, sel_out, o_win_out, o_long_out, ws)
    if out is None:
        out = _empty(q.shape, _torch_dtype(p.out_dtype), dev, stream)
    ws = new_workspace(p, dev, stream) if ws is None else ws
    _expect_ws(ws, workspace_bytes(p), dev)
    _check(lib().fsl_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), ctypes.byref(p), _ptr(ws), ws.numel(),
                              _ptr(sel_out), _ptr(o_win_out), _ptr(o_long_out), _stream(stream)), "fsl_attn_fwd")
    if check_range:
        with torch.cuda.stream(stream) if stream is not None else _nullcontext():
            st = range_status(ws, p)
        if st & FSL_STATUS_F16_RANGE:
            raise ValueError("fsl_attn_fwd: an element of k or v, or a rotated key, lies outside fp16's finite "
                             "range (|x| >= 65504 or not finite); the outputs of this call are undefined")
    return out


def make_fsb_params(tau: torch.Tensor, proj: torch.Tensor, beam: int = 16) -> FsbParams:
    """FS-B parameters: tau [H] and proj [32][d] device float32 tensors (kept alive by the block)."""
    for name, t in (("tau", tau), ("proj", proj)):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError(f"{name}: a contiguous float32 tensor is required")
    fb = FsbParams(beam=int(beam), reserved=0, tau=tau.data_ptr(), proj=proj.data_ptr())
    fb._keep = (tau, proj)
    return fb


def fsb_workspace_bytes(p: Params) -> int:
    return int(lib().fsl_fsb_workspace_bytes(ctypes.byref(p)))


def fsb_select(q: torch.Tensor, k: torch.Tensor, p: Params, fb: FsbParams, ws: Optional[torch.Tensor] = None,
               sel: Optional[torch.Tensor] = None, stream=None):
    """FS-B selections [H][N][K] (fsl_fsb_select)."""
    shp = _qkv_shape(p)
    _expect(q, "q", shp, _torch_dtype(p.dtype))
    _expect(k, "k", shp, _torch_dtype(p.dtype))
    _expect(sel, "sel", (p.H, p.N, p.K), torch.int32, optional=True)
    _expect(fb._keep[0], "tau", (p.H,), torch.float32)
    _expect(fb._keep[1], "proj", (32, p.d), torch.float32)
    dev = _on_gpu(q=q, k=k, sel=sel, ws=ws, tau=fb._keep[0], proj=fb._keep[1])
    need = fsb_workspace_bytes(p)
    ws = _empty(need, torch.uint8, dev, stream) if ws is None else ws
    _expect_ws(ws, need, dev)
    sel = _empty((p.H, p.N, p.K), torch.int32, dev, stream) if sel is None else sel
    _check(lib().fsl_fsb_select(_ptr(q), _ptr(k), ctypes.byref(p), ctypes.byref(fb), _ptr(sel), _ptr(ws), ws.numel(),
                                _stream(stream)), "fsl_fsb_select")
    return sel


def attn_fwd_fsb(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, p: Params, fb: FsbParams,
                 out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                 sel_out: Optional[torch.Tensor] = None, stream=None):
    """The forward with FS-B selections (fsl_attn_fwd_fsb)."""
    dev = _check_fwd_operands(q, k, v, out, p, sel_out, None, None, ws)
    _expect(fb._keep[0], "tau", (p.H,), torch.float32)
    _expect(fb._keep[1], "proj", (32, p.d), torch.float32)
    _on_gpu(q=q, tau=fb._keep[0], proj=fb._keep[1])
    out = _empty(q.shape, _torch_dtype(p.out_dtype), dev, stream) if out is None else out
    need = fsb_workspace_bytes(p)
    ws = _empty(need, torch.uint8, dev, stream) if ws is None else ws
    _expect_ws(ws, need, dev)
    _check(lib().fsl_attn_fwd_fsb(_ptr(q), _ptr(k), _ptr(v), _ptr(out), ctypes.byref(p), ctypes.byref(fb), _ptr(ws),
                                  ws.numel(), _ptr(sel_out), _stream(stream)), "fsl_attn_fwd_fsb")
    return out


def attn_bwd_workspace_bytes(p: Params) -> int:
    return int(lib().fsl_attn_bwd_workspace_bytes(ctypes.byref(p)))


def attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, dout: torch.Tensor, p: Params,
             fwd_ws: torch.Tensor, ws: Optional[torch.Tensor] = None, dq: Optional[torch.Tensor] = None,
             dk: Optional[torch.Tensor] = None, dv: Optional[torch.Tensor] = None,
             dgamma: Optional[torch.Tensor] = None, stream=None):
    """Backward (fsl_attn_bwd): dq, dk, dv [H][N][d] float32 and dgamma [H] float32 for the upstream
    gradient dout, with the selections of the forward whose workspace is fwd_ws held fixed."""
    shp = _qkv_shape(p)
    _check_fwd_operands(q, k, v, None, p)
    _expect(dout, "dout", shp, _torch_dtype(p.out_dtype))
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _expect(t, name, shp, torch.float32, optional=True)
    _expect(dgamma, "dgamma", (p.H,), torch.float32, optional=True)
    dev = _on_gpu(q=q, dout=dout, fwd_ws=fwd_ws, ws=ws, dq=dq, dk=dk, dv=dv, dgamma=dgamma)
    _expect_ws(fwd_ws, workspace_bytes(p), dev, "fwd_ws")
    need = attn_bwd_workspace_bytes(p)
    ws = _empty(need, torch.uint8, dev, stream) if ws is None else ws
    _expect_ws(ws, need, dev)
    dq = _empty(shp, torch.float32, dev, stream) if dq is None else dq
    dk = _empty(shp, torch.float32, dev, stream) if dk is None else dk
    dv = _empty(shp, torch.float32, dev, stream) if dv is None else dv
    dgamma = _empty((p.H,), torch.float32, dev, stream) if dgamma is None else dgamma
    _check(lib().fsl_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), ctypes.byref(p), _ptr(fwd_ws), fwd_ws.numel(),
                              _ptr(ws), ws.numel(), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dgamma), _stream(stream)),
           "fsl_attn_bwd")
    return dq, dk, dv, dgamma


NOALLOC_WORKSPACE_MAX = 256 << 20  # FSL_NOALLOC_WORKSPACE_MAX


def attn_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, p: Params, out: torch.Tensor,
                     sel_out: Optional[torch.Tensor] = None, o_win_out: Optional[torch.Tensor] = None,
                     o_long_out: Optional[torch.Tensor] = None, stream=None):
    """fsl_attn_fwd_noalloc: the forward with the library's own workspace array (no allocation, so the
    caller passes `out`). Overlapping calls on one GPU share that array and race."""
    _expect(out, "out", _qkv_shape(p), _torch_dtype(p.out_dtype))
    _check_fwd_operands(q, k, v, out, p, sel_out, o_win_out, o_long_out)
    _check(lib().fsl_attn_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), ctypes.byref(p), _ptr(sel_out),
                                      _ptr(o_win_out), _ptr(o_long_out), _stream(stream)), "fsl_attn_fwd_noalloc")
    return out


NUM_STAGES = 6
# Stages of fsl_attn_fwd_timed in launch order. fp32 inputs: the window branch, then the long
# branch with RMSNorm and the mix. bf16 inputs: the long branch as per-cell partial outputs,
# then the window kernel, which merges them and applies RMSNorm and the mix.
STAGES_F32 = ("cell_stats", "prune", "select", "kv_prep", "window", "readout_mix")
STAGES_BF16 = ("cell_stats", "prune", "select", "kv_prep", "readout", "window_mix")


def stage_names(p: Params):
    """Names of the NUM_STAGES stages fsl_attn_fwd_timed records for these parameters."""
    return STAGES_BF16 if p.dtype == FSL_BF16 else STAGES_F32


def attn_fwd_timed(q, k, v, p: Params, out: torch.Tensor, ws: torch.Tensor, events, stream=None):
    """fsl_attn_fwd recording NUM_STAGES + 1 hipEvent_t handles (a ctypes array) between its stages."""
    _expect(out, "out", _qkv_shape(p), _torch_dtype(p.out_dtype))
    dev = _check_fwd_operands(q, k, v, out, p, ws=ws)
    _expect_ws(ws, workspace_bytes(p), dev)
    if events is None:
        raise ValueError(f"events: a pointer to {NUM_STAGES + 1} hipEvent_t handles is required")
    _check(lib().fsl_attn_fwd_timed(_ptr(q), _ptr(k), _ptr(v), _ptr(out), ctypes.byref(p), _ptr(ws), ws.numel(),
                                    events, _stream(stream)), "fsl_attn_fwd_timed")
    return out


def workspace_views(ws: torch.Tensor, p: Params):
    """Named tensor views (kbar, amax, pool, sel) into a forward workspace."""
    L = workspace_layout(p)
    C = p.N // p.s
    nblk = (p.N + p.B - 1) // p.B
    _expect_ws(ws, L.total, ws.device)

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
        self.buf = _empty(n, torch.uint8, device, stream)
        _check(lib().fsl_decode_init(_ptr(self.buf), n, n_seq, ctypes.byref(p), _stream(stream)), "fsl_decode_init")

    @property
    def nbytes(self) -> int:
        return self.buf.numel()

    def prefill(self, seq: int, k_prefix: torch.Tensor, v_prefix: torch.Tensor, ws: Optional[torch.Tensor] = None,
                stream=None):
        """Load sequence seq from a prefix k_prefix, v_prefix [H][L][d]. Returns the workspace used; it must
        stay allocated until the stream has run the call's work (a workspace made here is tied to
        `stream`)."""
        if k_prefix.dim() != 3:
            raise ValueError(f"k_prefix: shape {tuple(k_prefix.shape)}, expected [H][L][d]")
        L = int(k_prefix.shape[1])
        dt = _torch_dtype(self.p.dtype)
        _expect(k_prefix, "k_prefix", (self.p.H, L, self.p.d), dt)
        _expect(v_prefix, "v_prefix", (self.p.H, L, self.p.d), dt)
        _on_gpu(state=self.buf, k_prefix=k_prefix, v_prefix=v_prefix, ws=ws)
        if not 0 <= seq < self.n_seq:
            raise ValueError(f"seq {seq} outside [0, {self.n_seq})")
        need = int(lib().fsl_decode_prefill_workspace_bytes(ctypes.byref(self.p), L))
        if ws is None or ws.numel() < need:
            ws = _empty(max(need, 1), torch.uint8, self.buf.device, stream)
        _expect_ws(ws, need, self.buf.device)
        _check(lib().fsl_decode_prefill(_ptr(self.buf), self.nbytes, seq, _ptr(k_prefix), _ptr(v_prefix), L,
                                        ctypes.byref(self.p), _ptr(ws), ws.numel(), _stream(stream)),
               "fsl_decode_prefill")
        return ws

    def append(self, seq: int, k: torch.Tensor, v: torch.Tensor, stream=None):
        """Append tokens without queries (streamed prefill): k, v [H][len][d] for sequence seq, or
        [n][H][len][d] for sequences seq .. seq + n - 1."""
        if k.dim() not in (3, 4):
            raise ValueError(f"k: shape {tuple(k.shape)}, expected [H][len][d] or [n][H][len][d]")
        n = 1 if k.dim() == 3 else int(k.shape[0])
        L = int(k.shape[-2])
        shp = (self.p.H, L, self.p.d) if k.dim() == 3 else (n, self.p.H, L, self.p.d)
        dt = _torch_dtype(self.p.dtype)
        _expect(k, "k", shp, dt)
        _expect(v, "v", shp, dt)
        _on_gpu(state=self.buf, k=k, v=v)
        if seq < 0 or seq + n > self.n_seq:
            raise ValueError(f"sequences {seq} .. {seq + n - 1} outside [0, {self.n_seq})")
        _check(lib().fsl_decode_append(_ptr(self.buf), self.nbytes, seq, n, _ptr(k), _ptr(v), L,
                                       ctypes.byref(self.p), _stream(stream)), "fsl_decode_append")

    def step(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: Optional[torch.Tensor] = None,
             sel_out: Optional[torch.Tensor] = None, stream=None):
        """Advance every sequence by one token: q, k, v [n_seq][H][d]."""
        shp = (self.n_seq, self.p.H, self.p.d)
        dt = _torch_dtype(self.p.dtype)
        _expect(q, "q", shp, dt)
        _expect(k, "k", shp, dt)
        _expect(v, "v", shp, dt)
        _expect(out, "out", shp, _torch_dtype(self.p.out_dtype), optional=True)
        _expect(sel_out, "sel_out", (self.n_seq, self.p.H, self.p.K), torch.int32, optional=True)
        dev = _on_gpu(state=self.buf, q=q, k=k, v=v, out=out, sel_out=sel_out)
        if out is None:
            out = _empty(shp, _torch_dtype(self.p.out_dtype), dev, stream)
        _check(lib().fsl_decode_step(_ptr(self.buf), self.nbytes, _ptr(q), _ptr(k), _ptr(v), _ptr(out), self.n_seq,
                                     ctypes.byref(self.p), _ptr(sel_out), _stream(stream)), "fsl_decode_step")
        return out

    def validate(self) -> int:
        return int(lib().fsl_decode_validate(_ptr(self.buf), self.nbytes, ctypes.byref(self.p), self.n_seq))
