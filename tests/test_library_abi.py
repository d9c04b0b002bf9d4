"""The C-ABI library loads on a machine without a GPU, exports every symbol
include/fsl.h declares, and rejects bad arguments on the host before any
launch (so no GPU is needed to exercise the error paths)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fsl.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(fsl_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def fsl():
    from long_context_sparse_cell_amd import fsl as mod
    if not os.path.exists(mod.LIB_PATH):
        pytest.fail("libfsl.so is not built (run __graft_entry__.build())")
    return mod


def test_every_declared_symbol_is_exported(fsl):
    names = declared_functions()
    assert "fsl_attn_fwd" in names and "fsl_cell_stats" in names and "fsl_prune_select" in names
    L = ctypes.CDLL(fsl.LIB_PATH)
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing


def test_version_and_messages(fsl):
    assert fsl.lib().fsl_version() == 1
    for code in (0, -1, -2, -3, -4, -5):
        assert fsl.strerror(code)
    assert fsl.strerror(-99) == "unknown status"


class FakeTensor:
    """Stands in for a device tensor: only its address is used by the host checks."""

    def __init__(self, addr=0x10000, n=1 << 20):
        self._addr = addr
        self._n = n

    def data_ptr(self):
        return self._addr


def params(fsl, **kw):
    base = dict(N=4096, H=2, d=64, w=512, s=32, P=64, W=8, K=4, B=128, dtype=1, out_dtype=1, scale=0.0, rho=1.0,
                rope_base=10000.0, rms_eps=1e-6)
    base.update(kw)
    p = fsl.Params(**{k: v for k, v in base.items()})
    p.sigma = p.lam = p.gamma = 0x20000
    return p


BAD = [
    (dict(N=0), -1), (dict(H=0), -1), (dict(d=63), -1), (dict(s=0), -1), (dict(B=100, s=32), -1),
    (dict(K=0), -1), (dict(W=-1), -1), (dict(P=-2), -1), (dict(dtype=7), -1), (dict(out_dtype=1, dtype=0), -1),
    (dict(rms_eps=0.0), -1), (dict(rope_base=0.0), -1), (dict(w=0), -1), (dict(scale=-1.0), -1),
    (dict(d=96), -2), (dict(s=8, B=128), -2), (dict(P=65), -2), (dict(K=9), -2),
    (dict(W=65), -2), (dict(B=288, s=32), -2), (dict(B=24, s=8), -2),
]


@pytest.mark.parametrize("over,code", BAD, ids=[str(b[0]) for b in BAD])
def test_bad_parameters_are_rejected(fsl, over, code):
    p = params(fsl, **over)
    assert fsl.check_params(p) == code
    assert fsl.workspace_bytes(p) == 0


def test_good_parameters_and_workspace_size(fsl):
    p = params(fsl)
    assert fsl.check_params(p) == 0
    n = fsl.workspace_bytes(p)
    L = fsl.workspace_layout(p)
    assert L.total == n
    C, nblk = 4096 // 32, 4096 // 128
    assert L.amax - L.kbar >= 2 * C * 64 * 4
    assert L.sel - L.pool >= 2 * nblk * 72 * 4
    assert all(getattr(L, f) % 256 == 0 for f in ("kbar", "amax", "pool", "sel", "rope", "scan_a", "scan_i", "o_win",
                                                  "status"))
    assert L.total - L.status >= 4  # the status word is the last array


@pytest.mark.parametrize("N,d", [(5000, 128), (4096, 64), (64, 64), (1, 128), (262144, 128)])
def test_prepared_key_value_arrays_cover_whole_tiles(fsl, N, d):
    """With bf16 inputs the workspace holds the rotated fp16 keys and transposed fp16
    values that the window and readout kernels copy in whole 64-token tiles: each
    needs H x Np x d fp16 elements, Np = 64 ceil(N/64), per-head extents back to back."""
    H = 3
    p = params(fsl, N=N, d=d, H=H, dtype=1, out_dtype=1)
    L = fsl.workspace_layout(p)
    need = H * (64 * ((N + 63) // 64)) * d * 2
    assert L.vt - L.kt >= need
    assert L.status - L.vt >= need
    assert L.kt % 256 == 0 and L.vt % 256 == 0
    # the fp32 path does not prepare them
    p32 = params(fsl, N=N, d=d, H=H, dtype=0, out_dtype=0)
    L32 = fsl.workspace_layout(p32)
    assert L32.status == L32.vt == L32.kt


@pytest.mark.parametrize("N,d,K", [(5000, 128, 4), (4096, 64, 8), (1, 64, 1)])
def test_branch_arrays_by_input_dtype(fsl, N, d, K):
    """fp32 inputs keep the window branch's fp32 output [H][N][d]; bf16 inputs keep instead,
    per (query, rank), the selected cell's normalised long-branch output (fp16 [H][N][K][d])
    and its base-2 log-sum-exp (float [H][N][K]), which the window kernel merges."""
    H = 3
    L = fsl.workspace_layout(params(fsl, N=N, d=d, H=H, K=K, dtype=1, out_dtype=1))
    assert L.rope_abs == L.o_win  # no fp32 window output
    assert L.plse - L.part >= H * N * K * d * 2 and L.fixups - L.plse >= H * N * K * 4
    assert L.part % 256 == 0 and L.plse % 256 == 0
    L32 = fsl.workspace_layout(params(fsl, N=N, d=d, H=H, K=K, dtype=0, out_dtype=0))
    assert L32.rope_abs - L32.o_win >= H * N * d * 4
    assert L32.part == L32.plse == L32.fixups  # no partial arrays


@pytest.mark.parametrize("dtype", [0, 1])
def test_unpruned_variant_workspace(fsl, dtype):
    """P = -1 (plain FS): no pool table; with bf16 inputs the workspace holds the split cell
    means (two bf16 [H][C][d] arrays), the per-cell bound constants (float4 [H][C]) and a
    near-tie list of 36-word entries (head, row, count, unused, 32 cell indices) per query."""
    H, N, d = 3, 5000, 128
    p = params(fsl, N=N, H=H, d=d, P=-1, W=8, dtype=dtype, out_dtype=dtype)
    assert fsl.check_params(p) == 0
    L = fsl.workspace_layout(p)
    assert L.sel == L.pool  # zero pool bytes
    C = N // 32
    if dtype == 1:
        regions = H * ((N + 127) // 128)
        assert L.khi - L.fixups >= 4 * ((regions + 63) // 64 * 64 + regions * 128 * 36)
        assert L.klo - L.khi >= H * C * d * 2 and L.kcf - L.klo >= H * C * d * 2
        assert L.status - L.kcf >= H * C * 16
        assert all(getattr(L, f) % 256 == 0 for f in ("fixups", "khi", "klo", "kcf"))
    else:
        assert L.status == L.kcf == L.klo == L.khi
    # the pruned variant has none of the split arrays
    Lp = fsl.workspace_layout(params(fsl, N=N, H=H, d=d, dtype=dtype, out_dtype=dtype))
    assert Lp.status == Lp.kcf == Lp.klo == Lp.khi
    # pool may be NULL without pruning, not with it
    lib = fsl.lib()
    a = ctypes.c_void_p(0x100000)
    n = fsl.workspace_bytes(p)
    assert lib.fsl_prune_select(a, a, a, None, a, ctypes.byref(p), a, n - 1, None) == -3
    pp = params(fsl, N=N, H=H, d=d, dtype=dtype, out_dtype=dtype)
    assert lib.fsl_prune_select(a, a, a, None, a, ctypes.byref(pp), a, fsl.workspace_bytes(pp), None) == -1


def test_null_pointers_and_small_workspace_fail_before_launch(fsl):
    L = fsl.lib()
    p = params(fsl)
    vp = ctypes.c_void_p
    a = vp(0x100000)
    n = fsl.workspace_bytes(p)
    # null q
    assert L.fsl_attn_fwd(None, a, a, a, ctypes.byref(p), a, n, None, None, None, None) == -1
    # misaligned k
    assert L.fsl_attn_fwd(a, vp(0x100004), a, a, ctypes.byref(p), a, n, None, None, None, None) == -1
    # workspace one byte short
    assert L.fsl_attn_fwd(a, a, a, a, ctypes.byref(p), a, n - 1, None, None, None, None) == -3
    assert L.fsl_prune_select(a, a, a, a, a, ctypes.byref(p), a, n - 1, None) == -3
    # missing per-head arrays
    p2 = params(fsl)
    p2.gamma = None
    assert L.fsl_attn_fwd(a, a, a, a, ctypes.byref(p2), a, n, None, None, None, None) == -1
    assert L.fsl_cell_stats(a, None, a, ctypes.byref(p), None) == -1


def test_decode_state_is_bounded_and_independent_of_prefix(fsl):
    """State per (sequence, head): ring of w+B+s tokens + P+W cell slots, whatever the prefix
    length (ai.info summary: bounded state O(((P+W)s + w + B + s)d))."""
    L = fsl.lib()
    sizes = []
    for N in (1, 4096, 131072, 1 << 30):
        p = params(fsl, N=N, H=16, d=64, dtype=1, out_dtype=1)
        sizes.append(int(L.fsl_decode_state_bytes(ctypes.byref(p), 64)))
    assert len(set(sizes)) == 1 and sizes[0] > 0
    per_head = sizes[0] / (64 * 16)
    tokens = (64 + 8) * 32 + 512 + 128 + 32  # (P+W)s + w + B + s
    kv_bytes = tokens * 64 * 2 * 2           # raw k and v, bf16
    rot_bytes = (512 + 128 + 32) * 64 * 2    # the ring's keys rotated at their positions, fp16
    need = kv_bytes + rot_bytes
    assert need <= per_head <= need * 1.1    # plus cell means/norms and alignment
    p = params(fsl, P=-1)
    assert int(L.fsl_decode_state_bytes(ctypes.byref(p), 4)) == 0
    p = params(fsl)
    assert int(L.fsl_decode_state_bytes(ctypes.byref(p), 0)) == 0


def test_decode_entry_points_reject_bad_arguments(fsl):
    L = fsl.lib()
    p = params(fsl)
    n = int(L.fsl_decode_state_bytes(ctypes.byref(p), 2))
    a = ctypes.c_void_p(0x100000)
    assert L.fsl_decode_init(a, n - 1, 2, ctypes.byref(p), None) == -3
    assert L.fsl_decode_init(None, n, 2, ctypes.byref(p), None) == -1
    assert L.fsl_decode_step(a, n, a, a, a, a, 3, ctypes.byref(p), None, None) == -3   # more sequences than the state holds
    assert L.fsl_decode_step(a, n, a, ctypes.c_void_p(0x100002), a, a, 2, ctypes.byref(p), None, None) == -1
    assert L.fsl_decode_prefill(a, n, 2, a, a, 100, ctypes.byref(p), a, 1 << 30, None) == -1  # seq out of range
    assert L.fsl_decode_prefill(a, n, 0, a, a, 100, ctypes.byref(p), a, 16, None) == -3      # workspace too small
    pw = params(fsl, w=70000)
    assert int(L.fsl_decode_state_bytes(ctypes.byref(pw), 1)) == 0
    # streamed prefill: pointers, length and sequence checked before any launch
    assert L.fsl_decode_append(a, n, 0, 1, None, a, 10, ctypes.byref(p), None) == -1
    assert L.fsl_decode_append(a, n, 0, 1, a, ctypes.c_void_p(0x100008), 10, ctypes.byref(p), None) == -1
    assert L.fsl_decode_append(a, n, 0, 1, a, a, 0, ctypes.byref(p), None) == -1
    assert L.fsl_decode_append(a, n, 2, 1, a, a, 10, ctypes.byref(p), None) == -1   # state holds sequences 0, 1
    assert L.fsl_decode_append(a, n, 1, 2, a, a, 10, ctypes.byref(p), None) == -1   # 1 .. 2 is past the end
    assert L.fsl_decode_append(a, n, 0, 0, a, a, 10, ctypes.byref(p), None) == -1
    assert L.fsl_decode_append(a, n, -1, 1, a, a, 10, ctypes.byref(p), None) == -1
    assert L.fsl_decode_append(a, n, 0, 1, a, a, 10, ctypes.byref(params(fsl, P=-1)), None) == -2


# ---------------------------------------------------------------------------
# the Python binding checks every tensor against the parameter block before any
# launch (a mismatch would otherwise be an out-of-bounds access on the device)

def _cpu_params(fsl, torch, **kw):
    H = kw.pop("H", 2)
    N = kw.pop("N", 512)
    d = kw.pop("d", 64)
    dt = kw.pop("dtype", torch.bfloat16)
    sig = torch.full((H,), 4.0)
    lam = torch.ones(H)
    gam = torch.ones(H)
    return fsl.make_params(N, H, d, dt, sig, lam, gam, **kw)


def test_binding_rejects_mismatched_tensors(fsl):
    import torch
    p = _cpu_params(fsl, torch)
    H, N, d = p.H, p.N, p.d
    good = torch.zeros((H, N, d), dtype=torch.bfloat16)
    cases = [
        (dict(q=torch.zeros((H, N + 1, d), dtype=torch.bfloat16)), "shape"),
        (dict(k=torch.zeros((H, N, d), dtype=torch.float32)), "dtype"),
        (dict(v=torch.zeros((H * N * d,), dtype=torch.bfloat16)), "shape"),
        (dict(out=torch.zeros((H, N, d), dtype=torch.float32)), "dtype"),
        (dict(sel_out=torch.zeros((H, N, p.K + 1), dtype=torch.int32)), "shape"),
        (dict(o_win_out=torch.zeros((H, N, d), dtype=torch.bfloat16)), "dtype"),
        (dict(o_long_out=torch.zeros((H, N - 1, d), dtype=torch.float32)), "shape"),
        (dict(q=good.t() if good.dim() == 2 else good.transpose(0, 1)), "shape"),
        (dict(), "GPU memory"),  # right shapes and dtypes, but host tensors
    ]
    for over, msg in cases:
        args = dict(q=good, k=good, v=good, out=torch.zeros((H, N, d), dtype=torch.bfloat16))
        args.update(over)
        with pytest.raises(ValueError, match=msg):
            fsl.attn_fwd(args["q"], args["k"], args["v"], p, out=args["out"], ws=torch.zeros(16, dtype=torch.uint8),
                         sel_out=args.get("sel_out"), o_win_out=args.get("o_win_out"),
                         o_long_out=args.get("o_long_out"))


def test_binding_rejects_bad_statistics_and_selection_buffers(fsl):
    import torch
    p = _cpu_params(fsl, torch, N=1024)
    H, N, d = p.H, p.N, p.d
    C = N // p.s
    nblk = (N + p.B - 1) // p.B
    k = torch.zeros((H, N, d), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="shape"):
        fsl.cell_stats(k, p, kbar=torch.zeros((H, C + 1, d)), amax=torch.zeros((H, C)))
    with pytest.raises(ValueError, match="dtype"):
        fsl.cell_stats(k, p, kbar=torch.zeros((H, C, d)), amax=torch.zeros((H, C), dtype=torch.float64))
    with pytest.raises(ValueError, match="shape"):
        fsl.cell_stats(k[:, :-1], p)
    kbar, amax = torch.zeros((H, C, d)), torch.zeros((H, C))
    with pytest.raises(ValueError, match="shape"):
        fsl.prune_select(k, kbar, amax, p, pool=torch.zeros((H, nblk, p.P + p.W - 1), dtype=torch.int32))
    with pytest.raises(ValueError, match="dtype"):
        fsl.prune_select(k, kbar, amax, p, sel=torch.zeros((H, N, p.K), dtype=torch.int64))
    with pytest.raises(ValueError, match="GPU memory"):
        fsl.prune_select(k, kbar, amax, p)


def test_binding_rejects_small_or_foreign_workspace(fsl):
    import torch
    p = _cpu_params(fsl, torch)
    with pytest.raises(ValueError, match="uint8"):
        fsl._expect_ws(torch.zeros(16, dtype=torch.int32), 8, torch.device("cpu"))
    with pytest.raises(ValueError, match="needs"):
        fsl._expect_ws(torch.zeros(16, dtype=torch.uint8), fsl.workspace_bytes(p), torch.device("cpu"))


def test_noalloc_size_and_pointer_checks_on_the_host(fsl):
    """fsl_attn_fwd_noalloc rejects a workspace beyond its array, and null pointers,
    before touching the device."""
    L = fsl.lib()
    a = ctypes.c_void_p(0x10000)
    big = params(fsl, N=65536, H=16, d=64)
    assert fsl.workspace_bytes(big) > fsl.NOALLOC_WORKSPACE_MAX
    assert L.fsl_attn_fwd_noalloc(a, a, a, a, ctypes.byref(big), None, None, None, None) == -3
    ok = params(fsl, N=4096, H=2, d=64)
    assert fsl.workspace_bytes(ok) <= fsl.NOALLOC_WORKSPACE_MAX
    assert L.fsl_attn_fwd_noalloc(None, a, a, a, ctypes.byref(ok), None, None, None, None) == -1
    assert L.fsl_attn_fwd_noalloc(a, a, a, a, ctypes.byref(params(fsl, K=0)), None, None, None, None) == -1
