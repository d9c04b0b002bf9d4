"""Helpers shared by the test modules: moving synth inputs to the GPU, running
the HIP path through the C ABI, and comparing against the oracle."""
import numpy as np
import torch

from long_context_sparse_cell_amd import synth

BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 1e-2
F32_MAX_ABS = 1e-4


def device_tensor(x: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """Upload float32 data already rounded to dtype (bf16 via its exact bit pattern)."""
    if dtype == synth.BF16:
        bits = synth.bf16_bits(x)
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(device)


def host_f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


class GpuRun:
    """One fsl_attn_fwd call on synth inputs, with every intermediate fetched."""

    def __init__(self, inp: synth.Inputs, device="cuda", want_internals=True, **over):
        from long_context_sparse_cell_amd import fsl
        sh = inp.shape
        self.shape = sh
        self.q = device_tensor(inp.q, sh.dtype, device)
        self.k = device_tensor(inp.k, sh.dtype, device)
        self.v = device_tensor(inp.v, sh.dtype, device)
        self.sigma = torch.from_numpy(inp.sigma).to(device)
        self.lam = torch.from_numpy(inp.lam).to(device)
        self.gamma = torch.from_numpy(inp.gamma).to(device)
        kw = dict(w=sh.w, s=sh.s, P=sh.P, W=sh.W, K=sh.K, B=sh.B, rho=sh.rho, rope_base=sh.rope_base,
                  rms_eps=sh.rms_eps)
        kw.update(over)
        self.p = fsl.make_params(sh.N, sh.H, sh.d, self.q.dtype, self.sigma, self.lam, self.gamma, **kw)
        self.ws = fsl.new_workspace(self.p, device)
        H, N, d, K = sh.H, sh.N, sh.d, self.p.K
        self.sel = torch.empty((H, N, K), dtype=torch.int32, device=device) if want_internals else None
        self.o_win = torch.empty((H, N, d), dtype=torch.float32, device=device) if want_internals else None
        self.o_long = torch.empty((H, N, d), dtype=torch.float32, device=device) if want_internals else None
        self.out = fsl.attn_fwd(self.q, self.k, self.v, self.p, ws=self.ws, sel_out=self.sel,
                                o_win_out=self.o_win, o_long_out=self.o_long)
        torch.cuda.synchronize()
        self.views = fsl.workspace_views(self.ws, self.p)


def oracle_head_params(oracle, sh, inp, h, **over):
    p = oracle.head_from_shape(sh, h, inp.sigma, inp.lam, inp.gamma)
    for k, v in over.items():
        setattr(p, "lam" if k == "lam" else k, v)
    return p


def check_out(got: np.ndarray, ref: np.ndarray, dtype: str, what: str):
    err = np.abs(got.astype(np.float64) - ref)
    at = np.unravel_index(int(np.argmax(err)), err.shape)
    info = f"{what}: max abs err {err.max():.3e} at {at} (oracle {ref[at]:.5f}, got {got[at]:.5f}), mean {err.mean():.3e}"
    if dtype == synth.BF16:
        assert err.max() <= BF16_MAX_ABS, info
        assert err.mean() <= BF16_MEAN_ABS, info
    else:
        assert err.max() <= F32_MAX_ABS, info
    return float(err.max()), float(err.mean())


def near_tie_rows(run, fs: bool):
    """(head, row) of every query the bf16 scoring passed to its exact fp64 fix-up: the
    queries whose certified MFMA filter left more than K contenders. Read from the
    workspace's near-tie list (a count per scoring region, then 128 entries of 6 words,
    or 36 without pruning, each starting with head and row)."""
    from long_context_sparse_cell_amd import fsl
    p = run.p
    L = fsl.workspace_layout(p)
    qw = p.B if p.B <= 128 else p.B // 2
    regions = p.H * ((p.N + qw - 1) // qw)
    words = 36 if fs else 6
    base = (regions + 63) // 64 * 64
    raw = run.ws[L.fixups: L.fixups + (base + regions * 128 * words) * 4].view(torch.int32).cpu().numpy()
    counts = raw[:regions]
    assert counts.min() >= 0 and counts.max() <= 128, "near-tie list counts out of range"
    ent = raw[base:].reshape(regions, 128, words)
    rows = [(int(ent[r, j, 0]), int(ent[r, j, 1])) for r in np.nonzero(counts)[0] for j in range(counts[r])]
    return rows
