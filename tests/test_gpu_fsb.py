"""Parity of the FS-B selection (beam search over two causal forests) and of
the forward that reads its cells, with the oracle.

Selections must equal the oracle's bit for bit; outputs are compared with the
oracle's forward for the same selections, within the fp32 / bf16 bars. tau_h
stands in for the pages' per-checkpoint threshold (the median cell norm of
training windows) as the median cell norm of the head's own first 4096
tokens; the code projections are seeded Gaussian rows.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from fsl_testlib import GpuRun, check_out, device_tensor, host_f32, oracle_head_params
from long_context_sparse_cell_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from long_context_sparse_cell_amd import fsl
    fsl.lib()  # a missing library is an error here, not a skip


def fsb_inputs(sh, inp, oracle, seed=3):
    """tau [H] (median cell norm of each head's first 4096 tokens) and proj [32][d]."""
    tau = np.zeros(sh.H, np.float32)
    for h in range(sh.H):
        n0 = min(sh.N, 4096)
        p0 = oracle_head_params(oracle, sh, inp, h)
        p0.N = n0
        _, am = oracle.cell_stats(inp.k[h][:n0], p0)
        tau[h] = np.float32(np.median(am)) if len(am) else np.float32(0.0)
    proj = np.random.default_rng(seed).standard_normal((32, sh.d)).astype(np.float32)
    return tau, proj


def run_and_compare(oracle, sh, inp, beam=16, rows=None):
    from long_context_sparse_cell_amd import fsl
    tau, proj = fsb_inputs(sh, inp, oracle)
    run = GpuRun(inp, want_internals=False)  # device tensors and parameters
    fb = fsl.make_fsb_params(torch.from_numpy(tau).cuda(), torch.from_numpy(proj).cuda(), beam)
    sel = torch.empty((sh.H, sh.N, sh.K), dtype=torch.int32, device="cuda")
    out = fsl.attn_fwd_fsb(run.q, run.k, run.v, run.p, fb, sel_out=sel)
    sel2 = fsl.fsb_select(run.q, run.k, run.p, fb)
    torch.cuda.synchronize()
    sel_h = sel.cpu().numpy()
    assert np.array_equal(sel_h, sel2.cpu().numpy()), "fsl_fsb_select and the forward select differently"
    out_h = host_f32(out)
    out_dtype = synth.F32 if run.p.out_dtype == 0 else synth.BF16

    def one(h):
        p = oracle_head_params(oracle, sh, inp, h)
        rh = np.arange(sh.N) if rows is None else rows
        rsel, _ = oracle.fsb_select(inp.q[h], inp.k[h], p, proj, float(tau[h]), beam=beam, rows=rh)
        ref_out, _, _ = oracle.forward_rows_sel(inp.q[h], inp.k[h], inp.v[h], p, rh, rsel)
        return rh, rsel, ref_out

    with ThreadPoolExecutor(max_workers=min(sh.H, 16)) as ex:
        res = list(ex.map(one, range(sh.H)))
    for h, (rh, rsel, ref_out) in enumerate(res):
        np.testing.assert_array_equal(sel_h[h][rh], rsel, err_msg=f"FS-B selections head {h}")
        mx, mean = check_out(out_h[h][rh], ref_out, out_dtype, f"out head {h}")
        print(f"  head {h}: out max err {mx:.3e}, mean {mean:.3e}, rows {len(rh)}", flush=True)
    return sel_h


SMALL = [
    ("bf16_d64_n4100", dict(H=2, N=4100, d=64, dtype=synth.BF16), 16),
    ("f32_d128_n3001", dict(H=2, N=3001, d=128, dtype=synth.F32), 16),
    ("bf16_d128_n5000_beam4", dict(H=1, N=5000, d=128, dtype=synth.BF16), 4),
    ("bf16_d64_small_window_s16", dict(H=2, N=3000, d=64, dtype=synth.BF16, w=64, s=16, B=64, K=3), 16),
    ("f32_d64_n2500_beam1", dict(H=1, N=2500, d=64, dtype=synth.F32), 1),
    ("bf16_d64_n6000_beam32_k8", dict(H=1, N=6000, d=64, dtype=synth.BF16, K=8), 32),
    ("bf16_d64_n1", dict(H=1, N=1, d=64, dtype=synth.BF16), 16),
    ("bf16_d64_n700", dict(H=2, N=700, d=64, dtype=synth.BF16), 16),
]


@pytest.mark.parametrize("name,shape,beam", SMALL, ids=[c[0] for c in SMALL])
def test_fsb_small_shapes_every_query(oracle, name, shape, beam):
    print(f"\n[case] fsb {name}", flush=True)
    sh = synth.Shape(name, seed=51, **shape)
    inp = synth.random_inputs(sh)
    rng = np.random.default_rng(52)
    inp.k = synth.to_dtype(inp.k * np.exp(rng.normal(0, 0.4, (sh.H, sh.N, 1))).astype(np.float32), sh.dtype)
    run_and_compare(oracle, sh, inp, beam=beam)


def test_fsb_sigma_small(oracle):
    print("\n[case] fsb sigma 0.05", flush=True)
    sh = synth.Shape("fsb_sigma005", H=2, N=4100, d=64, dtype=synth.BF16, seed=53)
    inp = synth.random_inputs(sh)
    inp.sigma[:] = 0.05
    run_and_compare(oracle, sh, inp)


def test_fsb_16384_workload_every_row_and_needles(oracle):
    sh = synth.CONFIGS["fwd_bf16_n16384"]
    print(f"\n[case] fsb workload {sh.name}", flush=True)
    inp = synth.make_inputs(sh)
    sel = run_and_compare(oracle, sh, inp)
    for h in range(sh.H):
        for m, pos in enumerate(inp.needles[h]):
            assert pos // sh.s in sel[h][inp.probes[h][m]], (h, pos)


def test_fsb_262144_workload_stripe(oracle):
    sh = synth.CONFIGS["fwd_bf16_n262144"]
    print(f"\n[case] fsb workload {sh.name}, 64 blocks", flush=True)
    inp = synth.make_inputs(sh)
    nblk = (sh.N + sh.B - 1) // sh.B
    blocks = np.unique(np.linspace(0, nblk - 1, 64).round().astype(np.int64))
    rows = np.concatenate([np.arange(b * sh.B, min(sh.N, (b + 1) * sh.B)) for b in blocks])
    sel = run_and_compare(oracle, sh, inp, rows=rows)
    for h in range(sh.H):
        pos = inp.needles[h][0]
        for row in inp.probes[h]:
            assert pos // sh.s in sel[h][row], (h, pos, row)
    torch.cuda.empty_cache()


def test_fsb_no_cells_ignores_stale_workspace(oracle):
    """With fewer than s tokens there are no cells and nothing is selected, whatever bytes the
    workspace held before: the per-cell list counts are not computed then, so the search must not
    read them (a regression test for exactly that read)."""
    from long_context_sparse_cell_amd import fsl
    for n in (1, 20):
        print(f"\n[case] fsb no cells N={n}, workspace filled with 0x7F", flush=True)
        sh = synth.Shape(f"fsb_nocells_n{n}", H=2, N=n, d=64, dtype=synth.BF16, seed=54)
        inp = synth.random_inputs(sh)
        tau, proj = fsb_inputs(sh, inp, oracle)
        run = GpuRun(inp, want_internals=False)
        fb = fsl.make_fsb_params(torch.from_numpy(tau).cuda(), torch.from_numpy(proj).cuda(), 16)
        ws = torch.full((fsl.fsb_workspace_bytes(run.p),), 0x7F, dtype=torch.uint8, device="cuda")
        sel = fsl.fsb_select(run.q, run.k, run.p, fb, ws=ws)
        torch.cuda.synchronize()
        assert (sel.cpu().numpy() == -1).all(), n
