"""fsl_attn_fwd_noalloc (the forward on the library's own workspace array)
against fsl_attn_fwd with a caller workspace, through the C ABI: two calls in
a row on one GPU, the second on a smaller input, must give the same selections
and bit-identical outputs; an input whose workspace exceeds the array is
rejected before any device work."""
import numpy as np
import pytest
import torch

from fsl_testlib import GpuRun, device_tensor
from long_context_sparse_cell_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from long_context_sparse_cell_amd import fsl
    fsl.lib()  # a missing library is an error here, not a skip


def _noalloc_run(run):
    from long_context_sparse_cell_amd import fsl
    sh = run.shape
    out = torch.empty_like(run.out)
    sel = torch.empty((sh.H, sh.N, run.p.K), dtype=torch.int32, device=run.q.device)
    o_win = torch.empty((sh.H, sh.N, sh.d), dtype=torch.float32, device=run.q.device)
    fsl.attn_fwd_noalloc(run.q, run.k, run.v, run.p, out, sel_out=sel, o_win_out=o_win)
    torch.cuda.synchronize()
    return out, sel, o_win


def _same(run, res, what):
    out, sel, o_win = res
    assert torch.equal(sel, run.sel), f"{what}: selections differ"
    assert torch.equal(o_win.view(torch.int32), run.o_win.view(torch.int32)), f"{what}: window outputs differ"
    assert torch.equal(out.view(torch.int16 if out.dtype == torch.bfloat16 else torch.int32),
                       run.out.view(torch.int16 if out.dtype == torch.bfloat16 else torch.int32)), \
        f"{what}: outputs differ"


def test_noalloc_matches_the_workspace_forward_twice():
    from long_context_sparse_cell_amd import fsl
    print("\n[case] noalloc: fwd_bf16_h16_n16384_d64, then bf16 H=2 N=3001 d=128, then fp32 H=1 N=2000", flush=True)
    big = GpuRun(synth.make_inputs(synth.CONFIGS["fwd_bf16_n16384"]))
    assert fsl.workspace_bytes(big.p) <= fsl.NOALLOC_WORKSPACE_MAX
    _same(big, _noalloc_run(big), "first call (16 heads x 16384 tokens)")
    sh = synth.Shape("noalloc_small", H=2, N=3001, d=128, dtype=synth.BF16, seed=31)
    small = GpuRun(synth.random_inputs(sh))
    _same(small, _noalloc_run(small), "second call (smaller)")
    sh3 = synth.Shape("noalloc_f32", H=1, N=2000, d=64, dtype=synth.F32, seed=32, w=100, s=16, B=64, P=8, W=2)
    third = GpuRun(synth.random_inputs(sh3))
    _same(third, _noalloc_run(third), "third call (fp32)")


def test_noalloc_rejects_a_workspace_beyond_its_array():
    from long_context_sparse_cell_amd import fsl
    sh = synth.CONFIGS["fwd_bf16_n65536"]
    dev = torch.device("cuda")
    sig, lam, gam = (torch.ones(sh.H, device=dev) for _ in range(3))
    p = fsl.make_params(sh.N, sh.H, sh.d, torch.bfloat16, sig, lam, gam)
    assert fsl.workspace_bytes(p) > fsl.NOALLOC_WORKSPACE_MAX
    x = torch.zeros((sh.H, sh.N, sh.d), dtype=torch.bfloat16, device=dev)
    with pytest.raises(fsl.FSLError) as e:
        fsl.attn_fwd_noalloc(x, x, x, p, torch.empty_like(x))
    assert e.value.code == fsl.FSL_E_WORKSPACE
