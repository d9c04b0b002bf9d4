"""Pins of the oracle's backward (orc_backward_head), on the CPU.

The backward differentiates the forward with the selection held fixed (the
pages: hard top-P / top-K indices receive no gradient; the routing scalars
sigma_h, lambda_h are fixed; the per-head mixing weight is learned). Each
pin checks it against something other than itself:
  1. torch.autograd in fp64 through an independent forward: RoPE as complex
     rotations, both branches as masked scaled_dot_product_attention, RMSNorm
     and the mix, with the oracle's selections as a fixed attention mask;
  2. central finite differences of the oracle's own forward output (whose
     arithmetic other pins fix), at coordinates whose perturbation leaves
     every selection unchanged;
  3. closed forms: a zero upstream gradient gives zero gradients; with
     gamma = 0 the long branch passes no gradient to q, k, v, and dgamma is the
     sum of dout . RMSNorm(o_long).
"""
import numpy as np
import pytest
import torch

from long_context_sparse_cell_amd import synth

TINY = dict(d=8, w=16, s=4, B=8, P=3, W=2, K=2)


def _inputs(N, seed, **over):
    par = dict(TINY)
    par.update(over)
    sh = synth.Shape(f"bwd_{N}_{seed}", H=1, N=N, dtype=synth.F32, seed=seed, **par)
    inp = synth.random_inputs(sh)
    inp.k[:, ::3] *= 2.0  # varied cell norms
    rng = np.random.default_rng(seed + 100)
    dout = rng.standard_normal((1, N, sh.d)).astype(np.float32)
    return sh, inp, dout


def rope_complex(x, pos, base):
    d = x.shape[-1]
    half = d // 2
    theta = base ** (-2.0 * torch.arange(half, dtype=torch.float64) / d)
    rot = torch.polar(torch.ones(len(pos), half, dtype=torch.float64), pos[:, None] * theta[None, :])
    xc = torch.complex(x[:, :half], x[:, half:]) * rot
    return torch.cat([xc.real, xc.imag], dim=1)


def torch_forward(q, k, v, gamma, sel, p):
    """FS-L forward in fp64 torch with the selection fixed: a differentiable reference."""
    N, d = q.shape
    pos = torch.arange(N, dtype=torch.float64)
    qr, kr = rope_complex(q, pos, p.rope_base), rope_complex(k, pos, p.rope_base)
    i = torch.arange(N)[:, None]
    j = torch.arange(N)[None, :]
    band = (j <= i) & (j > i - p.w)
    sdpa = torch.nn.functional.scaled_dot_product_attention
    o_win = sdpa(qr[None], kr[None], v[None], attn_mask=band[None], scale=p.scale)[0]
    sel_mask = torch.zeros(N, N, dtype=torch.bool)
    for r in range(N):
        for c in sel[r]:
            if c >= 0:
                sel_mask[r, c * p.s:(c + 1) * p.s] = True
    has = sel_mask.any(dim=1)
    safe = sel_mask.clone()
    safe[~has, 0] = True  # rows without cells attend to one dummy key, then are zeroed
    o_long = sdpa(q[None], k[None], v[None], attn_mask=safe[None], scale=p.scale)[0]
    o_long = torch.where(has[:, None], o_long, torch.zeros_like(o_long))
    y = o_long / torch.sqrt((o_long ** 2).mean(dim=1, keepdim=True) + p.rms_eps)
    return o_win + gamma * y


CASES = [
    ("n1", 1, dict()), ("n7", 7, dict()), ("n40", 40, dict()), ("n133", 133, dict()),
    ("n133_unpruned_k3", 133, dict(P=-1, K=3)), ("n90_w5", 90, dict(w=5)),
    ("n150_s8_b16", 150, dict(s=8, B=16, P=4, W=1, K=3)), ("n64_d16_wide", 64, dict(d=16, w=80)),
]


@pytest.mark.parametrize("name,N,over", CASES, ids=[c[0] for c in CASES])
def test_backward_matches_torch_autograd(oracle, name, N, over):
    sh, inp, dout = _inputs(N, 5 + N, **over)
    for sigma, gamma in [(4.0, 0.7), (0.05, 1.3)]:
        p = oracle.head_from_shape(sh, 0, inp.sigma * 0 + sigma, inp.lam, inp.gamma * 0 + gamma)
        fwd = oracle.forward_head(inp.q[0], inp.k[0], inp.v[0], p)
        g = oracle.backward_head(inp.q[0], inp.k[0], inp.v[0], dout[0], fwd["sel"], p)
        tq, tk, tv = (torch.tensor(a[0], dtype=torch.float64, requires_grad=True) for a in (inp.q, inp.k, inp.v))
        tg = torch.tensor(p.gamma, dtype=torch.float64, requires_grad=True)
        out = torch_forward(tq, tk, tv, tg, fwd["sel"], p)
        np.testing.assert_allclose(out.detach().numpy(), fwd["out"], rtol=1e-11, atol=1e-12)
        (out * torch.tensor(dout[0], dtype=torch.float64)).sum().backward()
        for name_, ref, got in [("dq", tq.grad, g["dq"]), ("dk", tk.grad, g["dk"]), ("dv", tv.grad, g["dv"])]:
            np.testing.assert_allclose(got, ref.numpy(), rtol=1e-9, atol=1e-11, err_msg=f"{name_} sigma={sigma}")
        assert abs(g["dgamma"] - float(tg.grad)) <= 1e-9 * max(1.0, abs(float(tg.grad)))


def test_backward_matches_finite_differences(oracle):
    """Central differences of L = sum(dout * out) through the oracle's forward, at
    coordinates where the perturbation changes no selection."""
    sh, inp, dout = _inputs(96, 11)
    p = oracle.head_from_shape(sh, 0, inp.sigma, inp.lam, inp.gamma * 0 + 0.8)
    base = oracle.forward_head(inp.q[0], inp.k[0], inp.v[0], p)
    g = oracle.backward_head(inp.q[0], inp.k[0], inp.v[0], dout[0], base["sel"], p)
    h = 2.0 ** -12
    rng = np.random.default_rng(3)

    def loss(q, k, v, pp):
        r = oracle.forward_head(q, k, v, pp)
        return float((r["out"] * dout[0]).sum()), r["sel"]

    checked = 0
    for which, grad in (("q", g["dq"]), ("k", g["dk"]), ("v", g["dv"])):
        for _ in range(25):
            i, x = int(rng.integers(0, sh.N)), int(rng.integers(0, sh.d))
            arrs = {"q": inp.q[0].copy(), "k": inp.k[0].copy(), "v": inp.v[0].copy()}
            a0 = arrs[which][i, x]
            arrs[which][i, x] = a0 + h
            lp, sp = loss(arrs["q"], arrs["k"], arrs["v"], p)
            arrs[which][i, x] = a0 - h
            lm, sm = loss(arrs["q"], arrs["k"], arrs["v"], p)
            if not (np.array_equal(sp, base["sel"]) and np.array_equal(sm, base["sel"])):
                continue  # a selection moved: no derivative defined there
            fd = (lp - lm) / (2 * h)
            assert abs(fd - grad[i, x]) <= 1e-5 * max(1.0, abs(fd)), (which, i, x, fd, grad[i, x])
            checked += 1
    assert checked >= 60
    # gamma
    pp, pm = oracle.head_from_shape(sh, 0, inp.sigma, inp.lam, inp.gamma * 0 + 0.8), None
    pp.gamma = 0.8 + h
    lp, _ = loss(inp.q[0], inp.k[0], inp.v[0], pp)
    pm = oracle.head_from_shape(sh, 0, inp.sigma, inp.lam, inp.gamma * 0 + 0.8)
    pm.gamma = 0.8 - h
    lm, _ = loss(inp.q[0], inp.k[0], inp.v[0], pm)
    assert abs((lp - lm) / (2 * h) - g["dgamma"]) <= 1e-6 * max(1.0, abs(g["dgamma"]))


def test_backward_closed_forms(oracle):
    sh, inp, dout = _inputs(120, 13)
    p = oracle.head_from_shape(sh, 0, inp.sigma, inp.lam, inp.gamma * 0 + 0.9)
    fwd = oracle.forward_head(inp.q[0], inp.k[0], inp.v[0], p)
    z = oracle.backward_head(inp.q[0], inp.k[0], inp.v[0], np.zeros_like(dout[0]), fwd["sel"], p)
    assert not z["dq"].any() and not z["dk"].any() and not z["dv"].any() and z["dgamma"] == 0.0
    # gamma = 0: q, k, v gradients come from the window branch alone, and equal those of
    # the same call with every selection emptied; dgamma is still sum(dout . RMSNorm(o_long))
    p0 = oracle.head_from_shape(sh, 0, inp.sigma, inp.lam, inp.gamma * 0)
    g0 = oracle.backward_head(inp.q[0], inp.k[0], inp.v[0], dout[0], fwd["sel"], p0)
    ge = oracle.backward_head(inp.q[0], inp.k[0], inp.v[0], dout[0], np.full_like(fwd["sel"], -1), p0)
    for key in ("dq", "dk", "dv"):
        np.testing.assert_array_equal(g0[key], ge[key])
    ol = fwd["o_long"]
    y = ol / np.sqrt((ol ** 2).mean(axis=1, keepdims=True) + p.rms_eps)
    np.testing.assert_allclose(g0["dgamma"], float((dout[0].astype(np.float64) * y).sum()), rtol=1e-12)
    assert ge["dgamma"] == 0.0
