"""Pins of the oracle's FS-B selection (beam search over two causal forests), on the CPU.

Each checks the oracle against something other than itself: the codes against
numpy's sign bits; every segment tree's leaf order against a brute-force sort
and its node statistics against numpy (means, largest norms, earliest
positions, and every leaf inside its ancestors' balls); the node bound against
the exact score of every cell beneath (it must never be lower, and equals it
at a leaf); an unbounded beam against the brute-force top-K of all eligible
cells by token-level log-sum-exp (scipy); and a planted high-norm needle that a
small beam must find.
"""
import numpy as np
import pytest
from scipy.special import logsumexp

from long_context_sparse_cell_amd import synth

PAR = dict(d=16, w=64, s=8, B=32, K=3)


def _setup(N, seed, **over):
    par = dict(PAR)
    par.update(over)
    sh = synth.Shape(f"fsb_{N}_{seed}", H=1, N=N, dtype=synth.F32, seed=seed, **par)
    inp = synth.random_inputs(sh)
    rng = np.random.default_rng(seed + 7)
    scale = np.exp(rng.normal(0, 0.4, size=(N, 1))).astype(np.float32)  # varied key norms
    inp.k[0] = (inp.k[0] * scale).astype(np.float32)
    proj = rng.standard_normal((32, sh.d)).astype(np.float32)
    return sh, inp, proj


def _codes(kbar, proj):
    bits = (proj.astype(np.float64) @ kbar.astype(np.float64).T) > 0  # [32][C]
    return (bits.astype(np.uint64) << (31 - np.arange(32, dtype=np.uint64))[:, None]).sum(axis=0).astype(np.uint32)


def test_codes_are_projection_sign_bits(oracle):
    sh, inp, proj = _setup(800, 1)
    p = oracle.head_from_shape(sh, 0, inp.sigma, inp.lam, inp.gamma)
    kbar, _ = oracle.cell_stats(inp.k[0], p)
    ref = _codes(kbar, proj)
    got = np.array([oracle.fsb_code(kbar[c], proj) for c in range(len(kbar))], dtype=np.uint32)
    np.testing.assert_array_equal(got, ref)
    assert oracle.fsb_code(np.zeros(sh.d, np.float32), proj) == 0
    assert oracle.fsb_code(proj[5], proj) & (1 << 26)  # |proj_5|^2 > 0 sets bit 31 - 5


@pytest.mark.parametrize("k,a", [(0, 3), (2, 1), (4, 0), (5, 2), (6, 0)])
def test_segment_trees_match_brute_force(oracle, k, a):
    sh, inp, proj = _setup(2600, 2)
    p = oracle.head_from_shape(sh, 0, inp.sigma, inp.lam, inp.gamma)
    kbar, amax = oracle.cell_stats(inp.k[0], p)
    codes = _codes(kbar, proj)
    tau = float(np.median(amax))
    lists = [np.arange(len(kbar), dtype=np.int32), np.nonzero(amax > tau)[0].astype(np.int32)]
    for lst in lists:
        L = 1 << k
        if (a + 1) * L > len(lst):
            continue
        t = oracle.fsb_tree(lst, a, k, codes, kbar, amax, p)
        seg = [(int(codes[c]), a * L + u, int(c)) for u, c in enumerate(lst[a * L:(a + 1) * L])]
        np.testing.assert_array_equal(t["cell"], [c for _, _, c in sorted(seg)])
        for j in range(1, 2 * L):
            depth = j.bit_length() - 1
            n = L >> depth
            leaves = t["cell"][(j - (1 << depth)) * n:(j - (1 << depth) + 1) * n]
            mean = kbar[leaves].astype(np.float64).mean(axis=0)
            np.testing.assert_allclose(t["mu"][j], mean, rtol=2e-7, atol=1e-7)
            assert t["amax"][j] == amax[leaves].max()
            assert t["pmin"][j] == leaves.min() * sh.s
            far = np.linalg.norm(kbar[leaves].astype(np.float64) - t["mu"][j].astype(np.float64), axis=1).max()
            assert far <= t["rad"][j], (j, far, t["rad"][j])
            if n == 1:
                assert t["rad"][j] == 0.0


def test_node_bound_never_below_a_cell_score_beneath(oracle):
    sh, inp, proj = _setup(2600, 3)
    rng = np.random.default_rng(9)
    for sigma, lam, rho in [(4.0, 1.0, 1.0), (0.05, 1.0, 1.0), (0.5, 2.0, 0.5), (4.0, 0.0, 1.0), (0.3, 1.0, 0.0)]:
        p = oracle.head_from_shape(sh, 0, inp.sigma * 0 + sigma, inp.lam * 0 + lam, inp.gamma)
        p.rho = rho
        kbar, amax = oracle.cell_stats(inp.k[0], p)
        codes = _codes(kbar, proj)
        lst = np.arange(len(kbar), dtype=np.int32)
        k = 5
        for a in range(2):
            i = int(rng.integers((a + 1) * 32 * sh.s + sh.w, sh.N))
            qi = inp.q[0, i]
            ub = oracle.fsb_tree_bounds(lst, a, k, codes, kbar, amax, p, qi, i)
            t = oracle.fsb_tree(lst, a, k, codes, kbar, amax, p)
            L = 1 << k
            sc = np.array([oracle.cell_score(qi, i, kbar[c], amax[c], c, p) for c in t["cell"]])
            for j in range(1, 2 * L):
                depth = j.bit_length() - 1
                n = L >> depth
                lo = (j - (1 << depth)) * n
                assert ub[j] >= sc[lo:lo + n].max(), (sigma, lam, rho, j)
            np.testing.assert_array_equal(ub[L:], sc)  # a leaf's bound is its cell score


@pytest.mark.parametrize("N,seed,tau_q", [(1500, 4, 0.5), (2600, 5, 0.3), (3001, 6, 0.8)])
def test_unbounded_beam_is_brute_force_token_lse_topk(oracle, N, seed, tau_q):
    sh, inp, proj = _setup(N, seed)
    p = oracle.head_from_shape(sh, 0, inp.sigma, inp.lam, inp.gamma)
    kbar, amax = oracle.cell_stats(inp.k[0], p)
    tau = float(np.quantile(amax, tau_q))
    rows = np.unique(np.linspace(0, N - 1, 60).astype(np.int64))
    sel, lse = oracle.fsb_select(inp.q[0], inp.k[0], p, proj, tau, beam=1 << 20, rows=rows)
    k = inp.k[0].astype(np.float64)
    for r, i in enumerate(rows):
        nb = oracle.eligible(int(i) // sh.B, p)
        if nb == 0:
            assert (sel[r] == -1).all()
            continue
        l = p.scale * (k[: nb * sh.s] @ inp.q[0, i].astype(np.float64)).reshape(nb, sh.s)
        cell_lse = logsumexp(l, axis=1)
        order = sorted(range(nb), key=lambda c: (-cell_lse[c], c))[: sh.K]
        np.testing.assert_array_equal(sel[r][: len(order)], sorted(order))
        for u, c in enumerate(sel[r]):
            if c >= 0:
                assert abs(lse[r, u] - cell_lse[c]) <= 1e-12 * max(1.0, abs(cell_lse[c]))


def test_selections_are_eligible_for_any_beam(oracle):
    sh, inp, proj = _setup(2600, 7)
    p = oracle.head_from_shape(sh, 0, inp.sigma, inp.lam, inp.gamma)
    kbar, amax = oracle.cell_stats(inp.k[0], p)
    for beam in (1, 2, 16):
        sel, _ = oracle.fsb_select(inp.q[0], inp.k[0], p, proj, float(np.median(amax)), beam=beam)
        for i in range(sh.N):
            nb = oracle.eligible(i // sh.B, p)
            got = sel[i][sel[i] >= 0]
            assert (got < nb).all() and (np.diff(got) > 0).all()
            # the full-prefix forest's beam ends with min(beam, nb) leaves; the union of the
            # two beams then holds at least that many cells and at most 2 beam
            if beam >= sh.K:
                assert len(got) == min(nb, sh.K)
            else:
                assert min(nb, beam) <= len(got) <= min(nb, 2 * beam, sh.K)


def test_planted_needle_is_found_by_a_small_beam(oracle):
    sh, inp, proj = _setup(3000, 8)
    p = oracle.head_from_shape(sh, 0, inp.sigma, inp.lam, inp.gamma)
    kbar0, amax0 = oracle.cell_stats(inp.k[0], p)
    tau = float(np.median(amax0))
    pos = 713
    inp.k[0, pos] = (inp.k[0, pos] / np.linalg.norm(inp.k[0, pos]) * 6 * amax0.max()).astype(np.float32)
    i = sh.N - 1
    inp.q[0, i] = (inp.k[0, pos] / np.linalg.norm(inp.k[0, pos])).astype(np.float32)
    sel, _ = oracle.fsb_select(inp.q[0], inp.k[0], p, proj, tau, beam=2, rows=[i])
    assert pos // sh.s in sel[0]


def test_forward_with_given_selection_equals_forward(oracle):
    sh, inp, proj = _setup(1500, 9)
    p = oracle.head_from_shape(sh, 0, inp.sigma, inp.lam, inp.gamma)
    fwd = oracle.forward_head(inp.q[0], inp.k[0], inp.v[0], p)
    out, ow, ol = oracle.forward_rows_sel(inp.q[0], inp.k[0], inp.v[0], p, np.arange(sh.N), fwd["sel"])
    np.testing.assert_array_equal(out, fwd["out"])
    np.testing.assert_array_equal(ow, fwd["o_win"])
    np.testing.assert_array_equal(ol, fwd["o_long"])
