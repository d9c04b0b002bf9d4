"""Planted mistakes in copies of the oracle must each fail at least one pin.

Every mutation below edits one line of fsl_oracle.c (a dropped term, a wrong
sign, an off-by-one, a transposed index), builds the copy into a temporary
directory, and runs the pin modules (forward and backward) against it in a
subprocess. The real oracle
is never touched.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "fsl_oracle.c")

MUTATIONS = {
    "rope_sign": ("out[m + half] = b * cs + a * sn;", "out[m + half] = b * cs - a * sn;"),
    "rope_theta": ("-2.0 * (double)m / (double)p->d);\n        double ang = (double)t * theta;\n        double cs = cos(ang), sn = sin(ang);\n        double a = (double)x[m]",
                   "-1.0 * (double)m / (double)p->d);\n        double ang = (double)t * theta;\n        double cs = cos(ang), sn = sin(ang);\n        double a = (double)x[m]"),
    "window_width": ("int64_t j0 = i - p->w + 1;\n    if (j0 < 0) j0 = 0;\n    const int64_t n",
                     "int64_t j0 = i - p->w;\n    if (j0 < 0) j0 = 0;\n    const int64_t n"),
    "eligible_edge": ("int64_t x = b * (int64_t)p->B - (int64_t)p->w + 1;",
                      "int64_t x = b * (int64_t)p->B - (int64_t)p->w + 2;"),
    "erf_width": ("double arg = (p->sigma * (double)(i - c * (int64_t)p->s)) / (2.0 * (double)p->s);",
                  "double arg = (p->sigma * (double)(i - c * (int64_t)p->s)) / ((double)p->s);"),
    "erf_dropped": ("* erf(arg);", "* 1.0;"),
    "pool_tie": ("return (a->idx < b->idx) ? -1 : (a->idx > b->idx);\n}\n\nstatic int cmp_i32",
                 "return (a->idx > b->idx) ? -1 : (a->idx < b->idx);\n}\n\nstatic int cmp_i32"),
    "pool_recent": ("const int64_t m = nb > p->W ? nb - p->W : 0;", "const int64_t m = nb > p->W ? nb - p->W + 1 : 0;"),
    "stats_mean": ("kbar[c * d + x] = (float)(acc / (double)s);", "kbar[c * d + x] = (float)(acc / (double)(s + 1));"),
    "stats_norm": ("if (ss > best) best = ss;", "if (ss > best) best = ss + 1e-3;"),
    "score_cell_stride": ("kbar + c * d, amax[c], c, p);", "kbar + c, amax[c], c, p);"),
    "select_order": ("if (a->sc > b->sc) return -1;\n    if (a->sc < b->sc) return 1;",
                     "if (a->sc < b->sc) return -1;\n    if (a->sc > b->sc) return 1;"),
    "readout_scale": ("double val = p->scale * dot;", "double val = dot;"),
    "readout_cell_token": ("((int64_t)sel[u] * s + j) * d;\n            double dot",
                           "((int64_t)sel[u] * s + j + 1) * d;\n            double dot"),
    "mix_mean": ("ms /= (double)d;", "ms /= (double)(d - 1);"),
    "mix_gamma": ("out[x] = o_win[x] + p->gamma * (o_long[x] / den);", "out[x] = o_win[x] + (o_long[x] / den);"),
    # the backward
    "bwd_rotate_back": ("out[m + half] = b * cs - a * sn;", "out[m + half] = b * cs + a * sn;"),
    "bwd_softmax_D": ("const double dS = l[t] * (dP - D);", "const double dS = l[t] * dP;"),
    "bwd_rmsnorm_projection": ("dO[x] = (p->gamma * (double)dout[i * d + x] - y * dyy / (double)d) / r;",
                               "dO[x] = (p->gamma * (double)dout[i * d + x]) / r;"),
    "bwd_dgamma": ("dg += (double)dout[i * d + x] * y;", "dg += (double)dout[i * d + x] * o[x];"),
    "bwd_scale": ("da[x] += p->scale * dS * bx;", "da[x] += dS * bx;"),
    "bwd_dv_weight": ("K->dv[j * d + x] += l[t] * dO[x];", "K->dv[j * d + x] += dO[x];"),
    # FS-B
    "fsb_radius_dropped": ("const double tt = fma(qn, t->rad[j], content);", "const double tt = content;"),
    "fsb_pmin": ("if ((int64_t)c * p->s < pm) pm = (int64_t)c * p->s;", "if ((int64_t)c * p->s > pm || pm == INT64_MAX) pm = (int64_t)c * p->s;"),
    "fsb_code_bit": ("if (dot > 0.0) code |= 1u << (31 - b);", "if (dot > 0.0) code |= 1u << b;"),
    "fsb_rerank_max": ("rk[u].sc = mx + log(sum);", "rk[u].sc = mx;"),
    "fsb_beam_width": ("                nbm = nc < B ? nc : B;\n                memcpy(beam, cand",
                       "                nbm = nc < 1 ? nc : 1;\n                memcpy(beam, cand"),
}
PIN_MODULES = ("test_oracle_pins.py", "test_oracle_backward_pins.py", "test_oracle_fsb_pins.py")


@pytest.mark.slow
@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    src = open(SRC).read()
    old, new = MUTATIONS[name]
    assert src.count(old) == 1, f"mutation {name} does not match exactly one place"
    mut = tmp_path / "mut.c"
    mut.write_text(src.replace(old, new))
    lib = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    "-o", str(lib), str(mut), "-lm"], check=True)
    env = dict(os.environ, FSL_ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider"] +
                       [os.path.join(ROOT, "tests", m) for m in PIN_MODULES],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"no pin failed for mutation {name}:\n{r.stdout[-2000:]}"
