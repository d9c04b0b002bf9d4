"""FS-L attention forward benchmark on one MI355X.

One step = one fsl_attn_fwd call over the whole workload (cell statistics,
norm prune, scoring + top-K, RoPE window attention, readout + RMSNorm + mix),
inputs already resident in HBM. Prints one JSON line with whole-job tokens/s,
per-stage kernel times measured with HIP events on the library's stream, the
roofline of the dominant kernel and the oracle timed on a bounded sample.

    python bench.py [--gpus 1] [--steps 10] [--warmup 3] [--workload fwd_bf16_n262144] [--no-cpu]
"""
import argparse
import hashlib
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_F16_PEAK_TFLOPS = 2500.0  # dense fp16/bf16 MFMA


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t handles through the HIP runtime's C API (torch's events only see torch's streams)."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.arr = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            rc = self.hip.hipEventCreate(ctypes.byref(h))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed ({rc})")
            self.arr[i] = h

    def sub(self, start, n):
        return ctypes.cast(ctypes.byref(self.arr, start * ctypes.sizeof(ctypes.c_void_p)),
                           ctypes.POINTER(ctypes.c_void_p))

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), self.arr[a], self.arr[b])
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def close(self):
        for h in self.arr:
            self.hip.hipEventDestroy(h)


def algorithmic_work(sh, sel_np=None):
    """Per-launch algorithmic bytes / flops of each stage: what the method must move or compute,
    each input read once and each output written once."""
    H, N, d, s, w, B, K = sh.H, sh.N, sh.d, sh.s, sh.w, sh.B, sh.K
    e = 2 if sh.dtype == "bf16" else 4
    C = N // s
    i = np.arange(N, dtype=np.float64)
    win_keys = np.minimum(i + 1, w).sum()
    nblk = (N + B - 1) // B
    nb = np.array([max(0, (b * B - w + 1) // s) for b in range(nblk)], dtype=np.int64)
    npool = np.minimum(nb, sh.P + sh.W)
    work = {
        # k read once; kbar and amax written once
        "cell_stats": ("hbm", H * N * d * e + H * C * (d + 1) * 4),
        # q and kbar/amax read once, the pools and selections written once
        "select": ("hbm", H * N * d * e + H * C * (d + 1) * 4 + H * nblk * (sh.P + sh.W) * 4 + H * N * K * 4),
        "window": ("mfma", H * 4.0 * d * win_keys),
    }
    if sh.dtype == "bf16":
        # the bf16 statistics are fused into one pass that also reads v and writes the fp16
        # rotated keys and transposed fp16 values (the key/value preparation stage is empty):
        # the statistics roofline counts the statistics' own bytes (k read, kbar/amax written),
        # the fused pass's whole traffic is reported beside it
        work["_cell_stats_fused_pass"] = H * N * d * (2 * e + 2 * 2) + H * C * (d + 1) * 4
    pairs = H * N * K
    if sel_np is not None:
        union_cells = 0
        distinct = 0
        for h in range(H):
            sh_sel = sel_np[h]
            distinct += int(np.unique(sh_sel[sh_sel >= 0]).size)
            pad = (-N) % B
            blocks = np.concatenate([sh_sel, np.full((pad, K), -1, sh_sel.dtype)]).reshape(nblk, B * K)
            srt = np.sort(blocks, axis=1)
            union_cells += int(((np.diff(srt, axis=1) != 0).sum(axis=1) + 1 - (srt[:, 0] < 0)).sum())
        pairs = int((sel_np >= 0).sum())
        work["_union_cells_per_block"] = union_cells / (H * nblk)
        work["_distinct_cells"] = distinct
    else:
        distinct = 0
    # the keys and values of every selected cell once per head (keys in the input dtype;
    # values fp16 on the bf16 path, fp32 otherwise)
    cells = distinct * s * d * (e + (2 if sh.dtype == "bf16" else 4))
    if sh.dtype == "bf16":
        # long branch: q read, each selected cell's keys and values, and per (query, selected
        # cell) the partial output it hands to the window kernel (fp16 d values and one float)
        work["readout"] = ("hbm", H * N * d * e + cells + pairs * (2 * d + 4))
        work["window_mix"] = work.pop("window")
        work["_partials_bytes"] = pairs * (2 * d + 4)
    else:
        # q and o_win read, out written, plus the keys and values of every selected cell
        work["readout_mix"] = ("hbm", H * N * d * (e + 4 + e) + cells)
    return work


# HBM bytes per launch measured with rocprofv3 --pmc (FETCH_SIZE x 2.00 + WRITE_SIZE x 1.00, the
# factors read off a plain 1 GiB device copy in the same run), for the kernel source they were taken
# on and the workload they were taken at; reported only for that workload while that source is unchanged.
TRAFFIC = {
    "readout": {"bytes": 4283625407, "workload": "fwd_bf16_h8_n262144_d128",
                "source": "long_context_sparse_cell_amd/csrc/readout_units.hip",
                "sha256": "67530fe0086f0ef45710561ad92adc5f4d8fd3ab111788e5d88f037858b604af",
                "profile": "profiles/fwd_n262144_hbm_traffic.md"},
    "window_mix": {"bytes": 4985320457, "workload": "fwd_bf16_h8_n262144_d128",
                   "source": "long_context_sparse_cell_amd/csrc/window_bf16.hip",
                   "sha256": "27b1d6235fc3f1b60f02f940b237fa58825a018a9196bcf2e4e388e368aa2a71",
                   "profile": "profiles/fwd_n262144_hbm_traffic.md"},
    "decode_step": {"bytes": 191697316, "workload": "decode_bf16_64seq_h16_d64_prefix131072",
                    "source": "long_context_sparse_cell_amd/csrc/decode.hip",
                    "sha256": "f18958cf685d90b25e9ab85b33099e375a5c0adf61f23c1441ebe0535fa3f4b9",
                    "profile": "profiles/decode_64seq_hbm_traffic.md"},
}


def measured_traffic(stage, workload):
    rec = TRAFFIC.get(stage)
    if rec is None or rec["workload"] != workload:
        return None
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), rec["source"])
    try:
        digest = hashlib.sha256(open(path, "rb").read()).hexdigest()
    except OSError:
        return None
    return rec["bytes"] if digest == rec["sha256"] else None


def cpu_baseline(inp, sample_rows):
    """The oracle as it stands, on a bounded sample of the workload, scaled to tokens/s."""
    from oracle import ref
    sh = inp.shape
    threads = len(os.sched_getaffinity(0))
    rows = np.arange(sh.N - sample_rows, sh.N, dtype=np.int64)
    t_fixed = 0.0
    t_rows = 0.0
    for h in range(sh.H):
        p = ref.head_from_shape(sh, h, inp.sigma, inp.lam, inp.gamma)
        t0 = time.perf_counter()
        ref.forward_head(inp.q[h], inp.k[h], inp.v[h], p, rows=rows[-1:], nthreads=threads)
        t1 = time.perf_counter()
        ref.forward_head(inp.q[h], inp.k[h], inp.v[h], p, rows=rows, nthreads=threads)
        t2 = time.perf_counter()
        t_fixed += t1 - t0
        t_rows += max(0.0, (t2 - t1) - (t1 - t0))
    full = t_fixed + t_rows * sh.N / sample_rows
    return {
        "value": sh.N / full,
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": ((f"all {sh.N} query rows x {sh.H} heads of the {sh.name} workload (the whole step)"
                    if sample_rows == sh.N else
                    f"{sample_rows} query rows (the last {sample_rows // sh.B} blocks) x {sh.H} heads of the "
                    f"{sh.name} workload, plus per-head cell statistics; rows time scaled by N/{sample_rows}")
                   + f"; measured {t_fixed + t_rows:.1f} s of oracle work"),
    }


def decode_bench(fsl, synth, torch, dev, steps_override=None):
    """Streaming decode workload: prefill every sequence, then time the steps."""
    sh = synth.CONFIGS["decode_64seq"]
    H, d, n, L = sh.H, sh.d, sh.n_seq, sh.prefix
    steps = sh.steps if steps_override is None else steps_override
    sig, lam, gam = (torch.from_numpy(a).to(dev) for a in synth.head_scalars(H))
    p = fsl.make_params(1, H, d, torch.bfloat16, sig, lam, gam, w=sh.w, s=sh.s, P=sh.P, W=sh.W, K=sh.K, B=sh.B)
    st = fsl.DecodeState(p, n, dev)
    gen = torch.Generator(device=dev)
    ws = None
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for r in range(n):
        gen.manual_seed(sh.seed * 1000 + r)
        kp = torch.randn((H, L, d), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
        vp = torch.randn((H, L, d), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
        ws = st.prefill(r, kp, vp, ws)
        del kp, vp
    torch.cuda.synchronize()
    t_prefill = time.perf_counter() - t0
    gen.manual_seed(sh.seed * 1000 + 999)
    qs = torch.randn((steps, n, H, d), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    ks = torch.randn((steps, n, H, d), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    vs = torch.randn((steps, n, H, d), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    out = torch.empty((n, H, d), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        st.step(qs[i], ks[i], vs[i], out=out)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    # streamed prefill: the same prefix length appended to a fresh state in chunks for every
    # sequence at once (one work-group per (sequence, head)); only the append calls are timed
    st2 = fsl.DecodeState(p, n, dev)
    chunk = 16384
    t_app = 0.0
    gen.manual_seed(sh.seed * 1000 + 998)
    for a in range(0, L, chunk):
        m = min(chunk, L - a)
        kc = torch.randn((n, H, m, d), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
        vc = torch.randn((n, H, m, d), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        st2.append(0, kc, vc)
        torch.cuda.synchronize()
        t_app += time.perf_counter() - t0
        del kc, vc
    del st2
    torch.cuda.empty_cache()
    e = 2
    pool_cells = sh.P + sh.W
    per_head = (sh.w * 2 * d * e) + pool_cells * (d + 1) * 4 + sh.K * sh.s * 2 * d * e + 4 * d * e
    step_bytes = per_head * n * H
    step_s = el / steps
    return {
        "workload": sh.name, "sequences": n, "steps": steps, "prefix": L,
        "tokens_per_s": round(n * steps / el, 1), "ms_per_step": round(step_s * 1e3, 4),
        "prefill_s_total": round(t_prefill, 3), "state_mib": round(st.nbytes / 2 ** 20, 1),
        "streamed_prefill": {"tokens_per_s": round(n * L / t_app, 1), "s_total": round(t_app, 4), "chunk": chunk,
                             "note": "fsl_decode_append of every sequence's prefix in chunks, no O(N d) workspace"},
        "roofline": {"bound": "hbm", "achieved": round(step_bytes / step_s / 1e9, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(step_bytes / step_s / 1e9 / HBM_PEAK_GBS, 4),
                     "bytes_per_step": step_bytes, "traffic": measured_traffic("decode_step", sh.name)},
        "data": "synthetic: k/v/q ~ N(0,1) from seeded device generators",
    }


def fs_bench(fsl, synth, torch, inp, q, k, v, dev, steps, warmup):
    """The same workload without pruning (P = -1, the plain FS variant): every query scores all
    eligible cells. Stage times from HIP events; the scoring stage's roofline counts the content
    dot products, 2 d flops per (query, eligible cell), against the bf16 MFMA peak."""
    sh = inp.shape
    sig, lam, gam = (torch.from_numpy(a).to(dev) for a in (inp.sigma, inp.lam, inp.gamma))
    p = fsl.make_params(sh.N, sh.H, sh.d, q.dtype, sig, lam, gam, w=sh.w, s=sh.s, P=-1, W=sh.W, K=sh.K, B=sh.B)
    ws = fsl.new_workspace(p, dev)
    out = torch.empty_like(q)
    nst = fsl.NUM_STAGES + 1
    ev = HipEvents(nst * max(steps, warmup, 1))
    for i in range(warmup):
        fsl.attn_fwd_timed(q, k, v, p, out, ws, ev.sub(0, nst))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        fsl.attn_fwd_timed(q, k, v, p, out, ws, ev.sub(i * nst, nst))
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    stage_ms = {name: round(float(np.mean([ev.elapsed_ms(i * nst + j, i * nst + j + 1) for i in range(steps)])), 4)
                for j, name in enumerate(fsl.stage_names(p))}
    ev.close()
    nblk = (sh.N + sh.B - 1) // sh.B
    pairs = 0
    for b in range(nblk):
        nb = max(0, (b * sh.B - sh.w + 1) // sh.s)
        pairs += nb * (min(sh.N, (b + 1) * sh.B) - b * sh.B)
    flops = sh.H * 2.0 * sh.d * pairs
    sel_tf = flops / (stage_ms["select"] * 1e-3) / 1e12
    del ws
    torch.cuda.empty_cache()
    return {
        "workload": sh.name + "_noprune", "P": -1,
        "tokens_per_s": round(sh.N * steps / el, 1), "ms_per_step": round(el * 1e3 / steps, 4),
        "stages": stage_ms,
        "select_roofline": {"bound": "mfma", "achieved": round(sel_tf, 2), "peak": MFMA_F16_PEAK_TFLOPS,
                            "unit": "TFLOP/s", "frac": round(sel_tf / MFMA_F16_PEAK_TFLOPS, 4),
                            "flops_per_launch": flops},
    }


def upload(inp, dev):
    import torch
    from long_context_sparse_cell_amd import synth

    def up(x):
        if inp.shape.dtype == synth.BF16:
            return torch.from_numpy(synth.bf16_bits(x).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(x).to(dev)
    return up(inp.q), up(inp.k), up(inp.v)


def time_forward(fsl, torch, sh, inp, q, k, v, dev, steps, warmup, with_work=False):
    """Time `steps` forwards of one workload (after `warmup`), with per-stage HIP events."""
    sig, lam, gam = (torch.from_numpy(a).to(dev) for a in (inp.sigma, inp.lam, inp.gamma))
    p = fsl.make_params(sh.N, sh.H, sh.d, q.dtype, sig, lam, gam, w=sh.w, s=sh.s, P=sh.P, W=sh.W, K=sh.K, B=sh.B)
    ws = fsl.new_workspace(p, dev)
    out = torch.empty_like(q)
    nst = fsl.NUM_STAGES + 1
    ev = HipEvents(nst * max(steps, warmup, 1))
    for i in range(warmup):
        fsl.attn_fwd_timed(q, k, v, p, out, ws, ev.sub(0, nst))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        fsl.attn_fwd_timed(q, k, v, p, out, ws, ev.sub(i * nst, nst))
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    stage_ms = {name: float(np.mean([ev.elapsed_ms(i * nst + j, i * nst + j + 1) for i in range(steps)]))
                for j, name in enumerate(fsl.stage_names(p))}
    gpu_ms = float(np.mean([ev.elapsed_ms(i * nst, i * nst + nst - 1) for i in range(steps)]))
    ev.close()
    res = {"workload": sh.name, "tokens_per_s": round(sh.N * steps / el, 1), "ms_per_step": round(el * 1e3 / steps, 4),
           "ns_per_token": round(el * 1e9 / steps / sh.N, 3), "gpu_ms_per_step": round(gpu_ms, 4),
           "stage_ms": {n: round(t, 4) for n, t in stage_ms.items()}, "elapsed_s": el}
    if with_work:
        sel_np = fsl.workspace_views(ws, p)["sel"].cpu().numpy()
        work = algorithmic_work(sh, sel_np)
        stages = {}
        for name, t in stage_ms.items():
            entry = {"ms": round(t, 4)}
            if name in work:
                kind, amount = work[name]
                if kind == "hbm":
                    entry.update(bound="hbm", achieved=amount / (t * 1e-3) / 1e9, peak=HBM_PEAK_GBS, unit="GB/s")
                else:
                    entry.update(bound="mfma", achieved=amount / (t * 1e-3) / 1e12, peak=MFMA_F16_PEAK_TFLOPS,
                                 unit="TFLOP/s")
                entry["frac"] = round(entry["achieved"] / entry["peak"], 4)
                entry["achieved"] = round(entry["achieved"], 2)
            stages[name] = entry
        if "_cell_stats_fused_pass" in work:
            gbs = work["_cell_stats_fused_pass"] / (stage_ms["cell_stats"] * 1e-3) / 1e9
            stages["cell_stats"]["fused_pass"] = {
                "note": "the bf16 statistics pass also reads v and writes the fp16 rotated keys and values",
                "bytes": work["_cell_stats_fused_pass"], "achieved": round(gbs, 2), "frac": round(gbs / HBM_PEAK_GBS, 4)}
        dominant = max((n for n in stages if "bound" in stages[n]), key=lambda n: stage_ms[n])
        dom = stages[dominant]
        res["stages"] = stages
        res["work"] = work
        res["roofline"] = {"kernel": dominant, "bound": dom["bound"], "achieved": dom["achieved"], "peak": dom["peak"],
                           "unit": dom["unit"], "frac": dom["frac"], "traffic": measured_traffic(dominant, sh.name)}
    del ws, out
    torch.cuda.empty_cache()
    return res


F32_PEAK_TFLOPS = 157.3  # fp32, on the matrix cores (dense) as on the vector ALUs


def backward_bench(fsl, synth, torch, sh, inp, q, k, v, dev, steps, warmup):
    """fsl_attn_bwd on one workload (after one forward whose selections it reuses): ms per call and
    the rate of algorithmic work, 10 d flops per (query, key) pair of both branches (scores, dP, and
    the dq, dk, dv products), against the fp32 peak (157.3 TFLOP/s on MI355X): every product of both
    branches runs on the fp32 matrix cores. The long branch's recomputed forward (scores and the
    weighted values once more) is not counted."""
    sig, lam, gam = (torch.from_numpy(a).to(dev) for a in (inp.sigma, inp.lam, inp.gamma))
    p = fsl.make_params(sh.N, sh.H, sh.d, q.dtype, sig, lam, gam, w=sh.w, s=sh.s, P=sh.P, W=sh.W, K=sh.K, B=sh.B)
    fws = fsl.new_workspace(p, dev)
    fsl.attn_fwd(q, k, v, p, ws=fws)
    gen = torch.Generator(device=dev)
    gen.manual_seed(4242)
    dout = torch.randn(q.shape, generator=gen, device=dev, dtype=torch.float32).to(q.dtype)
    bws = torch.empty(fsl.attn_bwd_workspace_bytes(p), dtype=torch.uint8, device=dev)
    grads = [torch.empty(q.shape, dtype=torch.float32, device=dev) for _ in range(3)]
    dg = torch.empty(sh.H, dtype=torch.float32, device=dev)
    for _ in range(warmup):
        fsl.attn_bwd(q, k, v, dout, p, fws, ws=bws, dq=grads[0], dk=grads[1], dv=grads[2], dgamma=dg)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fsl.attn_bwd(q, k, v, dout, p, fws, ws=bws, dq=grads[0], dk=grads[1], dv=grads[2], dgamma=dg)
    torch.cuda.synchronize()
    el = (time.perf_counter() - t0) / steps
    sel = fsl.workspace_views(fws, p)["sel"]
    long_tokens = int((sel >= 0).sum().item()) * sh.s
    i = np.arange(sh.N, dtype=np.float64)
    pairs = sh.H * float(np.minimum(i + 1, sh.w).sum()) + long_tokens
    flops = 10.0 * sh.d * pairs
    tf = flops / el / 1e12
    del fws, bws, grads, dout
    torch.cuda.empty_cache()
    return {"workload": sh.name, "ms_per_step": round(el * 1e3, 3), "tokens_per_s": round(sh.N / el, 1),
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": F32_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / F32_PEAK_TFLOPS, 4), "flops_per_launch": flops,
                         "note": "fp32 on the matrix cores, both branches"}}


def fsb_bench(fsl, synth, torch, sh, inp, q, k, v, dev, steps, warmup):
    """The forward with FS-B selections (beam 16 over two causal forests): ms per step and tokens/s,
    and the selection's own time (fsl_fsb_select, cell statistics and forests included)."""
    sig, lam, gam = (torch.from_numpy(a).to(dev) for a in (inp.sigma, inp.lam, inp.gamma))
    p = fsl.make_params(sh.N, sh.H, sh.d, q.dtype, sig, lam, gam, w=sh.w, s=sh.s, P=sh.P, W=sh.W, K=sh.K, B=sh.B)
    # tau: the median cell norm of each head's first 4096 tokens (a stand-in for the pages'
    # per-checkpoint median over training windows); projections: seeded Gaussian rows
    kb, am = fsl.cell_stats(k[:, :4096].contiguous(), fsl.make_params(4096, sh.H, sh.d, q.dtype, sig, lam, gam,
                                                                        s=sh.s, B=sh.B))
    tau = am.median(dim=1).values.contiguous()
    gen = torch.Generator(device=dev)
    gen.manual_seed(31)
    proj = torch.randn((32, sh.d), generator=gen, device=dev, dtype=torch.float32)
    fb = fsl.make_fsb_params(tau, proj, 16)
    ws = torch.empty(fsl.fsb_workspace_bytes(p), dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    sel = torch.empty((sh.H, sh.N, sh.K), dtype=torch.int32, device=dev)
    res = {"workload": sh.name + "_fsb", "beam": 16}
    for name, fn in (("forward", lambda: fsl.attn_fwd_fsb(q, k, v, p, fb, out=out, ws=ws)),
                     ("select", lambda: fsl.fsb_select(q, k, p, fb, ws=ws, sel=sel))):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        el = (time.perf_counter() - t0) / steps
        res[name] = {"ms_per_step": round(el * 1e3, 3), "tokens_per_s": round(sh.N / el, 1)}
    del ws, out, sel
    torch.cuda.empty_cache()
    return res


def other_workloads(fsl, synth, torch, dev, steps, warmup, skip):
    """The other forward workloads (4k fp32, 16k and 64k bf16), each timed on its own seeded inputs."""
    res = {}
    for name in ("fwd_f32_n4096", "fwd_bf16_n16384", "fwd_bf16_n65536"):
        if name == skip:
            continue
        sh = synth.CONFIGS[name]
        log(f"[bench] workload {sh.name}")
        inp = synth.make_inputs(sh)
        q, k, v = upload(inp, dev)
        r = time_forward(fsl, torch, sh, inp, q, k, v, dev, steps, warmup)
        r.pop("elapsed_s")
        res[sh.name] = r
        del q, k, v, inp
    torch.cuda.empty_cache()
    return res


def linearity_check(fsl, synth, torch, dev, steps, warmup):
    """The pages' O(N) cost claim: the 16-head, d=64 bf16 shape at N = 16384, 65536 and 262144
    (q, k, v ~ N(0,1) drawn on the device), time per token at each N; flat within ~20% is linear."""
    H, d = 16, 64
    sig, lam, gam = (torch.from_numpy(a).to(dev) for a in synth.head_scalars(H))
    gen = torch.Generator(device=dev)
    pts = []
    for N in (16384, 65536, 262144):
        gen.manual_seed(7000 + N)
        q, k, v = (torch.randn((H, N, d), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
                   for _ in range(3))
        sh = synth.Shape(f"linear_bf16_h{H}_n{N}_d{d}", H=H, N=N, d=d, dtype=synth.BF16, seed=0)
        inp = synth.Inputs(sh, None, None, None, *synth.head_scalars(H))
        r = time_forward(fsl, torch, sh, inp, q, k, v, dev, steps, warmup)
        log(f"[bench] O(N) check N={N}: {r['ns_per_token']:.3f} ns/token")
        pts.append({"N": N, "ms_per_step": r["ms_per_step"], "ns_per_token": r["ns_per_token"],
                    "stage_ms": r["stage_ms"]})
        del q, k, v
    torch.cuda.empty_cache()
    per = [x["ns_per_token"] for x in pts]
    return {"shape": f"H={H}, d={d}, bf16, q/k/v ~ N(0,1), pruned FS-L", "points": pts,
            "max_over_min_ns_per_token": round(max(per) / min(per), 3),
            "claim": "FS-L attention cost O(N) (FreeSolo digest, motivation; ai.info summary, Key Contributions)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="fwd_bf16_n262144", help="a forward workload of synth.CONFIGS (default fwd_bf16_n262144: N=262144, H=8, d=128, bf16)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--cpu-rows", type=int, default=262144)
    ap.add_argument("--no-decode", action="store_true", help="skip the streaming-decode measurement")
    ap.add_argument("--no-fs", action="store_true", help="skip the unpruned (P = -1) forward measurement")
    ap.add_argument("--no-others", action="store_true", help="skip the 4k/16k/64k workloads and the O(N) check")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward (fsl_attn_bwd) measurement")
    ap.add_argument("--no-fsb", action="store_true", help="skip the FS-B forward measurement")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="first run one plain device copy of this many MiB, the reference kernel for scaling "
                         "profiler byte counters (FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
              "the path would shard heads and sequences across GPUs with no exchange", file=sys.stderr)
        sys.exit(2)

    import torch
    from long_context_sparse_cell_amd import fsl, synth

    if args.calib_copy_mib > 0:
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy: {args.calib_copy_mib} MiB read, {args.calib_copy_mib} MiB written")
        del src, dst

    sh = synth.CONFIGS[args.workload]
    assert sh.kind == "fwd"
    log(f"[bench] generating {sh.name}")
    inp = synth.make_inputs(sh)
    dev = torch.device("cuda:0")
    q, k, v = upload(inp, dev)
    head = time_forward(fsl, torch, sh, inp, q, k, v, dev, args.steps, args.warmup, with_work=True)
    stages, roofline, work = head["stages"], head["roofline"], head["work"]
    t0, t1 = 0.0, head["elapsed_s"]
    # the decode workload next, before the other measurements' large allocations come and go: a
    # decode step reads about 190 MB spread over its 847 MiB state, and measured 5x slower on a
    # state allocated after that churn
    dec = None
    if not args.no_decode:
        log("[bench] streaming decode workload")
        torch.cuda.empty_cache()
        dec = decode_bench(fsl, synth, torch, dev)
        log(f"[bench] decode {dec['tokens_per_s']:.0f} tokens/s, {dec['ms_per_step']:.3f} ms/step")

    others = lin = None
    if not args.no_others:
        others = other_workloads(fsl, synth, torch, dev, args.steps, args.warmup, args.workload)
        lin = linearity_check(fsl, synth, torch, dev, args.steps, args.warmup)

    bwd = None
    if not args.no_backward:
        log("[bench] backward")
        bwd = {sh.name: backward_bench(fsl, synth, torch, sh, inp, q, k, v, dev, max(1, args.steps // 4), 1)}
        log(f"[bench] backward {sh.name}: {bwd[sh.name]['ms_per_step']} ms")
        if not args.no_others:
            sh2 = synth.CONFIGS["fwd_bf16_n16384"]
            inp2 = synth.make_inputs(sh2)
            q2, k2, v2 = upload(inp2, dev)
            bwd[sh2.name] = backward_bench(fsl, synth, torch, sh2, inp2, q2, k2, v2, dev, args.steps, args.warmup)
            log(f"[bench] backward {sh2.name}: {bwd[sh2.name]['ms_per_step']} ms")
            del q2, k2, v2, inp2

    fsb = None
    if not args.no_fsb:
        log("[bench] FS-B forward")
        fsb = {sh.name: fsb_bench(fsl, synth, torch, sh, inp, q, k, v, dev, max(1, args.steps // 4), 1)}
        log(f"[bench] FS-B {sh.name}: {fsb[sh.name]}")
        if not args.no_others:
            sh2 = synth.CONFIGS["fwd_bf16_n16384"]
            inp2 = synth.make_inputs(sh2)
            q2, k2, v2 = upload(inp2, dev)
            fsb[sh2.name] = fsb_bench(fsl, synth, torch, sh2, inp2, q2, k2, v2, dev, args.steps, args.warmup)
            log(f"[bench] FS-B {sh2.name}: {fsb[sh2.name]}")
            del q2, k2, v2, inp2

    fs = None
    if not args.no_fs and sh.dtype == synth.BF16:
        log("[bench] unpruned (P = -1) forward")
        torch.cuda.empty_cache()
        fs = fs_bench(fsl, synth, torch, inp, q, k, v, dev, args.steps, args.warmup)
        log(f"[bench] unpruned forward {fs['ms_per_step']:.3f} ms/step, stages {fs['stages']}")

    cpu = None
    if not args.no_cpu:
        log(f"[bench] oracle CPU baseline on {args.cpu_rows} rows")
        cpu = cpu_baseline(inp, min(args.cpu_rows, sh.N))

    tokens = sh.N
    line = {
        "metric": "FS-L attention fwd tokens/s at N=16k-256k; % of HBM/MFMA roofline",
        "value": round(tokens * args.steps / (t1 - t0), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": sh.dtype,
        "data": "synthetic (seeded q/k/v with planted needles; no dataset)",
        "config": {"workload": sh.name, "H": sh.H, "N": sh.N, "d": sh.d, "w": sh.w, "s": sh.s, "P": sh.P,
                   "W": sh.W, "K": sh.K, "B": sh.B, "batch": 1},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "stages": stages,
        "gpu_ms_per_step": head["gpu_ms_per_step"],
        "ns_per_token": head["ns_per_token"],
        "union_cells_per_block": round(work.get("_union_cells_per_block", 0.0), 2),
        "distinct_selected_cells": work.get("_distinct_cells"),
        "other_workloads": others,
        "backward": bwd,
        "fsb": fsb,
        "linearity": lin,
        "decode": dec,
        "noprune": fs,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
