"""Benchmark of the BitDelta hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload proj_4096]

A step is one pass of the whole path over one batch of synthetic input on the
workload's matrices: compression of a fine-tuned matrix (delta, packed signs,
alpha), the decode-shaped fused linear at each decode token count, a
mixed-variant decode batch (Zipf(1.1) over 14 variants), and the prefill GEMM
(M = 2048).  Inputs are resident in HBM before timing starts.  Weight copies
rotate so that the working set of consecutive calls exceeds the 256 MB
last-level cache several times: every call streams its weights from HBM.

Launches are captured in HIP graphs so that the GPU runs them back to back
(a Python launch costs more host time than a decode kernel takes).  Timed
region 1 replays K one-pass graphs (the steps), each bracketed by HIP events,
between synchronisations: ms_per_step.  Timed region 2 replays, per kernel,
a graph of back-to-back launches that cycles four times over the rotation
copies, with HIP events around each replay, on the stream the kernels run
on (the cost of starting a replay is spread over many launches): the average launch
duration of each kernel, which is what value and the rooflines use.  The line
printed reports decode effective HBM GB/s (algorithmic bytes / kernel time)
as `value`, the prefill TFLOP/s beside it, a roofline entry per kernel, and
the CPU oracle timed on a bounded sample of the same workload.

Outside the step, the line also carries the unfused A/B (`unfused_ab`): for
each decode token count and for prefill, the fused call's kernel time, the
time of bitdelta_reconstruct (W_eff written to HBM) plus the library GEMM on
it (torch.mm, hipBLASLt), and that GEMM alone on a stored W_eff (a dense bf16
layer of the same shape, no BitDelta at all).  Their graphs are checked
against eager launches after each timed range.

Counter runs (HBM traffic per launch, rocprofv3 FETCH_SIZE and WRITE_SIZE in
two separate runs), for W = proj_4096, layer70b_multi or layer70b_prefill:

    rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT_F -o run -- python bench.py --counter-pass --workload W
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT_W -o run -- python bench.py --counter-pass --workload W
    python bench.py --summarize-counters OUT_F OUT_W --workload W

`--counter-pass` launches each kernel of the workload (for a layer, each of
its five linears) eagerly, block by block, each launch on its own rotation
copy, then a plain elementwise kernel that reads and writes a known 256 MiB
(the calibration: the counters read a fixed fraction of the true bytes).
`--summarize-counters` scales the per-dispatch counters by that calibration
and writes profiles/<kernel>_<W>_pmc.json (with a digest of the kernel's
sources: a later change of the kernel voids the figure) and
profiles/counters_<W>.md.  `--summarize-pmc DIR...` turns --pmc runs of the
same pass with other counters (waves, waits, VALU/MFMA/TA busy, LDS) into
profiles/sq_counters_<W>.md, and `--summarize-trace DIR NAME COMMAND` a
--kernel-trace --stats run into profiles/NAME_kernel_trace.md.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synthetic as S  # noqa: E402
import tenant_linear_layers_amd as T  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
MALL_BYTES = 256 * 2**20
RANGE_CYCLES = 4               # passes over the rotation copies per timing graph
METRIC = "bitdelta_linear effective HBM GB/s (decode) + bf16 TFLOP/s (prefill), 1 GPU"
PROFILES = os.path.join(ROOT, "profiles")


def sources_digest(names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "tenant_linear_layers_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


KERNEL_SOURCES = {
    "decode": ("decode.hip", "common.h", "internal.h"),
    "multi": ("decode.hip", "common.h", "internal.h"),
    "compress": ("compress.hip", "common.h", "scale_round.h"),
    "prefill": ("prefill.hip", "common.h", "internal.h"),
    "reconstruct": ("reconstruct.hip", "common.h", "internal.h"),
}


def counter_traffic(kernel: str, workload: str):
    """HBM bytes per launch measured by rocprofv3 counters, from the committed
    summary for this kernel and workload, or None when there is none or the
    kernel's sources changed since it was taken."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_pmc.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    if rec.get("sources_digest") != sources_digest(KERNEL_SOURCES[kernel]):
        return None
    return rec.get("hbm_bytes_per_launch")


def capture(fn) -> torch.cuda.CUDAGraph:
    """HIP graph of the launches fn makes (run once eagerly first, on a side
    stream, as torch's capture rules ask)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def time_replays(graph, reps: int) -> list:
    """Milliseconds of each of `reps` replays, from HIP events recorded on the
    stream the graph runs on, around each replay."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for s, e in evs:
        s.record()
        graph.replay()
        e.record()
    torch.cuda.synchronize()
    return [s.elapsed_time(e) for s, e in evs]


def median(xs) -> float:
    v = sorted(xs)
    n = len(v)
    return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])


# ------------------------------------------------------------------ workload
class ProjWorkload:
    """The 4096x4096 projection: per-row alpha, decode M = 1, 4, 16, a
    14-variant mixed decode batch of 16 tokens, prefill M = 2048."""

    name = "proj_4096"
    multi_m = 16
    prefill_m = 2048
    n_variants = 14

    def __init__(self, dev):
        wl = S.WORKLOADS["proj_4096"]
        self.wl = wl
        self.dev = dev
        self.d_out = self.d_in = 4096
        self.mode = wl.alpha_mode
        self.decode_ms = wl.tokens
        g = S.generator(wl.seed)
        wb = S.draw_base(4096, 4096, wl.sigma, g)
        wf = S.draw_finetuned(wb, wl.b, g)
        xs = {m: S.draw_activations(m, 4096, g) for m in wl.tokens}
        # 13 more variants of the same base for the mixed batch (b as the workload's)
        more = [S.draw_finetuned(wb, wl.b, g) for _ in range(self.n_variants - 1)]
        x_multi = S.draw_activations(self.multi_m, 4096, g)
        x_prefill = S.draw_activations(self.prefill_m, 4096, g)
        ids = S.zipf_ids(self.multi_m, self.n_variants, wl.seed)

        per_copy = 4096 * 4096 * 2 + 4096 * 4096 // 8
        self.R = max(4, math.ceil(4 * MALL_BYTES / per_copy))
        wb_d, wf_d = wb.to(dev), wf.to(dev)
        packed, alpha = T.compress(wf_d, wb_d, self.mode)
        variants = [(packed, alpha)] + [T.compress(w.to(dev), wb_d, self.mode) for w in more]
        self.bases = [wb_d] + [wb_d.clone() for _ in range(self.R - 1)]
        self.fts = [wf_d] + [wf_d.clone() for _ in range(min(self.R, 16) - 1)]
        self.vsets = [variants] + [[(p.clone(), a.clone()) for p, a in variants]
                                   for _ in range(self.R - 1)]
        self.xs = {m: x.to(dev) for m, x in xs.items()}
        self.x_multi = x_multi.to(dev)
        self.x_prefill = x_prefill.to(dev)
        self.ids = torch.from_numpy(ids).to(dev)
        self.distinct = int(len(set(ids.tolist())))
        self.ys = {m: torch.empty(m, 4096, dtype=torch.bfloat16, device=dev) for m in wl.tokens}
        self.y_multi = torch.empty(self.multi_m, 4096, dtype=torch.bfloat16, device=dev)
        self.y_prefill = torch.empty(self.prefill_m, 4096, dtype=torch.bfloat16, device=dev)
        self.c_out = [(torch.empty_like(packed), torch.empty_like(alpha)) for _ in range(2)]
        # unfused A/B: W_eff written by bitdelta_reconstruct, and stored copies
        # of it (one per rotation copy) for a plain library GEMM
        self.w_eff = torch.empty(4096, 4096, dtype=torch.bfloat16, device=dev)
        self.w_effs = []
        for r in range(self.R):
            p, a = self.vsets[r][0]
            self.w_effs.append(T.reconstruct(self.bases[r], p, a, self.mode))
        self.ys_dense = {m: torch.empty(m, 4096, dtype=torch.bfloat16, device=dev)
                         for m in list(wl.tokens) + [self.prefill_m]}
        self.x_dense = dict(self.xs)
        self.x_dense[self.prefill_m] = self.x_prefill
        self.host = dict(wb=wb, wf=wf, xs=xs, more=more, x_multi=x_multi, ids=ids)
        self.k = 0

    @staticmethod
    def static_bytes():
        """Algorithmic bytes per launch of each kernel of the step, from the
        workload's shapes and seeded variant ids alone (no GPU needed)."""
        wl = S.WORKLOADS["proj_4096"]
        ids = S.zipf_ids(ProjWorkload.multi_m, ProjWorkload.n_variants, wl.seed)
        shell = ProjWorkload.__new__(ProjWorkload)
        shell.d_out = shell.d_in = 4096
        shell.mode = wl.alpha_mode
        shell.distinct = int(len(set(ids.tolist())))
        n = 4096 * 4096
        pm = ProjWorkload.prefill_m
        out = {"compress": shell.compress_bytes(), "multi": shell.multi_bytes(),
               "prefill": 2 * n + n // 8 + 4 * 4096 + 2 * pm * 4096 * 2,
               "reconstruct": shell.reconstruct_bytes()}
        for m in wl.tokens:
            out[f"decode_m{m}"] = shell.decode_bytes(m)
        return out

    # algorithmic bytes / flops per launch
    def decode_bytes(self, m):
        n = self.d_out * self.d_in
        alpha = 4 * (self.d_out if self.mode == 1 else 1)
        return 2 * n + n // 8 + alpha + 2 * m * self.d_in + 2 * m * self.d_out

    def multi_bytes(self):
        n = self.d_out * self.d_in
        alpha = 4 * (self.d_out if self.mode == 1 else 1)
        return (2 * n + self.distinct * (n // 8 + alpha) + 2 * self.multi_m * self.d_in
                + 2 * self.multi_m * self.d_out + 4 * self.multi_m)

    def compress_bytes(self):
        n = self.d_out * self.d_in
        alpha = 4 * (self.d_out if self.mode == 1 else 1)
        return 4 * n + n // 8 + alpha

    def reconstruct_bytes(self):
        n = self.d_out * self.d_in
        alpha = 4 * (self.d_out if self.mode == 1 else 1)
        return 2 * n + n // 8 + alpha + 2 * n

    def prefill_flops(self):
        return 2 * self.prefill_m * self.d_out * self.d_in

    # one launch of each kernel range on rotation copy r
    def run_compress(self, r):
        cp, ca = self.c_out[r % 2]
        T.compress(self.fts[r % len(self.fts)], self.bases[r % self.R], self.mode,
                   packed=cp, alpha=ca)

    def run_decode(self, m, r):
        p, a = self.vsets[r % self.R][0]
        T.linear(self.xs[m], self.bases[r % self.R], p, a, self.mode, y=self.ys[m])

    def run_multi(self, r):
        vs = self.vsets[r % self.R]
        T.linear_multi(self.x_multi, self.ids, self.bases[r % self.R], [p for p, _ in vs],
                       [a for _, a in vs], self.mode, y=self.y_multi)

    def run_prefill(self, r):
        p, a = self.vsets[r % self.R][0]
        T.linear(self.x_prefill, self.bases[r % self.R], p, a, self.mode, y=self.y_prefill)

    def run_reconstruct(self, r):
        p, a = self.vsets[r % self.R][0]
        T.reconstruct(self.bases[r % self.R], p, a, self.mode, w_eff=self.w_eff)

    def run_dense(self, m, r):
        """The library GEMM (torch.mm, hipBLASLt) on a stored W_eff copy."""
        torch.mm(self.x_dense[m], self.w_effs[r % self.R].t(), out=self.ys_dense[m])

    def one_pass(self, j):
        """One pass of the whole path (a step), on copies 6j .. 6j+5."""
        r = 6 * j
        self.run_compress(r)
        for i, m in enumerate(self.decode_ms):
            self.run_decode(m, r + 1 + i)
        self.run_multi(r + 4)
        self.run_prefill(r + 5)

    def ranges(self):
        """name -> (launches per graph, function making them back to back).
        Each graph cycles RANGE_CYCLES times through the rotation copies so
        that the cost of starting a replay is spread over many launches."""
        c = RANGE_CYCLES
        nf = len(self.fts)
        out = {"compress": (c * nf, lambda: [self.run_compress(r) for r in range(c * nf)])}
        for m in self.decode_ms:
            out[f"decode_m{m}"] = (c * self.R, lambda m=m: [self.run_decode(m, r)
                                                            for r in range(c * self.R)])
        out["multi"] = (c * self.R, lambda: [self.run_multi(r) for r in range(c * self.R)])
        out["prefill"] = (c * 8, lambda: [self.run_prefill(r % 8) for r in range(c * 8)])
        out["reconstruct"] = (c * self.R, lambda: [self.run_reconstruct(r)
                                                   for r in range(c * self.R)])
        for m in self.decode_ms:
            out[f"dense_m{m}"] = (c * self.R, lambda m=m: [self.run_dense(m, r)
                                                           for r in range(c * self.R)])
        out[f"dense_m{self.prefill_m}"] = (c * 8, lambda: [self.run_dense(self.prefill_m, r % 8)
                                                           for r in range(c * 8)])
        return out


class LayerWorkload:
    """One 70B-shaped decoder layer (QKV, O, gate, up, down).  mode "prefill":
    one variant, per-matrix alpha, M = 2048 through the prefill GEMM, reported
    in TFLOP/s.  mode "multi": 14 variants, per-row alpha, M = 32 tokens with
    Zipf(1.1) ids through the mixed-variant kernel, reported in GB/s.  The
    layer's weights (1.7 GB) exceed the last-level cache; each matrix's timing
    graph cycles over copies of that matrix's operands (W_base, packed signs,
    alpha, x) whose total is at least twice the cache, so consecutive launches
    of one matrix do not find its operands there."""

    def __init__(self, name, dev):
        wl = S.WORKLOADS[name]
        self.name, self.wl, self.dev = name, wl, dev
        self.mode = wl.alpha_mode
        self.kind = "prefill" if name == "layer70b_prefill" else "multi"
        self.m = wl.tokens[0]
        g = S.generator(wl.seed, dev)
        self.bases = S.draw_layer_bases(wl, g, dev)
        scales = S.variant_scales(wl)
        self.packs = [[None] * len(self.bases) for _ in scales]
        self.alphas = [[None] * len(self.bases) for _ in scales]
        for v, i, wf in S.iter_finetuned(self.bases, scales, g):
            self.packs[v][i], self.alphas[v][i] = T.compress(wf, self.bases[i], self.mode)
            del wf
        self.xs = S.draw_layer_inputs(wl, self.m, g, dev)
        ids = S.zipf_ids(self.m, wl.n_variants, wl.seed)
        self.ids = torch.from_numpy(ids).to(dev)
        self.distinct = int(len(set(ids.tolist())))
        self.ys = [torch.empty(self.m, d_out, dtype=torch.bfloat16, device=dev)
                   for _, d_out, _ in wl.matrices]
        self.ys_dense = [torch.empty_like(y) for y in self.ys]
        self.R = 1
        # operand copies per matrix: (x, W_base, packed list, alpha list)
        self.rot = []
        for i in range(len(self.bases)):
            ops = (self.xs[i], self.bases[i], [p[i] for p in self.packs],
                   [a[i] for a in self.alphas])
            nbytes = sum(t.numel() * t.element_size() for t in ops[:2]) + sum(
                t.numel() * t.element_size() for t in ops[2] + ops[3])
            copies = max(2, math.ceil(2 * MALL_BYTES / nbytes))
            self.rot.append([ops] + [(ops[0].clone(), ops[1].clone(), [t.clone() for t in ops[2]],
                                      [t.clone() for t in ops[3]]) for _ in range(copies - 1)])

    def run(self, i, c=0):
        x, wb, packs, alphas = self.rot[i][c % len(self.rot[i])]
        if self.kind == "prefill":
            T.linear(x, wb, packs[0], alphas[0], self.mode, y=self.ys[i])
        else:
            T.linear_multi(x, self.ids, wb, packs, alphas, self.mode, y=self.ys[i])

    def run_dense(self, i, c=0):
        """The library GEMM (torch.mm, hipBLASLt) on W_base alone: the base
        model's dense bf16 layer of the same shape and tokens."""
        x, wb, _, _ = self.rot[i][c % len(self.rot[i])]
        torch.mm(x, wb.t(), out=self.ys_dense[i])

    def setup_per_variant(self):
        """The per-variant fused alternative for the mixed batch: the tokens
        of each variant present gathered, one single-variant fused call
        (bitdelta_linear: W_base + alpha_v sign(Delta_v) formed in the
        kernel, W_base read again for every variant), the outputs scattered
        back."""
        ids = self.ids.cpu().numpy()
        self.groups = [(v, torch.from_numpy(np.nonzero(ids == v)[0]).to(self.dev))
                       for v in sorted(set(ids.tolist())) if v >= 0]
        if any(v < 0 for v in ids.tolist()):
            raise SystemExit("the per-variant comparison takes variant tokens only")
        self.ys_pv = [torch.empty_like(y) for y in self.ys]
        self.pv_bufs = {}
        for i, (_, d_out, d_in) in enumerate(self.wl.matrices):
            for v, idx in self.groups:
                self.pv_bufs[(i, v)] = (
                    torch.empty(len(idx), d_in, dtype=torch.bfloat16, device=self.dev),
                    torch.empty(len(idx), d_out, dtype=torch.bfloat16, device=self.dev))

    def run_per_variant(self, i, c=0):
        x, wb, packs, alphas = self.rot[i][c % len(self.rot[i])]
        for v, idx in self.groups:
            xv, yv = self.pv_bufs[(i, v)]
            torch.index_select(x, 0, idx, out=xv)
            T.linear(xv, wb, packs[v], alphas[v], self.mode, y=yv)
            self.ys_pv[i].index_copy_(0, idx, yv)

    def one_pass(self, j):
        for i in range(len(self.bases)):
            self.run(i)

    def ranges(self):
        out = {}
        for i, (nm, _, _) in enumerate(self.wl.matrices):
            n = len(self.rot[i]) * RANGE_CYCLES
            out[f"{self.kind}_{nm}"] = (n, lambda i=i, n=n: [self.run(i, c) for c in range(n)])
            out[f"dense_{nm}"] = (n, lambda i=i, n=n: [self.run_dense(i, c) for c in range(n)])
            if getattr(self, "groups", None) is not None:
                out[f"pervar_{nm}"] = (n, lambda i=i, n=n: [self.run_per_variant(i, c)
                                                            for c in range(n)])
        return out

    def work(self, i):
        _, d_out, d_in = self.wl.matrices[i]
        n = d_out * d_in
        if self.kind == "prefill":
            return 2.0 * self.m * n
        alpha = 4 * (d_out if self.mode == 1 else 1)
        return (2 * n + self.distinct * (n // 8 + alpha) + 2 * self.m * d_in
                + 2 * self.m * d_out + 4 * self.m)

    def report(self, avg_us, args, step_ms=None):
        names = [nm for nm, _, _ in self.wl.matrices]
        total_us = sum(avg_us[f"{self.kind}_{nm}"] for nm in names)
        total_work = sum(self.work(i) for i in range(len(names)))
        per = {nm: round(self.work(i) / (avg_us[f"{self.kind}_{nm}"] * 1e-6)
                         / (1e12 if self.kind == "prefill" else 1e9), 2)
               for i, nm in enumerate(names)}
        if self.kind == "prefill":
            val = total_work / (total_us * 1e-6) / 1e12
            roof = roofline_entry("mfma", val, BF16_PEAK_TFLOPS, "TFLOP/s",
                                  counter_traffic("prefill", self.name))
            unit = "TFLOP/s"
        else:
            val = total_work / (total_us * 1e-6) / 1e9
            roof = roofline_entry("hbm", val, HBM_PEAK_GBS, "GB/s",
                                  counter_traffic("multi", self.name))
            unit = "GB/s"
        cfg = {"workload": f"{self.name}: {self.wl.note}", "tokens": self.m,
               "alpha_mode": "per_row" if self.mode == 1 else "per_matrix",
               "matrices": [list(mm) for mm in self.wl.matrices]}
        if self.kind == "multi":
            cfg["distinct_variants"] = self.distinct
        out = {"value": round(val, 2), "unit": unit, "config": cfg, "per_matrix": per,
               "roofline": roof, "layer_us": round(total_us, 2)}
        if all(f"dense_{nm}" in avg_us for nm in names):
            # the fused BitDelta layer against the base model's own dense layer
            dense = {nm: avg_us[f"dense_{nm}"] for nm in names}
            d_tot = sum(dense.values())
            out["dense_base_ab"] = {
                "per_matrix_us": {nm: {"fused": round(avg_us[f"{self.kind}_{nm}"], 2),
                                       "dense_base": round(dense[nm], 2)} for nm in names},
                "layer_fused_us": round(total_us, 2), "layer_dense_base_us": round(d_tot, 2),
                "fused_over_dense_base": round(total_us / d_tot, 4)}
        if all(f"pervar_{nm}" in avg_us for nm in names):
            # the per-variant fused alternative on the same batch
            pv = {nm: avg_us[f"pervar_{nm}"] for nm in names}
            for i in range(len(names)):
                self.run(i)
                self.run_per_variant(i)
            torch.cuda.synchronize()
            rel = max(float(((self.ys_pv[i].float() - self.ys[i].float()).abs().max()
                             / self.ys[i].float().abs().max()).item())
                      for i in range(len(names)))
            out["per_variant_ab"] = {
                "per_matrix_us": {nm: {"grouped": round(avg_us[f"{self.kind}_{nm}"], 2),
                                       "per_variant": round(pv[nm], 2)} for nm in names},
                "layer_grouped_us": round(total_us, 2),
                "layer_per_variant_us": round(sum(pv.values()), 2),
                "per_variant_over_grouped": round(sum(pv.values()) / total_us, 4),
                "variant_calls_per_matrix": len(self.groups),
                "max_abs_diff_over_max_abs": rel}
        if step_ms:
            # the same work over the measured one-pass steps (launch gaps and
            # the matrices' order included)
            scale = 1e12 if self.kind == "prefill" else 1e9
            out["value_per_step"] = round(self.wl.layers * total_work / (step_ms * 1e-3) / scale,
                                          2)
        return out


class DecodeLayerWorkload(LayerWorkload):
    """One 70B-shaped layer, one variant, per-row alpha, through the decode
    kernel at M = 1, 4 and 16 tokens: the single-variant decode at the
    layer's shapes (the default workload measures it on 4096x4096).  Each
    (matrix, M) range cycles over operand copies of at least twice the
    last-level cache, as for the other layer workloads."""

    def __init__(self, name, dev):
        wl = S.WORKLOADS[name]
        self.name, self.wl, self.dev = name, wl, dev
        self.mode = wl.alpha_mode
        self.kind = "decode"
        self.ms = tuple(wl.tokens)
        self.m = max(self.ms)
        g = S.generator(wl.seed, dev)
        self.bases = S.draw_layer_bases(wl, g, dev)
        self.packs, self.alphas = [], []
        for _, i, wf in S.iter_finetuned(self.bases, S.variant_scales(wl), g):
            p, a = T.compress(wf, self.bases[i], self.mode)
            self.packs.append(p)
            self.alphas.append(a)
            del wf
        self.xs = S.draw_layer_inputs(wl, self.m, g, dev)
        self.distinct = 1
        self.ys = [torch.empty(self.m, d_out, dtype=torch.bfloat16, device=dev)
                   for _, d_out, _ in wl.matrices]
        self.R = 1
        self.rot = []
        for i in range(len(self.bases)):
            ops = (self.xs[i], self.bases[i], self.packs[i], self.alphas[i])
            nbytes = sum(t.numel() * t.element_size() for t in ops)
            copies = max(2, math.ceil(2 * MALL_BYTES / nbytes))
            self.rot.append([ops] + [tuple(t.clone() for t in ops) for _ in range(copies - 1)])

    def run_m(self, i, m, c=0):
        x, wb, p, a = self.rot[i][c % len(self.rot[i])]
        T.linear(x[:m], wb, p, a, self.mode, y=self.ys[i][:m])

    def one_pass(self, j):
        for m in self.ms:
            for i in range(len(self.bases)):
                self.run_m(i, m)

    def ranges(self):
        out = {}
        for i, (nm, _, _) in enumerate(self.wl.matrices):
            n = len(self.rot[i]) * RANGE_CYCLES
            for m in self.ms:
                out[f"decode_m{m}_{nm}"] = (n, lambda i=i, m=m, n=n: [self.run_m(i, m, c)
                                                                      for c in range(n)])
        return out

    def bytes_of(self, i, m):
        _, d_out, d_in = self.wl.matrices[i]
        n = d_out * d_in
        return 2 * n + n // 8 + 4 * d_out + 2 * m * d_in + 2 * m * d_out

    def report(self, avg_us, args, step_ms=None):
        names = [nm for nm, _, _ in self.wl.matrices]
        total_b = sum(self.bytes_of(i, m) for i in range(len(names)) for m in self.ms)
        total_us = sum(avg_us[f"decode_m{m}_{nm}"] for nm in names for m in self.ms)
        val = total_b / (total_us * 1e-6) / 1e9
        per = {f"{nm}_m{m}": round(self.bytes_of(i, m) / (avg_us[f"decode_m{m}_{nm}"] * 1e-6)
                                   / 1e9, 2)
               for i, nm in enumerate(names) for m in self.ms}
        layer_us = {f"m{m}": round(sum(avg_us[f"decode_m{m}_{nm}"] for nm in names), 2)
                    for m in self.ms}
        cfg = {"workload": f"{self.name}: {self.wl.note}", "tokens": list(self.ms),
               "alpha_mode": "per_row", "matrices": [list(mm) for mm in self.wl.matrices]}
        out = {"value": round(val, 2), "unit": "GB/s", "config": cfg, "per_matrix": per,
               "roofline": roofline_entry("hbm", val, HBM_PEAK_GBS, "GB/s", None),
               "layer_us": layer_us}
        if step_ms:
            out["value_per_step"] = round(total_b / (step_ms * 1e-3) / 1e9, 2)
        return out


class StackWorkload(LayerWorkload):
    """The 80-layer 70B-shaped stack resident on the GPU (137 GB of W_base and
    14 packed variants, about 257 GB), mixed-variant decode of 64 tokens with a
    Zipf(1.1) variant mix through every layer's five linears."""

    def __init__(self, name, dev):
        wl = S.WORKLOADS[name]
        self.name, self.wl, self.dev = name, wl, dev
        self.mode = wl.alpha_mode
        self.kind = "multi"
        self.m = wl.tokens[0]
        g = S.generator(wl.seed, dev)
        self.stack = S.draw_stack_bases(wl, g, dev)
        scales = S.variant_scales(wl)
        nm = len(wl.matrices)
        self.packs = [[[None] * nm for _ in scales] for _ in range(wl.layers)]
        self.alphas = [[[None] * nm for _ in scales] for _ in range(wl.layers)]
        for l, v, i, wf in S.iter_stack_finetuned(self.stack, scales, g):
            self.packs[l][v][i], self.alphas[l][v][i] = T.compress(wf, self.stack[l][i], self.mode)
            del wf
            if v == len(scales) - 1 and i == nm - 1 and l % 10 == 9:
                print(f"[bench] layers 0..{l} drawn and compressed", file=sys.stderr, flush=True)
        self.xs = S.draw_stack_inputs(wl, self.m, g, dev)
        ids = S.zipf_ids(self.m, wl.n_variants, wl.seed)
        self.ids = torch.from_numpy(ids).to(dev)
        self.distinct = int(len(set(ids.tolist())))
        self.ys = [torch.empty(self.m, d_out, dtype=torch.bfloat16, device=dev)
                   for _, d_out, _ in wl.matrices]
        self.R = 1

    def run_li(self, l, i):
        nv = len(self.packs[l])
        T.linear_multi(self.xs[l][i], self.ids, self.stack[l][i],
                       [self.packs[l][v][i] for v in range(nv)],
                       [self.alphas[l][v][i] for v in range(nv)], self.mode, y=self.ys[i])

    def one_pass(self, j):
        for l in range(self.wl.layers):
            for i in range(len(self.wl.matrices)):
                self.run_li(l, i)

    def ranges(self):
        L = self.wl.layers
        return {f"multi_{nm}": (L, lambda i=i: [self.run_li(l, i) for l in range(L)])
                for i, (nm, _, _) in enumerate(self.wl.matrices)}

    def report(self, avg_us, args, step_ms=None):
        rep = super().report(avg_us, args, step_ms)
        L = self.wl.layers
        rep["layer_us"] = round(rep["layer_us"], 2)
        rep["stack_ms"] = round(rep["layer_us"] * L / 1e3, 3)
        rep["config"]["layers"] = L
        rep["config"]["resident_bytes"] = sum(
            t.numel() * t.element_size() for layer in self.stack for t in layer) + sum(
            p.numel() * p.element_size() for layer in self.packs for vs in layer for p in vs)
        return rep


def serve_layer70b(args, dev):
    """The serving loop around the path on one 70B-shaped layer: the 14
    variants' deltas of the layer (QKV, O, gate, up, down; per-row alpha;
    Laplace b_v log-uniform in [2e-4, 2e-3], as layer70b_multi) live in
    page-locked host blobs; a delta cache of 8 device slots with the top 6
    variants pinned (the page's split of 14) loads them on demand; a router
    forms decode batches of up to 64 ready requests from a Zipf(1.1) request
    stream arriving 64 per batch slot; every batch runs the layer's five
    mixed-variant linears on the cached slots.  Two passes over 4096
    requests each: cold (empty cache) and warm (the cache as the first left
    it).  value is the linears' algorithmic HBM bytes over the pass's wall
    time; tokens_per_s is requests served per second through the layer."""
    wl = S.WORKLOADS["layer70b_multi"]
    mode = wl.alpha_mode
    g = S.generator(wl.seed, dev)
    bases = S.draw_layer_bases(wl, g, dev)
    shapes = [(d_out, d_in) for _, d_out, d_in in wl.matrices]
    _, total = T.delta_layout(shapes, mode)
    V = wl.n_variants
    packs = [[None] * len(shapes) for _ in range(V)]
    alphas = [[None] * len(shapes) for _ in range(V)]
    for v, i, wf in S.iter_finetuned(bases, S.variant_scales(wl), g):
        packs[v][i], alphas[v][i] = T.compress(wf, bases[i], mode)
        del wf
    blobs = [torch.empty(total, dtype=torch.uint8, pin_memory=True) for _ in range(V)]
    for v in range(V):
        for (hp, ha), p, a in zip(T.delta_views(blobs[v], shapes, mode), packs[v], alphas[v]):
            hp.copy_(p.cpu())
            ha.copy_(a.cpu())
    n_slots, n_pinned, max_m, n_req = 8, 6, 64, 4096
    cache = T.DeltaCache(V, n_slots, n_pinned, 0)
    slots = [torch.empty(total, dtype=torch.uint8, device=dev) for _ in range(n_slots)]
    cache.attach(slots, blobs)
    router = T.Router(cache)
    copy = torch.cuda.Stream()
    xs = S.draw_layer_inputs(wl, max_m, g, dev)
    ys = [torch.empty(max_m, d_out, dtype=torch.bfloat16, device=dev) for d_out, _ in shapes]
    slot_views = [T.delta_views(t, shapes, mode) for t in slots]
    torch.cuda.synchronize()
    print(f"[bench] serve_layer70b: {V} variants, {n_slots} slots ({n_pinned} pinned), "
          f"delta {total:,} B per variant", file=sys.stderr, flush=True)

    def one_pass(seed, rid0, checks):
        ids_all = S.zipf_ids(n_req, V, seed)
        submitted = served = batches = 0
        nbytes = 0
        distinct = []
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while served < n_req:
            for _ in range(max_m):
                if submitted < n_req:
                    router.submit(rid0 + submitted, int(ids_all[submitted]))
                    submitted += 1
            batch = router.next_batch(max_m, copy)
            if not batch:
                copy.synchronize()   # every queued request waits for a load
                continue
            m = len(batch)
            local = sorted({b[1] for b in batch})
            slot_of = {b[1]: b[2] for b in batch}
            ids = torch.tensor([local.index(b[1]) for b in batch], dtype=torch.int32,
                               device=dev)
            for i, (d_out, d_in) in enumerate(shapes):
                pl = [slot_views[slot_of[v]][i][0] for v in local]
                al = [slot_views[slot_of[v]][i][1] for v in local]
                T.linear_multi(xs[i][:m], ids, bases[i], pl, al, mode, y=ys[i][:m])
                n = d_out * d_in
                nbytes += (2 * n + len(local) * (n // 8 + 4 * d_out) + 2 * m * d_in
                           + 2 * m * d_out + 4 * m)
            if batches in checks:
                # the cached slots against the variants' own tensors, bit for bit
                i = 2
                y_ref = T.linear_multi(xs[i][:m], ids, bases[i], [packs[v][i] for v in local],
                                       [alphas[v][i] for v in local], mode)
                torch.cuda.synchronize()
                if not torch.equal(ys[i][:m].view(torch.int16), y_ref.view(torch.int16)):
                    raise RuntimeError("served batch differs from the direct call")
            router.complete(batch)
            served += m
            batches += 1
            distinct.append(len(local))
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return {"requests": n_req, "batches": batches, "mean_batch": round(n_req / batches, 2),
                "mean_distinct_variants": round(sum(distinct) / len(distinct), 2),
                "wall_ms": round(wall * 1e3, 3), "tokens_per_s": round(n_req / wall, 1),
                "linears_gbs": round(nbytes / wall / 1e9, 2)}

    cold = one_pass(101, 0, {0, 5})
    warm = one_pass(102, n_req, {0, 7, 30})
    print(f"[bench] cold {cold['wall_ms']} ms, warm {warm['wall_ms']} ms", file=sys.stderr,
          flush=True)
    out = {"metric": METRIC, "value": warm["linears_gbs"], "unit": "GB/s", "n_gpus": 1,
           "steps": 1, "warmup": 1, "ms_per_step": warm["wall_ms"], "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "serve_layer70b: one 70B-shaped layer, 14 variants' deltas "
                                  "in pinned host memory, delta cache of 8 slots (top 6 "
                                  "pinned), router batches of up to 64 Zipf(1.1) requests "
                                  "through the layer's five mixed-variant linears",
                      "variants": V, "slots": n_slots, "pinned": n_pinned, "max_batch": max_m,
                      "delta_bytes_per_variant": total},
           "cold": cold, "warm": warm,
           "roofline": roofline_entry("hbm", warm["linears_gbs"], HBM_PEAK_GBS, "GB/s", None),
           "cpu_baseline": None}
    print(json.dumps(out), flush=True)


def monosoup_4096(args, dev):
    """MonoSoup merge of 4 fine-tuned checkpoints of a 4096x4096 matrix at
    rank 16 with 4 power iterations (task vectors with a planted rank-16
    part plus Laplace noise).  The merge is captured in a HIP graph and timed
    with HIP events.  Algorithmic bytes per merge: each checkpoint's task
    vector is streamed from its two bf16 matrices (4 bytes per element) once
    per product, 2 * (power_iters + 1) products, and the merge reads the base
    and writes the merged weights (4 bytes per element)."""
    d, k, rank, q = 4096, 4, 16, 4
    g = S.generator(31, dev)
    wb = S.draw_base(d, d, 0.02, g, dev)
    wf = [S.draw_lowrank_checkpoint(wb, rank, 2e-3, 2e-4, g) for _ in range(k)]
    omega = S.draw_gaussian(d, rank, g, dev)
    out = torch.empty_like(wb)
    ws = torch.empty(T.monosoup_workspace_size(d, d, k, rank), dtype=torch.uint8, device=dev)
    T.monosoup_merge(wf, wb, rank, q, omega, out=out, workspace=ws)
    ref = out.clone()
    graph = capture(lambda: T.monosoup_merge(wf, wb, rank, q, omega, out=out, workspace=ws))
    for _ in range(args.warmup):
        graph.replay()
    ms = median(time_replays(graph, max(REPS, args.steps)))
    if not torch.equal(out.view(torch.int16), ref.view(torch.int16)):
        raise RuntimeError("graph replays of the merge differ from the eager call")
    nbytes = k * 2 * (q + 1) * 4 * d * d + 4 * d * d
    gbs = nbytes / (ms * 1e-3) / 1e9
    cpu = None
    if args.cpu_budget > 0:
        import oracle.monosoup as M
        t0 = time.perf_counter()
        M.merge([S.bf16_bits(w) for w in wf[:1]], S.bf16_bits(wb), rank)
        t1 = time.perf_counter() - t0
        cpu = {"value": round(nbytes / k / t1 / 1e9, 3), "unit": "GB/s", "cores":
               len(os.sched_getaffinity(0)), "kind": "oracle",
               "sample": f"oracle merge of one of the {k} checkpoints (exact float64 SVD of the "
                         f"4096x4096 task vector), {t1:.1f} s; value is that merge's share of "
                         f"the bytes over its time"}
    out_line = {"metric": "monosoup merge effective HBM GB/s, 1 GPU", "value": round(gbs, 2),
                "unit": "GB/s", "n_gpus": 1, "steps": max(3, args.steps), "warmup": args.warmup,
                "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
                "vs_baseline": None, "dtype": "f32", "data": "synthetic",
                "config": {"workload": "monosoup_4096: 4 checkpoints of a 4096x4096 matrix, "
                                       "rank 16, 4 power iterations, planted rank-16 task "
                                       "vectors plus Laplace(0, 2e-4) noise",
                           "d_out": d, "d_in": d, "checkpoints": k, "rank": rank,
                           "power_iters": q, "bytes_per_merge": nbytes},
                "roofline": roofline_entry("hbm", gbs, HBM_PEAK_GBS, "GB/s", None),
                "cpu_baseline": cpu}
    print(json.dumps(out_line), flush=True)


# ------------------------------------------------------------------ CPU oracle
def cpu_baseline(w: ProjWorkload, budget_s: float):
    """The oracle, as it stands, on a bounded sample of the same workload:
    compression of the projection and the three decode products (all 4096 rows),
    repeated while the time budget lasts.  Reported in the metric's unit."""
    import oracle as O
    wb = S.bf16_bits(w.host["wb"])
    wf = S.bf16_bits(w.host["wf"])
    xs = {m: S.bf16_bits(x) for m, x in w.host["xs"].items()}
    t0 = time.perf_counter()
    packed, alpha = O.compress(wf, wb, w.mode)
    t_comp = time.perf_counter() - t0
    passes, t_dec, nbytes = 0, 0.0, 0
    while True:
        t0 = time.perf_counter()
        for m in w.decode_ms:
            O.linear(xs[m], wb, packed, alpha, w.mode)
            nbytes += w.decode_bytes(m)
        t_dec += time.perf_counter() - t0
        passes += 1
        if t_dec + t_comp > budget_s or passes >= 200:
            break
    return _cpu_record(
        round(nbytes / t_dec / 1e9, 4), "GB/s",
        f"oracle decode products M={list(w.decode_ms)} on the full 4096x4096 projection, "
        f"{passes} pass(es), {t_dec:.1f} s; oracle compression of the same matrix "
        f"{t_comp:.1f} s ({w.compress_bytes() / t_comp / 1e9:.3f} GB/s)")


# ------------------------------------------------------------------ counters
COUNTER_WORKLOADS = ("proj_4096", "layer70b_multi", "layer70b_prefill")
CALIB_BYTES = 256 * 2**20
# kernel-name substring that every launch of a counter block must carry
KERNEL_OF = {"compress": "compress_rows_kernel", "decode": "linear_decode_",
             "multi": "linear_multi_", "prefill": "prefill_", "reconstruct": "reconstruct_kernel"}


def layer_work_static(name: str):
    """Per matrix of a layer workload: (label, algorithmic bytes per launch),
    from the shapes and seeded variant ids alone (no GPU needed).  A mixed
    decode launch reads W_base once and each distinct variant's signs and
    alpha once; a prefill launch reads x, W_base, the signs and alpha and
    writes y."""
    wl = S.WORKLOADS[name]
    m = wl.tokens[0]
    out = []
    for nm, d_out, d_in in wl.matrices:
        n = d_out * d_in
        alpha = 4 * (d_out if wl.alpha_mode == 1 else 1)
        if name == "layer70b_prefill":
            out.append((f"prefill_{nm}", 2 * n + n // 8 + alpha + 2 * m * d_in + 2 * m * d_out))
        else:
            ids = S.zipf_ids(m, wl.n_variants, wl.seed)
            distinct = len(set(ids.tolist()))
            out.append((f"multi_{nm}", 2 * n + distinct * (n // 8 + alpha) + 2 * m * d_in
                        + 2 * m * d_out + 4 * m))
    return out


def counter_plan(workload: str):
    """Blocks of a counter pass: [(block, kernel family, algorithmic bytes per
    launch)], and how blocks group into one roofline unit per kernel family:
    {family: (blocks, unit)}."""
    if workload == "proj_4096":
        sb = ProjWorkload.static_bytes()
        blocks = [(b, b.split("_")[0], sb[b]) for b in
                  ("compress", "decode_m1", "decode_m4", "decode_m16", "multi", "prefill",
                   "reconstruct")]
        groups = {"decode": (["decode_m1", "decode_m4", "decode_m16"],
                             "one launch of each decode token count (M = 1, 4, 16), as the "
                             "decode roofline's unit")}
        for f in ("compress", "multi", "prefill", "reconstruct"):
            groups[f] = ([f], "one launch")
        return blocks, groups
    fam = "prefill" if workload == "layer70b_prefill" else "multi"
    blocks = [(b, fam, v) for b, v in layer_work_static(workload)]
    return blocks, {fam: ([b for b, _, _ in blocks],
                          "one pass of the layer's five linears (one launch each), as the "
                          "layer roofline's unit")}


def clock_pass(dev, n: int = 6):
    """For a GRBM_GUI_ACTIVE counter run: n fused prefills (M = 2048) of a
    gate-shaped 28672x8192 matrix with finite weights and per-matrix alpha,
    then n library GEMMs (torch.mm) of the same shape on W_base."""
    g = S.generator(45, dev)
    M, d_out, d_in = 2048, 28672, 8192
    wb = S.draw_base(d_out, d_in, 0.015, g, dev)
    wf = S.draw_finetuned(wb, 1e-3, g)
    p, a = T.compress(wf, wb, 0)
    del wf
    x = S.draw_activations(M, d_in, g, dev)
    y = torch.empty(M, d_out, dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    for _ in range(n):
        T.linear(x, wb, p, a, 0, y=y)
    torch.cuda.synchronize()
    for _ in range(n):
        torch.mm(x, wb.t(), out=y)
    torch.cuda.synchronize()


SEPARATOR_KERNEL = "FillFunctor<unsigned char>"
CALIB_KERNEL = "neg_kernel"


def counter_pass(workload: str, dev, n: int):
    """n eager calls of each block of the workload, block by block, each call
    on its own rotation copy of the operands; then n launches of the
    calibration kernel (a plain elementwise kernel reading and writing
    CALIB_BYTES each).  A one-byte fill separates the blocks (a call may make
    more than one launch), and one comes before the first."""
    if workload == "proj_4096":
        w = ProjWorkload(dev)
        run = {"compress": w.run_compress, "multi": w.run_multi, "prefill": w.run_prefill,
               "reconstruct": w.run_reconstruct}
        for m in w.decode_ms:
            run[f"decode_m{m}"] = lambda r, m=m: w.run_decode(m, r)
    else:
        w = LayerWorkload(workload, dev)
        run = {f"{w.kind}_{nm}": (lambda r, i=i: w.run(i, r))
               for i, (nm, _, _) in enumerate(w.wl.matrices)}
    blocks, _ = counter_plan(workload)
    sep = torch.empty(1, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    sep.fill_(0)
    for b, (name, _, _) in enumerate(blocks):
        for r in range(n):
            run[name](r)
        sep.fill_(b + 1)
        torch.cuda.synchronize()
    src = torch.zeros(CALIB_BYTES // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(n):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()


def _counter_rows(d: str):
    """(dispatch id, kernel name, counter, value) of every row of a --pmc run."""
    import csv
    rows = []
    for dirpath, _, files in os.walk(d):
        for f in files:
            if f.endswith("counter_collection.csv"):
                for r in csv.DictReader(open(os.path.join(dirpath, f))):
                    rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], r["Counter_Name"],
                                 float(r["Counter_Value"])))
    rows.sort()
    return rows


def _split_blocks(d: str, workload: str, n: int):
    """Per-dispatch counter values of a counter-pass run, cut into its blocks
    at the separators and summed per call: ({block: [{counter: value} per
    call]}, [calibration launches], calibration kernel name).  Raises when a
    block holds a kernel of another family or a launch count that n calls
    cannot make."""
    blocks, _ = counter_plan(workload)
    per = {}
    names = {}
    for did, kname, c, v in _counter_rows(d):
        per.setdefault(did, {})
        per[did][c] = per[did].get(c, 0.0) + v
        names[did] = kname
    ids = sorted(per)
    seps = [i for i in ids if SEPARATOR_KERNEL in names[i]][-(len(blocks) + 1):]
    if len(seps) != len(blocks) + 1:
        raise SystemExit(f"{d}: expected {len(blocks) + 1} separators, found {len(seps)}")
    calib = [i for i in ids if i > seps[-1]][-n:]
    if len(calib) != n or any(CALIB_KERNEL not in names[i] for i in calib):
        raise SystemExit(f"{d}: expected {n} calibration dispatches ({CALIB_KERNEL}) after "
                         f"the last separator")
    out = {}
    for b, (name, fam, _) in enumerate(blocks):
        chunk = [i for i in ids if seps[b] < i < seps[b + 1]]
        wrong = [names[i] for i in chunk if KERNEL_OF[fam] not in names[i]]
        if wrong:
            raise SystemExit(f"{d}: block {name} holds other kernels: {wrong[0][:80]}")
        if not chunk or len(chunk) % n:
            raise SystemExit(f"{d}: block {name} holds {len(chunk)} launches for {n} calls")
        k = len(chunk) // n
        counters = per[chunk[0]].keys()
        out[name] = [{c: sum(per[i][c] for i in chunk[j * k:(j + 1) * k]) for c in counters}
                     for j in range(n)]
        out[name + "#kernel"] = sorted({_short_kernel(names[i]) for i in chunk})
    return out, [per[i] for i in calib], names[calib[0]]


def _short_kernel(name: str) -> str:
    name = name.replace("void ", "").replace("bd::(anonymous namespace)::", "")
    return name.split("(")[0]


def summarize_counters(fetch_dir: str, write_dir: str, workload: str, n: int):
    """Per-launch HBM bytes of each block from the two counter runs, each
    counter scaled by the calibration kernel's true bytes over its counted
    bytes."""
    blocks, _ = counter_plan(workload)
    res = {name: {"algorithmic_bytes": v} for name, _, v in blocks}
    per = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        got, calib, ck = _split_blocks(d, workload, n)
        factor = CALIB_BYTES / (1024.0 * sum(c[counter] for c in calib) / n)
        per[counter] = {"factor": factor, "calib_kernel": ck[:80]}
        for name, _, _ in blocks:
            res[name][counter] = sum(c[counter] for c in got[name]) / n
            res[name]["kernels"] = got[name + "#kernel"]
    for name, r in res.items():
        r["hbm_bytes"] = round(r["FETCH_SIZE"] * 1024 * per["FETCH_SIZE"]["factor"]
                               + r["WRITE_SIZE"] * 1024 * per["WRITE_SIZE"]["factor"])
        r["fetch_kib"] = round(r.pop("FETCH_SIZE"), 1)
        r["write_kib"] = round(r.pop("WRITE_SIZE"), 1)
    return res, per


def write_counter_profiles(res, per, workload: str, n: int):
    cmd = ("rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT_F -o run -- python -u "
           f"bench.py --counter-pass --workload {workload} --counter-launches {n}; the same "
           f"with WRITE_SIZE into OUT_W; python bench.py --summarize-counters OUT_F OUT_W "
           f"--workload {workload} --counter-launches {n}")
    _, groups = counter_plan(workload)
    for fam, (labels, unit) in groups.items():
        rec = {"kernel": fam, "workload": workload,
               "sources_digest": sources_digest(KERNEL_SOURCES[fam]),
               "hbm_bytes_per_launch": sum(res[l]["hbm_bytes"] for l in labels),
               "algorithmic_bytes_per_launch": sum(res[l]["algorithmic_bytes"] for l in labels),
               "launches": {l: res[l] for l in labels},
               "calibration": {k: {"factor": round(v["factor"], 4), "kernel": v["calib_kernel"],
                                   "bytes": CALIB_BYTES} for k, v in per.items()},
               "unit_note": unit, "command": cmd}
        with open(os.path.join(PROFILES, f"{fam}_{workload}_pmc.json"), "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
    lines = [f"# HBM traffic per launch from rocprofv3 counters: bench.py, workload {workload}",
             "", "Commands (on one MI355X, from the repository root):", "", "    " + cmd, "",
             "FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by the ratio of true bytes "
             "to counter bytes measured on a plain elementwise kernel reading and writing 256 MiB "
             f"(FETCH x{per['FETCH_SIZE']['factor']:.3f}, WRITE x{per['WRITE_SIZE']['factor']:.3f}). "
             f"Averages over {n} calls, each on its own operand copy (a call may make more "
             "than one launch: their counters are summed).", "",
             "| Call | Kernels | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | HBM bytes (scaled) "
             "| Algorithmic bytes | Ratio |", "|---|---|---|---|---|---|---|"]
    for l, r in res.items():
        kname = ", ".join(f"`{k}`" for k in r["kernels"])
        lines.append(f"| {l} | {kname} | {r['fetch_kib']:.0f} | {r['write_kib']:.0f} | "
                     f"{r['hbm_bytes']:,} | {r['algorithmic_bytes']:,} | "
                     f"{r['hbm_bytes'] / r['algorithmic_bytes']:.3f} |")
    with open(os.path.join(PROFILES, f"counters_{workload}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")


# Derived figures of a counter summary, each from counters of one run.
# GRBM_GUI_ACTIVE sums the eight XCDs' busy cycles, so one eighth of it is the
# dispatch's length in GPU clocks; the chip has 256 CUs of 4 SIMDs and one
# texture addresser (TA) per CU.
DERIVED = (
    ("clocks", ("GRBM_GUI_ACTIVE",), lambda c: c["GRBM_GUI_ACTIVE"] / 8,
     "GRBM_GUI_ACTIVE / 8", "{:,.0f}"),
    ("MFMA pipe busy per SIMD", ("SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE"),
     lambda c: c["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024 * c["GRBM_GUI_ACTIVE"] / 8),
     "SQ_VALU_MFMA_BUSY_CYCLES / (1024 x clocks)", "{:.1%}"),
    ("VALU busy per SIMD", ("SQ_ACTIVE_INST_VALU", "GRBM_GUI_ACTIVE"),
     lambda c: 4 * c["SQ_ACTIVE_INST_VALU"] / (1024 * c["GRBM_GUI_ACTIVE"] / 8),
     "4 x SQ_ACTIVE_INST_VALU / (1024 x clocks)", "{:.1%}"),
    ("waves waiting on anything", ("SQ_WAIT_ANY", "SQ_WAVE_CYCLES"),
     lambda c: c["SQ_WAIT_ANY"] / c["SQ_WAVE_CYCLES"], "SQ_WAIT_ANY / SQ_WAVE_CYCLES", "{:.1%}"),
    ("waves waiting to issue", ("SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES"),
     lambda c: c["SQ_WAIT_INST_ANY"] / c["SQ_WAVE_CYCLES"], "SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES",
     "{:.1%}"),
    ("TA busy per CU", ("TA_TA_BUSY_sum", "GRBM_GUI_ACTIVE"),
     lambda c: c["TA_TA_BUSY_sum"] / (256 * c["GRBM_GUI_ACTIVE"] / 8),
     "TA_TA_BUSY_sum / (256 x clocks)", "{:.1%}"),
    ("TA cycles per vector memory read", ("TA_TA_BUSY_sum", "SQ_INSTS_VMEM_RD"),
     lambda c: c["TA_TA_BUSY_sum"] / c["SQ_INSTS_VMEM_RD"],
     "TA_TA_BUSY_sum / SQ_INSTS_VMEM_RD", "{:.1f}"),
    ("LDS bank conflicts per LDS cycle", ("SQ_LDS_BANK_CONFLICT", "SQ_ACTIVE_INST_LDS"),
     lambda c: c["SQ_LDS_BANK_CONFLICT"] / c["SQ_ACTIVE_INST_LDS"],
     "SQ_LDS_BANK_CONFLICT / SQ_ACTIVE_INST_LDS", "{:.3f}"),
)


def summarize_pmc(dirs, workload: str, n: int):
    """profiles/sq_counters_<workload>.md: per block, the average per dispatch
    of every counter of the given --pmc runs of a counter pass, and the
    derived figures whose counters one run holds."""
    blocks, _ = counter_plan(workload)
    runs = []
    for d in dirs:
        got, _, _ = _split_blocks(d, workload, n)
        counters = sorted(next(iter(got[blocks[0][0]])).keys())
        avg = {name: {c: sum(x[c] for x in got[name]) / n for c in counters}
               for name, _, _ in blocks}
        runs.append((d, counters, avg, got))
    lines = [f"# Counters per dispatch: bench.py counter pass, workload {workload}", "",
             "Commands (on one MI355X, from the repository root), one run per counter set:", ""]
    for i, (_, counters, _, _) in enumerate(runs):
        lines.append(f"    rocprofv3 --pmc {','.join(counters)} --output-format csv -d OUT_{i + 1} "
                     f"-o run -- python -u bench.py --counter-pass --workload {workload} "
                     f"--counter-launches {n}")
    lines += ["", "    python bench.py --summarize-pmc " + " ".join(
        f"OUT_{i + 1}" for i in range(len(runs))) + f" --workload {workload} "
        f"--counter-launches {n}", "",
        f"Averages over the {n} calls of each block (each on its own operand copy; the "
        "launches of a call summed).", ""]
    head = "| Counter | " + " | ".join(b for b, _, _ in blocks) + " |"
    sep = "|---" * (len(blocks) + 1) + "|"
    lines += ["## Raw counters", "", head, sep]
    for ri, (_, counters, avg, _) in enumerate(runs):
        for c in counters:
            lines.append(f"| {c} (run {ri + 1}) | " + " | ".join(
                f"{avg[b][c]:,.0f}" for b, _, _ in blocks) + " |")
    lines += ["", "## Derived", "",
              "GRBM_GUI_ACTIVE sums the eight XCDs' busy cycles: one eighth of it is the "
              "dispatch's length in GPU clocks (clocks below). The chip has 256 CUs of 4 SIMDs "
              "and one texture addresser per CU.", "", "| Figure (formula) | " +
              " | ".join(b for b, _, _ in blocks) + " |", sep]
    for label, need, fn, formula, fmt in DERIVED:
        for ri, (_, counters, avg, _) in enumerate(runs):
            if all(k in counters for k in need):
                def cell(c):
                    try:
                        return fmt.format(fn(c))
                    except ZeroDivisionError:
                        return "—"
                lines.append(f"| {label} ({formula}; run {ri + 1}) | " + " | ".join(
                    cell(avg[b]) for b, _, _ in blocks) + " |")
                break
    with open(os.path.join(PROFILES, f"sq_counters_{workload}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")


def summarize_trace(d: str, name: str, command: str):
    """profiles/<name>_kernel_trace.md from the *_kernel_stats.csv of a
    rocprofv3 --kernel-trace --stats run: calls and durations of the
    library's kernels (and the calibration probes)."""
    import csv
    rows = []
    for dirpath, _, files in os.walk(d):
        for f in files:
            if f.endswith("kernel_stats.csv"):
                rows += list(csv.DictReader(open(os.path.join(dirpath, f))))
    if not rows:
        raise SystemExit(f"{d}: no kernel_stats.csv")
    keep = [r for r in rows if "bd::" in r["Name"] or any(
        k in r["Name"] for k in KERNEL_OF.values())]
    lines = [f"# rocprofv3 kernel trace: {name}", "", "Command (one MI355X, repository root):", "",
             "    " + command, "",
             "Library kernels from the run's kernel statistics (every launch of the process: "
             "set-up, eager runs, graph captures, timed steps and ranges; durations in "
             "microseconds).", "", "| Kernel | Calls | Average | Min | Max | Total (ms) |",
             "|---|---|---|---|---|---|"]
    for r in sorted(keep, key=lambda r: -float(r["TotalDurationNs"])):
        kname = _short_kernel(r["Name"])
        lines.append(f"| `{kname}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['TotalDurationNs']) / 1e6:.2f} |")
    with open(os.path.join(PROFILES, f"{name}_kernel_trace.md"), "w") as f:
        f.write("\n".join(lines) + "\n")


PCIE_PEAK_GBS = 64.0           # PCIe 5.0 x16 host link, one direction, published


def measure_delta_loads(decode_graph, n_decode: int, decode_alone_us: float):
    """Cold loads through the delta cache (bitdelta_cache_acquire): one
    70B-shaped layer's delta per variant (packed signs of its five linears
    and per-row alpha, laid out by delta_layout), from page-locked host
    memory into device slots on a copy stream.  Four variants cycle through
    two slots, so every request is a miss that loads (a request that finds
    both slots still loading is refused by the policy and retried once the
    copy stream is idle).  Then the same loads
    run while the decode range (back-to-back decode launches) replays on the
    compute stream: the decode's launch time with loads in flight against
    its time alone.  The bytes are checked after the loads."""
    shapes = [(d_out, d_in) for _, d_out, d_in in S.LAYER_70B]
    _, total = T.delta_layout(shapes, T.ALPHA_PER_ROW)
    n_var, n_slots = 4, 2
    blobs = [torch.full((total,), v + 1, dtype=torch.uint8, pin_memory=True)
             for v in range(n_var)]
    slots = [torch.empty(total, dtype=torch.uint8, device="cuda") for _ in range(n_slots)]
    cache = T.DeltaCache(n_var, n_slots, 0, 0)
    cache.attach(slots, blobs)
    copy = torch.cuda.Stream()
    use = torch.cuda.Stream()   # the consumer of the loaded deltas (not the decode's stream)

    def loads(first: int, k: int):
        evs = []
        for j in range(k):
            v = (first + j) % n_var
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            act, slot = T.CACHE_FULL, None
            while act == T.CACHE_FULL:   # both slots still loading: wait, as a router would
                a.record(copy)
                act, slot, _ = cache.acquire(v, copy, use)
                if act == T.CACHE_FULL:
                    copy.synchronize()
            b.record(copy)
            if act != T.CACHE_LOAD:
                raise RuntimeError(f"expected a load of variant {v}, got action {act}")
            cache.release(v, use)
            evs.append((a, b, v, slot))
        return evs

    loads(0, 4)   # warm-up: first touch of every slot and source
    torch.cuda.synchronize()
    evs = loads(0, 8)
    torch.cuda.synchronize()
    load_ms = [a.elapsed_time(b) for a, b, _, _ in evs]
    for _, _, v, slot in evs[-2:]:
        if not bool((slot[:: 1 << 20] == v + 1).all()):
            raise RuntimeError("loaded delta bytes differ from the source")
    # loads during decode
    d0 = torch.cuda.Event(enable_timing=True)
    d1 = torch.cuda.Event(enable_timing=True)
    evs2 = loads(0, 4)
    d0.record()
    decode_graph.replay()
    d1.record()
    torch.cuda.synchronize()
    # the first two loads fill both slots and the host waits for them before
    # the last two can be requested; the last two overlap the decode replay
    load_ms_during = [a.elapsed_time(b) for a, b, _, _ in evs2[2:]]
    decode_during_us = 1e3 * d0.elapsed_time(d1) / n_decode
    mean_ms = sum(load_ms) / len(load_ms)
    gbs = total / (mean_ms * 1e-3) / 1e9
    variant_80 = 80 * total
    cache.close()
    return {
        "what": "one 70B-shaped layer's delta per load (packed signs of QKV, O, gate, up, "
                "down + per-row alpha), page-locked host -> HBM via bitdelta_cache_acquire "
                "on a copy stream, 4 variants cycling through 2 slots (every request loads)",
        "bytes_per_load": total,
        "load_ms": round(mean_ms, 4),
        "achieved_gbs": round(gbs, 2),
        "pcie_peak_gbs": PCIE_PEAK_GBS,
        "frac": round(gbs / PCIE_PEAK_GBS, 4),
        "variant_80_layers_bytes": variant_80,
        "variant_80_layers_ms_at_this_rate": round(variant_80 / (gbs * 1e9) * 1e3, 1),
        "load_ms_during_decode": round(sum(load_ms_during) / len(load_ms_during), 4),
        "decode_m16_us_alone": round(decode_alone_us, 3),
        "decode_m16_us_during_loads": round(decode_during_us, 3),
    }


REPS = 50                      # replays per timing graph; the median is reported


def roofline_entry(bound, achieved, peak, unit, traffic=None, measured=None):
    """Roofline of one kernel: achieved against the published peak, and
    against the ceiling measured on this GPU by the calibration probes."""
    e = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
         "frac": round(achieved / peak, 4), "traffic": traffic}
    if measured:
        e["measured_peak"] = round(measured, 2)
        e["frac_vs_measured"] = round(achieved / measured, 4)
    return e


# ------------------------------------------------------------------ ceilings
def measure_ceilings(dev):
    """What this GPU reaches on plain work: a stream read of 1 GiB (the best
    of several workgroup counts), the same read as 32 MiB launches cycling
    over 32 distinct buffers (the size of one decode launch on the
    projection), and back-to-back bf16 MFMA (the best of two grid sizes)."""
    sink = torch.zeros(256, dtype=torch.int32, device=dev)
    big = torch.zeros(2**30 // 2, dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    res = {}
    best = (0.0, 0)
    for wg in (1024, 2048, 4096, 8192):
        g = capture(lambda wg=wg: [T.probe_stream_read(big, wg, sink) for _ in range(4)])
        ms = median(time_replays(g, 20)) / 4
        best = max(best, (2**30 / (ms * 1e-3) / 1e9, wg))
    res["hbm_read_gbs"] = round(best[0], 1)
    res["hbm_read_workgroups"] = best[1]
    chunks = [big[i * 2**24:(i + 1) * 2**24] for i in range(32)]
    best32 = (0.0, 0)
    for wg in (256, 512, 1024, 2048):
        g = capture(lambda wg=wg: [T.probe_stream_read(c, wg, sink) for _ in range(4)
                                   for c in chunks])
        ms = median(time_replays(g, 20)) / 128
        best32 = max(best32, (2**25 / (ms * 1e-3) / 1e9, wg))
    res["hbm_read_32mib_gbs"] = round(best32[0], 1)
    res["hbm_read_32mib_workgroups"] = best32[1]
    del big, chunks
    bestm = (0.0, 0)
    for wg in (512, 1024):
        iters = 2048
        flops = [0]
        g = capture(lambda wg=wg: flops.__setitem__(0, sum(T.probe_mfma_bf16(wg, iters, sink)
                                                          for _ in range(4))))
        ms = median(time_replays(g, 10))
        bestm = max(bestm, (flops[0] / (ms * 1e-3) / 1e12, wg))
    res["bf16_mfma_tflops"] = round(bestm[0], 1)
    res["bf16_mfma_workgroups"] = bestm[1]
    res["bf16_mfma_implied_ghz"] = round(2.4 * bestm[0] / BF16_PEAK_TFLOPS, 3)
    # The single-variant decode's loads on the 4096 x 4096 projection without
    # its arithmetic, in six patterns (bitdelta_probe_decode_loads), over 12
    # matrix copies in turn; microseconds per launch.
    gen = torch.Generator(device=dev)
    gen.manual_seed(17)
    ws = [torch.randn(4096, 4096, generator=gen, device=dev).to(torch.bfloat16) for _ in range(12)]
    ss = [torch.randint(0, 2 ** 31 - 1, (1 << 19,), generator=gen, device=dev, dtype=torch.int32)
          for _ in range(12)]
    xv = torch.randn(4096, generator=gen, device=dev).to(torch.bfloat16)
    orders = {}
    for mode, name in enumerate(DECODE_LOAD_PATTERNS):
        g = capture(lambda mode=mode: [T.probe_decode_loads(ws[c % 12], ss[c % 12], xv, mode, sink)
                                       for c in range(24)])
        orders[name] = round(median(time_replays(g, 20)) / 24 * 1e3, 3)
    res["decode_loads_us"] = orders
    del ws, ss
    torch.cuda.synchronize()
    return res


# bitdelta_probe_decode_loads modes 0..5 (include/bitdelta.h)
DECODE_LOAD_PATTERNS = ("contiguous", "blocks_consecutive_rows", "blocks_interleaved_rows",
                        "interleaved_to_lds", "interleaved_with_signs", "ring_loads")


# ------------------------------------------------------------------ timing
def time_workload(w, args, n_pass=1, check=None):
    """Graphs of one pass of the path (the steps) and of each kernel range;
    K timed steps (HIP events around each replay, between synchronisations),
    then REPS timed replays of each range: the median replay divided by its
    launches is the kernel's launch duration.  check(name) runs after a
    range's replays (the graphs must reproduce eager results)."""
    passes = [capture(lambda j=j: w.one_pass(j)) for j in range(n_pass)]
    range_graphs = {name: (n, capture(fn)) for name, (n, fn) in w.ranges().items()}
    for i in range(args.warmup):
        passes[i % n_pass].replay()
    torch.cuda.synchronize()
    step_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step_ev[i][0].record()
        passes[i % n_pass].replay()
        step_ev[i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_list = [s.elapsed_time(e) for s, e in step_ev]
    avg_us = {}
    for name, (n, g) in range_graphs.items():
        g.replay()
        avg_us[name] = 1e3 * median(time_replays(g, REPS)) / n
        if check:
            check(name)
    print(f"[bench] {w.name}: timed {args.steps} steps in {wall:.3f} s "
          f"(GPU {sum(step_list) / len(step_list):.3f} ms per step)", file=sys.stderr, flush=True)
    return {"step_ms": sum(step_list) / len(step_list), "step_ms_median": median(step_list),
            "wall_s": wall, "avg_us": avg_us, "range_graphs": range_graphs}


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        return 1


def _cpu_record(value, unit, sample):
    return {"value": value, "unit": unit, "cores": int(_blas_threads()), "kind": "oracle",
            "sample": sample, "host_cores_available": len(os.sched_getaffinity(0)),
            "cores_note": "cores = numpy BLAS threads the oracle's float64 products ran on; "
                          "host_cores_available = CPUs this process may use"}


# ------------------------------------------------------------------ proj_4096
def bench_proj(args, dev, ceil):
    """The 4096x4096 projection (the metric's decode configuration): the
    whole path per step, each kernel's launch duration, the unfused A/B and
    the delta loads.  Returns (record, workload)."""
    w = ProjWorkload(dev)
    torch.cuda.synchronize()
    print(f"[bench] proj_4096: rotation copies R={w.R}, distinct variants in the mixed batch "
          f"D={w.distinct}", file=sys.stderr, flush=True)
    n_pass = max(1, w.R // 6)
    # eager references of the unfused A/B outputs, checked after each range
    eager_ref = {}
    for m in list(w.decode_ms) + [w.prefill_m]:
        w.run_dense(m, 0)
        eager_ref[f"dense_m{m}"] = (w.ys_dense[m], w.ys_dense[m].clone())
    w.run_reconstruct(0)
    eager_ref["reconstruct"] = (w.w_eff, w.w_eff.clone())
    w.run_decode(16, 0)
    eager_ref["decode_m16"] = (w.ys[16], w.ys[16].clone())
    torch.cuda.synchronize()

    def check(name):
        if name in eager_ref:
            buf, ref = eager_ref[name]
            assert torch.equal(buf.view(torch.int16), ref.view(torch.int16)), (
                f"graph replays of {name} differ from the eager launch")

    t = time_workload(w, args, n_pass, check)
    avg_us = t["avg_us"]
    dec_bytes = sum(w.decode_bytes(m) for m in w.decode_ms)
    dec_us = sum(avg_us[f"decode_m{m}"] for m in w.decode_ms)
    dec_gbs = dec_bytes / (dec_us * 1e-6) / 1e9
    pre_tflops = w.prefill_flops() / (avg_us["prefill"] * 1e-6) / 1e12
    hbm = ceil.get("hbm_read_32mib_gbs")
    mfma = ceil.get("bf16_mfma_tflops")
    rooflines = {
        "decode": roofline_entry("hbm", dec_gbs, HBM_PEAK_GBS, "GB/s",
                                 counter_traffic("decode", w.name), hbm),
        "compress": roofline_entry("hbm", w.compress_bytes() / (avg_us["compress"] * 1e-6) / 1e9,
                                   HBM_PEAK_GBS, "GB/s", counter_traffic("compress", w.name),
                                   ceil.get("hbm_read_gbs")),
        "multi": roofline_entry("hbm", w.multi_bytes() / (avg_us["multi"] * 1e-6) / 1e9,
                                HBM_PEAK_GBS, "GB/s", counter_traffic("multi", w.name), hbm),
        "prefill": roofline_entry("mfma", pre_tflops, BF16_PEAK_TFLOPS, "TFLOP/s",
                                  counter_traffic("prefill", w.name), mfma),
        "reconstruct": roofline_entry("hbm", w.reconstruct_bytes() / (avg_us["reconstruct"] * 1e-6)
                                      / 1e9, HBM_PEAK_GBS, "GB/s",
                                      counter_traffic("reconstruct", w.name),
                                      ceil.get("hbm_read_gbs")),
    }
    # Unfused A/B: the fused call against W_eff materialised by
    # bitdelta_reconstruct and multiplied by the library GEMM (torch.mm on
    # hipBLASLt), and against that GEMM alone on a stored W_eff.
    rec_us = avg_us["reconstruct"]
    unfused = {}
    for m in list(w.decode_ms) + [w.prefill_m]:
        key = f"decode_m{m}" if m in w.decode_ms else "prefill"
        dense = avg_us[f"dense_m{m}"]
        unfused[key] = {"tokens": m, "fused_us": round(avg_us[key], 3),
                        "reconstruct_plus_gemm_us": round(rec_us + dense, 3),
                        "gemm_on_stored_weff_us": round(dense, 3)}
    print("[bench] proj_4096: delta-cache loads", file=sys.stderr, flush=True)
    n16, g16 = t["range_graphs"]["decode_m16"]
    delta_load = measure_delta_loads(g16, n16, avg_us["decode_m16"])
    rec = {
        "value": round(dec_gbs, 2), "unit": "GB/s",
        "ms_per_step": round(t["step_ms"], 4), "ms_per_step_median": round(t["step_ms_median"], 4),
        "config": {
            "workload": "proj_4096: Llama-style 4096x4096 projection, bf16 W_base~N(0,0.02), "
                        "Laplace(0,5e-4) delta, per-row alpha; step = compress W_ft + decode "
                        "M=1,4,16 + 14-variant Zipf(1.1) decode M=16 + prefill M=2048",
            "d_out": 4096, "d_in": 4096, "decode_tokens": list(w.decode_ms),
            "multi_tokens": w.multi_m, "multi_variants": w.n_variants,
            "multi_distinct_variants": w.distinct, "prefill_tokens": w.prefill_m,
            "alpha_mode": "per_row", "rotation_copies": w.R,
        },
        "prefill_tflops": round(pre_tflops, 2),
        "roofline": rooflines["decode"],
        "roofline_by_kernel": rooflines,
        "unfused_ab": unfused,
        "kernel_us": {k: round(v, 3) for k, v in avg_us.items()},
        "delta_load": delta_load,
    }
    return rec, w


# ------------------------------------------------------------------ layers
def sample_rows(d_out: int, k: int, seed: int) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    return np.sort(rng.choice(d_out, size=min(k, d_out), replace=False))


def _host_rows(t: torch.Tensor, rows):
    return t[torch.as_tensor(rows, device=t.device)].cpu()


def layer_samples(w, layer_ops, k: int, seed: int):
    """Host copies of what the oracle needs for k sampled output rows of each
    matrix (every output row depends on its weight row only): x, the rows of
    W_base, their packed signs and alpha.  layer_ops: per matrix (x, W_base,
    [packed per variant], [alpha per variant])."""
    out = []
    for i, (x, wb, packs, alphas) in enumerate(layer_ops):
        d_out = wb.shape[0]
        rows = sample_rows(d_out, k, seed + i)
        out.append({
            "x": S.bf16_bits(x), "wb": S.bf16_bits(_host_rows(wb, rows)),
            "packs": [_host_rows(p, rows).numpy().view(np.uint64) for p in packs],
            "alphas": [(_host_rows(a, rows) if w.mode == 1 else a.cpu()).numpy()
                       for a in alphas],
            "rows": len(rows), "d_in": wb.shape[1], "d_out": d_out})
    return out


def cpu_layer(kind, samples, mode, ids, budget_s: float, what: str):
    """The oracle on the sampled rows, repeated while the budget lasts: prefill
    in TFLOP/s (2*M*rows*d_in per matrix), mixed decode in GB/s (the rows'
    share of the algorithmic bytes: W_base, the signs and alpha of every
    variant present, x and y)."""
    import oracle as O
    work, t_all, passes = 0.0, 0.0, 0
    distinct = len(set(int(v) for v in ids)) if ids is not None else 1
    while True:
        t0 = time.perf_counter()
        for smp in samples:
            r, d_in = smp["rows"], smp["d_in"]
            m = smp["x"].shape[0]
            if kind == "prefill":
                O.linear(smp["x"], smp["wb"], smp["packs"][0], smp["alphas"][0], mode)
                work += 2.0 * m * r * d_in
            else:
                O.linear_multi(smp["x"], ids, smp["wb"], smp["packs"], smp["alphas"], mode)
                alpha = 4 * (r if mode == 1 else 1)
                work += (2 * r * d_in + distinct * (r * d_in // 8 + alpha) + 2 * m * d_in
                         + 2 * m * r + 4 * m)
        t_all += time.perf_counter() - t0
        passes += 1
        if t_all > budget_s or passes >= 50:
            break
    scale, unit = (1e12, "TFLOP/s") if kind == "prefill" else (1e9, "GB/s")
    rows = samples[0]["rows"]
    return _cpu_record(round(work / t_all / scale, 5), unit,
                       f"{what}: oracle on {rows} sampled output rows of each matrix, "
                       f"{passes} pass(es), {t_all:.1f} s")


def bench_layer(name, args, dev, ceil):
    """One of the layer configurations (70B-shaped layer prefill, layer
    mixed decode, the 80-layer stack's mixed decode): steps, each matrix's
    launch duration, the roofline, and host samples for the oracle."""
    t0 = time.perf_counter()
    if name == "stack70b_multi":
        w = StackWorkload(name, dev)
    else:
        w = LayerWorkload(name, dev)
        if args.ab_per_variant and w.kind == "multi":
            w.setup_per_variant()
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t0
    print(f"[bench] {name}: set up in {setup_s:.1f} s, distinct variants D={w.distinct}",
          file=sys.stderr, flush=True)
    t = time_workload(w, args)
    rep = w.report(t["avg_us"], args, t["step_ms"])
    measured = ceil.get("bf16_mfma_tflops") if w.kind == "prefill" else ceil.get("hbm_read_gbs")
    rep["roofline"] = roofline_entry(rep["roofline"]["bound"], rep["value"],
                                     rep["roofline"]["peak"], rep["roofline"]["unit"],
                                     rep["roofline"]["traffic"], measured)
    rep["ms_per_step"] = round(t["step_ms"], 4)
    rep["ms_per_step_median"] = round(t["step_ms_median"], 4)
    rep["kernel_us"] = {k: round(v, 3) for k, v in t["avg_us"].items()}
    rep["setup_s"] = round(setup_s, 1)
    # host samples for the oracle, taken before the device memory is freed
    if name == "stack70b_multi":
        layers = (0, w.wl.layers // 2, w.wl.layers - 1)
        samples = []
        for l in layers:
            ops = [(w.xs[l][i], w.stack[l][i], [w.packs[l][v][i] for v in range(len(w.packs[l]))],
                    [w.alphas[l][v][i] for v in range(len(w.alphas[l]))])
                   for i in range(len(w.wl.matrices))]
            samples += layer_samples(w, ops, 32, 1000 + 10 * l)
        what = f"layers {list(layers)} of the 80-layer stack, M={w.m}"
    else:
        ops = [w.rot[i][0] for i in range(len(w.bases))]
        samples = layer_samples(w, ops, 64 if w.kind == "prefill" else 128, 1000)
        what = f"one 70B-shaped layer, M={w.m}"
    ids = w.ids.cpu().numpy() if w.kind == "multi" else None
    meta = {"kind": w.kind, "mode": w.mode, "ids": ids, "samples": samples, "what": what}
    return rep, meta


def free_device():
    import gc
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


DEFAULT_CONFIGS = ("proj_4096", "layer70b_prefill", "layer70b_multi", "stack70b_multi")


def run_default(args, dev):
    """The default line: value is the decode figure of the projection (the
    metric's decode configuration); the 70B-shaped layer's prefill gives the
    metric's TFLOP/s; the layer's and the 80-layer stack's mixed-variant
    decode are reported beside them, each with its roofline and the oracle on
    a bounded sample."""
    configs = [c for c in args.configs.split(",") if c]
    for c in configs:
        if c not in DEFAULT_CONFIGS:
            raise SystemExit(f"unknown configuration {c}")
    print("[bench] measuring ceilings", file=sys.stderr, flush=True)
    ceil = measure_ceilings(dev)
    print(f"[bench] ceilings {ceil}", file=sys.stderr, flush=True)
    free_device()
    recs, metas, proj_w = {}, {}, None
    for c in configs:
        print(f"[bench] setting up {c}", file=sys.stderr, flush=True)
        if c == "proj_4096":
            recs[c], proj_w = bench_proj(args, dev, ceil)
            proj_host = proj_w.host
            proj_meta = {"mode": proj_w.mode, "decode_ms": proj_w.decode_ms}
            proj_w = None
        else:
            recs[c], metas[c] = bench_layer(c, args, dev, ceil)
        free_device()
    if args.cpu_budget > 0:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        if "proj_4096" in recs:
            shell = ProjWorkload.__new__(ProjWorkload)
            shell.host, shell.mode, shell.decode_ms = proj_host, proj_meta["mode"], \
                proj_meta["decode_ms"]
            shell.d_out = shell.d_in = 4096
            recs["proj_4096"]["cpu_baseline"] = cpu_baseline(shell, args.cpu_budget)
        for c, m in metas.items():
            recs[c]["cpu_baseline"] = cpu_layer(m["kind"], m["samples"], m["mode"], m["ids"],
                                                args.cpu_budget / 2, m["what"])
    head = recs.get("proj_4096") or next(iter(recs.values()))
    out = {
        "metric": METRIC, "value": head["value"], "unit": head["unit"], "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic", "config": head["config"],
        "roofline": head["roofline"], "cpu_baseline": head.get("cpu_baseline"),
    }
    if "layer70b_prefill" in recs:
        r = recs["layer70b_prefill"]
        out["prefill_tflops"] = r["value"]
        out["prefill_roofline"] = r["roofline"]
    if "layer70b_multi" in recs:
        out["multi_layer_gbs"] = recs["layer70b_multi"]["value"]
        out["multi_layer_roofline"] = recs["layer70b_multi"]["roofline"]
    if "stack70b_multi" in recs:
        out["multi_stack_gbs"] = recs["stack70b_multi"]["value"]
        out["multi_stack_roofline"] = recs["stack70b_multi"]["roofline"]
    out["ceilings"] = ceil
    out["timing"] = (f"medians of {REPS} HIP-event-timed graph replays per kernel range "
                     f"(each replay = back-to-back launches over distinct operand copies); "
                     f"ms_per_step = mean of the K timed steps")
    out["configs"] = recs
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="default",
                    choices=["default", "proj_4096", "layer70b_prefill", "layer70b_multi",
                             "layer70b_decode", "stack70b_multi", "serve_layer70b",
                             "monosoup_4096", "ceilings"])
    ap.add_argument("--configs", default=",".join(DEFAULT_CONFIGS),
                    help="configurations of the default line (comma-separated)")
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of oracle work for the projection's cpu_baseline leg (half "
                         "that for each layer configuration; 0 skips them)")
    ap.add_argument("--counter-pass", action="store_true",
                    help="eager launches for a rocprofv3 --pmc run (--workload proj_4096, "
                         "layer70b_multi or layer70b_prefill; default proj_4096), then exit")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/*_<workload>_pmc.json and counters_<workload>.md "
                         "from a FETCH_SIZE and a WRITE_SIZE run of the counter pass, then exit")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="DIR",
                    help="write profiles/sq_counters_<workload>.md from --pmc runs of the "
                         "counter pass, then exit")
    ap.add_argument("--summarize-trace", nargs=3, metavar=("DIR", "NAME", "COMMAND"),
                    help="write profiles/NAME_kernel_trace.md from a --kernel-trace --stats "
                         "run made by COMMAND, then exit")
    ap.add_argument("--counter-launches", type=int, default=8)
    ap.add_argument("--ab-per-variant", action="store_true",
                    help="layer70b_multi: also time the per-variant fused alternative (one "
                         "single-variant fused call per variant present) on the same batch")
    ap.add_argument("--clock-pass", action="store_true",
                    help="six fused gate-shaped prefills then six library GEMMs, for a "
                         "rocprofv3 --pmc GRBM_GUI_ACTIVE run, then exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the kernels would shard by output rows); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    cw = "proj_4096" if args.workload == "default" else args.workload
    if (args.counter_pass or args.summarize_counters or args.summarize_pmc) \
            and cw not in COUNTER_WORKLOADS:
        raise SystemExit(f"counter runs cover {', '.join(COUNTER_WORKLOADS)}")
    if args.summarize_counters:
        res, per = summarize_counters(*args.summarize_counters, cw, args.counter_launches)
        write_counter_profiles(res, per, cw, args.counter_launches)
        print(json.dumps({"counters": res, "calibration": per}), flush=True)
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc, cw, args.counter_launches)
        print(f"[bench] wrote profiles/sq_counters_{cw}.md", flush=True)
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        print(f"[bench] wrote profiles/{args.summarize_trace[1]}_kernel_trace.md", flush=True)
        return
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    T.lib()
    if args.clock_pass:
        clock_pass(dev)
        print("[bench] clock pass done", file=sys.stderr, flush=True)
        return
    if args.counter_pass:
        counter_pass(cw, dev, args.counter_launches)
        print(f"[bench] counter pass done ({cw}, {args.counter_launches} launches per block)",
              file=sys.stderr, flush=True)
        return
    if args.workload == "default":
        run_default(args, dev)
        return
    if args.workload == "ceilings":
        # the measured ceilings alone (stream read of HBM, bf16 MFMA), as the
        # default line reports them beside the published peaks
        ceil = measure_ceilings(dev)
        print(json.dumps({"ceilings": ceil, "published": {"hbm_gbs": HBM_PEAK_GBS,
                                                         "bf16_tflops": BF16_PEAK_TFLOPS}}),
              flush=True)
        return
    print(f"[bench] setting up {args.workload}", file=sys.stderr, flush=True)
    if args.workload == "serve_layer70b":
        serve_layer70b(args, dev)
        return
    if args.workload == "monosoup_4096":
        monosoup_4096(args, dev)
        return
    if args.workload == "layer70b_decode":
        w = DecodeLayerWorkload(args.workload, dev)
        torch.cuda.synchronize()
        t = time_workload(w, args)
        rep = w.report(t["avg_us"], args, t["step_ms"])
        rep["kernel_us"] = {k: round(v, 3) for k, v in t["avg_us"].items()}
        out = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
               "ms_per_step": round(t["step_ms"], 4), "higher_is_better": True,
               "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
               **rep, "cpu_baseline": None}
        print(json.dumps(out), flush=True)
        return
    # one configuration of the default line alone
    args.configs = args.workload
    run_default(args, dev)


if __name__ == "__main__":
    main()
