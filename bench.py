"""Benchmark of the attention block on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]

A step is one pass of the hot path over one batch of synthetic input resident in HBM:
  split-GQA workloads: the k and v headnorms in one launch, then split-GQA attention that
    applies the q headnorm + rope as it stages q (--norm one_launch: q, k and v in one launch,
    then plain attention; --norm separate: the page's three headnorm dispatches);
  dg_layers: the same for each layer of a sliding/global layer stack (one step = all layers);
  sam_relpos: one rel-pos flash attention (bias-row pass + flash kernel);
  sam_windowed: the same over the SAM windowed block's 25 windows of 14x14 tokens.
The default workload is the long-cache split-GQA canvas step (4 canvases, T=256, ctx=8192,
nh=32, nkv=8, hd=128).  W untimed steps, then K steps timed with HIP events on the stream the
kernels run on (torch's current stream), bracketed by device synchronisation.  By default W
covers about half a second (the GPU raises its clock over the first tens of milliseconds of
sustained load) and K about a quarter second; both are reported.  A second pass of K steps
times each launch of the dominant call with its own events (kept out of the first pass: an
event pair between launches adds a few microseconds to a step).

A third pass records an event at every step boundary (median and minimum step time), and
--cold N times N more steps one at a time, each after a read of a 512 MiB buffer has evicted
the L2s and the MALL.  The DiffusionGemma-like workload cycles through 48 pre-staged denoising
steps (fresh canvas q, k, v each step, one fixed cache).  Before the main workload, the
workloads named by --also (default: the other configurations) are measured the same way with
time-based step counts and reported under "also".

Prints ONE JSON line: metric/value/unit (algorithmic TFLOP/s of the step, or GB/s for the
HBM-bound depformer workload), roofline of the dominant kernel against MI355X peaks, timing
statistics, and the oracle timed on the host cores over a bounded sample of the same workload
(a reported baseline, not the target; with the host CPU's model and the threads it used).
Parity of this launch configuration is the GPU tests' job.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s and HBM GB/s (% of MI355X roofline) per canvas step"
PEAK_F32_MFMA = 157.3      # TFLOP/s, dense f32 matrix
PEAK_BF16_MFMA = 2500.0    # TFLOP/s, dense bf16 matrix
CLOCK_SETTLE_S = 0.3       # untimed load before the warmup steps (see run())


def mfma_ceiling(plan_kernel, kv16=None):
    """(TFLOP/s of algorithmic flops, description) that bound the split-GQA kernel a plan names.
    The 32-key tile kernel forms each f32 product from bf16 matrix products: six for f32 K/V
    (both operands in three bf16 terms), three for bf16 K/V (q and p in three terms); the other
    kernels, and f16 K/V, use f32 MFMA."""
    from gqa_flash_attention_dg_amd import DG_KERNEL_TILE32
    if plan_kernel != DG_KERNEL_TILE32 or kv16 == "f16":
        return PEAK_F32_MFMA, "f32 MFMA"
    if kv16 == "bf16":
        return PEAK_BF16_MFMA / 3, "bf16 MFMA / 3 (three bf16 products per f32 product)"
    return PEAK_BF16_MFMA / 6, "bf16 MFMA / 6 (six bf16 products per f32 product)"


ARITH = {
    "f32 MFMA": "f32 (f32 MFMA)",
    "bf16 MFMA / 6 (six bf16 products per f32 product)":
        "f32 operands as three bf16 terms each; every product as six exact bf16 MFMA products "
        "summed in f32 (within 2^-23 |a||b| of the f32 product, typically 2^-29)",
    "bf16 MFMA / 3 (three bf16 products per f32 product)":
        "bf16 K/V; q and p as three bf16 terms; exact bf16 MFMA products summed in f32",
}


def combined_ceiling(parts):
    """Ceiling of a step made of launches [(flops, (peak, name))]: total flops over the sum of
    each launch's minimum time."""
    flops = sum(f for f, _ in parts)
    tmin = sum(f / pk for f, (pk, _) in parts)
    names = sorted(set(n for _, (_, n) in parts))
    return flops / tmin, " + ".join(names)
PEAK_HBM = 8000.0          # GB/s
CSRC = os.path.join(ROOT, "gqa_flash_attention_dg_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


def _code_tokens(text: str) -> str:
    """C/C++ source with comments removed and whitespace collapsed (string and character
    literals kept as written), so that an edit of comments alone keeps the hash."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


# The source file each measured kernel family is built from; its local includes are followed.
KERNEL_SOURCES = {"attn_split_gqa": "attn_split_gqa.hip", "attn_small": "attn_split_gqa.hip",
                  "relpos_flash": "relpos_flash.hip", "hbm_copy": None}


def _source_files(kernel):
    """Names under CSRC that kernel's code comes from: its file and, transitively, every
    `#include "..."` found there (all files when kernel is None)."""
    if kernel is None:
        return sorted(os.listdir(CSRC))
    todo, seen = [KERNEL_SOURCES[kernel]] if KERNEL_SOURCES[kernel] else [], set()
    while todo:
        name = todo.pop()
        if name in seen:
            continue
        seen.add(name)
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            todo += re.findall(r'^\s*#\s*include\s*"([^"]+)"', f.read(), flags=re.M)
    return sorted(seen)


def source_hash(kernel=None) -> str:
    """Hash of a kernel family's source code (comments and layout excluded; every kernel
    source when kernel is None): a profile's traffic record is used only while the hash of the
    kernel it measured matches the one it was taken on."""
    h = hashlib.sha256()
    for name in _source_files(kernel):
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            h.update(name.encode() + b"\0" + _code_tokens(f.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if taken on this source."""
    p = os.path.join(PROFILES, "traffic_%s_%s.json" % (kernel, workload))
    if not os.path.exists(p):
        return None
    with open(p) as f:
        rec = json.load(f)
    if rec.get("source_hash") != source_hash(kernel):
        return None
    return rec.get("hbm_bytes_per_launch")


def split_counts(c, norm_mode="in_attention"):
    """Algorithmic flops and bytes of one attention launch and of the headnorm work: q, k and v
    each read and written once, or with the q norm inside attention only k and v (q is read by
    the attention launch either way), or none with all three norms inside attention."""
    if c.causal:
        pairs = c.B * c.nh * (c.T * c.ctx + c.T * (c.T + 1) // 2)
    else:
        pairs = c.B * c.nh * c.T * (c.ctx + c.T)
    flops = 4 * c.hd * pairs
    f32 = 4
    q = c.B * c.T * c.nh * c.hd
    kv = c.B * c.T * c.nkv * c.hd
    cache = c.B * c.nkv * c.ctx * c.hd
    attn_bytes = f32 * (q + 2 * kv + 2 * cache + q)
    qn = 0 if norm_mode == "in_attention" else q
    norm_bytes = (f32 * 2 * (qn + 2 * kv)) if c.normed and norm_mode != "fused" else 0
    return flops, attn_bytes, norm_bytes


class SplitWork:
    dominant = "attn_split_gqa"

    def __init__(self, name, case, norm_mode="auto", kv16=None):
        import numpy as np
        import torch
        from gqa_flash_attention_dg_amd.canvas import CanvasBlock

        if kv16 and norm_mode in ("auto", "fused", "in_attention"):
            norm_mode = "one_launch"   # the 16-bit attention takes a normed q
        self.name, self.c, self.kv16 = name, case, kv16
        # ctx + T <= 8 runs the short-key-set kernel, longer key sets the tiled MFMA kernel
        self.dominant = "attn_small" if case.ctx + case.T <= 8 else "attn_split_gqa"
        d = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()
        c = case
        self.blk = CanvasBlock(c.B, c.T, c.ctx, c.nh, c.nkv, c.hd, d(c.kc), d(c.vc), d(c.wq),
                               d(c.wk), eps=c.eps, theta=c.theta, scale=c.scale,
                               causal=c.causal, rope_cache=c.rope_cache, normed=c.normed,
                               norm_mode=norm_mode, kv16=kv16)
        self.norm_mode = norm_mode = self.blk.norm_mode   # "auto" resolved by the block
        # Canvas inputs of every pre-staged denoising step (one set unless the case holds
        # several); step i of a run reads set i mod len(sets), against the fixed cache.
        draws = c.steps if c.steps else [{"q": c.q, "k": c.k, "v": c.v}]
        self.sets = [(d(st["q"]), d(st["k"]), d(st["v"])) for st in draws]
        self.q, self.k, self.v = self.sets[0]
        self.t = 0
        self.out = torch.empty((c.B, c.T, c.nh * c.hd), device="cuda")
        self.flops, self.attn_bytes, self.norm_bytes = split_counts(c, norm_mode)
        if kv16:  # K/V read as 16-bit values; the canvas twins are written by the one-launch
            # norm (2 bytes per element) or by a pack pass (4 read + 2 written)
            kvn = c.B * c.T * c.nkv * c.hd
            self.attn_bytes -= 2 * (2 * kvn + 2 * c.B * c.nkv * c.ctx * c.hd)
            fused = norm_mode == "one_launch" and c.normed
            self.norm_bytes += 2 * kvn * (2 if fused else 4 + 2)
        self.bound = "mfma" if self.flops / self.attn_bytes > 20 else "hbm"
        from gqa_flash_attention_dg_amd import DG_KV_BF16, DG_KV_F16, dg_attn_split_gqa_plan
        fmt = {None: 0, "f16": DG_KV_F16, "bf16": DG_KV_BF16}[kv16]
        plan = dg_attn_split_gqa_plan(c.B, c.T, c.ctx, c.nh, c.nkv, c.hd, int(c.causal), fmt)
        self.mfma_peak, self.mfma_peak_name = mfma_ceiling(plan.kernel, kv16)

    def config(self):
        c = self.c
        cfg = {"workload": c.name, "batch": c.B, "T": c.T, "ctx": c.ctx, "nh": c.nh,
               "nkv": c.nkv, "hd": c.hd, "scale": c.scale, "causal": bool(c.causal),
               "step": self.step_name()}
        if len(self.sets) > 1:
            cfg["staged_steps"] = len(self.sets)
        return cfg

    def step_name(self):
        if getattr(self, "kv16", None):
            if self.norm_mode == "one_launch" and getattr(self.c, "normed", True):
                return ("dg_qkv_headnorm_rope_kv16(q, k, v -> k16, v16) + "
                        "dg_attn_split_gqa_kv16 (%s K/V)" % self.kv16)
            return ("norms as --norm %s + dg_pack_kv16(k), dg_pack_kv16(v) + "
                    "dg_attn_split_gqa_kv16 (%s K/V)" % (self.norm_mode, self.kv16))
        if not getattr(self.c, "normed", True):
            return "dg_attn_split_gqa"
        names = {"fused": "dg_attn_split_gqa_qkvnorm (q, k, v norms inside attention)",
                 "one_launch": "dg_qkv_headnorm_rope(q, k, v) + dg_attn_split_gqa",
                 "in_attention": "dg_qkv_headnorm_rope(k, v) + dg_attn_split_gqa_qnorm",
                 "separate": "dg_headnorm_rope x3 (q, k, v) + dg_attn_split_gqa"}
        return " / ".join(names[m] for m in self.norm_mode.split("/"))

    def step(self, ev=None):
        self.q, self.k, self.v = self.sets[self.t % len(self.sets)]
        self.t += 1
        normed_q = self.c.normed and self.norm_mode == "in_attention"
        normed_all = self.c.normed and self.norm_mode == "fused"
        fused16 = self.kv16 and self.c.normed and self.norm_mode == "one_launch"
        if fused16:   # one launch: the norms and the 16-bit twins of k and v
            self.blk.norm_qkv_kv16(self.q, self.k, self.v)
        elif normed_all:
            pass      # every norm runs inside the attention launch
        elif self.c.normed:
            if self.norm_mode == "in_attention":
                self.blk.norm_qkv(None, self.k, self.v)
            elif self.norm_mode == "one_launch":
                self.blk.norm_qkv(self.q, self.k, self.v)
            else:
                self.blk.norm(self.q, self.k, self.v)
        if self.kv16 and not fused16:
            self.blk.pack_canvas(self.k, self.v)
        if ev:
            ev[0].record()
        if self.kv16:
            self.blk.attend_kv16(self.q, self.out)
        elif normed_all:
            self.blk.attend_qkvnorm(self.q, self.k, self.v, self.out)
        elif normed_q:
            self.blk.attend_qnorm(self.q, self.k, self.v, self.out)
        else:
            self.blk.attend(self.q, self.k, self.v, self.out)
        if ev:
            ev[1].record()

    def cpu_baseline(self, budget_s):
        """The oracle on the host: all three headnorms plus attention for a row sample."""
        import numpy as np
        import oracle
        sys.path.insert(0, os.path.join(ROOT, "tests"))
        from helpers import oracle_prepare, oracle_step

        c = self.c
        cs, kc = oracle_prepare(c)
        nrows = c.B * c.T
        per_row = self.flops / nrows
        probe = np.arange(0, nrows, max(1, nrows // 8), dtype=np.int64)[:8]
        t0 = time.perf_counter()
        oracle_step(c, c.q, c.k, c.v, cs, kc, rows=probe)
        dt = time.perf_counter() - t0
        n = int(min(nrows, max(len(probe), len(probe) * budget_s / max(dt, 1e-3))))
        rows = np.linspace(0, nrows - 1, n).astype(np.int64)
        rows = np.unique(rows)
        t0 = time.perf_counter()
        oracle_step(c, c.q, c.k, c.v, cs, kc, rows=rows)
        dt = time.perf_counter() - t0
        if self.bound == "hbm":
            value, unit = self.attn_bytes / nrows * rows.size / dt / 1e9, "GB/s"
        else:
            value, unit = per_row * rows.size / dt / 1e12, "TFLOP/s"
        return {"value": value, "unit": unit, "cores": oracle.threads(), "kind": "oracle",
                "sample": "%d of %d canvas rows (all %d heads) of one step, plus the q/k/v "
                          "headnorms of the whole step; %.2f s wall" % (rows.size, nrows, c.nh, dt)}


class LayerStackWork:
    """One canvas step through a sliding/global layer stack: per layer the k/v norm launch and
    the attention (with the q norm inside, by default).  The attention launches of all layers
    are timed together as the dominant kernel."""
    dominant = "attn_split_gqa"

    def __init__(self, name, case, norm_mode="auto"):
        import numpy as np
        import torch
        from gqa_flash_attention_dg_amd.canvas import CanvasStack

        self.name, self.c = name, case
        d = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()
        c = case
        self.stack = CanvasStack(c.B, c.T, c.nh, c.pos0, c.layers,
                                 [(d(p["kc"]), d(p["vc"])) for p in c.per_layer],
                                 [(d(p["wq"]), d(p["wk"])) for p in c.per_layer],
                                 theta_sliding=c.theta_sliding, theta_full=c.theta_full,
                                 eps=c.eps, scale=c.scale, norm_mode=norm_mode)
        from gqa_flash_attention_dg_amd import dg_attn_split_gqa_plan
        self.io = []
        self.flops = self.attn_bytes = self.norm_bytes = 0
        parts = []
        modes = [blk.norm_mode for blk in self.stack.blocks]   # "auto" resolved per layer
        self.norm_mode = modes[0] if len(set(modes)) == 1 else "/".join(modes)
        for l, p, norm_mode in zip(c.layers, c.per_layer, modes):
            v = torch.empty((c.B, c.T, l.nkv * l.hd), device="cuda") if l.k_eq_v else d(p["v"])
            out = torch.empty((c.B, c.T, c.nh * l.hd), device="cuda")
            self.io.append((d(p["q"]), d(p["k"]), v, out))
            q, kv = c.B * c.T * c.nh * l.hd, c.B * c.T * l.nkv * l.hd
            cache = c.B * l.nkv * l.ctx * l.hd
            lflops = 4 * l.hd * c.B * c.nh * c.T * (l.ctx + c.T)
            self.flops += lflops
            plan = dg_attn_split_gqa_plan(c.B, c.T, l.ctx, c.nh, l.nkv, l.hd, 0, 0)
            parts.append((lflops, mfma_ceiling(plan.kernel)))
            self.attn_bytes += 4 * (2 * q + 2 * kv + 2 * cache)
            qn = 0 if norm_mode == "in_attention" else q
            if norm_mode != "fused":
                self.norm_bytes += 4 * 2 * (qn + kv) + 4 * (kv if l.k_eq_v else 2 * kv)
        self.bound = "mfma"
        self.mfma_peak, self.mfma_peak_name = combined_ceiling(parts)

    def config(self):
        c = self.c
        return {"workload": c.name, "batch": c.B, "T": c.T, "nh": c.nh, "pos0": c.pos0,
                "layers": [{"type": "sliding" if l.sliding else "global", "hd": l.hd,
                            "nkv": l.nkv, "ctx": l.ctx, "k_eq_v": l.k_eq_v} for l in c.layers],
                "rope_base": {"sliding": c.theta_sliding, "global": c.theta_full},
                "step": "per layer: " + SplitWork.step_name(self)}

    def step(self, ev=None):
        blocks = self.stack.blocks
        for li, (q, k, v, out) in enumerate(self.io):
            blk = blocks[li]
            mode = blk.norm_mode
            if mode == "fused":
                pass
            elif mode == "in_attention":
                blk.norm_qkv(None, k, v)
            elif mode == "one_launch":
                blk.norm_qkv(q, k, v)
            else:
                blk.norm(q, k, v)
            if ev:
                ev[li][0].record()
            if mode == "fused":
                blk.attend_qkvnorm(q, k, v, out)
            elif mode == "in_attention":
                blk.attend_qnorm(q, k, v, out)
            else:
                blk.attend(q, k, v, out)
            if ev:
                ev[li][1].record()

    def cpu_baseline(self, budget_s):
        return None


class RelposWork:
    """Rel-pos flash attention over one grid (sam_relpos) or a batch of windows
    (sam_windowed), one relpos_flash_attn_windows call with a workspace: the 64 x 64 grid's
    workgroups and the windows' form their bias rows themselves, other grids go through a
    bias pass into the workspace."""
    dominant = "relpos_flash"

    def __init__(self, name, case):
        import numpy as np
        import torch
        import gqa_flash_attention_dg_amd as dg
        self.name, self.c = name, case
        self.nwin = getattr(case, "nwin", 1)
        d = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()
        self.qkv, self.rh, self.rw = d(case.qkv), d(case.rh), d(case.rw)
        n, W = case.gh * case.gw, case.heads * case.hd
        self.out = torch.empty((self.nwin, n, W), device="cuda")
        self.ws_bytes = dg.relpos_flash_attn_windows_workspace_size(
            self.nwin, case.gh, case.gw, case.heads, case.hd)
        self.ws = torch.empty((max(self.ws_bytes, 4) // 4,), device="cuda")
        attn = self.nwin * case.heads * n * n * 4 * case.hd
        bias = self.nwin * case.heads * n * 2 * case.hd * (case.gh + case.gw) if case.rh is not None else 0
        self.flops = attn + bias
        # q.k and p.v take six bf16 products each; the bias rows are f32 MFMA
        self.mfma_peak, self.mfma_peak_name = combined_ceiling(
            [(attn, (PEAK_BF16_MFMA / 6, "bf16 MFMA / 6 (six bf16 products per f32 product)"))] +
            ([(bias, (PEAK_F32_MFMA, "f32 MFMA"))] if bias else []))
        # every input read once, the output written once (the bias rows it keeps in its
        # workspace are the method's own intermediate, not counted)
        self.attn_bytes = 4 * (self.nwin * (n * 3 * W + n * W) +
                               (case.gh ** 2 + case.gw ** 2) * case.hd)
        self.norm_bytes = 0
        self.bound = "mfma"

    def config(self):
        c = self.c
        cfg = {"workload": c.name, "grid": [c.gh, c.gw], "heads": c.heads, "hd": c.hd,
               "scale": c.scale}
        if self.nwin > 1:
            cfg["windows"] = self.nwin
            cfg["step"] = "relpos_flash_attn_windows"
        else:
            cfg["step"] = "relpos_flash_attn"
        return cfg

    def _call(self, out):
        import gqa_flash_attention_dg_amd as dg
        c = self.c
        dg.relpos_flash_attn_windows(self.qkv, self.rh, self.rw, out, self.nwin, c.gh, c.gw,
                                     c.heads, c.hd, c.scale, self.ws, self.ws_bytes)

    def step(self, ev=None):
        if ev:
            ev[0].record()
        self._call(self.out)
        if ev:
            ev[1].record()

    def cpu_baseline(self, budget_s):
        import numpy as np
        import oracle
        c = self.c
        n = c.gh * c.gw
        qkv0 = c.qkv if self.nwin == 1 else c.qkv[0]
        probe = np.arange(0, n, n // 8 or 1, dtype=np.int64)[:8]
        t0 = time.perf_counter()
        oracle.relpos_attn(qkv0, c.rh, c.rw, c.gh, c.gw, c.heads, c.hd, c.scale, rows=probe)
        dt = time.perf_counter() - t0
        m = int(min(n, max(len(probe), len(probe) * budget_s / max(dt, 1e-3))))
        rows = np.unique(np.linspace(0, n - 1, m).astype(np.int64))
        t0 = time.perf_counter()
        oracle.relpos_attn(qkv0, c.rh, c.rw, c.gh, c.gw, c.heads, c.hd, c.scale, rows=rows)
        dt = time.perf_counter() - t0
        per_row = self.flops / (self.nwin * n)
        where = "" if self.nwin == 1 else " of window 0 (of %d)" % self.nwin
        return {"value": per_row * rows.size / dt / 1e12, "unit": "TFLOP/s",
                "cores": oracle.threads(), "kind": "oracle",
                "sample": "%d of %d query rows%s (all %d heads); %.2f s wall"
                          % (rows.size, n, where, c.heads, dt)}


class CopyWork:
    """Device-to-device copy of a 512 MiB buffer: calibrates the HBM byte counters and gives
    the achievable copy bandwidth.  Not part of the attention block."""
    dominant = "hbm_copy"

    def __init__(self, name, nbytes=512 << 20):
        import torch
        self.name = name
        self.src = torch.ones(nbytes // 4, device="cuda")
        self.dst = torch.empty_like(self.src)
        self.flops, self.attn_bytes, self.norm_bytes = 0, 2 * nbytes, 0
        self.bound = "hbm"

    def config(self):
        return {"workload": "hbm_copy_512MiB", "bytes_read": self.attn_bytes // 2,
                "bytes_written": self.attn_bytes // 2, "step": "torch copy_"}

    def step(self, ev=None):
        if ev:
            ev[0].record()
        self.dst.copy_(self.src)
        if ev:
            ev[1].record()

    def cpu_baseline(self, budget_s):
        return None


def make_work(name, norm_mode="auto", kv16=None):
    from gqa_flash_attention_dg_amd import synth
    if name == "long_cache":
        return SplitWork(name, synth.long_cache(), norm_mode, kv16)
    if name == "dg_canvas":
        return SplitWork(name, synth.dg_canvas_steps(48), norm_mode, kv16)
    if name == "tiny":
        return SplitWork(name, synth.tiny_canvas_step(), norm_mode)
    if name == "depformer":
        return SplitWork(name, synth.depformer_frames(), norm_mode)
    if name == "dg_layers":
        return LayerStackWork(name, synth.dg_layer_stack(), norm_mode)
    if name == "sam_relpos":
        return RelposWork(name, synth.sam_global())
    if name == "sam_windowed":
        return RelposWork(name, synth.sam_windowed())
    if name == "hbm_copy":
        return CopyWork(name)
    raise SystemExit("unknown workload %s" % name)


def host_cpu_model() -> str:
    """Model name of the host CPU (from /proc/cpuinfo), or what the platform reports."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def _stats(xs):
    xs = sorted(xs)
    n = len(xs)
    med = xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])
    return {"mean": sum(xs) / n, "median": med, "min": xs[0]}


def attach_graph(work, nsteps):
    """Replace work.step by replays of a HIP graph of `nsteps` consecutive canvas steps (split-GQA
    workloads); the events of a replay are split evenly over its steps."""
    from gqa_flash_attention_dg_amd.canvas import CanvasGraph
    sets = [work.sets[j % len(work.sets)] for j in range(nsteps)]
    cg = CanvasGraph(work.blk, [s[0] for s in sets], [s[1] for s in sets], [s[2] for s in sets],
                     work.out, steps=nsteps)
    work.graph = nsteps
    state = {"n": 0}

    def graph_step(ev=None):
        if state["n"] % nsteps == 0:
            if ev:
                ev[0].record()
            cg.replay()
            if ev:
                ev[1].record()
        elif ev:
            ev[0].record()
            ev[1].record()
        state["n"] += 1
    work.step = graph_step
    work.graph_state = state


def run(work, steps=None, warmup=None, cold=0):
    """Times `work` on the GPU.  W untimed warmup steps, then three passes of K steps:
    pass 1 times all K steps between two events (nothing queued between their launches) and
    gives the mean step time; pass 2 puts an event pair around each launch of the dominant
    call; pass 3 records one event at every step boundary, for the median and minimum step.
    With `cold` > 0, that many more steps each follow a read of a 512 MiB buffer that evicts
    the L2s and the MALL, and are timed alone."""
    import torch
    per = getattr(work, "graph", 0) or 1
    nprobe = 0
    if warmup is None or steps is None:
        # default counts from the wall time of a few probe steps (which count as warmup; the
        # first, which loads the code objects, is not timed); with a graph a probe is a replay
        nprobe = 4 * per if warmup is None else min(4 * per, warmup // per * per)
        est = None
        if nprobe >= 2 * per:
            for _ in range(per):
                work.step()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(nprobe - per):
                work.step()
            torch.cuda.synchronize()
            est = max((time.perf_counter() - t0) / (nprobe - per), 1e-6)
        else:
            nprobe = 0
        if warmup is None:
            warmup = max(nprobe, min(5000, int(0.5 / est)))
        if steps is None:
            steps = max(20, min(2000, int(0.25 / est))) if est else 20
            steps = -(-steps // per) * per
    # The GPU raises its clock over tens of milliseconds of load, so a few warmup steps leave
    # the timed ones on a ramping clock (long cache: 0.80 ms per step after 5 warmup steps,
    # 0.71 ms once settled).  Before the W warmup steps the step therefore runs untimed for at
    # least CLOCK_SETTLE_S of wall time; the count is reported as clock_settle_steps.
    settle = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < CLOCK_SETTLE_S:
        for _ in range(per):
            work.step()
        settle += per
        if settle % (16 * per) == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    for _ in range(warmup - nprobe):
        work.step()
    torch.cuda.synchronize()
    reset = lambda: getattr(work, "graph_state", {}).update(n=0)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    # pass 1
    reset()
    t_start, t_end = ev(), ev()
    torch.cuda.synchronize()
    t_start.record()
    for _ in range(steps):
        work.step()
    t_end.record()
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / steps
    # pass 2
    reset()
    nev = len(work.io) if isinstance(work, LayerStackWork) else 0
    evs = [[(ev(), ev()) for _ in range(nev)] if nev else (ev(), ev()) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        work.step(evs[i])
    torch.cuda.synchronize()
    if nev:
        kern_ms = [sum(a.elapsed_time(b) for a, b in st) for st in evs]
    else:
        kern_ms = [a.elapsed_time(b) for a, b in evs]
    # pass 3 (per-step boundaries; a graph replay is one boundary per replay)
    reset()
    marks = [ev() for _ in range(steps // per + 1)]
    torch.cuda.synchronize()
    marks[0].record()
    for i in range(steps):
        work.step()
        if (i + 1) % per == 0:
            marks[(i + 1) // per].record()
    torch.cuda.synchronize()
    step_ms = [marks[j].elapsed_time(marks[j + 1]) / per for j in range(len(marks) - 1)]
    r = {"steps": steps, "warmup": warmup, "ms_step": ms_step, "kern_ms": kern_ms,
         "step_ms": step_ms, "clock_settle_steps": settle}
    if cold > 0:
        flush = torch.ones((512 << 20) // 4, device="cuda")
        cold_ms = []
        for _ in range(cold):
            # Reading 512 MiB leaves other lines in the L2s and the MALL.  The step's launches
            # queue behind that read, so the events time the step alone, with no host gap.
            flush.sum()
            a, b = ev(), ev()
            a.record()
            for _ in range(per):
                work.step()
            b.record()
            torch.cuda.synchronize()
            cold_ms.append(a.elapsed_time(b) / per)
        del flush
        r["cold_ms"] = cold_ms
    return r


def rates(work, r):
    """value/unit of the step and the roofline of the dominant kernel from run()'s times."""
    kern_avg = sum(r["kern_ms"]) / len(r["kern_ms"])
    step_bytes = work.attn_bytes + work.norm_bytes
    if work.bound == "mfma":
        achieved = work.flops / (kern_avg * 1e-3) / 1e12
        peak = getattr(work, "mfma_peak", PEAK_F32_MFMA)
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                "frac": achieved / peak,
                "peak_of": getattr(work, "mfma_peak_name", "f32 MFMA")}
        per_ms = lambda ms: work.flops / (ms * 1e-3) / 1e12
        unit = "TFLOP/s"
    else:
        achieved = work.attn_bytes / (kern_avg * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM, "unit": "GB/s",
                "frac": achieved / PEAK_HBM}
        per_ms = lambda ms: step_bytes / (ms * 1e-3) / 1e9
        unit = "GB/s"
    roof["kernel"] = work.dominant
    roof["avg_launch_ms"] = kern_avg
    timing = {"step_ms": _stats(r["step_ms"]), "dominant_ms": _stats(r["kern_ms"])}
    timing["step_ms"]["mean_first_pass"] = r["ms_step"]
    if "cold_ms" in r:
        cold = _stats(r["cold_ms"])
        timing["cold"] = dict(cold, value_at_median=per_ms(cold["median"]), runs=len(r["cold_ms"]))
        timing["warm_value_at_median"] = per_ms(timing["step_ms"]["median"])
    return per_ms(r["ms_step"]), unit, roof, timing


ALSO_DEFAULT = "dg_canvas,sam_relpos,sam_windowed,depformer"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: about 0.25 s of steps, at least 20)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps before them (default: about 0.5 s of steps, at least 3, "
                         "so the timed steps run at the clock the GPU holds under sustained load)")
    ap.add_argument("--workload", default="long_cache",
                    choices=["long_cache", "dg_canvas", "dg_layers", "tiny", "depformer",
                             "sam_relpos", "sam_windowed", "hbm_copy"])
    ap.add_argument("--norm", default="auto",
                    choices=["auto", "fused", "in_attention", "one_launch", "separate"],
                    help="auto (default): fused when the attention splits its key range across "
                         "workgroups, else in_attention; "
                         "fused: q, k and v norms inside the attention launch; "
                         "in_attention: k/v norms in one launch + q norm inside attention; "
                         "one_launch: q, k, v norms in one launch; separate: the page's three "
                         "headnorm dispatches")
    ap.add_argument("--graph", type=int, default=0, metavar="STEPS",
                    help="split-GQA workloads: capture STEPS consecutive steps as one HIP graph "
                         "and replay it (timed per step; the dominant-kernel events then cover "
                         "the whole replay)")
    ap.add_argument("--kv16", default=None, choices=["f16", "bf16"],
                    help="long_cache / dg_canvas: keys and values stored in 16 bits, widened to "
                         "f32 inside attention")
    ap.add_argument("--cold", type=int, default=10,
                    help="extra steps of the main workload timed one at a time after the L2s "
                         "and the MALL are evicted (0 = skip)")
    ap.add_argument("--also", default=ALSO_DEFAULT,
                    help="comma-separated workloads measured first, in the same run, with "
                         "default step counts and reported under 'also' ('' = none)")
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of oracle wall time for the CPU baseline (0 = skip)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import gqa_flash_attention_dg_amd as dg
    if not os.path.exists(dg.LIB_PATH):
        from gqa_flash_attention_dg_amd import build
        build.build()
    dg.lib()
    torch.cuda.set_device(0)

    # The main workload's inputs are staged first, so that no host-side input generation
    # separates the other configurations' runs from its timed steps.
    work = make_work(args.workload, norm_mode=args.norm, kv16=args.kv16)
    # The other configurations next, each with its own time-based warmup and step counts.
    also = {}
    for name in [n for n in args.also.split(",") if n and n != args.workload]:
        w = make_work(name)
        r = run(w)
        value, unit, roof, timing = rates(w, r)
        also[name] = {"value": value, "unit": unit, "ms_per_step": r["ms_step"],
                      "steps": r["steps"], "warmup": r["warmup"], "step": w.config()["step"],
                      "workload": w.config()["workload"],
                      "roofline": {k: roof[k] for k in ("kernel", "bound", "achieved", "unit",
                                                        "peak", "frac", "avg_launch_ms")
                                   if k in roof},
                      "timing": timing}
        del w, r
        torch.cuda.empty_cache()

    if args.graph:
        if not isinstance(work, SplitWork):
            raise SystemExit("--graph applies to the split-GQA workloads")
        if args.steps is not None and args.steps % args.graph:
            raise SystemExit("--steps must be a multiple of --graph")
        attach_graph(work, args.graph)
    r = run(work, args.steps, args.warmup, cold=args.cold)
    value, unit, roof, timing = rates(work, r)
    roof["traffic"] = measured_traffic(work.dominant, work.name + (
        "_kv16" + args.kv16 if getattr(args, "kv16", None) else ""))

    cpu = None
    if args.cpu_budget > 0:
        cpu = work.cpu_baseline(args.cpu_budget)
        if cpu is not None:
            cpu["cpu_model"] = host_cpu_model()

    step_bytes = work.attn_bytes + work.norm_bytes
    rec = {
        "metric": METRIC, "value": value, "unit": unit, "n_gpus": 1, "steps": r["steps"],
        "warmup": r["warmup"], "clock_settle_steps": r["clock_settle_steps"],
        "ms_per_step": r["ms_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "arith": "; ".join(ARITH.get(n, n) for n in
                           getattr(work, "mfma_peak_name", "f32 MFMA").split(" + ")),
        "config": dict(work.config(), **({"hip_graph_steps": work.graph} if getattr(work, "graph", 0) else {})),
        "step_flops": work.flops, "step_hbm_bytes_algorithmic": step_bytes,
        "step_hbm_gbps_algorithmic": step_bytes / (r["ms_step"] * 1e-3) / 1e9,
        "roofline": roof, "timing": timing, "cpu_baseline": cpu, "also": also,
        "source_hash": source_hash(work.dominant),
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
