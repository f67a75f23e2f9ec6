"""Canvas steps of the attention block, as sequences of C-ABI calls on the GPU.

Follows the per-layer dispatch order of `canvas_forward` in inferencelayer 0.2.3,
src/diffusion_gemma_gpu.rs: the per-token rope tables for positions seq_len + t are built once
per forward, one per layer type (sliding layers: head_dim and the sliding rope base; global
layers: head_dim_global and the full rope base); then each layer's step normalises q (weighted
+ rope) and k (weighted + rope), runs the weightless, un-roped norm on v, and the split-GQA
attention over that layer's [cache | canvas].  A k_eq_v layer has no v projection: its v is
the raw k projection, normalised without weight or rope.

Set-up work (rope tables, roping a cache that is stored un-roped) happens once per canvas
block in the constructor; `step` is the per-denoising-step hot path.  Four ways to run the
norms of a step (`norm_mode`), plus "auto" (the default), which takes "fused" when each
attention workgroup meets at most AUTO_FUSED_KEYS canvas keys (a split key range, or a short
canvas: normalising them in place costs less than a launch) and "in_attention" otherwise (a
workgroup that walks many canvas tiles would norm each itself):
  "fused"         all three norms inside the attention launch: q as it is staged, the canvas
                  k and v rows as their tiles land in on-chip memory (q, k and v are not
                  written; a k_eq_v layer's v buffer is neither read nor written);
  "in_attention"  k and v normalised by one launch, the q norm and rope applied by the
                  attention kernel as it stages q (q is left un-normalised in memory);
  "one_launch"    q, k and v normalised in place by one launch, then plain attention;
  "separate"      the page's three in-place headnorm dispatches, then plain attention.
This module only orders calls into libdgattn.so; it does no arithmetic of its own.
"""
from __future__ import annotations

import torch

from . import (DG_KV_BF16, DG_KV_F16, DG_NORM_ROPE, DG_NORM_SKIP,
               DG_NORM_V_FROM_K, DG_NORM_WEIGHTED, dg_attn_split_gqa, dg_attn_split_gqa_kv16,
               dg_attn_split_gqa_plan,
               dg_attn_split_gqa_qkvnorm, dg_attn_split_gqa_qnorm,
               dg_attn_split_gqa_workspace_size, dg_headnorm_rope,
               dg_pack_kv16, dg_qkv_headnorm_rope, dg_qkv_headnorm_rope_kv16, dg_rope_table)

KV_FORMATS = {"f16": DG_KV_F16, "bf16": DG_KV_BF16}

NORM_MODES = ("auto", "fused", "in_attention", "one_launch", "separate")
# Canvas keys per attention workgroup up to which "auto" norms k and v inside the kernel:
# measured faster at one or two 32-key tiles (a split key range, or a short canvas); slower at
# 8 tiles of 32.
AUTO_FUSED_KEYS = 64


def auto_norm_mode(B, T, ctx, nh, nkv, hd, causal=False, cus=0, split=True):
    """The norm mode "auto" stands for: "fused" when one attention workgroup of the call's
    launch plan (dg_attn_split_gqa_plan; cus = 0: the current device) meets at most
    AUTO_FUSED_KEYS canvas keys, "in_attention" otherwise.  Splits deal the canvas tiles round
    robin, so a workgroup meets about T / nsplit of them; causal calls do not split, nor do
    calls without a workspace (split=False)."""
    if B * T * nh == 0:
        return "fused"
    p = dg_attn_split_gqa_plan(B, T, ctx, nh, nkv, hd, int(causal), 0, cus)
    tile = 32
    nsplit = p.nsplit if split else 1
    tiles = (T + tile - 1) // tile                   # canvas tiles
    per_wg = (tiles + nsplit - 1) // nsplit          # ... met by one workgroup
    return "fused" if per_wg * tile <= AUTO_FUSED_KEYS else "in_attention"


def rope_table(pos0, T, hd, theta, device="cuda"):
    """[T, 2*hd] cos|sin table for positions pos0..pos0+T-1 (one launch)."""
    cs = torch.empty((T, 2 * hd), dtype=torch.float32, device=device)
    dg_rope_table(cs, pos0, T, hd, theta)
    return cs


class CanvasBlock:
    """Device-resident state of one layer's canvas attention: cache, norm weights, rope table,
    workspace.

    kc, vc: [B, nkv, ctx, hd] float32 GPU tensors (None when ctx == 0); wq, wk: [hd] or None.
    pos0: absolute position of canvas row 0 (default ctx: the cache holds positions before it).
    cs: a [T, 2*hd] rope table to share (e.g. one per layer type); built here when None.
    rope_cache: the cache keys are stored un-roped and get roped here, in place on kc, at the
    ctx positions just before pos0.  normed: normalise q, k and v in each step, as `norm_mode`
    says.  k_eq_v: the layer has no v projection; each step's v buffer is written with the
    weightless norm of the raw k (its input contents are ignored).
    workspace: an optional GPU tensor to use as the split-KV scratch (e.g. one shared by the
    layers of a stack, which run one after another on one stream); one is allocated otherwise.
    kv16: None (f32 K/V) or "f16" / "bf16": the cache is packed once into 16-bit twins here, each
    step's one-launch norm also writes 16-bit twins of its normalised canvas k and v (with
    "separate" norms a pack pass writes them), and the attention reads the 16-bit twins
    (dg_attn_split_gqa_kv16; the q norm then runs in the norm launch, not inside attention).
    """

    def __init__(self, B, T, ctx, nh, nkv, hd, kc=None, vc=None, wq=None, wk=None, *,
                 eps=1e-6, theta=10000.0, scale=1.0, causal=False, rope_cache=False,
                 normed=True, norm_mode="auto", use_workspace=True, pos0=None, cs=None,
                 k_eq_v=False, kv16=None, workspace=None, device="cuda"):
        if kv16 is not None and kv16 not in KV_FORMATS:
            raise ValueError("kv16 must be None, 'f16' or 'bf16'")
        if kv16 is not None and norm_mode in ("auto", "fused", "in_attention"):
            norm_mode = "one_launch"
        if norm_mode not in NORM_MODES:
            raise ValueError("unknown norm_mode %r" % (norm_mode,))
        if k_eq_v and not normed:
            raise ValueError("k_eq_v needs the norms (v is derived from the raw k)")
        self.B, self.T, self.ctx, self.nh, self.nkv, self.hd = B, T, ctx, nh, nkv, hd
        self.kc, self.vc, self.wq, self.wk = kc, vc, wq, wk
        self.eps, self.scale, self.causal, self.normed = eps, scale, int(causal), normed
        self.norm_mode, self.k_eq_v = norm_mode, k_eq_v
        pos0 = ctx if pos0 is None else pos0
        if cs is not None:
            if tuple(cs.shape) != (T, 2 * hd):
                raise ValueError("cs must be [T, 2*hd] = [%d, %d]" % (T, 2 * hd))
            self.cs = cs
        else:
            self.cs = rope_table(pos0, T, hd, theta, device) if normed else None
        if rope_cache and ctx > 0:
            if pos0 < ctx:
                raise ValueError("rope_cache needs pos0 >= ctx")
            cs_cache = rope_table(pos0 - ctx, ctx, hd, theta, device)
            dg_headnorm_rope(kc, None, cs_cache, B * nkv, ctx, 1, hd,
                             DG_NORM_ROPE | DG_NORM_SKIP, 0.0)
        self.kv16 = KV_FORMATS[kv16] if kv16 else 0
        if self.kv16:
            half = lambda n: torch.empty(n, dtype=torch.int16, device=device)
            nc, nk = B * nkv * ctx * hd, B * T * nkv * hd
            self.kc16, self.vc16 = (half(nc), half(nc)) if ctx > 0 else (None, None)
            if ctx > 0:
                dg_pack_kv16(kc, self.kc16, nc, self.kv16)
                dg_pack_kv16(vc, self.vc16, nc, self.kv16)
            self.k16, self.v16 = half(nk), half(nk)
        self.ws_bytes = dg_attn_split_gqa_workspace_size(B, T, ctx, nh, nkv, hd) \
            if use_workspace else 0
        if self.ws_bytes > 0 and workspace is not None:
            if workspace.numel() * workspace.element_size() < self.ws_bytes:
                raise ValueError("workspace holds fewer than the %d bytes needed" % self.ws_bytes)
            self.ws = workspace
        else:
            self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device) \
                if self.ws_bytes > 0 else None
        if self.norm_mode == "auto":
            self.norm_mode = auto_norm_mode(B, T, ctx, nh, nkv, hd, causal,
                                            split=self.ws_bytes > 0)

    def norm(self, q, k, v):
        """The page's per-step headnorm calls, in place on q, k and v (for a k_eq_v layer the
        k and v norms share one launch, since v is derived from the raw k)."""
        B, T, nh, nkv, hd = self.B, self.T, self.nh, self.nkv, self.hd
        flags = DG_NORM_WEIGHTED | DG_NORM_ROPE
        dg_headnorm_rope(q, self.wq, self.cs, B, T, nh, hd, flags, self.eps)
        if self.k_eq_v:
            self.norm_qkv(None, k, v)
            return
        dg_headnorm_rope(k, self.wk, self.cs, B, T, nkv, hd, flags, self.eps)
        dg_headnorm_rope(v, None, None, B, T, nkv, hd, 0, self.eps)

    def norm_qkv(self, q, k, v):
        """q, k (weighted + rope) and v (weightless) norms in one launch, in place; q may be
        None to leave it for the attention kernel."""
        flags = DG_NORM_WEIGHTED | DG_NORM_ROPE | (DG_NORM_V_FROM_K if self.k_eq_v else 0)
        dg_qkv_headnorm_rope(q, self.wq, k, self.wk, v, self.cs, self.B, self.T, self.nh,
                             self.nkv, self.hd, flags, self.eps)

    def attend_qnorm(self, q, k, v, out):
        """Attention on the raw q, normalised and roped inside the kernel (q is not written)."""
        dg_attn_split_gqa_qnorm(q, self.wq, self.cs, self.kc, self.vc, k, v, out, self.B,
                                self.T, self.ctx, self.nh, self.nkv, self.hd,
                                DG_NORM_WEIGHTED | DG_NORM_ROPE, self.eps, self.scale,
                                self.causal, self.ws, self.ws_bytes)

    def attend_qkvnorm(self, q, k, v, out):
        """Attention on the raw q, k and v, all three normalised inside the kernel (none of them
        is written); a k_eq_v layer's v is the raw k."""
        dg_attn_split_gqa_qkvnorm(q, self.wq, k, self.wk, k if self.k_eq_v else v, self.cs,
                                  self.kc, self.vc, out, self.B, self.T, self.ctx, self.nh,
                                  self.nkv, self.hd, DG_NORM_WEIGHTED | DG_NORM_ROPE, self.eps,
                                  self.scale, self.causal, self.ws, self.ws_bytes)

    def norm_qkv_kv16(self, q, k, v):
        """norm_qkv that also writes the 16-bit twins of the normalised k and v (kv16 blocks)."""
        flags = DG_NORM_WEIGHTED | DG_NORM_ROPE | (DG_NORM_V_FROM_K if self.k_eq_v else 0)
        dg_qkv_headnorm_rope_kv16(q, self.wq, k, self.wk, v, self.cs, self.k16, self.v16, self.B,
                                  self.T, self.nh, self.nkv, self.hd, flags, self.eps, self.kv16)

    def pack_canvas(self, k, v):
        """16-bit twins of this step's normed canvas k and v (kv16 blocks)."""
        nk = self.B * self.T * self.nkv * self.hd
        dg_pack_kv16(k, self.k16, nk, self.kv16)
        dg_pack_kv16(v, self.v16, nk, self.kv16)

    def attend_kv16(self, q, out):
        dg_attn_split_gqa_kv16(q, self.kc16, self.vc16, self.k16, self.v16, out, self.B, self.T,
                               self.ctx, self.nh, self.nkv, self.hd, self.scale, self.causal,
                               self.kv16, self.ws, self.ws_bytes)

    def attend(self, q, k, v, out):
        if self.kv16:
            self.pack_canvas(k, v)
            self.attend_kv16(q, out)
            return
        dg_attn_split_gqa(q, self.kc, self.vc, k, v, out, self.B, self.T, self.ctx, self.nh,
                          self.nkv, self.hd, self.scale, self.causal, self.ws, self.ws_bytes)

    def step(self, q, k, v, out):
        """One canvas step: norms (when enabled), then attention into `out`.

        What the step leaves in the caller's buffers depends on the norm mode (a normed block):
          "fused"         q, k and v are read only and keep their raw contents; a k_eq_v
                          layer's v buffer is neither read nor written;
          "in_attention"  k holds the normed, weighted, roped k and v the weightless norm of v
                          (k_eq_v: of the raw k); q keeps its raw contents;
          "one_launch", "separate"  as "in_attention", and q holds the normed, weighted, roped q.
        `out` is written in every mode."""
        if self.normed and self.norm_mode == "fused":
            self.attend_qkvnorm(q, k, v, out)
            return
        if self.normed and self.norm_mode == "in_attention":
            self.norm_qkv(None, k, v)
            self.attend_qnorm(q, k, v, out)
            return
        if self.normed and self.norm_mode == "one_launch" and self.kv16:
            self.norm_qkv_kv16(q, k, v)
            self.attend_kv16(q, out)
            return
        if self.normed and self.norm_mode == "one_launch":
            self.norm_qkv(q, k, v)
        elif self.normed:
            self.norm(q, k, v)
        self.attend(q, k, v, out)


class CanvasGraph:
    """`steps` canvas steps of a CanvasBlock captured as one HIP graph (through
    torch.cuda.CUDAGraph): the steps' launches (norms, attention, split-KV combine; no memset or
    host work) replay with one submission.  The graph is bound to the tensors given at capture:
    q, k and v are either single tensors, used by every step, or lists of `steps` tensors, one
    set per step (e.g. pre-staged denoising steps); a caller refreshes their contents in place
    between replays."""

    def __init__(self, blk, q, k, v, out, warmup=2, steps=1):
        per = lambda x: list(x) if isinstance(x, (list, tuple)) else [x] * steps
        qs, ks, vs = per(q), per(k), per(v)
        if not len(qs) == len(ks) == len(vs) == steps:
            raise ValueError("q, k and v lists must hold one tensor per step")
        self.blk, self.io, self.steps = blk, (qs, ks, vs, out), steps
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):      # launch once outside capture (loads the code objects)
            for _ in range(warmup):
                blk.step(qs[0], ks[0], vs[0], out)
        torch.cuda.current_stream().wait_stream(side)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            for i in range(steps):   # `steps` consecutive steps, step i on set i
                blk.step(qs[i], ks[i], vs[i], out)

    def replay(self):
        self.graph.replay()


class CanvasStack:
    """The attention blocks of a stack of decoder layers over one canvas.

    Each layer has its own type (sliding or global), head dim, kv heads, cache and k_eq_v
    flag (`layers`: objects with fields sliding, hd, nkv, ctx, k_eq_v).  Layers of one type
    share one rope table, built once for canvas positions pos0..pos0+T-1 with that type's
    head dim and rope base, as `canvas_forward` builds `cs_sliding` and `cs_full`.
    caches[i] = (kc, vc) and weights[i] = (wq, wk) are layer i's GPU tensors.
    """

    def __init__(self, B, T, nh, pos0, layers, caches, weights, *, theta_sliding, theta_full,
                 eps=1e-6, scale=1.0, norm_mode="auto", use_workspace=True,
                 device="cuda"):
        self.layers = list(layers)
        tables = {}
        for l in self.layers:
            key = (l.sliding, l.hd)
            if key not in tables:
                theta = theta_sliding if l.sliding else theta_full
                tables[key] = rope_table(pos0, T, l.hd, theta, device)
        for sliding in (True, False):
            if len({l.hd for l in self.layers if l.sliding == sliding}) > 1:
                raise ValueError("all layers of one type share one head dim (one rope table)")
        self.tables = tables
        # Layers of one shape share a split-KV scratch (they run in order on one stream): the
        # partials then land in the lines the last such layer's combine read on the same XCD.
        self.ws = {}
        if use_workspace:
            for l in self.layers:
                key = (l.ctx, l.nkv, l.hd)
                need = dg_attn_split_gqa_workspace_size(B, T, l.ctx, nh, l.nkv, l.hd)
                if key not in self.ws and need > 0:
                    self.ws[key] = torch.empty(need, dtype=torch.uint8, device=device)
        self.blocks = []
        for l, (kc, vc), (wq, wk) in zip(self.layers, caches, weights):
            self.blocks.append(CanvasBlock(
                B, T, l.ctx, nh, l.nkv, l.hd, kc, vc, wq, wk, eps=eps, scale=scale,
                norm_mode=norm_mode, use_workspace=use_workspace, pos0=pos0,
                cs=tables[(l.sliding, l.hd)], k_eq_v=l.k_eq_v,
                workspace=self.ws.get((l.ctx, l.nkv, l.hd)), device=device))

    def step(self, li, q, k, v, out):
        """Layer li's attention for this canvas step (q, k, v are its projections; a k_eq_v
        layer ignores v's contents).  Which of q, k and v are left normed depends on the layer's
        norm mode, as CanvasBlock.step says; with "fused" (what "auto" picks at the
        DiffusionGemma-like shapes) none of them is written, and a k_eq_v layer's v neither."""
        self.blocks[li].step(q, k, v, out)
