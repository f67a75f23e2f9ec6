"""One canvas step of the attention block, as a sequence of C-ABI calls on the GPU.

Follows the per-layer dispatch order of `canvas_forward` in inferencelayer 0.2.3,
src/diffusion_gemma_gpu.rs: the per-token rope table for positions seq_len + t is built once
per forward, then each step runs the headnorm on q (weighted + rope), on k (weighted + rope),
the weightless, un-roped norm on v, and the split-GQA attention over [cache | canvas].

Set-up work (rope tables, roping a cache that is stored un-roped) happens once per canvas
block in the constructor; `step` is the per-denoising-step hot path.  Three ways to run the
norms of a step (`norm_mode`):
  "one_launch"    q, k and v normalised in place by one launch, then plain attention;
  "in_attention"  k and v normalised by one launch, the q norm and rope applied in registers
                  by the attention kernel as it loads q (q is left un-normalised in memory);
  "separate"      the page's three in-place headnorm dispatches, then plain attention.  This module only orders
calls into libdgattn.so; it does no arithmetic of its own.
"""
from __future__ import annotations

import torch

from . import (DG_NORM_ROPE, DG_NORM_SKIP, DG_NORM_WEIGHTED, dg_attn_split_gqa,
               dg_attn_split_gqa_qnorm, dg_attn_split_gqa_workspace_size, dg_headnorm_rope,
               dg_qkv_headnorm_rope, dg_rope_table)


class CanvasBlock:
    """Device-resident state of one canvas block: cache, norm weights, rope table, workspace.

    kc, vc: [B, nkv, ctx, hd] float32 GPU tensors (None when ctx == 0); wq, wk: [hd] or None.
    rope_cache: the cache keys are stored un-roped and get roped at positions 0..ctx-1 here
    (in place on kc).  normed: normalise q, k and v in each step, as `norm_mode` says.
    """

    def __init__(self, B, T, ctx, nh, nkv, hd, kc=None, vc=None, wq=None, wk=None, *,
                 eps=1e-6, theta=10000.0, scale=1.0, causal=False, rope_cache=False,
                 normed=True, norm_mode="one_launch", use_workspace=True, device="cuda"):
        if norm_mode not in ("one_launch", "in_attention", "separate"):
            raise ValueError("unknown norm_mode %r" % (norm_mode,))
        self.B, self.T, self.ctx, self.nh, self.nkv, self.hd = B, T, ctx, nh, nkv, hd
        self.kc, self.vc, self.wq, self.wk = kc, vc, wq, wk
        self.eps, self.scale, self.causal, self.normed = eps, scale, int(causal), normed
        self.norm_mode = norm_mode
        self.cs = torch.empty((T, 2 * hd), dtype=torch.float32, device=device)
        if normed:
            dg_rope_table(self.cs, ctx, T, hd, theta)
        if rope_cache and ctx > 0:
            cs_cache = torch.empty((ctx, 2 * hd), dtype=torch.float32, device=device)
            dg_rope_table(cs_cache, 0, ctx, hd, theta)
            dg_headnorm_rope(kc, None, cs_cache, B * nkv, ctx, 1, hd,
                             DG_NORM_ROPE | DG_NORM_SKIP, 0.0)
        self.ws_bytes = dg_attn_split_gqa_workspace_size(B, T, ctx, nh, nkv, hd) \
            if use_workspace else 0
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device) \
            if self.ws_bytes > 0 else None

    def norm(self, q, k, v):
        """The three per-step headnorm calls, in place on q, k and v."""
        B, T, nh, nkv, hd = self.B, self.T, self.nh, self.nkv, self.hd
        flags = DG_NORM_WEIGHTED | DG_NORM_ROPE
        dg_headnorm_rope(q, self.wq, self.cs, B, T, nh, hd, flags, self.eps)
        dg_headnorm_rope(k, self.wk, self.cs, B, T, nkv, hd, flags, self.eps)
        dg_headnorm_rope(v, None, None, B, T, nkv, hd, 0, self.eps)

    def norm_qkv(self, q, k, v):
        """q, k (weighted + rope) and v (weightless) norms in one launch, in place; q may be
        None to leave it for the attention kernel."""
        dg_qkv_headnorm_rope(q, self.wq, k, self.wk, v, self.cs, self.B, self.T, self.nh,
                             self.nkv, self.hd, DG_NORM_WEIGHTED | DG_NORM_ROPE, self.eps)

    def attend_qnorm(self, q, k, v, out):
        """Attention on the raw q, normalised and roped inside the kernel (q is not written)."""
        dg_attn_split_gqa_qnorm(q, self.wq, self.cs, self.kc, self.vc, k, v, out, self.B,
                                self.T, self.ctx, self.nh, self.nkv, self.hd,
                                DG_NORM_WEIGHTED | DG_NORM_ROPE, self.eps, self.scale,
                                self.causal, self.ws, self.ws_bytes)

    def attend(self, q, k, v, out):
        dg_attn_split_gqa(q, self.kc, self.vc, k, v, out, self.B, self.T, self.ctx, self.nh,
                          self.nkv, self.hd, self.scale, self.causal, self.ws, self.ws_bytes)

    def step(self, q, k, v, out):
        """One canvas step: norms (when enabled), then attention into `out`."""
        if self.normed and self.norm_mode == "in_attention":
            self.norm_qkv(None, k, v)
            self.attend_qnorm(q, k, v, out)
            return
        if self.normed and self.norm_mode == "one_launch":
            self.norm_qkv(q, k, v)
        elif self.normed:
            self.norm(q, k, v)
        self.attend(q, k, v, out)
