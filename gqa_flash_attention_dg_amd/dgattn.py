"""Tensor-level calls of the attention block: the hot path's operations with their extents
taken from the tensors' shapes.

    from gqa_flash_attention_dg_amd import dgattn
    dgattn.headnorm_rope_(x, w, cs, heads, eps, rope=True)      # in place, like the page's kernel
    out = dgattn.attn_split_gqa(q, kc, vc, k, v, out=None, scale=1.0, causal=False)
    out = dgattn.relpos_flash_attn(qkv, rh, rw, heads, scale)
    out = dgattn.relpos_flash_attn_windows(qkv, rh, rw, heads, scale)

They follow kernels DG_HEADNORM_ROPE and DG_ATTN of "inferencelayer 0.2.3 -- src/diffusion_gemma_gpu.rs"
and the rel-pos flash attention of "inferencelayer 0.2.8 -- src/deepencoder_gpu.rs"
(`sam_attn_buf`).  Each reads the extents from the shapes, allocates the output and any
split-KV or bias-row workspace with torch on the tensors' device, and calls the C entry point
of the same operation in libdgattn.so through this package's binding, on torch's current
stream.  No arithmetic happens here: everything runs in the library's HIP kernels, and a
missing library raises.
"""
from __future__ import annotations

import torch

from . import (DG_NORM_ROPE, DG_NORM_WEIGHTED, dg_attn_split_gqa,
               dg_attn_split_gqa_workspace_size, dg_headnorm_rope,
               relpos_flash_attn_windows_workspace_size, relpos_flash_attn_workspace_size,
               relpos_flash_attn_ws)
from . import relpos_flash_attn_windows as _relpos_windows   # the C call of the same name


def _scratch(nbytes: int, device):
    return torch.empty(nbytes, dtype=torch.uint8, device=device) if nbytes else None


def headnorm_rope_(x, w, cs, heads: int, eps: float, rope: bool = True):
    """Per-(token, head) RMSNorm of x [..., T, heads*hd] in place, times w [hd] when w is given,
    then the NeoX rope from cs [T, 2*hd] when `rope` (dg_headnorm_rope).  Returns x."""
    if x.dim() < 2:
        raise ValueError("x must be [..., T, heads*hd]")
    T, width = x.shape[-2], x.shape[-1]
    if heads <= 0 or width % heads:
        raise ValueError("the last dim of x (%d) is not heads (%d) times hd" % (width, heads))
    hd = width // heads
    batch = x.numel() // (T * width) if T * width else 0
    flags = (DG_NORM_WEIGHTED if w is not None else 0) | (DG_NORM_ROPE if rope else 0)
    dg_headnorm_rope(x, w, cs if rope else None, batch, T, heads, hd, flags, eps)
    return x


def attn_split_gqa(q, kc, vc, k, v, out=None, scale: float = 1.0, causal: bool = False):
    """GQA attention over [cache | canvas] (dg_attn_split_gqa).  q [B, T, nh, hd] or
    [B, T, nh*hd]; kc, vc [B, nkv, ctx, hd] (None for an empty cache, then q must be 4-D to give
    hd); k, v [B, T, nkv*hd].  Returns out, shaped like q (allocated when not given)."""
    if kc is not None:
        B, nkv, ctx, hd = kc.shape
    else:
        if q.dim() != 4:
            raise ValueError("without a cache, q must be [B, T, nh, hd] to give hd")
        B, hd, ctx = q.shape[0], q.shape[3], 0
        nkv = k.shape[-1] // hd
    T = q.shape[1]
    nh = (q.shape[2] * q.shape[3] if q.dim() == 4 else q.shape[2]) // hd
    if out is None:
        out = torch.empty_like(q)
    need = dg_attn_split_gqa_workspace_size(B, T, ctx, nh, nkv, hd)
    dg_attn_split_gqa(q, kc, vc, k, v, out, B, T, ctx, nh, nkv, hd, scale, int(causal),
                      _scratch(need, q.device), need)
    return out


def _grid(rh, rw, qkv, heads: int, grid):
    if rh is not None and rw is not None:
        return rh.shape[0], rw.shape[0], rh.shape[2]
    if grid is None:
        raise ValueError("without tables the grid (gh, gw) must be given")
    return grid[0], grid[1], qkv.shape[-1] // (3 * heads)


def relpos_flash_attn(qkv, rh, rw, heads: int, scale: float, grid=None):
    """Vision attention with the decomposed rel-pos bias over one grid.  qkv [gh*gw,
    3*heads*hd]; rh [gh, gh, hd] and rw [gw, gw, hd] give the grid (both None: no bias, and
    `grid` = (gh, gw) must be passed).  The bias rows go to a torch-allocated workspace
    (relpos_flash_attn_ws).  Returns out [gh*gw, heads*hd]."""
    gh, gw, hd = _grid(rh, rw, qkv, heads, grid)
    out = torch.empty((gh * gw, heads * hd), dtype=qkv.dtype, device=qkv.device)
    need = relpos_flash_attn_workspace_size(gh, gw, heads, hd) if rh is not None else 0
    relpos_flash_attn_ws(qkv, rh, rw, out, gh, gw, heads, hd, scale, _scratch(need, qkv.device),
                         need)
    return out


def relpos_flash_attn_windows(qkv, rh, rw, heads: int, scale: float, grid=None):
    """relpos_flash_attn over a batch of windows: qkv [nwin, gh*gw, 3*heads*hd], tables shared.
    Returns out [nwin, gh*gw, heads*hd]."""
    gh, gw, hd = _grid(rh, rw, qkv, heads, grid)
    nwin = qkv.shape[0]
    out = torch.empty((nwin, gh * gw, heads * hd), dtype=qkv.dtype, device=qkv.device)
    need = (relpos_flash_attn_windows_workspace_size(nwin, gh, gw, heads, hd)
            if rh is not None else 0)
    _relpos_windows(qkv, rh, rw, out, nwin, gh, gw, heads, hd, scale, _scratch(need, qkv.device),
                    need)
    return out
