"""Seeded synthetic inputs for the attention block.

This module only draws random numbers: it holds none of the method's arithmetic (no norm, no
rope, no attention).  Both the HIP path and the CPU oracle consume the same host arrays made
here, so a parity comparison sees identical input bits.

Every workload draws from one ``torch.Generator`` seeded with ``seed`` (default 0) using
``torch.randn(dtype=float32)`` in a fixed order, then hands back contiguous float32 numpy
arrays.  Norm weights are ``1 + 0.1 * N(0, 1)``; rel-pos tables are ``0.02 * N(0, 1)``.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np
import torch


def _randn(g: torch.Generator, *shape) -> np.ndarray:
    return torch.randn(*shape, generator=g, dtype=torch.float32).numpy()


def _weight(g: torch.Generator, hd: int) -> np.ndarray:
    return (1.0 + 0.1 * torch.randn(hd, generator=g, dtype=torch.float32)).numpy()


@dataclass
class SplitCase:
    """One canvas step of the split-GQA block: shapes plus host tensors.

    q [B,T,nh*hd], k/v [B,T,nkv*hd]; kc/vc [B,nkv,ctx,hd] (None when ctx == 0);
    wq/wk [hd] norm weights; ``steps`` holds extra (q, k, v) draws for repeated canvas steps.
    ``rope_cache`` marks caches stored un-roped that a set-up pass must rope at positions
    0..ctx-1 before the first step.
    """
    name: str
    B: int
    T: int
    ctx: int
    nh: int
    nkv: int
    hd: int
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    kc: Optional[np.ndarray]
    vc: Optional[np.ndarray]
    wq: Optional[np.ndarray] = None
    wk: Optional[np.ndarray] = None
    scale: float = 1.0
    causal: bool = False
    eps: float = 1e-6
    theta: float = 10000.0
    rope_cache: bool = False
    normed: bool = True
    steps: List[Dict[str, np.ndarray]] = field(default_factory=list)

    @property
    def S(self) -> int:
        return self.ctx + self.T


@dataclass
class RelposCase:
    name: str
    gh: int
    gw: int
    heads: int
    hd: int
    qkv: np.ndarray
    rh: Optional[np.ndarray]
    rw: Optional[np.ndarray]
    scale: float


def split_case(B, T, ctx, nh, nkv, hd, seed=0, scale=1.0, causal=False, normed=True,
               rope_cache=False, name="split") -> SplitCase:
    """Generic split-GQA case: kc, vc, q, k, v per batch entry, then wq, wk."""
    g = torch.Generator().manual_seed(seed)
    kcs, vcs, qs, ks, vs = [], [], [], [], []
    for _ in range(B):
        kcs.append(_randn(g, nkv, ctx, hd))
        vcs.append(_randn(g, nkv, ctx, hd))
        qs.append(_randn(g, T, nh * hd))
        ks.append(_randn(g, T, nkv * hd))
        vs.append(_randn(g, T, nkv * hd))
    wq = _weight(g, hd)
    wk = _weight(g, hd)
    kc = np.ascontiguousarray(np.stack(kcs)) if ctx > 0 else None
    vc = np.ascontiguousarray(np.stack(vcs)) if ctx > 0 else None
    return SplitCase(name, B, T, ctx, nh, nkv, hd, np.stack(qs), np.stack(ks), np.stack(vs),
                     kc, vc, wq, wk, scale=scale, causal=causal, normed=normed,
                     rope_cache=rope_cache)


def tiny_canvas_step(seed=0) -> SplitCase:
    """Tiny split-GQA canvas step: T=16, ctx=32, nh=4, nkv=2, hd=64.

    Draw order: kc[2,32,64], vc[2,32,64], q[16,256], k[16,128], v[16,128], wq[64], wk[64].
    The cache K is roped at positions 0..31 by the set-up pass; canvas positions are 32..47.
    """
    g = torch.Generator().manual_seed(seed)
    kc = _randn(g, 2, 32, 64)
    vc = _randn(g, 2, 32, 64)
    q = _randn(g, 16, 256)
    k = _randn(g, 16, 128)
    v = _randn(g, 16, 128)
    wq = _weight(g, 64)
    wk = _weight(g, 64)
    return SplitCase("tiny_split_gqa_T16_ctx32_h4_kv2_hd64", 1, 16, 32, 4, 2, 64,
                     q[None], k[None], v[None], kc[None], vc[None], wq, wk,
                     rope_cache=True)


def dg_canvas_steps(nsteps=48, seed=0) -> SplitCase:
    """DiffusionGemma-like canvas: T=256, ctx=1024, nh=16, nkv=8, hd=128, ``nsteps`` steps.

    Draw order: kc[8,1024,128], vc, wq[128], wk[128], then per step q[256,2048],
    k[256,1024], v[256,1024].  The fixed cache K is roped at positions 0..1023 by the set-up
    pass; canvas positions are 1024..1279.  Step 0's draw is also exposed as q/k/v.
    """
    g = torch.Generator().manual_seed(seed)
    kc = _randn(g, 8, 1024, 128)
    vc = _randn(g, 8, 1024, 128)
    wq = _weight(g, 128)
    wk = _weight(g, 128)
    steps = []
    for _ in range(nsteps):
        steps.append({"q": _randn(g, 256, 2048)[None], "k": _randn(g, 256, 1024)[None],
                      "v": _randn(g, 256, 1024)[None]})
    c = SplitCase("dg_canvas_T256_ctx1024_h16_kv8_hd128", 1, 256, 1024, 16, 8, 128,
                  steps[0]["q"], steps[0]["k"], steps[0]["v"], kc[None], vc[None], wq, wk,
                  rope_cache=True)
    c.steps = steps
    return c


def long_cache(seed=0, B=4, ctx=8192) -> SplitCase:
    """Long-cache split-GQA: B=4 canvases, T=256, ctx=8192, nh=32, nkv=8, hd=128.

    Draw order: for each canvas kc[8,ctx,128], vc, q[256,4096], k[256,1024], v[256,1024];
    then wq[128], wk[128].  The cache is used as drawn; canvas positions ctx..ctx+255.
    """
    c = split_case(B, 256, ctx, 32, 8, 128, seed=seed,
                   name="long_cache_B%d_T256_ctx%d_h32_kv8_hd128" % (B, ctx))
    return c


def depformer_frames(seed=0, frames=4096) -> SplitCase:
    """Batched causal-within-frame attention: ``frames`` x 8 steps x 16 heads x hd 64.

    Draw order: q[frames,8,1024], k, v.  Scale 0.125, causal, no cache, no norms.
    """
    g = torch.Generator().manual_seed(seed)
    q = _randn(g, frames, 8, 1024)
    k = _randn(g, frames, 8, 1024)
    v = _randn(g, frames, 8, 1024)
    return SplitCase("depformer_frames%d_steps8_h16_hd64" % frames, frames, 8, 0, 16, 16, 64,
                     q, k, v, None, None, None, None, scale=0.125, causal=True, normed=False)


@dataclass
class LayerSpec:
    """Attention geometry of one decoder layer over a shared canvas: its type (sliding layers
    use the sliding rope table, global layers the full one), head dim, kv heads, cache length,
    and whether it lacks a v projection (k_eq_v: v is the raw k projection)."""
    sliding: bool
    hd: int
    nkv: int
    ctx: int
    k_eq_v: bool = False


@dataclass
class LayerStackCase:
    """One canvas step through a stack of layers.  ``per_layer[i]`` holds layer i's host
    tensors: q [B,T,nh*hd], k [B,T,nkv*hd], v (None for k_eq_v), kc/vc [B,nkv,ctx,hd], wq, wk.
    Canvas row t sits at position pos0 + t in every layer."""
    name: str
    B: int
    T: int
    nh: int
    pos0: int
    theta_sliding: float
    theta_full: float
    layers: List[LayerSpec]
    per_layer: List[Dict[str, Optional[np.ndarray]]]
    eps: float = 1e-6
    scale: float = 1.0


def layer_stack(B, T, nh, pos0, layers, seed=0, theta_sliding=1e4, theta_full=1e6,
                name="layer_stack") -> LayerStackCase:
    """Per layer in order: kc, vc [B,nkv,ctx,hd], q, k, then v unless k_eq_v, then wq, wk."""
    g = torch.Generator().manual_seed(seed)
    per = []
    for l in layers:
        d = {"kc": _randn(g, B, l.nkv, l.ctx, l.hd) if l.ctx > 0 else None}
        d["vc"] = _randn(g, B, l.nkv, l.ctx, l.hd) if l.ctx > 0 else None
        d["q"] = _randn(g, B, T, nh * l.hd)
        d["k"] = _randn(g, B, T, l.nkv * l.hd)
        d["v"] = None if l.k_eq_v else _randn(g, B, T, l.nkv * l.hd)
        d["wq"] = _weight(g, l.hd)
        d["wk"] = _weight(g, l.hd)
        per.append(d)
    return LayerStackCase(name, B, T, nh, pos0, theta_sliding, theta_full, list(layers), per)


def dg_layer_stack(seed=0) -> LayerStackCase:
    """DiffusionGemma-like layer types over one canvas (T=256, nh=16, positions 1024..1279):
    sliding layers hd 128, nkv 8, rope base 1e4, a 512-entry cache; one global layer hd 96
    (run padded in the 128-wide kernel), nkv 4, rope base 1e6, a 1024-entry cache, k_eq_v."""
    layers = [LayerSpec(True, 128, 8, 512), LayerSpec(False, 96, 4, 1024, k_eq_v=True),
              LayerSpec(True, 128, 8, 512)]
    return layer_stack(1, 256, 16, 1024, layers, seed=seed,
                       name="dg_layers_T256_h16_sliding128kv8ctx512_global96kv4ctx1024")


def relpos_case(gh, gw, heads, hd, seed=0, scale=None, bias=True, table_std=0.02,
                name="relpos") -> RelposCase:
    """Fused qkv [gh*gw, 3*heads*hd] ~ N(0,1), then Rh [gh,gh,hd], Rw [gw,gw,hd]."""
    g = torch.Generator().manual_seed(seed)
    n = gh * gw
    qkv = _randn(g, n, 3 * heads * hd)
    rh = (table_std * torch.randn(gh, gh, hd, generator=g)).numpy() if bias else None
    rw = (table_std * torch.randn(gw, gw, hd, generator=g)).numpy() if bias else None
    if scale is None:
        scale = float(hd) ** -0.5
    return RelposCase(name, gh, gw, heads, hd, qkv, rh, rw, float(scale))


@dataclass
class WindowsCase:
    """A batch of windows for windowed rel-pos attention: qkv [nwin, gh*gw, 3*heads*hd]."""
    name: str
    nwin: int
    gh: int
    gw: int
    heads: int
    hd: int
    qkv: np.ndarray
    rh: Optional[np.ndarray]
    rw: Optional[np.ndarray]
    scale: float


def windows_case(nwin, gh, gw, heads, hd, seed=0, scale=None, bias=True, table_std=0.02,
                 name="relpos_windows") -> WindowsCase:
    """qkv [nwin, gh*gw, 3*heads*hd] ~ N(0,1), then Rh [gh,gh,hd], Rw [gw,gw,hd] (0.02*N)."""
    g = torch.Generator().manual_seed(seed)
    qkv = _randn(g, nwin, gh * gw, 3 * heads * hd)
    rh = (table_std * torch.randn(gh, gh, hd, generator=g)).numpy() if bias else None
    rw = (table_std * torch.randn(gw, gw, hd, generator=g)).numpy() if bias else None
    if scale is None:
        scale = float(hd) ** -0.5
    return WindowsCase(name, nwin, gh, gw, heads, hd, qkv, rh, rw, float(scale))


def sam_windowed(seed=0) -> WindowsCase:
    """SAM windowed attention: 25 windows of 14x14 tokens (a 64x64 map padded to 70x70),
    12 heads, hd 64, scale 1/8."""
    return windows_case(25, 14, 14, 12, 64, seed=seed, scale=0.125,
                        name="sam_windowed_25x14x14_h12_hd64")


def sam_global(seed=0) -> RelposCase:
    """SAM-style windowless attention: 64x64 grid, 12 heads, hd 64, scale 1/8."""
    return relpos_case(64, 64, 12, 64, seed=seed, scale=0.125,
                       name="sam_relpos_64x64_h12_hd64")
