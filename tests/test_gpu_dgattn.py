"""GPU parity of the tensor-level calls (gqa_flash_attention_dg_amd.dgattn) against the oracle:
extents come from the tensors' shapes, outputs and workspaces are allocated by the calls, and
every compared element meets the same bar as the C entry points (2e-4 + 1e-4*|oracle|)."""
import numpy as np
import pytest
import torch

import oracle
from gqa_flash_attention_dg_amd import dgattn, synth

from helpers import assert_parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def dev(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


@pytest.mark.parametrize("rope,weighted", [(True, True), (False, False), (True, False)])
def test_headnorm_rope_in_place(rope, weighted):
    rng = np.random.default_rng(7)
    B, T, heads, hd = 2, 19, 3, 128
    x = (rng.standard_normal((B, T, heads * hd)) * 2.0).astype(np.float32)
    w = (1 + 0.1 * rng.standard_normal(hd)).astype(np.float32)
    cs = oracle.rope_table(5, T, hd, 10000.0)
    flags = (1 if weighted else 0) | (2 if rope else 0)
    ref = oracle.headnorm_rope(x, w, cs, heads, hd, flags, 1e-6)
    xd = dev(x)
    got = dgattn.headnorm_rope_(xd, dev(w) if weighted else None, dev(cs), heads, 1e-6, rope=rope)
    assert got is xd
    assert_parity(host(xd), ref, "headnorm_rope_")


@pytest.mark.parametrize("B,T,ctx,nh,nkv,hd,causal", [(1, 40, 300, 8, 2, 128, False),
                                                      (2, 9, 0, 4, 4, 64, True),
                                                      (1, 256, 1024, 16, 8, 128, False)])
@pytest.mark.parametrize("q4d", [False, True])
def test_attn_split_gqa(B, T, ctx, nh, nkv, hd, causal, q4d):
    scale = 0.125 if causal else 1.0
    c = synth.split_case(B, T, ctx, nh, nkv, hd, seed=T + ctx, scale=scale, causal=causal)
    ref = oracle.attn_split_gqa(c.q, c.kc, c.vc, c.k, c.v, nh, nkv, hd, scale, causal)
    q = dev(c.q)
    if q4d:
        q = q.view(B, T, nh, hd)
    elif ctx == 0:
        pytest.skip("without a cache hd comes from a 4-D q")
    out = dgattn.attn_split_gqa(q, dev(c.kc), dev(c.vc), dev(c.k), dev(c.v), scale=scale,
                                causal=causal)
    assert out.shape == q.shape
    assert_parity(host(out).reshape(B, T, nh * hd), ref, "attn_split_gqa")
    # a given output is written and returned
    out2 = torch.full_like(q, float("nan"))
    assert dgattn.attn_split_gqa(q, dev(c.kc), dev(c.vc), dev(c.k), dev(c.v), out=out2,
                                 scale=scale, causal=causal) is out2
    assert_parity(host(out2).reshape(B, T, nh * hd), ref, "attn_split_gqa out=")


@pytest.mark.parametrize("gh,gw,heads,bias", [(14, 14, 3, True), (64, 64, 2, True),
                                              (9, 7, 2, False), (20, 33, 1, True)])
def test_relpos_flash_attn(gh, gw, heads, bias):
    c = synth.relpos_case(gh, gw, heads, 64, seed=gh + gw, bias=bias, table_std=0.3)
    ref = oracle.relpos_attn(c.qkv, c.rh, c.rw, gh, gw, heads, 64, c.scale)
    out = dgattn.relpos_flash_attn(dev(c.qkv), dev(c.rh), dev(c.rw), heads, c.scale,
                                   grid=None if bias else (gh, gw))
    assert out.shape == (gh * gw, heads * 64)
    assert_parity(host(out), ref, "relpos_flash_attn")


def test_relpos_flash_attn_windows():
    c = synth.windows_case(6, 14, 14, 2, 64, seed=3, bias=True, table_std=0.3)
    ref = np.stack([oracle.relpos_attn(c.qkv[w], c.rh, c.rw, c.gh, c.gw, c.heads, c.hd, c.scale)
                    for w in range(c.nwin)])
    out = dgattn.relpos_flash_attn_windows(dev(c.qkv), dev(c.rh), dev(c.rw), c.heads, c.scale)
    assert out.shape == (6, 196, 128)
    assert_parity(host(out), ref, "relpos_flash_attn_windows")
