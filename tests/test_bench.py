"""Host logic of bench.py (no GPU): the one-GPU contract, the code-only source hash that ties
the committed traffic records to the kernels they were measured on, and the algorithmic
flop/byte counts the roofline divides by, checked against brute-force counting."""
import json
import os
import subprocess
import sys
from types import SimpleNamespace

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_code_tokens_drop_comments_and_layout_only():
    src = 'int a = 1; // note\n/* block\n comment */  float  b=2;\nconst char* s = "x // y /* z */";'
    assert bench._code_tokens(src) == 'int a = 1; float b=2; const char* s = "x // y /* z */";'
    # character literals and escaped quotes stay whole
    assert bench._code_tokens("char q = '\"'; // c") == "char q = '\"';"
    assert bench._code_tokens('s = "a\\"//b"; // c') == 's = "a\\"//b";'
    # a change of code is a change of tokens; a change of comments or spacing is not
    assert bench._code_tokens("x = y + 1;") != bench._code_tokens("x = y + 2;")
    assert bench._code_tokens("x = y + 1; // one") == bench._code_tokens("x  =  y + 1;   /* 1 */")


def test_source_hash_follows_code_not_comments(tmp_path, monkeypatch):
    d = tmp_path / "csrc"
    d.mkdir()
    (d / "k.hip").write_text("__global__ void k() { int i = 0; }  // first\n")
    monkeypatch.setattr(bench, "CSRC", str(d))
    h0 = bench.source_hash()
    (d / "k.hip").write_text("// another comment\n__global__ void k() {\n  int i = 0;\n}\n")
    assert bench.source_hash() == h0
    (d / "k.hip").write_text("__global__ void k() { int i = 1; }\n")
    assert bench.source_hash() != h0
    (d / "k.hip").write_text("__global__ void k() { int i = 0; }\n")
    (d / "extra.hpp").write_text("// only a comment\n")
    assert bench.source_hash() != h0   # a new file is part of the kernel sources


def test_source_hash_per_kernel_follows_its_file_and_includes(tmp_path, monkeypatch):
    d = tmp_path / "csrc"
    d.mkdir()
    (d / "common.hpp").write_text("int shared = 0;\n")
    (d / "attn_split_gqa.hip").write_text('#include "common.hpp"\n__global__ void a() {}\n')
    (d / "relpos_flash.hip").write_text('#include "common.hpp"\n__global__ void r() {}\n')
    monkeypatch.setattr(bench, "CSRC", str(d))
    a0, r0 = bench.source_hash("attn_split_gqa"), bench.source_hash("relpos_flash")
    assert bench.source_hash("attn_small") == a0          # built from the same file
    (d / "relpos_flash.hip").write_text('#include "common.hpp"\n\n__global__  void r()  {}  // r\n')
    assert bench.source_hash("relpos_flash") == r0        # layout and comments only
    (d / "relpos_flash.hip").write_text('#include "common.hpp"\n__global__ void r(int) {}\n')
    assert bench.source_hash("relpos_flash") != r0
    assert bench.source_hash("attn_split_gqa") == a0      # the other kernel's record stays valid
    (d / "common.hpp").write_text("int shared = 1;\n")
    assert bench.source_hash("attn_split_gqa") != a0      # a shared include changes both
    (d / "unrelated.hip").write_text("__global__ void u() {}\n")
    a1 = bench.source_hash("attn_split_gqa")
    (d / "unrelated.hip").write_text("__global__ void u(int) {}\n")
    assert bench.source_hash("attn_split_gqa") == a1
    assert bench.source_hash("hbm_copy") == bench.source_hash("hbm_copy")   # no source of ours


def test_traffic_record_used_only_on_matching_source(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    rec = {"source_hash": bench.source_hash("attn_split_gqa"), "hbm_bytes_per_launch": 12345.0}
    (tmp_path / "traffic_attn_split_gqa_w.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("attn_split_gqa", "w") == 12345.0
    rec["source_hash"] = "0" * 16
    (tmp_path / "traffic_attn_split_gqa_w.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("attn_split_gqa", "w") is None
    assert bench.measured_traffic("attn_split_gqa", "missing") is None


def _case(B, T, ctx, nh, nkv, hd, causal, normed=True):
    return SimpleNamespace(B=B, T=T, ctx=ctx, nh=nh, nkv=nkv, hd=hd, causal=causal,
                           normed=normed)


@pytest.mark.parametrize("B,T,ctx,nh,nkv,hd,causal", [(1, 16, 32, 4, 2, 64, 0),
                                                      (2, 5, 7, 6, 3, 8, 0),
                                                      (3, 8, 0, 2, 2, 4, 1),
                                                      (1, 6, 3, 2, 1, 12, 1)])
def test_split_counts_match_brute_force(B, T, ctx, nh, nkv, hd, causal):
    # every (batch, q head, canvas row, key) pair the attention evaluates, counted one by one
    pairs = 0
    for _b in range(B):
        for _h in range(nh):
            for i in range(T):
                for j in range(ctx + T):
                    if not causal or j < ctx or j - ctx <= i:
                        pairs += 1
    flops, attn_bytes, norm_bytes = bench.split_counts(_case(B, T, ctx, nh, nkv, hd, causal))
    assert flops == 4 * hd * pairs              # q.k and p.v: 2 * hd flops each
    q, kv, cache = B * T * nh * hd, B * T * nkv * hd, B * nkv * ctx * hd
    assert attn_bytes == 4 * (2 * q + 2 * kv + 2 * cache)   # q, k, v, kc, vc in; out
    # with the q norm inside attention only k and v make a norm round trip; otherwise q too
    assert norm_bytes == 4 * 2 * 2 * kv
    _, _, nb_sep = bench.split_counts(_case(B, T, ctx, nh, nkv, hd, causal), "separate")
    assert nb_sep == 4 * 2 * (q + 2 * kv)
    _, _, nb_none = bench.split_counts(_case(B, T, ctx, nh, nkv, hd, causal, normed=False))
    assert nb_none == 0
    # with every norm inside attention nothing makes a separate round trip
    f2, a2, nb_fused = bench.split_counts(_case(B, T, ctx, nh, nkv, hd, causal), "fused")
    assert (f2, a2, nb_fused) == (flops, attn_bytes, 0)


def test_auto_norm_mode_counts_canvas_keys_per_workgroup():
    """'auto' norms k and v inside attention when one workgroup of the launch plan meets at most
    64 canvas keys (the key range split over workgroups, or a short canvas), else keeps the k/v
    norm launch.  Plans are taken for a 256-CU device; causal calls and calls without a
    workspace do not split."""
    from gqa_flash_attention_dg_amd.canvas import auto_norm_mode
    m = lambda *a, **k: auto_norm_mode(*a, cus=256, **k)
    assert m(1, 16, 32, 4, 2, 64) == "fused"                       # tiny: 1 tile
    assert m(1, 256, 1024, 16, 8, 128) == "fused"                  # 8 tiles over 8 splits
    assert m(1, 256, 512, 16, 8, 128) == "fused"                   # 16-key tiles, 4 per split
    assert m(4, 256, 8192, 32, 8, 128) == "in_attention"           # long cache: unsplit
    assert m(1, 64, 0, 8, 8, 64) == "fused"                        # 2 tiles, unsplit
    assert m(1, 65, 0, 8, 8, 64) == "in_attention"                 # 3 tiles, unsplit
    assert m(1, 256, 1024, 16, 8, 128, causal=True) == "in_attention"   # causal: no split
    assert m(1, 256, 1024, 16, 8, 128, split=False) == "in_attention"   # no workspace
    assert m(0, 16, 32, 4, 2, 64) == "fused"                       # empty: no launch


def test_stats_mean_median_min():
    assert bench._stats([3.0, 1.0, 2.0]) == {"mean": 2.0, "median": 2.0, "min": 1.0}
    assert bench._stats([4.0, 1.0, 2.0, 3.0]) == {"mean": 2.5, "median": 2.5, "min": 1.0}


def test_host_cpu_model_is_named():
    m = bench.host_cpu_model()
    assert isinstance(m, str) and m and m != "unknown"
