"""Launch plans of the split-GQA entry points and the workgroup placement (host only, no GPU).

dg_attn_split_gqa_plan takes the device's compute-unit count as an argument, so the plans of a
full MI355X (256 CUs) and of one partition of it (32 CUs) are checked here without a device:
the kernel chosen, the key-range splits and the workspace they need.  The XCD placement every
kernel applies is checked to be a bijection by a small host program built from the library's
own header.
"""
import os
import shutil
import subprocess

import pytest

import gqa_flash_attention_dg_amd as dg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def lib():
    if not os.path.exists(dg.LIB_PATH):
        from gqa_flash_attention_dg_amd import build
        build.build()
    dg.lib()


def plan(B, T, ctx, nh, nkv, hd, cus, causal=0, kv=0):
    return dg.dg_attn_split_gqa_plan(B, T, ctx, nh, nkv, hd, causal, kv, cus)


# (shape, CUs) -> (kernel, query block, nsplit, workgroups)
EXPECTED = [
    # the DiffusionGemma-like step: 32 workgroups of 128 query vectors, 8 splits fill 256 CUs;
    # on 32 CUs they already fill the device
    ((1, 256, 1024, 16, 8, 128), 256, (dg.DG_KERNEL_TILE32, 128, 8, 256)),
    ((1, 256, 1024, 16, 8, 128), 32, (dg.DG_KERNEL_TILE32, 128, 1, 32)),
    # the long cache fills 256 CUs without a split
    ((4, 256, 8192, 32, 8, 128), 256, (dg.DG_KERNEL_TILE32, 128, 1, 256)),
    ((4, 256, 8192, 32, 8, 128), 32, (dg.DG_KERNEL_TILE32, 128, 1, 256)),
    # a sliding layer (768 keys): 128-query workgroups cap at 6 splits (192 of 256 CUs)
    ((1, 256, 512, 16, 8, 128), 256, (dg.DG_KERNEL_TILE32, 128, 6, 192)),
    ((1, 256, 512, 16, 8, 128), 32, (dg.DG_KERNEL_TILE32, 128, 1, 32)),
    # the global hd-96 layer (G = 4): 32 workgroups of 128, 8 splits fill the device
    ((1, 256, 1024, 16, 4, 96), 256, (dg.DG_KERNEL_TILE32, 128, 8, 256)),
    # causal calls do not split
    ((1, 256, 1024, 16, 8, 128, 1), 256, (dg.DG_KERNEL_TILE32, 128, 1, 32)),
    # 16-bit K/V stay on the 32-key tiles
    ((1, 256, 1024, 16, 8, 128, 0, dg.DG_KV_BF16), 256, (dg.DG_KERNEL_TILE32, 128, 8, 256)),
    # hd 64 stays on the 32-key tiles; short key sets take the small kernel
    ((1, 16, 32, 4, 2, 64), 256, (dg.DG_KERNEL_TILE32, 128, 1, 2)),
    ((4096, 8, 0, 16, 16, 64, 1), 256, (dg.DG_KERNEL_SMALL, 0, 1, 16384)),
]


@pytest.mark.parametrize("shape,cus,want", EXPECTED)
def test_plan_at_256_and_32_cus(shape, cus, want):
    B, T, ctx, nh, nkv, hd = shape[:6]
    causal = shape[6] if len(shape) > 6 else 0
    kv = shape[7] if len(shape) > 7 else 0
    p = plan(B, T, ctx, nh, nkv, hd, cus, causal, kv)
    assert (p.kernel, p.query_block, p.nsplit, p.workgroups) == want
    G = nh // nkv
    if p.kernel != dg.DG_KERNEL_SMALL:
        qblocks = -(-T * G // p.query_block)
        assert p.workgroups == B * nkv * qblocks * p.nsplit
    if p.nsplit > 1:
        # at least two 64-key stages per split; the partials are (hd + 2) floats per vector
        assert p.nsplit <= (ctx + T + 63) // 64 // 2
        assert p.workspace_bytes == p.nsplit * B * T * nh * (hd + 2) * 4
    else:
        assert p.workspace_bytes == 0


@pytest.mark.parametrize("cus", [32, 64, 128, 256, 304])
def test_plan_invariants_over_shapes(cus):
    for B in (1, 2):
        for T in (1, 40, 256, 1000):
            for ctx in (0, 100, 1024):
                for nh, nkv in ((16, 8), (8, 1), (4, 4)):
                    for hd in (64, 96, 128):
                        for causal in (0, 1):
                            p = plan(B, T, ctx, nh, nkv, hd, cus, causal)
                            assert p.nsplit >= 1 and p.workgroups >= 1
                            if causal or p.kernel == dg.DG_KERNEL_SMALL:
                                assert p.nsplit == 1
                            if p.nsplit > 1:   # a split only where the device would idle
                                assert p.workgroups // p.nsplit < cus


def test_workspace_size_covers_both_kv_formats():
    # the size query serves the f32 and the 16-bit entry points alike
    need = dg.dg_attn_split_gqa_workspace_size(1, 256, 512, 16, 8, 128)
    f32 = plan(1, 256, 512, 16, 8, 128, 0).workspace_bytes
    b16 = plan(1, 256, 512, 16, 8, 128, 0, kv=dg.DG_KV_BF16).workspace_bytes
    assert need == max(f32, b16) > 0


def test_plan_rejects_bad_arguments():
    for args in [(-1, 4, 4, 2, 1, 64), (1, 4, 4, 3, 2, 64), (1, 4, 4, 2, 0, 64)]:
        with pytest.raises(dg.DgError) as e:
            plan(*args, 256)
        assert e.value.status == dg.DG_EINVAL
    with pytest.raises(dg.DgError) as e:
        plan(1, 4, 4, 2, 1, 130, 256)
    assert e.value.status == dg.DG_EUNSUPPORTED
    with pytest.raises(dg.DgError):
        plan(1, 4, 4, 2, 1, 64, -1)
    p = plan(0, 4, 4, 2, 1, 64, 256)     # empty output: nothing launched
    assert p.kernel == dg.DG_KERNEL_NONE and p.workgroups == 0


def test_xcd_remap_is_a_bijection(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = tmp_path / "xcd_remap_check"
    subprocess.run([hipcc, "--cuda-host-only", "-x", "hip", "-std=c++17", "-O1",
                    os.path.join(ROOT, "tests", "xcd_remap_check.cpp"), "-o", str(exe)],
                   check=True, capture_output=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
