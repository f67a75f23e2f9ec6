"""Host-side argument checks of the C ABI, run by tests/test_abi.py in a child process that
sees no GPU.

Every check passes made-up, never-dereferenced device addresses (FAKE) into the real entry
points together with an argument the library must reject, or extents that describe an empty
output; the library validates before any launch, so nothing reaches a device.  The child
process hides every GPU (HIP_VISIBLE_DEVICES empty), so a regression in the validation shows
up as a launch error (DG_ELAUNCH) rather than as a kernel touching an unmapped address.

    python tests/abi_checks.py     # prints one JSON object: {check name: "ok" or the failure}
"""
import json
import os
import sys
import traceback

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import gqa_flash_attention_dg_amd as dg  # noqa: E402

FAKE = 0x10000000  # a non-NULL address that is never dereferenced (validation fails first)


def _err(L):
    return L.dg_last_error().decode()


def check_headnorm_validation(L):
    f = L.dg_headnorm_rope
    assert f(FAKE, FAKE, FAKE, -1, 4, 2, 64, 3, 1e-6, None) == dg.DG_EINVAL
    assert "negative" in _err(L)
    assert f(FAKE, FAKE, FAKE, 1, 4, 2, 0, 3, 1e-6, None) == dg.DG_EINVAL
    assert f(FAKE, FAKE, FAKE, 1, 4, 2, 256, 3, 1e-6, None) == dg.DG_EUNSUPPORTED
    assert f(FAKE, FAKE, FAKE, 1, 4, 2, 64, 8, 1e-6, None) == dg.DG_EINVAL          # bad flag
    assert f(FAKE, FAKE, FAKE, 1, 4, 2, 63, 2, 1e-6, None) == dg.DG_EINVAL          # odd + rope
    assert f(FAKE, None, FAKE, 1, 4, 2, 64, 3, 1e-6, None) == dg.DG_EINVAL          # w NULL
    assert f(FAKE, FAKE, None, 1, 4, 2, 64, 3, 1e-6, None) == dg.DG_EINVAL          # cs NULL
    assert f(None, FAKE, FAKE, 1, 4, 2, 64, 3, 1e-6, None) == dg.DG_EINVAL          # x NULL
    assert f(FAKE, FAKE, FAKE, 1, 4, 2, 64, 3, -1.0, None) == dg.DG_EINVAL          # eps < 0
    assert f(FAKE, FAKE + 64, FAKE, 1, 4, 2, 64, 1, 1e-6, None) == dg.DG_EINVAL     # w inside x
    assert "overlaps" in _err(L)
    # empty outputs are a successful no-op
    assert f(None, None, None, 0, 4, 2, 64, 3, 1e-6, None) == dg.DG_OK
    assert f(None, None, None, 3, 0, 2, 64, 3, 1e-6, None) == dg.DG_OK
    assert _err(L) == ""


def check_rope_table_validation(L):
    f = L.dg_rope_table
    assert f(FAKE, -1, 4, 64, 1e4, None) == dg.DG_EINVAL
    assert f(FAKE, 0, 4, 63, 1e4, None) == dg.DG_EINVAL
    assert f(FAKE, 0, 4, 64, 0.0, None) == dg.DG_EINVAL
    assert f(None, 0, 4, 64, 1e4, None) == dg.DG_EINVAL
    assert f(None, 0, 0, 64, 1e4, None) == dg.DG_OK


def check_attn_split_validation(L):
    f = L.dg_attn_split_gqa
    args = lambda **kw: [kw.get(k, d) for k, d in (
        ("q", FAKE), ("kc", FAKE + (1 << 24)), ("vc", FAKE + (2 << 24)), ("k", FAKE + (3 << 24)),
        ("v", FAKE + (4 << 24)), ("out", FAKE + (5 << 24)), ("batch", 1), ("T", 16),
        ("ctx", 32), ("nh", 4), ("nkv", 2), ("hd", 64), ("scale", 1.0), ("causal", 0),
        ("ws", None), ("wsb", 0), ("stream", None))]
    assert f(*args(nh=5)) == dg.DG_EINVAL                   # nh % nkv != 0
    assert "multiple" in _err(L)
    assert f(*args(nkv=0)) == dg.DG_EINVAL
    assert f(*args(T=-1)) == dg.DG_EINVAL
    assert f(*args(hd=98)) == dg.DG_EUNSUPPORTED            # not a multiple of 4
    assert f(*args(hd=132)) == dg.DG_EUNSUPPORTED
    assert f(*args(hd=0)) == dg.DG_EINVAL
    assert f(*args(scale=float("nan"))) == dg.DG_EINVAL
    assert f(*args(causal=2)) == dg.DG_EINVAL
    assert f(*args(kc=None)) == dg.DG_EINVAL                # ctx > 0 needs a cache
    assert f(*args(q=None)) == dg.DG_EINVAL
    assert f(*args(out=FAKE + 16)) == dg.DG_EINVAL          # out overlaps q
    assert "overlaps" in _err(L)
    assert f(*args(out=FAKE + (3 << 24) + 4)) == dg.DG_EINVAL  # out overlaps canvas k
    assert f(*args(ws=FAKE + (6 << 24) + 8, wsb=1 << 20)) == dg.DG_EINVAL  # misaligned
    assert f(*args(ctx=(1 << 30))) == dg.DG_EUNSUPPORTED    # 32-bit key indices
    assert f(*args(T=(1 << 29), nh=8, nkv=2)) == dg.DG_EUNSUPPORTED
    assert f(*args(T=0)) == dg.DG_OK                        # zero canvas: no-op
    assert f(*args(batch=0)) == dg.DG_OK
    assert L.dg_attn_split_gqa_workspace_size(1, 16, 32, 5, 2, 64) == 0


def check_qkv_headnorm_validation(L):
    f = L.dg_qkv_headnorm_rope
    base = dict(q=FAKE, wq=FAKE + (1 << 24), k=FAKE + (2 << 24), wk=FAKE + (3 << 24),
                v=FAKE + (4 << 24), cs=FAKE + (5 << 24), batch=1, T=4, nh=4, nkv=2, hd=64,
                flags=3, eps=1e-6, stream=None)
    call = lambda **kw: f(*[{**base, **kw}[k] for k in base])
    assert call(nh=-1) == dg.DG_EINVAL
    assert call(hd=256) == dg.DG_EUNSUPPORTED
    assert call(flags=16) == dg.DG_EINVAL                  # unknown bit
    assert call(wq=None) == dg.DG_EINVAL                   # WEIGHTED needs wq for q
    assert call(cs=None) == dg.DG_EINVAL
    assert call(k=FAKE + 64) == dg.DG_EINVAL               # k inside q
    assert "overlap" in _err(L)
    assert call(cs=FAKE + (2 << 24) + 256) == dg.DG_EINVAL  # table inside k
    assert call(eps=float("nan")) == dg.DG_EINVAL
    assert call(q=None, k=None, v=None) == dg.DG_OK        # nothing to do
    vfk = dg.DG_NORM_V_FROM_K
    assert call(flags=3 | vfk, v=None) == dg.DG_EINVAL      # V_FROM_K needs an output v
    assert call(flags=4 | vfk) == dg.DG_EINVAL              # ... and the norm
    assert L.dg_headnorm_rope(FAKE, FAKE + (1 << 24), FAKE + (2 << 24), 1, 4, 2, 64, 3 | vfk,
                              1e-6, None) == dg.DG_EINVAL   # single-tensor entry: unknown bit
    assert call(T=0) == dg.DG_OK
    assert _err(L) == ""


def check_qkv_headnorm_kv16_validation(L):
    f = L.dg_qkv_headnorm_rope_kv16
    base = dict(q=FAKE, wq=FAKE + (1 << 24), k=FAKE + (2 << 24), wk=FAKE + (3 << 24),
                v=FAKE + (4 << 24), cs=FAKE + (5 << 24), k16=FAKE + (6 << 24),
                v16=FAKE + (7 << 24), batch=1, T=4, nh=4, nkv=2, hd=64, flags=3, eps=1e-6,
                fmt=dg.DG_KV_BF16, stream=None)
    call = lambda **kw: f(*[{**base, **kw}[k] for k in base])
    assert call(fmt=0) == dg.DG_EINVAL                      # unknown format
    assert call(fmt=3) == dg.DG_EINVAL
    assert "kv_format" in _err(L)
    assert call(k16=None) == dg.DG_EINVAL                   # k given without its twin
    assert call(v16=None) == dg.DG_EINVAL                   # v given without its twin
    assert call(k16=FAKE + (2 << 24) + 64) == dg.DG_EINVAL  # twin inside k
    assert "overlap" in _err(L)
    assert call(v16=FAKE + (6 << 24) + 32) == dg.DG_EINVAL  # twin inside the other twin
    assert call(k16=FAKE + (5 << 24)) == dg.DG_EINVAL       # twin on the rope table
    assert call(flags=16) == dg.DG_EINVAL                   # the checks of the plain entry
    assert call(wq=None) == dg.DG_EINVAL
    assert call(flags=3 | dg.DG_NORM_V_FROM_K, v=None) == dg.DG_EINVAL
    assert call(q=None, k=None, v=None, k16=None, v16=None) == dg.DG_OK   # nothing to do
    assert call(T=0) == dg.DG_OK
    assert _err(L) == ""


def check_attn_qnorm_validation(L):
    f = L.dg_attn_split_gqa_qnorm
    base = dict(q=FAKE, wq=FAKE + (1 << 24), cs=FAKE + (2 << 24), kc=FAKE + (3 << 24),
                vc=FAKE + (4 << 24), k=FAKE + (5 << 24), v=FAKE + (6 << 24),
                out=FAKE + (7 << 24), batch=1, T=16, ctx=32, nh=4, nkv=2, hd=64, qflags=3,
                eps=1e-6, scale=1.0, causal=0, ws=None, wsb=0, stream=None)
    call = lambda **kw: f(*[{**base, **kw}[k] for k in base])
    assert call(qflags=16) == dg.DG_EINVAL
    assert call(eps=-1.0) == dg.DG_EINVAL
    assert call(wq=None) == dg.DG_EINVAL
    assert call(cs=None) == dg.DG_EINVAL
    assert call(out=FAKE + (1 << 24)) == dg.DG_EINVAL       # out overlaps wq
    assert call(out=FAKE + (2 << 24) + 512) == dg.DG_EINVAL # out overlaps the rope table
    assert call(hd=66) == dg.DG_EUNSUPPORTED
    assert call(nh=3) == dg.DG_EINVAL
    assert call(q=FAKE + 4, out=FAKE + (8 << 24)) == dg.DG_EINVAL   # misaligned q
    assert "aligned" in _err(L)
    assert call(T=0) == dg.DG_OK


def check_attn_qkvnorm_validation(L):
    f = L.dg_attn_split_gqa_qkvnorm
    base = dict(q=FAKE, wq=FAKE + (1 << 24), k=FAKE + (2 << 24), wk=FAKE + (3 << 24),
                v=FAKE + (4 << 24), cs=FAKE + (5 << 24), kc=FAKE + (6 << 24),
                vc=FAKE + (7 << 24), out=FAKE + (8 << 24), batch=1, T=16, ctx=32, nh=4, nkv=2,
                hd=64, flags=3, eps=1e-6, scale=1.0, causal=0, ws=None, wsb=0, stream=None)
    call = lambda **kw: f(*[{**base, **kw}[k] for k in base])
    assert call(flags=4) == dg.DG_EINVAL                    # SKIP is not accepted here
    assert call(flags=8) == dg.DG_EINVAL                    # nor V_FROM_K (pass k as v)
    assert call(eps=float("nan")) == dg.DG_EINVAL
    assert call(wq=None) == dg.DG_EINVAL
    assert call(wk=None) == dg.DG_EINVAL
    assert call(cs=None) == dg.DG_EINVAL
    assert call(out=FAKE + (3 << 24)) == dg.DG_EINVAL       # out overlaps wk
    assert call(out=FAKE + (2 << 24) + 256) == dg.DG_EINVAL # out overlaps the canvas keys
    assert call(out=FAKE + (5 << 24) + 512) == dg.DG_EINVAL # out overlaps the rope table
    assert call(hd=66) == dg.DG_EUNSUPPORTED
    assert call(nh=3) == dg.DG_EINVAL
    assert call(wk=FAKE + (3 << 24) + 4) == dg.DG_EINVAL     # misaligned wk
    assert "aligned" in _err(L)
    assert call(T=0, wq=None, wk=None, cs=None) == dg.DG_OK
    assert call(flags=0, T=0) == dg.DG_OK


def check_attn_alignment_validation(L):
    f = L.dg_attn_split_gqa
    assert f(FAKE, FAKE + (1 << 24), FAKE + (2 << 24), FAKE + (3 << 24) + 8, FAKE + (4 << 24),
             FAKE + (5 << 24), 1, 16, 32, 4, 2, 64, 1.0, 0, None, 0, None) == dg.DG_EINVAL
    assert "aligned" in _err(L)


def check_relpos_validation(L):
    # the form without a workspace
    g = L.relpos_flash_attn
    base0 = dict(qkv=FAKE, rh=FAKE + (1 << 26), rw=FAKE + (2 << 26), out=FAKE + (3 << 26),
                 gh=8, gw=8, heads=2, hd=64, scale=0.125, stream=None)
    call0 = lambda **kw: g(*[{**base0, **kw}[k] for k in base0])
    assert call0(hd=32) == dg.DG_EUNSUPPORTED
    assert call0(rw=None) == dg.DG_EINVAL
    assert call0(out=FAKE + 4) == dg.DG_EINVAL
    assert call0(gw=0) == dg.DG_OK
    # the form with a workspace
    f = L.relpos_flash_attn_ws
    base = dict(qkv=FAKE, rh=FAKE + (1 << 26), rw=FAKE + (2 << 26), out=FAKE + (3 << 26),
                gh=8, gw=8, heads=2, hd=64, scale=0.125, ws=None, wsb=0, stream=None)
    call = lambda **kw: f(*[{**base, **kw}[k] for k in base])
    assert call(hd=32) == dg.DG_EUNSUPPORTED
    assert call(gh=65) == dg.DG_EUNSUPPORTED
    assert call(rh=None) == dg.DG_EINVAL                   # exactly one table
    assert call(gw=-1) == dg.DG_EINVAL
    assert call(scale=float("inf")) == dg.DG_EINVAL
    assert call(out=FAKE + 4) == dg.DG_EINVAL              # overlaps qkv
    assert call(qkv=None) == dg.DG_EINVAL
    assert call(ws=FAKE + (4 << 26) + 4, wsb=1 << 20) == dg.DG_EINVAL   # misaligned workspace
    assert call(ws=FAKE + (4 << 26), wsb=16) == dg.DG_EINVAL           # too small
    assert call(ws=FAKE + 64, wsb=1 << 20) == dg.DG_EINVAL              # overlaps qkv
    assert call(rw=FAKE + (2 << 26) + 4) == dg.DG_EINVAL                # misaligned table
    assert "aligned" in _err(L)
    assert call(gh=0) == dg.DG_OK
    assert call(heads=0) == dg.DG_OK
    assert L.relpos_flash_attn_workspace_size(64, 64, 12, 64) == 12 * 4096 * (64 + 64) * 4
    assert L.relpos_flash_attn_workspace_size(14, 20, 2, 64) == 2 * 280 * (14 + 20) * 4
    assert L.relpos_flash_attn_workspace_size(64, 64, 12, 32) == 0


def check_relpos_windows_validation(L):
    f = L.relpos_flash_attn_windows
    base = dict(qkv=FAKE, rh=FAKE + (1 << 26), rw=FAKE + (2 << 26), out=FAKE + (3 << 26),
                nwin=4, gh=8, gw=8, heads=2, hd=64, scale=0.125, ws=None, wsb=0, stream=None)
    call = lambda **kw: f(*[{**base, **kw}[k] for k in base])
    assert call(nwin=-1) == dg.DG_EINVAL
    assert "negative" in _err(L)
    assert call(hd=32) == dg.DG_EUNSUPPORTED
    assert call(gw=65) == dg.DG_EUNSUPPORTED
    assert call(rw=None) == dg.DG_EINVAL
    assert call(out=FAKE + 4 * 8 * 8 * 3 * 128 * 4 - 16) == dg.DG_EINVAL   # inside the last window
    assert call(ws=FAKE + (4 << 26), wsb=1024) == dg.DG_EINVAL             # too small for 4 windows
    assert call(nwin=0) == dg.DG_OK
    # grids of at most 16 x 16: dh and dw rows each padded to 4 floats (14 -> 16)
    assert L.relpos_flash_attn_windows_workspace_size(25, 14, 14, 12, 64) == 25 * 12 * 196 * 32 * 4
    assert L.relpos_flash_attn_windows_workspace_size(0, 14, 14, 12, 64) == 0


def check_kv16_validation(L):
    assert L.dg_pack_kv16(FAKE, FAKE + (1 << 24), 100, 3, None) == dg.DG_EINVAL       # format
    assert L.dg_pack_kv16(FAKE, FAKE + 8, 100, dg.DG_KV_F16, None) == dg.DG_EINVAL     # misaligned
    assert L.dg_pack_kv16(FAKE, FAKE + 16, 100, dg.DG_KV_F16, None) == dg.DG_EINVAL    # overlap
    assert L.dg_pack_kv16(None, None, 0, dg.DG_KV_BF16, None) == dg.DG_OK
    f = L.dg_attn_split_gqa_kv16
    base = dict(q=FAKE, kc=FAKE + (1 << 24), vc=FAKE + (2 << 24), k=FAKE + (3 << 24),
                v=FAKE + (4 << 24), out=FAKE + (5 << 24), batch=1, T=16, ctx=32, nh=4, nkv=2,
                hd=64, scale=1.0, causal=0, fmt=dg.DG_KV_BF16, ws=None, wsb=0, stream=None)
    call = lambda **kw: f(*[{**base, **kw}[k] for k in base])
    assert call(fmt=0) == dg.DG_EINVAL
    assert call(hd=20) == dg.DG_EUNSUPPORTED                 # 16-bit rows need hd % 8 == 0
    assert call(out=FAKE + (3 << 24) + 16 * 2 * 64 * 2 - 16) == dg.DG_EINVAL   # 2-byte extents
    assert call(kc=FAKE + (1 << 24) + 8) == dg.DG_EINVAL     # misaligned
    assert call(T=0) == dg.DG_OK


CHECKS = [check_headnorm_validation, check_rope_table_validation, check_attn_split_validation, check_qkv_headnorm_validation, check_qkv_headnorm_kv16_validation, check_attn_qnorm_validation, check_attn_qkvnorm_validation, check_attn_alignment_validation, check_relpos_validation, check_relpos_windows_validation, check_kv16_validation]


def main():
    L = dg.lib()
    res = {}
    for fn in CHECKS:
        try:
            fn(L)
            res[fn.__name__] = "ok"
        except Exception:  # report every check, whatever it raised
            res[fn.__name__] = traceback.format_exc(limit=3)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
