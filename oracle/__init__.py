"""CPU oracle for the attention block -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package.  The product library (``gqa_flash_attention_dg_amd``) never loads it and
has no CPU fallback.

The arithmetic lives in ``oracle.c`` (plain C, f32, sequential sums, OpenMP across independent
output units only).  This module builds it with gcc and wraps it for numpy arrays; it holds no
arithmetic of its own.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

NORM_WEIGHTED = 1
NORM_ROPE = 2
NORM_SKIP = 4
KV_F16 = 1      # IEEE binary16 storage
KV_BF16 = 2     # bfloat16 storage

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so (gcc -O2 -fopenmp, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        f32p = ctypes.POINTER(ctypes.c_float)
        lp = ctypes.POINTER(ctypes.c_long)
        I, F, D, U = ctypes.c_int, ctypes.c_float, ctypes.c_double, ctypes.c_uint
        lib.oracle_threads.argtypes = [I]
        lib.oracle_threads.restype = I
        lib.oracle_rope_table.argtypes = [f32p, I, I, I, D]
        lib.oracle_rope_table.restype = None
        lib.oracle_headnorm_rope.argtypes = [f32p, f32p, f32p, I, I, I, I, U, F]
        lib.oracle_headnorm_rope.restype = None
        lib.oracle_attn_split_gqa.argtypes = [f32p, f32p, f32p, f32p, f32p, f32p,
                                              I, I, I, I, I, I, F, I, lp, ctypes.c_long]
        lib.oracle_attn_split_gqa.restype = None
        u16p = ctypes.POINTER(ctypes.c_uint16)
        lib.oracle_pack16.argtypes = [f32p, u16p, ctypes.c_long, I]
        lib.oracle_pack16.restype = None
        lib.oracle_widen16.argtypes = [u16p, f32p, ctypes.c_long, I]
        lib.oracle_widen16.restype = None
        lib.oracle_relpos_attn.argtypes = [f32p, f32p, f32p, f32p, I, I, I, I, F, lp,
                                           ctypes.c_long]
        lib.oracle_relpos_attn.restype = None
        _lib = lib
    return _lib


def _f32(a):
    if a is None:
        return None
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def _rows(rows):
    if rows is None:
        return None, None, 0
    r = np.ascontiguousarray(rows, dtype=np.int64)
    return r, r.ctypes.data_as(ctypes.POINTER(ctypes.c_long)), int(r.size)


def threads(n: int = 0) -> int:
    """Set (n > 0) and return the OpenMP thread count the oracle uses."""
    return int(_load().oracle_threads(int(n)))


def rope_table(pos0: int, T: int, hd: int, theta: float = 10000.0) -> np.ndarray:
    """cs[T, 2*hd] = cos | sin of positions pos0 .. pos0+T-1 (NeoX pairing)."""
    cs = np.empty((T, 2 * hd), dtype=np.float32)
    _load().oracle_rope_table(_ptr(cs), int(pos0), int(T), int(hd), float(theta))
    return cs


def headnorm_rope(x, w, cs, heads: int, hd: int, flags: int, eps: float) -> np.ndarray:
    """Return a normed/roped copy of x [..., T, heads*hd] (leading dims are the batch)."""
    x = np.array(x, dtype=np.float32, copy=True, order="C")
    T = x.shape[-2]
    assert x.shape[-1] == heads * hd
    batch = int(np.prod(x.shape[:-2])) if x.ndim > 2 else 1
    w = _f32(w)
    cs = _f32(cs)
    _load().oracle_headnorm_rope(_ptr(x), _ptr(w), _ptr(cs), batch, T, heads, hd,
                                 int(flags), float(eps))
    return x


def attn_split_gqa(q, kc, vc, k, v, nh: int, nkv: int, hd: int, scale: float = 1.0,
                   causal: bool = False, rows=None, out=None) -> np.ndarray:
    """q [B,T,nh*hd], kc/vc [B,nkv,ctx,hd] (or None when ctx == 0), k/v [B,T,nkv*hd]."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    B, T = q.shape[0], q.shape[1]
    ctx = 0 if kc is None else kc.shape[2]
    kc, vc = _f32(kc), _f32(vc)
    if out is None:
        out = np.zeros((B, T, nh * hd), dtype=np.float32)
    rr, rp, nr = _rows(rows)
    _load().oracle_attn_split_gqa(_ptr(q), _ptr(kc), _ptr(vc), _ptr(k), _ptr(v), _ptr(out),
                                  B, T, ctx, nh, nkv, hd, float(scale), int(bool(causal)),
                                  rp, nr)
    return out


def relpos_attn(qkv, rh, rw, gh: int, gw: int, heads: int, hd: int, scale: float,
                rows=None, out=None) -> np.ndarray:
    """qkv [gh*gw, 3*heads*hd]; rh [gh,gh,hd], rw [gw,gw,hd] (both None => no bias)."""
    qkv, rh, rw = _f32(qkv), _f32(rh), _f32(rw)
    n = gh * gw
    if out is None:
        out = np.zeros((n, heads * hd), dtype=np.float32)
    rr, rp, nr = _rows(rows)
    _load().oracle_relpos_attn(_ptr(qkv), _ptr(rh), _ptr(rw), _ptr(out), gh, gw, heads, hd,
                               float(scale), rp, nr)
    return out


def pack16(x, fmt: int) -> np.ndarray:
    """f32 -> 16-bit storage (uint16 bit patterns), round to nearest, ties to even."""
    x = _f32(x)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().oracle_pack16(_ptr(x), out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)), x.size,
                          int(fmt))
    return out


def widen16(h, fmt: int) -> np.ndarray:
    """16-bit storage (uint16 bit patterns) -> the f32 values they hold (exact)."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, dtype=np.float32)
    _load().oracle_widen16(h.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)), _ptr(out), h.size,
                           int(fmt))
    return out
