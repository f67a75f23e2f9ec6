"""Python binding of libdgattn.so: the MI355X (gfx950) attention block.

The functions carry the names and the argument order of the C ABI in include/dgattn.h.  They
only marshal arguments: torch tensors become device pointers, the stream defaults to torch's
current stream, and every tensor is checked (float32, on the GPU, contiguous, large enough for
the extents passed) before the C call, so no launch can read or write past a tensor.  All
computation runs in the library's HIP kernels; there is no CPU path.  A missing library raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdgattn.so")

DG_OK, DG_EINVAL, DG_EUNSUPPORTED, DG_ELAUNCH = 0, -1, -2, -3
DG_NORM_WEIGHTED, DG_NORM_ROPE, DG_NORM_SKIP, DG_NORM_V_FROM_K = 1, 2, 4, 8
DG_KV_F16, DG_KV_BF16 = 1, 2
DG_NOALLOC_SCRATCH_BYTES = 32 << 20
DG_KERNEL_NONE, DG_KERNEL_SMALL, DG_KERNEL_TILE32 = 0, 1, 2


class AttnPlan(ctypes.Structure):
    """dg_attn_plan: how a split-GQA attention call is launched."""
    _fields_ = [("kernel", ctypes.c_int), ("query_block", ctypes.c_int), ("nsplit", ctypes.c_int),
                ("workgroups", ctypes.c_longlong), ("workspace_bytes", ctypes.c_size_t)]

EXPORTS = ("dg_rope_table", "dg_headnorm_rope", "dg_qkv_headnorm_rope", "dg_pack_kv16",
           "dg_qkv_headnorm_rope_kv16",
           "dg_attn_split_gqa_workspace_size", "dg_attn_split_gqa_plan", "dg_attn_split_gqa",
           "dg_attn_split_gqa_qnorm",
           "dg_attn_split_gqa_qkvnorm", "dg_attn_split_gqa_kv16", "dg_attn_split_gqa_noalloc",
           "relpos_flash_attn_workspace_size", "relpos_flash_attn", "relpos_flash_attn_ws",
           "relpos_flash_attn_windows_workspace_size", "relpos_flash_attn_windows",
           "dg_last_error")


class DgError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("status %d: %s" % (status, message))
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libdgattn.so (built by ``python -m gqa_flash_attention_dg_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libdgattn.so is not built (run: python -m "
                               "gqa_flash_attention_dg_amd.build); there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        vp, I, F, D, U, Z = (ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_double,
                             ctypes.c_uint, ctypes.c_size_t)
        L.dg_rope_table.argtypes = [vp, I, I, I, D, vp]
        L.dg_headnorm_rope.argtypes = [vp, vp, vp, I, I, I, I, U, F, vp]
        L.dg_qkv_headnorm_rope.argtypes = [vp, vp, vp, vp, vp, vp, I, I, I, I, I, U, F, vp]
        L.dg_pack_kv16.argtypes = [vp, vp, Z, I, vp]
        L.dg_qkv_headnorm_rope_kv16.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, I, I, I, I, I, U,
                                                F, I, vp]
        L.dg_attn_split_gqa_kv16.argtypes = [vp, vp, vp, vp, vp, vp, I, I, I, I, I, I, F, I, I, vp,
                                             Z, vp]
        L.dg_attn_split_gqa_workspace_size.argtypes = [I, I, I, I, I, I]
        L.dg_attn_split_gqa_workspace_size.restype = Z
        L.dg_attn_split_gqa_plan.argtypes = [I, I, I, I, I, I, I, I, I, ctypes.POINTER(AttnPlan)]
        L.dg_attn_split_gqa_plan.restype = I
        L.dg_attn_split_gqa.argtypes = [vp, vp, vp, vp, vp, vp, I, I, I, I, I, I, F, I, vp, Z, vp]
        L.dg_attn_split_gqa_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, I, I, I, I, I, I, F, I, vp]
        L.dg_attn_split_gqa_qnorm.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, I, I, I, I, I, I, U,
                                              F, F, I, vp, Z, vp]
        L.dg_attn_split_gqa_qkvnorm.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, I, I, I, I, I,
                                                I, U, F, F, I, vp, Z, vp]
        L.relpos_flash_attn_workspace_size.argtypes = [I, I, I, I]
        L.relpos_flash_attn_workspace_size.restype = Z
        L.relpos_flash_attn.argtypes = [vp, vp, vp, vp, I, I, I, I, F, vp]
        L.relpos_flash_attn_ws.argtypes = [vp, vp, vp, vp, I, I, I, I, F, vp, Z, vp]
        L.relpos_flash_attn_windows_workspace_size.argtypes = [I, I, I, I, I]
        L.relpos_flash_attn_windows_workspace_size.restype = Z
        L.relpos_flash_attn_windows.argtypes = [vp, vp, vp, vp, I, I, I, I, I, F, vp, Z, vp]
        for name in ("dg_rope_table", "dg_headnorm_rope", "dg_qkv_headnorm_rope", "dg_pack_kv16",
                     "dg_qkv_headnorm_rope_kv16",
                     "dg_attn_split_gqa", "dg_attn_split_gqa_qnorm", "dg_attn_split_gqa_qkvnorm",
                     "dg_attn_split_gqa_kv16", "dg_attn_split_gqa_noalloc", "relpos_flash_attn",
                     "relpos_flash_attn_ws",
                     "relpos_flash_attn_windows"):
            getattr(L, name).restype = I
        L.dg_last_error.argtypes = []
        L.dg_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def dg_last_error() -> str:
    return lib().dg_last_error().decode()


def _check(status: int) -> None:
    if status != DG_OK:
        raise DgError(status, dg_last_error())


def _ptr(t, name: str, need: int):
    """Device pointer of a float32 tensor holding at least `need` elements (None -> NULL)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor or None" % name)
    if t.dtype != torch.float32:
        raise TypeError("%s must be float32, got %s" % (name, t.dtype))
    if t.device.type != "cuda":
        raise ValueError("%s must be on the GPU, got %s" % (name, t.device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if t.numel() < need:
        raise ValueError("%s holds %d elements, the call needs %d" % (name, t.numel(), need))
    return t.data_ptr() if t.numel() > 0 else None


def _ptr16(t, name: str, need: int):
    """Device pointer of a tensor of 16-bit elements (uint16/int16/float16/bfloat16 storage of
    f16 or bf16 bit patterns) holding at least `need` elements (None -> NULL)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor or None" % name)
    if t.element_size() != 2:
        raise TypeError("%s must have 2-byte elements, got %s" % (name, t.dtype))
    if t.device.type != "cuda":
        raise ValueError("%s must be on the GPU, got %s" % (name, t.device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if t.numel() < need:
        raise ValueError("%s holds %d elements, the call needs %d" % (name, t.numel(), need))
    return t.data_ptr() if t.numel() > 0 else None


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _nonneg(**kw):
    for k, v in kw.items():
        if int(v) < 0:
            # the C side reports this too; refuse here before sizing any buffer check
            raise DgError(DG_EINVAL, "%s must be >= 0, got %d" % (k, v))


def dg_rope_table(cs, pos0: int, T: int, hd: int, theta: float, stream=None) -> None:
    _nonneg(T=T, hd=hd)
    _check(lib().dg_rope_table(_ptr(cs, "cs", T * 2 * hd), pos0, T, hd, float(theta),
                               _stream(stream)))


def dg_headnorm_rope(x, w, cs, batch: int, T: int, heads: int, hd: int, flags: int, eps: float,
                     stream=None) -> None:
    _nonneg(batch=batch, T=T, heads=heads, hd=hd)
    need_w = (flags & DG_NORM_WEIGHTED) and not (flags & DG_NORM_SKIP)
    need_cs = flags & DG_NORM_ROPE
    _check(lib().dg_headnorm_rope(_ptr(x, "x", batch * T * heads * hd),
                                  _ptr(w, "w", hd if need_w else 0),
                                  _ptr(cs, "cs", T * 2 * hd if need_cs else 0),
                                  batch, T, heads, hd, flags, float(eps), _stream(stream)))


def dg_qkv_headnorm_rope(q, wq, k, wk, v, cs, batch: int, T: int, nh: int, nkv: int, hd: int,
                         flags: int, eps: float, stream=None) -> None:
    _nonneg(batch=batch, T=T, nh=nh, nkv=nkv, hd=hd)
    need_w = (flags & DG_NORM_WEIGHTED) and not (flags & DG_NORM_SKIP)
    need_cs = (flags & DG_NORM_ROPE) and (q is not None or k is not None)
    nq, nk = batch * T * nh * hd, batch * T * nkv * hd
    _check(lib().dg_qkv_headnorm_rope(
        _ptr(q, "q", nq), _ptr(wq, "wq", hd if need_w and q is not None else 0),
        _ptr(k, "k", nk), _ptr(wk, "wk", hd if need_w and k is not None else 0),
        _ptr(v, "v", nk), _ptr(cs, "cs", T * 2 * hd if need_cs else 0),
        batch, T, nh, nkv, hd, flags, float(eps), _stream(stream)))


def dg_qkv_headnorm_rope_kv16(q, wq, k, wk, v, cs, k16, v16, batch: int, T: int, nh: int,
                              nkv: int, hd: int, flags: int, eps: float, kv_format: int,
                              stream=None) -> None:
    _nonneg(batch=batch, T=T, nh=nh, nkv=nkv, hd=hd)
    need_w = (flags & DG_NORM_WEIGHTED) and not (flags & DG_NORM_SKIP)
    need_cs = (flags & DG_NORM_ROPE) and (q is not None or k is not None)
    nq, nk = batch * T * nh * hd, batch * T * nkv * hd
    _check(lib().dg_qkv_headnorm_rope_kv16(
        _ptr(q, "q", nq), _ptr(wq, "wq", hd if need_w and q is not None else 0),
        _ptr(k, "k", nk), _ptr(wk, "wk", hd if need_w and k is not None else 0),
        _ptr(v, "v", nk), _ptr(cs, "cs", T * 2 * hd if need_cs else 0),
        _ptr16(k16, "k16", nk if k is not None else 0),
        _ptr16(v16, "v16", nk if v is not None else 0),
        batch, T, nh, nkv, hd, flags, float(eps), int(kv_format), _stream(stream)))


def dg_pack_kv16(src, dst, n: int, format: int, stream=None) -> None:
    _nonneg(n=n)
    _check(lib().dg_pack_kv16(_ptr(src, "src", n), _ptr16(dst, "dst", n), n, int(format),
                              _stream(stream)))


def dg_attn_split_gqa_workspace_size(batch: int, T: int, ctx: int, nh: int, nkv: int,
                                     hd: int) -> int:
    return int(lib().dg_attn_split_gqa_workspace_size(batch, T, ctx, nh, nkv, hd))


def dg_attn_split_gqa_plan(batch: int, T: int, ctx: int, nh: int, nkv: int, hd: int,
                           causal: int = 0, kv_format: int = 0, cus: int = 0) -> AttnPlan:
    """The launch plan of a split-GQA attention call (cus = 0: the current device's CUs)."""
    p = AttnPlan()
    _check(lib().dg_attn_split_gqa_plan(batch, T, ctx, nh, nkv, hd, int(causal), int(kv_format),
                                        int(cus), ctypes.byref(p)))
    return p


def _workspace(workspace, workspace_bytes):
    if workspace is None:
        return None, 0
    if not isinstance(workspace, torch.Tensor) or workspace.device.type != "cuda" or \
            not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    if workspace.numel() * workspace.element_size() < workspace_bytes:
        raise ValueError("workspace is smaller than workspace_bytes")
    return workspace.data_ptr(), int(workspace_bytes)


def dg_attn_split_gqa(q, kc, vc, k, v, out, batch: int, T: int, ctx: int, nh: int, nkv: int,
                      hd: int, scale: float, causal: int, workspace=None,
                      workspace_bytes: int = 0, stream=None) -> None:
    _nonneg(batch=batch, T=T, ctx=ctx, nh=nh, nkv=nkv, hd=hd)
    nq, nkvc, nc = batch * T * nh * hd, batch * T * nkv * hd, batch * nkv * ctx * hd
    ws, wsb = _workspace(workspace, workspace_bytes)
    _check(lib().dg_attn_split_gqa(_ptr(q, "q", nq), _ptr(kc, "kc", nc), _ptr(vc, "vc", nc),
                                   _ptr(k, "k", nkvc), _ptr(v, "v", nkvc), _ptr(out, "out", nq),
                                   batch, T, ctx, nh, nkv, hd, float(scale), int(causal), ws,
                                   wsb, _stream(stream)))


def dg_attn_split_gqa_noalloc(q, kc, vc, k, v, out, batch: int, T: int, ctx: int, nh: int,
                              nkv: int, hd: int, scale: float, causal: int, stream=None) -> None:
    _nonneg(batch=batch, T=T, ctx=ctx, nh=nh, nkv=nkv, hd=hd)
    nq, nkvc, nc = batch * T * nh * hd, batch * T * nkv * hd, batch * nkv * ctx * hd
    _check(lib().dg_attn_split_gqa_noalloc(_ptr(q, "q", nq), _ptr(kc, "kc", nc), _ptr(vc, "vc", nc),
                                           _ptr(k, "k", nkvc), _ptr(v, "v", nkvc),
                                           _ptr(out, "out", nq), batch, T, ctx, nh, nkv, hd,
                                           float(scale), int(causal), _stream(stream)))


def dg_attn_split_gqa_qnorm(q, wq, cs, kc, vc, k, v, out, batch: int, T: int, ctx: int, nh: int,
                            nkv: int, hd: int, qflags: int, eps: float, scale: float,
                            causal: int, workspace=None, workspace_bytes: int = 0,
                            stream=None) -> None:
    _nonneg(batch=batch, T=T, ctx=ctx, nh=nh, nkv=nkv, hd=hd)
    nq, nkvc, nc = batch * T * nh * hd, batch * T * nkv * hd, batch * nkv * ctx * hd
    need_w = (qflags & DG_NORM_WEIGHTED) and not (qflags & DG_NORM_SKIP)
    need_cs = qflags & DG_NORM_ROPE
    ws, wsb = _workspace(workspace, workspace_bytes)
    _check(lib().dg_attn_split_gqa_qnorm(
        _ptr(q, "q", nq), _ptr(wq, "wq", hd if need_w else 0),
        _ptr(cs, "cs", T * 2 * hd if need_cs else 0), _ptr(kc, "kc", nc), _ptr(vc, "vc", nc),
        _ptr(k, "k", nkvc), _ptr(v, "v", nkvc), _ptr(out, "out", nq), batch, T, ctx, nh, nkv, hd,
        qflags, float(eps), float(scale), int(causal), ws, wsb, _stream(stream)))


def dg_attn_split_gqa_qkvnorm(q, wq, k, wk, v, cs, kc, vc, out, batch: int, T: int, ctx: int,
                              nh: int, nkv: int, hd: int, flags: int, eps: float, scale: float,
                              causal: int, workspace=None, workspace_bytes: int = 0,
                              stream=None) -> None:
    _nonneg(batch=batch, T=T, ctx=ctx, nh=nh, nkv=nkv, hd=hd)
    nq, nkvc, nc = batch * T * nh * hd, batch * T * nkv * hd, batch * nkv * ctx * hd
    need_w = flags & DG_NORM_WEIGHTED
    need_cs = flags & DG_NORM_ROPE
    ws, wsb = _workspace(workspace, workspace_bytes)
    _check(lib().dg_attn_split_gqa_qkvnorm(
        _ptr(q, "q", nq), _ptr(wq, "wq", hd if need_w else 0), _ptr(k, "k", nkvc),
        _ptr(wk, "wk", hd if need_w else 0), _ptr(v, "v", nkvc),
        _ptr(cs, "cs", T * 2 * hd if need_cs else 0), _ptr(kc, "kc", nc), _ptr(vc, "vc", nc),
        _ptr(out, "out", nq), batch, T, ctx, nh, nkv, hd, flags, float(eps), float(scale),
        int(causal), ws, wsb, _stream(stream)))


def dg_attn_split_gqa_kv16(q, kc, vc, k, v, out, batch: int, T: int, ctx: int, nh: int, nkv: int,
                           hd: int, scale: float, causal: int, kv_format: int, workspace=None,
                           workspace_bytes: int = 0, stream=None) -> None:
    _nonneg(batch=batch, T=T, ctx=ctx, nh=nh, nkv=nkv, hd=hd)
    nq, nkvc, nc = batch * T * nh * hd, batch * T * nkv * hd, batch * nkv * ctx * hd
    ws, wsb = _workspace(workspace, workspace_bytes)
    _check(lib().dg_attn_split_gqa_kv16(
        _ptr(q, "q", nq), _ptr16(kc, "kc", nc), _ptr16(vc, "vc", nc), _ptr16(k, "k", nkvc),
        _ptr16(v, "v", nkvc), _ptr(out, "out", nq), batch, T, ctx, nh, nkv, hd, float(scale),
        int(causal), int(kv_format), ws, wsb, _stream(stream)))


def relpos_flash_attn_workspace_size(gh: int, gw: int, heads: int, hd: int) -> int:
    return int(lib().relpos_flash_attn_workspace_size(gh, gw, heads, hd))


def relpos_flash_attn(qkv, rh, rw, out, gh: int, gw: int, heads: int, hd: int, scale: float,
                      stream=None) -> None:
    _nonneg(gh=gh, gw=gw, heads=heads, hd=hd)
    n, W = gh * gw, heads * hd
    _check(lib().relpos_flash_attn(_ptr(qkv, "qkv", n * 3 * W), _ptr(rh, "rh", gh * gh * hd),
                                   _ptr(rw, "rw", gw * gw * hd), _ptr(out, "out", n * W),
                                   gh, gw, heads, hd, float(scale), _stream(stream)))


def relpos_flash_attn_ws(qkv, rh, rw, out, gh: int, gw: int, heads: int, hd: int, scale: float,
                         workspace=None, workspace_bytes: int = 0, stream=None) -> None:
    _nonneg(gh=gh, gw=gw, heads=heads, hd=hd)
    n, W = gh * gw, heads * hd
    ws, wsb = _workspace(workspace, workspace_bytes)
    _check(lib().relpos_flash_attn_ws(_ptr(qkv, "qkv", n * 3 * W), _ptr(rh, "rh", gh * gh * hd),
                                      _ptr(rw, "rw", gw * gw * hd), _ptr(out, "out", n * W),
                                      gh, gw, heads, hd, float(scale), ws, wsb, _stream(stream)))


def relpos_flash_attn_windows_workspace_size(nwin: int, gh: int, gw: int, heads: int,
                                             hd: int) -> int:
    return int(lib().relpos_flash_attn_windows_workspace_size(nwin, gh, gw, heads, hd))


def relpos_flash_attn_windows(qkv, rh, rw, out, nwin: int, gh: int, gw: int, heads: int, hd: int,
                              scale: float, workspace=None, workspace_bytes: int = 0,
                              stream=None) -> None:
    _nonneg(nwin=nwin, gh=gh, gw=gw, heads=heads, hd=hd)
    n, W = gh * gw, heads * hd
    ws, wsb = _workspace(workspace, workspace_bytes)
    _check(lib().relpos_flash_attn_windows(
        _ptr(qkv, "qkv", nwin * n * 3 * W), _ptr(rh, "rh", gh * gh * hd),
        _ptr(rw, "rw", gw * gw * hd), _ptr(out, "out", nwin * n * W), nwin, gh, gw, heads, hd,
        float(scale), ws, wsb, _stream(stream)))
