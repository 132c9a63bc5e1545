"""Python binding of ``libkvx.so`` (argument marshalling only).

Every function here converts torch tensors to raw pointers and sizes, picks
the current HIP stream and calls the C entry point of the same name; all
computation runs in the library's HIP kernels.  Device workspaces are
allocated with torch when the caller does not pass one.

Raises ``KvxError`` with the library's status when a call fails, and
``RuntimeError`` at import of a call when the library has not been built
(there is no other implementation to fall back on).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkvx.so")

F32, BF16 = 0, 1
OK, ERR_INVALID, ERR_SHAPE, ERR_WORKSPACE, ERR_NOT_SPD, ERR_HIP, ERR_UNSUPPORTED, ERR_NOT_CONVERGED = range(8)

EXPORTS = (
    "kvx_status_string", "kvx_align_workspace_size", "kvx_align_tokens", "kvx_align_batched_workspace_size",
    "kvx_align_tokens_batched", "kvx_layer_map", "kvx_translate_workspace_size", "kvx_translate",
    "kvx_translate_timed", "kvx_translate_placed_workspace_size", "kvx_translate_placed", "kvx_gather_features",
    "kvx_fit_ridge_workspace_size", "kvx_fit_ridge", "kvx_fit_ridge_batched_workspace_size",
    "kvx_fit_ridge_batched", "kvx_fit_recolor_workspace_size", "kvx_fit_recolor", "kvx_fold_lowrank",
    "kvx_quantize_fp8", "kvx_translate_fp8", "kvx_align_tokens_async", "kvx_translate_recorded",
    "kvx_align_tokens_noalloc", "kvx_prepared_maps_size", "kvx_prepare_maps",
    "kvx_translate_prepared_workspace_size", "kvx_translate_prepared", "kvx_probe_hbm", "kvx_probe_mfma",
    "kvx_probe_scratch_words", "kvx_fit_ridge_caches_workspace_size", "kvx_fit_ridge_caches",
    "kvx_fit_recolor_caches_workspace_size", "kvx_fit_recolor_caches",
)


class KvxError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class CacheDesc(ctypes.Structure):
    _fields_ = [("layers", ctypes.c_int32), ("tokens", ctypes.c_int32), ("kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32), ("rope_base", ctypes.c_double),
                ("k_norm", ctypes.c_void_p), ("k_norm_eps", ctypes.c_double)]


class Placement(ctypes.Structure):
    _fields_ = [("slot", ctypes.c_void_p), ("pool_rows", ctypes.c_int64), ("recv_pos", ctypes.c_void_p),
                ("send_pos", ctypes.c_void_p), ("pos_limit", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (built beforehand by ``cross_model_kv_kvx_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m cross_model_kv_kvx_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz, dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_double
        dp = ctypes.POINTER(CacheDesc)
        ip = ctypes.POINTER(ctypes.c_int32)
        vpp = ctypes.POINTER(ctypes.c_void_p)
        sig = {
            "kvx_status_string": (ctypes.c_char_p, [ctypes.c_int]),
            "kvx_align_workspace_size": (sz, [i32]),
            "kvx_align_tokens": (ctypes.c_int, [vp, i32, vp, i32, vp, vp, sz, vp]),
            "kvx_align_batched_workspace_size": (sz, [ip, i32]),
            "kvx_align_tokens_batched": (ctypes.c_int, [vp, ip, vp, ip, i32, vp, vp, sz, vp]),
            "kvx_layer_map": (ctypes.c_int, [i32, i32, i32, i32, ip]),
            "kvx_translate_workspace_size": (sz, [dp, dp, i32, i32]),
            "kvx_translate": (ctypes.c_int, [dp, vp, vp, dp, vp, vp, vp, ip, i32, i32, i32, vp, vp, vp, vp,
                                             vp, sz, vp]),
            "kvx_translate_timed": (ctypes.c_int, [dp, vp, vp, dp, vp, vp, vp, ip, i32, i32, i32, vp, vp, vp, vp,
                                                   vp, sz, vp, ctypes.POINTER(ctypes.c_float)]),
            "kvx_translate_placed_workspace_size": (sz, [dp, dp, i32, i32, i32]),
            "kvx_translate_placed": (ctypes.c_int, [dp, vp, vp, dp, vp, vp, vp, ip, i32, i32, i32, vp, vp, vp, vp,
                                                    vp, sz, vp, ctypes.POINTER(Placement)]),
            "kvx_gather_features": (ctypes.c_int, [dp, vp, i32, vp, i32, ip, i32, vp, vp]),
            "kvx_fit_ridge_workspace_size": (sz, [i32, i32]),
            "kvx_fit_ridge": (ctypes.c_int, [vp, i64, vp, i64, i32, i64, i32, i32, dbl, dbl, i32, vp, vp, vp, sz,
                                             vp]),
            "kvx_fit_ridge_batched_workspace_size": (sz, [i32, i32, i32]),
            "kvx_fit_ridge_caches_workspace_size": (sz, [dp, dp, i32]),
            "kvx_fit_ridge_caches": (ctypes.c_int, [dp, vp, vp, dp, vp, vp, vp, ip, i32, dbl, dbl, vp, vp, ip, vp,
                                                    sz, vp]),
            "kvx_fit_recolor_caches_workspace_size": (sz, [dp, dp, i32]),
            "kvx_fit_recolor_caches": (ctypes.c_int, [dp, vp, vp, dp, vp, vp, vp, ip, i32, dbl, dbl, vp, vp, vp, vp,
                                                      ip, ip, vp, sz, vp]),
            "kvx_fit_ridge_batched": (ctypes.c_int, [i32, vpp, i64, vpp, i64, i32, i64, i32, i32, dbl, dbl, i32,
                                                     vpp, vpp, ip, vp, sz, vp]),
            "kvx_fit_recolor_workspace_size": (sz, [i32, i32, i32]),
            "kvx_fit_recolor": (ctypes.c_int, [i32, vpp, i64, vpp, i64, i32, i64, i32, i32, dbl, dbl, vpp, vpp,
                                               ip, ip, vp, sz, vp]),
            "kvx_fold_lowrank": (ctypes.c_int, [vp, vp, vp, i32, i32, i32, i32, vp, i32, vp]),
            "kvx_quantize_fp8": (ctypes.c_int, [vp, i32, i32, i32, vp, vp, vp]),
            "kvx_prepared_maps_size": (sz, [dp, dp, i32, i32, i32, i32]),
            "kvx_probe_hbm": (ctypes.c_int, [i32, vp, vp, i64, i32, ctypes.POINTER(ctypes.c_float), vp]),
            "kvx_probe_mfma": (ctypes.c_int, [vp, i32, i32, ctypes.POINTER(ctypes.c_float),
                                              ctypes.POINTER(ctypes.c_double), vp]),
            "kvx_probe_scratch_words": (i32, []),
            "kvx_prepare_maps": (ctypes.c_int, [dp, dp, i32, i32, i32, i32, vp, vp, sz, vp]),
            "kvx_translate_prepared_workspace_size": (sz, [dp, dp, i32, i32, i32]),
            "kvx_translate_prepared": (ctypes.c_int, [dp, vp, vp, dp, vp, vp, vp, ip, i32, i32, i32, vp, vp, vp,
                                                      vp, vp, sz, vp, ctypes.POINTER(Placement), vpp]),
            "kvx_align_tokens_async": (ctypes.c_int, [vp, i32, vp, i32, vp, vp, vp, sz, vp]),
            "kvx_align_tokens_noalloc": (ctypes.c_int, [vp, i32, vp, i32, vp, vp, vp]),
            "kvx_translate_recorded": (ctypes.c_int, [dp, vp, vp, dp, vp, vp, vp, ip, i32, i32, i32, vp, vp, vp,
                                                      vp, vp, sz, vp, vpp]),
            "kvx_translate_fp8": (ctypes.c_int, [dp, vp, vp, dp, vp, vp, vp, ip, i32, vp, vp, vp, vp, vp, vp, vp,
                                                 sz, vp, ctypes.POINTER(ctypes.c_float)]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().kvx_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != OK:
        raise KvxError(status, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _need(t: torch.Tensor, name: str, dtype=None, device=True):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if device and not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]) -> torch.Tensor:
    if ws is not None:
        return ws
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def cache_desc(cache: torch.Tensor, rope_base: float = 0.0, tokens: Optional[int] = None) -> CacheDesc:
    """Descriptor of a [layers][tokens][heads][head_dim] cache tensor."""
    L, N, H, d = cache.shape
    return CacheDesc(int(L), int(N if tokens is None else tokens), int(H), int(d), _dtype_code(cache),
                     float(rope_base))


# ---------------------------------------------------------------- entry points


def align_tokens(send_end: torch.Tensor, recv_end: torch.Tensor, out: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None, stream=None,
                 invalid: Optional[torch.Tensor] = None) -> torch.Tensor:
    """kvx_align_tokens: receiver->sender token map (device int32).  With a
    device int32 tensor ``invalid`` (one element), kvx_align_tokens_async
    instead: no synchronisation, the validity flag is left in ``invalid``."""
    _need(send_end, "send_end", torch.int32)
    _need(recv_end, "recv_end", torch.int32)
    n_r = recv_end.numel()
    if out is None:
        out = torch.empty(n_r, dtype=torch.int32, device=recv_end.device)
    _need(out, "out", torch.int32)
    ws = _workspace(lib().kvx_align_workspace_size(n_r), recv_end.device, workspace)
    if invalid is not None:
        _need(invalid, "invalid", torch.int32)
        st = lib().kvx_align_tokens_async(_ptr(send_end), send_end.numel(), _ptr(recv_end), n_r, _ptr(out),
                                          _ptr(invalid), _ptr(ws), ws.numel(), _stream(stream))
        _check(st, "kvx_align_tokens_async")
        return out
    st = lib().kvx_align_tokens(_ptr(send_end), send_end.numel(), _ptr(recv_end), n_r, _ptr(out), _ptr(ws),
                                ws.numel(), _stream(stream))
    _check(st, "kvx_align_tokens")
    return out


def align_tokens_noalloc(send_end: torch.Tensor, recv_end: torch.Tensor, out: torch.Tensor,
                         invalid: torch.Tensor, stream=None) -> torch.Tensor:
    """kvx_align_tokens_noalloc: the asynchronous alignment with the library's
    static scratch; ``out`` (device int32 [n_recv]) and ``invalid`` (device
    int32, one element) are the caller's, nothing is allocated."""
    _need(send_end, "send_end", torch.int32)
    _need(recv_end, "recv_end", torch.int32)
    _need(out, "out", torch.int32)
    _need(invalid, "invalid", torch.int32)
    if out.numel() != recv_end.numel():
        raise ValueError("out must have one entry per receiver token")
    st = lib().kvx_align_tokens_noalloc(_ptr(send_end), send_end.numel(), _ptr(recv_end), recv_end.numel(),
                                        _ptr(out), _ptr(invalid), _stream(stream))
    _check(st, "kvx_align_tokens_noalloc")
    return out


def align_tokens_batched(send_end: torch.Tensor, send_off, recv_end: torch.Tensor, recv_off,
                         out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                         stream=None) -> torch.Tensor:
    """kvx_align_tokens_batched: sequences concatenated (host offsets of
    n_seq + 1 entries); returns the map into the concatenated sender tokens."""
    _need(send_end, "send_end", torch.int32)
    _need(recv_end, "recv_end", torch.int32)
    so = np.ascontiguousarray(send_off, dtype=np.int32)
    ro = np.ascontiguousarray(recv_off, dtype=np.int32)
    n_seq = ro.size - 1
    if so.size != ro.size or n_seq < 1:
        raise ValueError("send_off and recv_off need n_seq + 1 entries")
    ip = ctypes.POINTER(ctypes.c_int32)
    if out is None:
        out = torch.empty(int(ro[-1]), dtype=torch.int32, device=recv_end.device)
    _need(out, "out", torch.int32)
    ws = _workspace(lib().kvx_align_batched_workspace_size(ro.ctypes.data_as(ip), n_seq), recv_end.device, workspace)
    st = lib().kvx_align_tokens_batched(_ptr(send_end), so.ctypes.data_as(ip), _ptr(recv_end), ro.ctypes.data_as(ip),
                                        n_seq, _ptr(out), _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "kvx_align_tokens_batched")
    return out


def layer_map(send_layers: int, recv_layers: int, n_taps: int = 3, tap_stride: int = 4) -> np.ndarray:
    """kvx_layer_map: host int32 [recv_layers][n_taps]."""
    out = np.zeros((recv_layers, n_taps), dtype=np.int32)
    st = lib().kvx_layer_map(int(send_layers), int(recv_layers), int(n_taps), int(tap_stride),
                             out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
    _check(st, "kvx_layer_map")
    return out


def translate_workspace_size(send: CacheDesc, recv: CacheDesc, n_taps: int, per_head: bool) -> int:
    return int(lib().kvx_translate_workspace_size(ctypes.byref(send), ctypes.byref(recv), int(n_taps),
                                                   int(bool(per_head))))


def translate(k_send: Optional[torch.Tensor], v_send: Optional[torch.Tensor], recv_to_send: torch.Tensor,
              taps, w_k: Optional[torch.Tensor], w_v: Optional[torch.Tensor],
              b_k: Optional[torch.Tensor] = None, b_v: Optional[torch.Tensor] = None, *,
              recv_layers: Optional[int] = None, recv_heads: Optional[int] = None,
              recv_head_dim: Optional[int] = None, per_head: bool = False,
              send_rope_base: float = 0.0, recv_rope_base: float = 0.0,
              k_recv: Optional[torch.Tensor] = None, v_recv: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None, stream=None, stage_ms: Optional[list] = None,
              recv_key_norm: Optional[torch.Tensor] = None, key_norm_eps: float = 1e-6,
              slot: Optional[torch.Tensor] = None, pool_rows: Optional[int] = None,
              recv_pos: Optional[torch.Tensor] = None, send_pos: Optional[torch.Tensor] = None,
              pos_limit: Optional[int] = None, events=None, prepared: bool = False,
              w_dtype: Optional[int] = None):
    """kvx_translate.  Returns (k_recv, v_recv) (either None when its role is
    skipped).  ``taps``: host int32 [L_R][n_taps] (numpy).  ``w_k``, ``w_v``:
    row-major maps [L_R][F_in][F_out] (per head [L_R][H][d][d], w[l][h][c][o]),
    fp32 or bf16.  With a list ``stage_ms``, calls kvx_translate_timed
    instead (synchronous) and appends the [preparation, translation kernel]
    device times in ms.  With three recorded torch.cuda.Event objects
    ``events``, calls kvx_translate_recorded (asynchronous; the events mark
    the phases).  With ``prepared`` (and ``w_dtype``, F32 or BF16, the type
    they were prepared from), ``w_k``/``w_v`` are buffers from
    ``prepare_maps`` and kvx_translate_prepared runs (placement and events
    allowed, no stage timing)."""
    ref = k_send if k_send is not None else v_send
    if ref is None:
        raise ValueError("at least one role is needed")
    taps = np.ascontiguousarray(taps, dtype=np.int32)
    L_R, n_taps = taps.shape
    if recv_layers is not None and recv_layers != L_R:
        raise ValueError("taps rows must equal recv_layers")
    _need(recv_to_send, "recv_to_send", torch.int32)
    for name, t in (("k_send", k_send), ("v_send", v_send)):
        if t is not None:
            _need(t, name, ref.dtype)
    w_ref = w_k if w_k is not None else w_v
    H_R = recv_heads if recv_heads is not None else ref.shape[2]
    d_R = recv_head_dim if recv_head_dim is not None else ref.shape[3]
    N_R = recv_to_send.numel()
    send = cache_desc(ref, send_rope_base)
    recv = CacheDesc(int(L_R), int(N_R), int(H_R), int(d_R), _dtype_code(ref), float(recv_rope_base))
    if recv_key_norm is not None:
        _need(recv_key_norm, "recv_key_norm", torch.float32)
        if tuple(recv_key_norm.shape) != (L_R, d_R):
            raise ValueError("recv_key_norm must be [recv_layers][head_dim]")
        recv.k_norm = recv_key_norm.data_ptr()
        recv.k_norm_eps = float(key_norm_eps)
    for name, t in (("w_k", w_k), ("w_v", w_v)):
        if t is not None:
            _need(t, name, w_ref.dtype)
    if prepared:
        if w_dtype not in (F32, BF16) or w_ref.dtype != torch.uint8:
            raise ValueError("prepared maps are uint8 buffers from prepare_maps, with w_dtype F32 or BF16")
        if stage_ms is not None:
            raise ValueError("stage timing is not available with prepared maps (use events)")
        code = int(w_dtype)
    else:
        code = _dtype_code(w_ref)
    for name, t in (("b_k", b_k), ("b_v", b_v)):
        if t is not None:
            _need(t, name, torch.float32)
    placed = any(x is not None for x in (slot, pool_rows, recv_pos, send_pos, pos_limit))
    rows = N_R if pool_rows is None else int(pool_rows)
    if k_send is not None and k_recv is None:
        k_recv = torch.empty((L_R, rows, H_R, d_R), dtype=ref.dtype, device=ref.device)
    if v_send is not None and v_recv is None:
        v_recv = torch.empty((L_R, rows, H_R, d_R), dtype=ref.dtype, device=ref.device)
    place = None
    if placed:
        if stage_ms is not None or (events is not None and not prepared):
            raise ValueError("stage timing is not available with a placement")
        for name, t, dt in (("slot", slot, torch.int64), ("recv_pos", recv_pos, torch.int32),
                            ("send_pos", send_pos, torch.int32)):
            if t is not None:
                _need(t, name, dt)
        place = Placement(slot.data_ptr() if slot is not None else None, 0 if pool_rows is None else rows,
                          recv_pos.data_ptr() if recv_pos is not None else None,
                          send_pos.data_ptr() if send_pos is not None else None,
                          int(pos_limit) if pos_limit is not None else 0)
    pl = place.pos_limit if place is not None else 0
    if prepared:
        nbytes = lib().kvx_translate_prepared_workspace_size(ctypes.byref(send), ctypes.byref(recv), int(n_taps),
                                                             int(bool(per_head)), pl)
    elif placed:
        nbytes = lib().kvx_translate_placed_workspace_size(ctypes.byref(send), ctypes.byref(recv), int(n_taps),
                                                           int(bool(per_head)), pl)
    else:
        nbytes = translate_workspace_size(send, recv, n_taps, per_head)
    ws = _workspace(nbytes, ref.device, workspace)
    args = [ctypes.byref(send), _ptr(k_send), _ptr(v_send), ctypes.byref(recv),
            _ptr(k_recv) if k_send is not None else None, _ptr(v_recv) if v_send is not None else None,
            _ptr(recv_to_send), taps.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), int(n_taps),
            int(bool(per_head)), code, _ptr(w_k), _ptr(w_v), _ptr(b_k), _ptr(b_v),
            _ptr(ws), ws.numel(), _stream(stream)]
    ev = None
    if events is not None:
        if len(events) != 3 or any(not e.cuda_event for e in events):
            raise ValueError("events must be three torch.cuda.Event objects that have been recorded once")
        ev = (ctypes.c_void_p * 3)(*[e.cuda_event for e in events])
    if prepared:
        _check(lib().kvx_translate_prepared(*args, ctypes.byref(place) if place is not None else None, ev),
               "kvx_translate_prepared")
    elif placed:
        _check(lib().kvx_translate_placed(*args, ctypes.byref(place)), "kvx_translate_placed")
    elif ev is not None:
        _check(lib().kvx_translate_recorded(*args, ev), "kvx_translate_recorded")
    elif stage_ms is None:
        _check(lib().kvx_translate(*args), "kvx_translate")
    else:
        ms = (ctypes.c_float * 2)()
        _check(lib().kvx_translate_timed(*args, ms), "kvx_translate_timed")
        stage_ms.extend([float(ms[0]), float(ms[1])])
    return (k_recv if k_send is not None else None), (v_recv if v_send is not None else None)


def prepare_maps(w: torch.Tensor, role: str, send: CacheDesc, recv: CacheDesc, n_taps: int,
                 per_head: bool = False, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """kvx_prepare_maps: the maps of one role ("k" or "v"; row-major as
    ``translate`` takes them, fp32 or bf16) in the kernel layout for
    translations with these descriptors; returns the device uint8 buffer to
    pass to ``translate(..., prepared=True, w_dtype=...)``."""
    _need(w, "w")
    r = {"k": 0, "v": 1}[role]
    code = _dtype_code(w)
    n = int(lib().kvx_prepared_maps_size(ctypes.byref(send), ctypes.byref(recv), int(n_taps), int(bool(per_head)), r,
                                         code))
    if n == 0:
        raise ValueError("invalid descriptors for prepared maps")
    if out is None:
        out = torch.empty(n, dtype=torch.uint8, device=w.device)
    _check(lib().kvx_prepare_maps(ctypes.byref(send), ctypes.byref(recv), int(n_taps), int(bool(per_head)), r, code,
                                  _ptr(w), _ptr(out), out.numel(), _stream(stream)), "kvx_prepare_maps")
    return out


def quantize_fp8(w: torch.Tensor, stream=None):
    """kvx_quantize_fp8 on row-major fp32 maps [count][f_in][f_out] (a single
    map may drop the leading dimension): returns (codes uint8
    [count][f_out][f_in], output-major, and scales fp32 [count][f_out])."""
    _need(w, "w", torch.float32)
    squeeze = w.dim() == 2
    if squeeze:
        w = w[None]
    count, f_in, f_out = w.shape
    q = torch.empty((count, f_out, f_in), dtype=torch.uint8, device=w.device)
    sc = torch.empty((count, f_out), dtype=torch.float32, device=w.device)
    _check(lib().kvx_quantize_fp8(_ptr(w), count, f_in, f_out, _ptr(q), _ptr(sc), _stream(stream)),
           "kvx_quantize_fp8")
    return (q[0], sc[0]) if squeeze else (q, sc)


def translate_fp8(k_send: Optional[torch.Tensor], v_send: Optional[torch.Tensor], recv_to_send: torch.Tensor,
                  taps, wq_k: Optional[torch.Tensor], wq_v: Optional[torch.Tensor], s_k: Optional[torch.Tensor],
                  s_v: Optional[torch.Tensor], b_k: Optional[torch.Tensor] = None,
                  b_v: Optional[torch.Tensor] = None, *, recv_heads: Optional[int] = None,
                  recv_head_dim: Optional[int] = None, send_rope_base: float = 0.0, recv_rope_base: float = 0.0,
                  k_recv: Optional[torch.Tensor] = None, v_recv: Optional[torch.Tensor] = None,
                  recv_key_norm: Optional[torch.Tensor] = None, key_norm_eps: float = 1e-6,
                  workspace: Optional[torch.Tensor] = None, stream=None, stage_ms: Optional[list] = None):
    """kvx_translate_fp8 (flattened maps stored as E4M3 codes wq [L_R][F_out][F_in]
    uint8 with scales s [L_R][F_out] fp32).  Returns (k_recv, v_recv).  With a
    list ``stage_ms`` the call is timed (synchronous) and the [preparation,
    translation kernel] device times in ms are appended."""
    ref = k_send if k_send is not None else v_send
    if ref is None:
        raise ValueError("at least one role is needed")
    taps = np.ascontiguousarray(taps, dtype=np.int32)
    L_R, n_taps = taps.shape
    _need(recv_to_send, "recv_to_send", torch.int32)
    for name, t, dt in (("k_send", k_send, ref.dtype), ("v_send", v_send, ref.dtype), ("wq_k", wq_k, torch.uint8),
                        ("wq_v", wq_v, torch.uint8), ("s_k", s_k, torch.float32), ("s_v", s_v, torch.float32),
                        ("b_k", b_k, torch.float32), ("b_v", b_v, torch.float32)):
        if t is not None:
            _need(t, name, dt)
    H_R = recv_heads if recv_heads is not None else ref.shape[2]
    d_R = recv_head_dim if recv_head_dim is not None else ref.shape[3]
    N_R = recv_to_send.numel()
    send = cache_desc(ref, send_rope_base)
    recv = CacheDesc(int(L_R), int(N_R), int(H_R), int(d_R), _dtype_code(ref), float(recv_rope_base))
    if recv_key_norm is not None:
        _need(recv_key_norm, "recv_key_norm", torch.float32)
        recv.k_norm = recv_key_norm.data_ptr()
        recv.k_norm_eps = float(key_norm_eps)
    if k_send is not None and k_recv is None:
        k_recv = torch.empty((L_R, N_R, H_R, d_R), dtype=ref.dtype, device=ref.device)
    if v_send is not None and v_recv is None:
        v_recv = torch.empty((L_R, N_R, H_R, d_R), dtype=ref.dtype, device=ref.device)
    ws = _workspace(translate_workspace_size(send, recv, n_taps, False), ref.device, workspace)
    ms = (ctypes.c_float * 2)() if stage_ms is not None else None
    st = lib().kvx_translate_fp8(ctypes.byref(send), _ptr(k_send), _ptr(v_send), ctypes.byref(recv),
                                 _ptr(k_recv) if k_send is not None else None,
                                 _ptr(v_recv) if v_send is not None else None, _ptr(recv_to_send),
                                 taps.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), int(n_taps), _ptr(wq_k),
                                 _ptr(wq_v), _ptr(s_k), _ptr(s_v), _ptr(b_k), _ptr(b_v), _ptr(ws), ws.numel(),
                                 _stream(stream), ms)
    _check(st, "kvx_translate_fp8")
    if ms is not None:
        stage_ms.extend([float(ms[0]), float(ms[1])])
    return (k_recv if k_send is not None else None), (v_recv if v_send is not None else None)


def gather_features(kv_send: torch.Tensor, recv_to_send: torch.Tensor, taps_of_layer: Sequence[int], *,
                    derotate: bool = False, rope_base: float = 0.0, out: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    """kvx_gather_features: [n_rows][n_taps*H*d] in the cache dtype."""
    _need(kv_send, "kv_send")
    _need(recv_to_send, "recv_to_send", torch.int32)
    taps = np.ascontiguousarray(taps_of_layer, dtype=np.int32).ravel()
    n = recv_to_send.numel()
    L, N, H, d = kv_send.shape
    if out is None:
        out = torch.empty((n, taps.size * H * d), dtype=kv_send.dtype, device=kv_send.device)
    _need(out, "out", kv_send.dtype)
    send = cache_desc(kv_send, rope_base)
    st = lib().kvx_gather_features(ctypes.byref(send), _ptr(kv_send), int(bool(derotate)), _ptr(recv_to_send), n,
                                   taps.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), taps.size, _ptr(out),
                                   _stream(stream))
    _check(st, "kvx_gather_features")
    return out


def fit_ridge(x: torch.Tensor, y: torch.Tensor, *, lambda_abs: float = 0.0, lambda_rel: float = 0.0,
              fit_intercept: bool = False, w_out: Optional[torch.Tensor] = None,
              b_out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None, stream=None):
    """kvx_fit_ridge on row-major 2-D x [n][f_in], y [n][f_out].  Returns
    (w fp32 [f_in][f_out], y = x w + b; b fp32 [f_out] or None)."""
    if x.dim() != 2 or y.dim() != 2 or x.shape[0] != y.shape[0]:
        raise ValueError("x and y must be 2-D with equal row counts")
    if x.stride(1) != 1 or y.stride(1) != 1:
        raise ValueError("rows of x and y must be contiguous")
    if x.dtype != y.dtype:
        raise TypeError("x and y must share a dtype")
    n, f_in = x.shape
    f_out = y.shape[1]
    if w_out is None:
        w_out = torch.empty((f_in, f_out), dtype=torch.float32, device=x.device)
    if fit_intercept and b_out is None:
        b_out = torch.empty(f_out, dtype=torch.float32, device=x.device)
    ws = _workspace(lib().kvx_fit_ridge_workspace_size(f_in, f_out), x.device, workspace)
    st = lib().kvx_fit_ridge(_ptr(x), x.stride(0), _ptr(y), y.stride(0), _dtype_code(x), n, f_in, f_out,
                             float(lambda_abs), float(lambda_rel), int(bool(fit_intercept)), _ptr(w_out),
                             _ptr(b_out) if fit_intercept else None, _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "kvx_fit_ridge")
    return w_out, (b_out if fit_intercept else None)


def fit_ridge_batched(xs, ys, *, lambda_abs: float = 0.0, lambda_rel: float = 0.0, fit_intercept: bool = False,
                      w_outs=None, b_outs=None, workspace: Optional[torch.Tensor] = None, stream=None,
                      status: Optional[list] = None):
    """kvx_fit_ridge_batched on lists of row-major 2-D x [n][f_in] and
    y [n][f_out] (one shape, one dtype, one row stride each).  Returns the
    lists (w fp32 [f_in][f_out], b fp32 [f_out] or None).  With a list
    ``status``, appends each problem's status and raises only for other
    errors."""
    count = len(xs)
    if count == 0 or len(ys) != count:
        raise ValueError("xs and ys must be non-empty lists of equal length")
    x0, y0 = xs[0], ys[0]
    for x, y in zip(xs, ys):
        if x.dim() != 2 or y.dim() != 2 or x.shape != x0.shape or y.shape != y0.shape:
            raise ValueError("every x (and every y) must be 2-D of one shape")
        if x.stride() != x0.stride() or y.stride() != y0.stride() or x.stride(1) != 1 or y.stride(1) != 1:
            raise ValueError("rows must be contiguous with one row stride per operand")
        if x.dtype != x0.dtype or y.dtype != x0.dtype:
            raise TypeError("x and y must share a dtype")
    n, f_in = x0.shape
    f_out = y0.shape[1]
    dev = x0.device
    if w_outs is None:
        w_outs = [torch.empty((f_in, f_out), dtype=torch.float32, device=dev) for _ in range(count)]
    if fit_intercept and b_outs is None:
        b_outs = [torch.empty(f_out, dtype=torch.float32, device=dev) for _ in range(count)]
    arr = ctypes.c_void_p * count
    xp, yp = arr(*[x.data_ptr() for x in xs]), arr(*[y.data_ptr() for y in ys])
    wp = arr(*[w.data_ptr() for w in w_outs])
    bp = arr(*[b.data_ptr() for b in b_outs]) if fit_intercept else None
    st_arr = (ctypes.c_int32 * count)()
    ws = _workspace(lib().kvx_fit_ridge_batched_workspace_size(count, f_in, f_out), dev, workspace)
    st = lib().kvx_fit_ridge_batched(count, xp, x0.stride(0), yp, y0.stride(0), _dtype_code(x0), n, f_in, f_out,
                                     float(lambda_abs), float(lambda_rel), int(bool(fit_intercept)), wp, bp, st_arr,
                                     _ptr(ws), ws.numel(), _stream(stream))
    if status is not None:
        status.extend(int(v) for v in st_arr)
        if st not in (OK, ERR_NOT_SPD):
            _check(st, "kvx_fit_ridge_batched")
    else:
        _check(st, "kvx_fit_ridge_batched")
    return w_outs, (b_outs if fit_intercept else [None] * count)


def fit_ridge_caches_workspace_size(send: CacheDesc, recv: CacheDesc, n_taps: int) -> int:
    return int(lib().kvx_fit_ridge_caches_workspace_size(ctypes.byref(send), ctypes.byref(recv), int(n_taps)))


class _CacheFit:
    """Arguments shared by the fits from the caches: the descriptors, the
    per-role pointers (null for a role not requested) and the shapes."""

    def __init__(self, k_send, v_send, k_recv, v_recv, taps, roles, send_rope=0.0, recv_rope=0.0):
        taps = np.ascontiguousarray(taps, dtype=np.int32)
        if taps.ndim != 2:
            raise ValueError("taps must be [L_R][n_taps]")
        self.taps = taps
        self.L_R, self.n_taps = taps.shape
        self.do_k, self.do_v = "k" in roles, "v" in roles
        if not (self.do_k or self.do_v):
            raise ValueError("roles must name k, v or both")
        ref_send = k_send if self.do_k else v_send
        ref_recv = k_recv if self.do_k else v_recv
        self.send, self.recv = cache_desc(ref_send, send_rope), cache_desc(ref_recv, recv_rope)
        if self.recv.layers != self.L_R:
            raise ValueError("taps rows must equal the receiver's layers")
        for t in (k_send, v_send, k_recv, v_recv):
            if t is not None and not t.is_contiguous():
                raise ValueError("caches must be contiguous")
        self.f_in = self.n_taps * self.send.kv_heads * self.send.head_dim
        self.f_out = self.recv.kv_heads * self.recv.head_dim
        self.dev = ref_send.device
        self.ptrs = (_ptr(k_send if self.do_k else None), _ptr(v_send if self.do_v else None),
                     _ptr(k_recv if self.do_k else None), _ptr(v_recv if self.do_v else None))

    def out(self, given, present, shape):
        if not present:
            return None
        return given if given is not None else torch.empty(shape, dtype=torch.float32, device=self.dev)

    def taps_ptr(self):
        return self.taps.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def fit_ridge_caches(k_send: Optional[torch.Tensor], v_send: Optional[torch.Tensor], k_recv: Optional[torch.Tensor],
                     v_recv: Optional[torch.Tensor], recv_to_send: torch.Tensor, taps, *, lambda_abs: float = 0.0,
                     lambda_rel: float = 0.0, w_k: Optional[torch.Tensor] = None, w_v: Optional[torch.Tensor] = None,
                     roles=("k", "v"), send_rope: float = 0.0, recv_rope: float = 0.0,
                     workspace: Optional[torch.Tensor] = None, stream=None, status: Optional[list] = None):
    """kvx_fit_ridge_caches: the ridge maps of every receiver layer of the
    requested ``roles`` from the calibration caches (bf16 [L][N][H][d]; the
    sender's N_S tokens, the receiver's N), the alignment ``recv_to_send``
    (device int32 [N]) and ``taps`` (host int32 [L_R][n_taps]).  Returns
    (w_k, w_v), fp32 [L_R][F_in][F_out] (None for a role not requested).
    ``send_rope`` / ``recv_rope`` > 0: the keys are stored rotated with that
    base (turned back at the sender / receiver position before the fit).
    With a list ``status``, appends the [2][L_R] per-problem statuses and
    raises only for other errors."""
    a = _CacheFit(k_send, v_send, k_recv, v_recv, taps, roles, send_rope, recv_rope)
    w_k = a.out(w_k, a.do_k, (a.L_R, a.f_in, a.f_out))
    w_v = a.out(w_v, a.do_v, (a.L_R, a.f_in, a.f_out))
    ws = _workspace(fit_ridge_caches_workspace_size(a.send, a.recv, a.n_taps), a.dev, workspace)
    st_arr = (ctypes.c_int32 * (2 * a.L_R))()
    ks, vs, kr, vr = a.ptrs
    st = lib().kvx_fit_ridge_caches(ctypes.byref(a.send), ks, vs, ctypes.byref(a.recv), kr, vr, _ptr(recv_to_send),
                                    a.taps_ptr(), int(a.n_taps), float(lambda_abs), float(lambda_rel), _ptr(w_k),
                                    _ptr(w_v), st_arr, _ptr(ws), ws.numel(), _stream(stream))
    if status is not None:
        status.extend(int(v) for v in st_arr)
        if st not in (OK, ERR_NOT_SPD):
            _check(st, "kvx_fit_ridge_caches")
    else:
        _check(st, "kvx_fit_ridge_caches")
    return w_k, w_v


def fit_recolor_caches_workspace_size(send: CacheDesc, recv: CacheDesc, n_taps: int) -> int:
    return int(lib().kvx_fit_recolor_caches_workspace_size(ctypes.byref(send), ctypes.byref(recv), int(n_taps)))


def fit_recolor_caches(k_send: Optional[torch.Tensor], v_send: Optional[torch.Tensor],
                       k_recv: Optional[torch.Tensor], v_recv: Optional[torch.Tensor], recv_to_send: torch.Tensor,
                       taps, *, rho_x: float = 0.0, rho_y: float = 0.0, w_k: Optional[torch.Tensor] = None,
                       w_v: Optional[torch.Tensor] = None, b_k: Optional[torch.Tensor] = None,
                       b_v: Optional[torch.Tensor] = None, roles=("k", "v"), send_rope: float = 0.0,
                       recv_rope: float = 0.0, workspace: Optional[torch.Tensor] = None, stream=None,
                       status: Optional[list] = None, info: Optional[dict] = None):
    """kvx_fit_recolor_caches: the Recolor maps of every receiver layer of
    the requested ``roles`` from the calibration caches, arguments as for
    fit_ridge_caches.  Returns (w_k, w_v, b_k, b_v): fp32 [L_R][F_in][F_out]
    and [L_R][F_out] (None for a role not requested).  With a list
    ``status``, appends the [2][L_R] per-problem statuses and raises only for
    other errors; with a dict ``info``, stores the polar iterations under
    "iters"."""
    a = _CacheFit(k_send, v_send, k_recv, v_recv, taps, roles, send_rope, recv_rope)
    w_k = a.out(w_k, a.do_k, (a.L_R, a.f_in, a.f_out))
    w_v = a.out(w_v, a.do_v, (a.L_R, a.f_in, a.f_out))
    b_k = a.out(b_k, a.do_k, (a.L_R, a.f_out))
    b_v = a.out(b_v, a.do_v, (a.L_R, a.f_out))
    ws = _workspace(fit_recolor_caches_workspace_size(a.send, a.recv, a.n_taps), a.dev, workspace)
    st_arr = (ctypes.c_int32 * (2 * a.L_R))()
    iters = ctypes.c_int32(0)
    ks, vs, kr, vr = a.ptrs
    st = lib().kvx_fit_recolor_caches(ctypes.byref(a.send), ks, vs, ctypes.byref(a.recv), kr, vr,
                                      _ptr(recv_to_send), a.taps_ptr(), int(a.n_taps), float(rho_x), float(rho_y),
                                      _ptr(w_k), _ptr(w_v), _ptr(b_k), _ptr(b_v), st_arr, ctypes.byref(iters),
                                      _ptr(ws), ws.numel(), _stream(stream))
    if info is not None:
        info["iters"] = int(iters.value)
    if status is not None:
        status.extend(int(v) for v in st_arr)
        if st not in (OK, ERR_NOT_SPD, ERR_NOT_CONVERGED):
            _check(st, "kvx_fit_recolor_caches")
    else:
        _check(st, "kvx_fit_recolor_caches")
    return w_k, w_v, b_k, b_v


def fit_recolor(xs, ys, *, rho_x: float = 0.0, rho_y: float = 0.0, w_outs=None, b_outs=None,
                workspace: Optional[torch.Tensor] = None, stream=None, status: Optional[list] = None,
                info: Optional[dict] = None):
    """kvx_fit_recolor on lists of row-major 2-D x [n][f_in] and y [n][f_out]
    (one shape, one dtype, one row stride each).  Returns the lists
    (w fp32 [f_in][f_out], b fp32 [f_out]).  With a list ``status``, appends
    each problem's status and raises only for other errors; with a dict
    ``info``, stores the number of polar iterations under "iters"."""
    count = len(xs)
    if count == 0 or len(ys) != count:
        raise ValueError("xs and ys must be non-empty lists of equal length")
    x0, y0 = xs[0], ys[0]
    for x, y in zip(xs, ys):
        if x.dim() != 2 or y.dim() != 2 or x.shape != x0.shape or y.shape != y0.shape:
            raise ValueError("every x (and every y) must be 2-D of one shape")
        if x.stride() != x0.stride() or y.stride() != y0.stride() or x.stride(1) != 1 or y.stride(1) != 1:
            raise ValueError("rows must be contiguous with one row stride per operand")
        if x.dtype != x0.dtype or y.dtype != x0.dtype:
            raise TypeError("x and y must share a dtype")
    n, f_in = x0.shape
    f_out = y0.shape[1]
    dev = x0.device
    if w_outs is None:
        w_outs = [torch.empty((f_in, f_out), dtype=torch.float32, device=dev) for _ in range(count)]
    if b_outs is None:
        b_outs = [torch.empty(f_out, dtype=torch.float32, device=dev) for _ in range(count)]
    arr = ctypes.c_void_p * count
    xp, yp = arr(*[x.data_ptr() for x in xs]), arr(*[y.data_ptr() for y in ys])
    wp, bp = arr(*[w.data_ptr() for w in w_outs]), arr(*[b.data_ptr() for b in b_outs])
    st_arr = (ctypes.c_int32 * count)()
    iters = ctypes.c_int32(0)
    ws = _workspace(lib().kvx_fit_recolor_workspace_size(count, f_in, f_out), dev, workspace)
    st = lib().kvx_fit_recolor(count, xp, x0.stride(0), yp, y0.stride(0), _dtype_code(x0), n, f_in, f_out,
                               float(rho_x), float(rho_y), wp, bp, st_arr, ctypes.byref(iters), _ptr(ws), ws.numel(),
                               _stream(stream))
    if info is not None:
        info["iters"] = int(iters.value)
    if status is not None:
        status.extend(int(v) for v in st_arr)
        if st not in (OK, ERR_NOT_SPD, ERR_NOT_CONVERGED):
            _check(st, "kvx_fit_recolor")
    else:
        _check(st, "kvx_fit_recolor")
    return w_outs, b_outs


def fold_lowrank(w: torch.Tensor, a: torch.Tensor, b: torch.Tensor, out_dtype=torch.bfloat16,
                 out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """kvx_fold_lowrank: W + A B on row-major [count][f_in][f_out] maps with
    a [count][f_in][r], b [count][r][f_out] (a single map may drop the
    leading dimension)."""
    squeeze = w.dim() == 2
    if squeeze:
        w, a, b = w[None], a[None], b[None]
    for name, t in (("w", w), ("a", a), ("b", b)):
        _need(t, name, torch.float32)
    count, f_in, f_out = w.shape
    rank = a.shape[-1]
    if tuple(a.shape) != (count, f_in, rank) or tuple(b.shape) != (count, rank, f_out):
        raise ValueError("a must be [count][f_in][rank] and b [count][rank][f_out]")
    if out is None:
        out = torch.empty((count, f_in, f_out), dtype=out_dtype, device=w.device)
    code = BF16 if out.dtype == torch.bfloat16 else F32
    st = lib().kvx_fold_lowrank(_ptr(w), _ptr(a), _ptr(b), count, f_in, f_out, rank, _ptr(out), code,
                                _stream(stream))
    _check(st, "kvx_fold_lowrank")
    return out[0] if squeeze else out


def probe_hbm(mode: str, a: torch.Tensor, b: Optional[torch.Tensor] = None, iters: int = 10,
              stream=None) -> float:
    """kvx_probe_hbm: "copy" (a -> b), "read" (a; b a sink the binding
    allocates) or "fill" (a).  Returns the mean ms per launch."""
    m = {"copy": 0, "read": 1, "fill": 2}[mode]
    _need(a, "a")
    nbytes = a.numel() * a.element_size()
    if m == 1 and b is None:
        b = torch.empty(int(lib().kvx_probe_scratch_words()), dtype=torch.int32, device=a.device)
    ms = ctypes.c_float(0.0)
    _check(lib().kvx_probe_hbm(m, _ptr(a), _ptr(b), nbytes, int(iters), ctypes.byref(ms), _stream(stream)),
           "kvx_probe_hbm")
    return float(ms.value)


def probe_mfma(reps: int = 100000, iters: int = 8, device="cuda", stream=None):
    """kvx_probe_mfma: returns (ms per launch, flops per launch)."""
    out = torch.empty(int(lib().kvx_probe_scratch_words()), dtype=torch.float32, device=device)
    ms, fl = ctypes.c_float(0.0), ctypes.c_double(0.0)
    _check(lib().kvx_probe_mfma(_ptr(out), int(reps), int(iters), ctypes.byref(ms), ctypes.byref(fl),
                                _stream(stream)), "kvx_probe_mfma")
    return float(ms.value), float(fl.value)
