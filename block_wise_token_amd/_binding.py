"""ctypes binding of libuniprefill (argument marshalling only)."""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libuniprefill.so")

KERNEL_IDS = {
    "score_partial": 0, "row_stats": 1, "block_mass": 2, "normalize": 3, "select": 4,
    "select_finalize": 5, "block_dst": 6, "gather": 7, "compose": 8, "score_plan": 9,
    "score_partial_lse": 10, "lse_finalize": 11, "attn_plan": 12, "rope_layout": 13,
    "attention": 14, "swiglu": 15, "gemm": 16, "select_fused": 17, "attention_window": 18,
}

_lib = None


class UniPrefillError(RuntimeError):
    pass


def lib():
    """Load libuniprefill.so (built in-tree by ``python -m block_wise_token_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise UniPrefillError(f"{LIB_PATH} is missing: build it with "
                              "`python -m block_wise_token_amd.build` (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32p, u8p, f32p = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
    ci, cf, cs = ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.up_status_string.restype = ctypes.c_char_p
    L.up_status_string.argtypes = [ci]
    L.up_abi_version.restype = ci
    L.up_block_scores_workspace.restype = cs
    L.up_block_scores_workspace.argtypes = [vp, ci, ci, ci, ci, ci, ci]
    L.up_block_scores.restype = ci
    L.up_block_scores.argtypes = [vp, vp, i32p, vp, ci, ci, ci, ci, ci, ci, cf, f32p, f32p, vp, cs,
                                  vp]
    L.up_block_scores_chunks.restype = ci
    L.up_block_scores_chunks.argtypes = [vp, ci, ci, ci, ci, ci, ci, vp]
    L.up_block_scores_paged.restype = ci
    L.up_block_scores_paged.argtypes = [vp, vp, ctypes.c_int64, ci, i32p, ci, i32p, vp, ci, ci, ci,
                                        ci, ci, ci, cf, f32p, f32p, vp, cs, vp]
    L.up_block_scores_lse_workspace.restype = cs
    L.up_block_scores_lse_workspace.argtypes = [vp, ci, ci, ci, ci, ci, ci]
    L.up_block_scores_lse.restype = ci
    L.up_block_scores_lse.argtypes = [vp, vp, f32p, i32p, vp, ci, ci, ci, ci, ci, ci, cf, f32p, vp,
                                      cs, vp]
    L.up_block_scores_lse_paged.restype = ci
    L.up_block_scores_lse_paged.argtypes = [vp, vp, ctypes.c_int64, ci, i32p, ci, f32p, i32p, vp,
                                            ci, ci, ci, ci, ci, ci, cf, f32p, vp, cs, vp]
    L.up_topp_select.restype = ci
    L.up_topp_select.argtypes = [f32p, i32p, vp, ci, ci, ci, cf, u8p, i32p, vp]
    L.up_topk_select.restype = ci
    L.up_topk_select.argtypes = [f32p, i32p, vp, ci, ci, ci, ci, u8p, i32p, vp]
    L.up_expand_compact_workspace.restype = cs
    L.up_expand_compact_workspace.argtypes = [vp, ci, ci]
    L.up_expand_compact.restype = ci
    L.up_expand_compact.argtypes = [vp, ci, ci, i32p, u8p, i32p, i32p, vp, ci, ci, i32p, vp, i32p,
                                    i32p, i32p, vp, cs, vp]
    L.up_expand_compact_noalloc.restype = ci
    L.up_expand_compact_noalloc.argtypes = [vp, ci, ci, i32p, u8p, i32p, i32p, vp, ci, ci, i32p,
                                            vp, i32p, i32p, i32p, vp]
    L.up_compose_drops.restype = ci
    L.up_compose_drops.argtypes = [i32p, ci, i32p, i32p, ci, i32p, vp]
    L.up_device_error.restype = ci
    L.up_device_error.argtypes = [vp, vp]
    L.up_profile_enable.restype = ci
    L.up_profile_enable.argtypes = [ci]
    L.up_profile_read.restype = ci
    L.up_profile_read.argtypes = [ci, vp, vp]
    L.up_profile_reset.restype = ci
    L.up_profile_reset.argtypes = []
    i64 = ctypes.c_int64
    L.up_rope_attention_workspace.restype = cs
    L.up_rope_attention_workspace.argtypes = [vp, ci, ci, ci, ci]
    L.up_rope_attention_scores_workspace.restype = cs
    L.up_rope_attention_scores_workspace.argtypes = [vp, ci, ci, ci, ci, ci, ci]
    L.up_rope_attention_scores.restype = ci
    L.up_rope_attention_scores.argtypes = [vp, vp, vp, i32p, i32p, vp, ci, ci, ci, ci, cf, cf, ci,
                                           ci, vp, f32p, f32p, vp, cs, vp]
    L.up_rope_attention.restype = ci
    L.up_rope_attention.argtypes = [vp, vp, vp, i32p, i32p, vp, ci, ci, ci, ci, cf, cf, vp, vp, cs,
                                    vp]
    L.up_swiglu.restype = ci
    L.up_swiglu.argtypes = [vp, i64, ci, vp, vp]
    L.up_layer_decision_workspace.restype = cs
    L.up_layer_decision_workspace.argtypes = [vp, ci, ci, ci, ci, ci, ci]
    L.up_layer_decision.restype = ci
    L.up_layer_decision.argtypes = [vp, vp, i32p, vp, ci, ci, ci, ci, ci, ci, cf, cf, vp, ci, ci,
                                    i32p, i32p, f32p, u8p, i32p, i32p, vp, i32p, i32p, vp, cs, vp]
    _lib = L
    return L


LAYER_LIB_PATH = os.path.join(_HERE, "libuniprefill_layer.so")
_layer = None


def layer_lib():
    """Load libuniprefill_layer.so (the layer's hipBLASLt GEMMs; it loads
    libuniprefill.so itself, which lib() loads first so both share one copy)."""
    global _layer
    if _layer is not None:
        return _layer
    lib()
    if not os.path.exists(LAYER_LIB_PATH):
        raise UniPrefillError(f"{LAYER_LIB_PATH} is missing: build it with "
                              "`python -m block_wise_token_amd.build` (hipcc, gfx950)")
    L = ctypes.CDLL(LAYER_LIB_PATH)
    vp, ci, cs, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_int64
    L.up_linear.restype = ci
    L.up_linear.argtypes = [vp, vp, vp, i64, ci, ci, vp, vp, cs, vp]
    L.up_swiglu_ffn_workspace.restype = cs
    L.up_swiglu_ffn_workspace.argtypes = [i64, ci, ci]
    L.up_swiglu_ffn.restype = ci
    L.up_swiglu_ffn.argtypes = [vp, vp, vp, vp, i64, ci, ci, vp, vp, cs, vp]
    _layer = L
    return L


def _check(status: int, what: str):
    if status != 0:
        raise UniPrefillError(f"{what}: {lib().up_status_string(status).decode()}")


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t: torch.Tensor, dtype, name: str):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if t.device.index is not None and t.device.index != torch.cuda.current_device():
        # the library launches on the current device and stream
        raise ValueError(f"{name} is on {t.device}, the current device is "
                         f"cuda:{torch.cuda.current_device()}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _buf(t: torch.Tensor, dtype, min_numel: int, name: str):
    """A contiguous device tensor of `dtype` with room for `min_numel` elements: the
    library writes or reads that many through a plain pointer."""
    _dev(t, dtype, name)
    if t.numel() < min_numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs at least {min_numel}")
    return t


def _rank(t: torch.Tensor, ndim: int, name: str):
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    return t


def _check_scores_inputs(qwin, k, h, n, d_k_axis=2):
    """qwin [sum W_i, Hq, d] and token-major keys with the same d."""
    _rank(qwin, 3, "qwin")
    if int(qwin.shape[0]) < h.win_rows(n):
        raise ValueError(f"qwin has {int(qwin.shape[0])} rows, the window needs {h.win_rows(n)}")
    if int(k.shape[d_k_axis]) != int(qwin.shape[2]):
        raise ValueError("k and qwin differ in head dimension")


class _HostCu:
    """Host copy of cu_seqlens as a C int32 array (kept alive with its pointer)."""

    def __init__(self, cu_h):
        a = np.ascontiguousarray(np.asarray(cu_h.cpu() if isinstance(cu_h, torch.Tensor) else cu_h,
                                            dtype=np.int32))
        self.arr = a
        self.B = int(a.size - 1)
        self.ptr = a.ctypes.data_as(ctypes.c_void_p)

    @property
    def T(self) -> int:
        return int(self.arr[-1]) if self.arr.size else 0

    def nb_tot(self, G: int) -> int:
        return int(sum((int(L) + G - 1) // G for L in np.diff(self.arr)))

    def win_rows(self, n: int) -> int:
        return int(sum(min(int(n), int(L)) for L in np.diff(self.arr)))


def block_scores_chunks(cu_h, Hq, Hkv, d, n, G) -> np.ndarray:
    """Per-request statistics-chunk length in blocks (int32 [B]); see
    up_block_scores_chunks.  Host only."""
    h = _HostCu(cu_h)
    out = np.zeros(max(h.B, 0), dtype=np.int32)
    _check(lib().up_block_scores_chunks(h.ptr, h.B, Hq, Hkv, d, n, G,
                                        out.ctypes.data_as(ctypes.c_void_p)),
           "up_block_scores_chunks")
    return out


def block_scores_workspace_bytes(cu_h, Hq, Hkv, d, n, G) -> int:
    h = _HostCu(cu_h)
    return int(lib().up_block_scores_workspace(h.ptr, h.B, Hq, Hkv, d, n, G))


def expand_compact_workspace_bytes(cu_h, G) -> int:
    h = _HostCu(cu_h)
    return int(lib().up_expand_compact_workspace(h.ptr, h.B, G))


def block_scores_lse_workspace_bytes(cu_h, Hq, Hkv, d, n, G) -> int:
    h = _HostCu(cu_h)
    return int(lib().up_block_scores_lse_workspace(h.ptr, h.B, Hq, Hkv, d, n, G))


def block_scores(qwin, k, cu_seqlens, cu_h, n, G, scale=0.0, out=None, workspace=None,
                 stream=None, row_lse=None):
    """Per-block importance scores (float32 [NB_tot]); see up_block_scores.  With
    ``row_lse`` (float32 [sum W, Hq]) each window row's log-sum-exp is written too."""
    _dev(qwin, torch.bfloat16, "qwin")
    _dev(k, torch.bfloat16, "k")
    _dev(cu_seqlens, torch.int32, "cu_seqlens")
    h = _HostCu(cu_h)
    _buf(cu_seqlens, torch.int32, h.B + 1, "cu_seqlens")
    _check_scores_inputs(qwin, _rank(k, 3, "k"), h, n)
    if int(k.shape[0]) < h.T:
        raise ValueError(f"k has {int(k.shape[0])} rows, cu_seqlens needs {h.T}")
    Hq, d = int(qwin.shape[1]), int(qwin.shape[2])
    Hkv = int(k.shape[1])
    if out is None:
        out = torch.empty(h.nb_tot(G), dtype=torch.float32, device=qwin.device)
    _buf(out, torch.float32, h.nb_tot(G), "out")
    need = int(lib().up_block_scores_workspace(h.ptr, h.B, Hq, Hkv, d, n, G))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=qwin.device)
    _buf(workspace, torch.uint8, need, "workspace")
    if row_lse is not None:
        _buf(row_lse, torch.float32, h.win_rows(n) * Hq, "row_lse")
    st = lib().up_block_scores(_ptr(qwin), _ptr(k), _ptr(cu_seqlens), h.ptr, h.B, Hq, Hkv, d, n,
                               G, float(scale), _ptr(out), _ptr(row_lse), _ptr(workspace),
                               workspace.numel(), _stream(stream))
    _check(st, "up_block_scores")
    return out


def block_scores_paged(qwin, k_pages, block_table, cu_seqlens, cu_h, n, G, scale=0.0, out=None,
                       workspace=None, stream=None, row_lse=None):
    """Block scores with keys in a paged cache: k_pages bf16 [num_pages, page_size, Hkv,
    d], block_table int32 [B, max_pages]; see up_block_scores_paged."""
    _dev(qwin, torch.bfloat16, "qwin")
    _dev(k_pages, torch.bfloat16, "k_pages")
    _dev(block_table, torch.int32, "block_table")
    _dev(cu_seqlens, torch.int32, "cu_seqlens")
    h = _HostCu(cu_h)
    _buf(cu_seqlens, torch.int32, h.B + 1, "cu_seqlens")
    _check_scores_inputs(qwin, _rank(k_pages, 4, "k_pages"), h, n, d_k_axis=3)
    _rank(block_table, 2, "block_table")
    if int(block_table.shape[0]) < h.B:
        raise ValueError("block_table needs one row per request")
    Hq, d = int(qwin.shape[1]), int(qwin.shape[2])
    num_pages, page_size, Hkv = int(k_pages.shape[0]), int(k_pages.shape[1]), int(k_pages.shape[2])
    if out is None:
        out = torch.empty(h.nb_tot(G), dtype=torch.float32, device=qwin.device)
    _buf(out, torch.float32, h.nb_tot(G), "out")
    need = int(lib().up_block_scores_workspace(h.ptr, h.B, Hq, Hkv, d, n, G))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=qwin.device)
    _buf(workspace, torch.uint8, need, "workspace")
    if row_lse is not None:
        _buf(row_lse, torch.float32, h.win_rows(n) * Hq, "row_lse")
    st = lib().up_block_scores_paged(_ptr(qwin), _ptr(k_pages), num_pages, page_size,
                                     _ptr(block_table), int(block_table.shape[1]), _ptr(cu_seqlens),
                                     h.ptr, h.B, Hq, Hkv, d, n, G, float(scale), _ptr(out),
                                     _ptr(row_lse), _ptr(workspace), workspace.numel(),
                                     _stream(stream))
    _check(st, "up_block_scores_paged")
    return out


def block_scores_lse(qwin, k, row_lse, cu_seqlens, cu_h, n, G, scale=0.0, out=None,
                     workspace=None, stream=None):
    """Block scores from given window-row log-sum-exp (float32 [sum W, Hq], natural
    log); see up_block_scores_lse."""
    _dev(qwin, torch.bfloat16, "qwin")
    _dev(k, torch.bfloat16, "k")
    _dev(row_lse, torch.float32, "row_lse")
    _dev(cu_seqlens, torch.int32, "cu_seqlens")
    h = _HostCu(cu_h)
    _buf(cu_seqlens, torch.int32, h.B + 1, "cu_seqlens")
    _check_scores_inputs(qwin, _rank(k, 3, "k"), h, n)
    if int(k.shape[0]) < h.T:
        raise ValueError(f"k has {int(k.shape[0])} rows, cu_seqlens needs {h.T}")
    Hq, d = int(qwin.shape[1]), int(qwin.shape[2])
    Hkv = int(k.shape[1])
    _buf(row_lse, torch.float32, h.win_rows(n) * Hq, "row_lse")
    if out is None:
        out = torch.empty(h.nb_tot(G), dtype=torch.float32, device=qwin.device)
    _buf(out, torch.float32, h.nb_tot(G), "out")
    need = int(lib().up_block_scores_lse_workspace(h.ptr, h.B, Hq, Hkv, d, n, G))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=qwin.device)
    _buf(workspace, torch.uint8, need, "workspace")
    st = lib().up_block_scores_lse(_ptr(qwin), _ptr(k), _ptr(row_lse), _ptr(cu_seqlens), h.ptr,
                                   h.B, Hq, Hkv, d, n, G, float(scale), _ptr(out),
                                   _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st, "up_block_scores_lse")
    return out


def block_scores_lse_paged(qwin, k_pages, block_table, row_lse, cu_seqlens, cu_h, n, G,
                           scale=0.0, out=None, workspace=None, stream=None):
    """Block scores from given window-row log-sum-exp with the keys in a paged cache
    (k_pages and block_table as for block_scores_paged); see up_block_scores_lse_paged."""
    _dev(qwin, torch.bfloat16, "qwin")
    _dev(k_pages, torch.bfloat16, "k_pages")
    _dev(block_table, torch.int32, "block_table")
    _dev(row_lse, torch.float32, "row_lse")
    _dev(cu_seqlens, torch.int32, "cu_seqlens")
    h = _HostCu(cu_h)
    _buf(cu_seqlens, torch.int32, h.B + 1, "cu_seqlens")
    _check_scores_inputs(qwin, _rank(k_pages, 4, "k_pages"), h, n, d_k_axis=3)
    _rank(block_table, 2, "block_table")
    if int(block_table.shape[0]) < h.B:
        raise ValueError("block_table needs one row per request")
    Hq, d = int(qwin.shape[1]), int(qwin.shape[2])
    num_pages, page_size, Hkv = int(k_pages.shape[0]), int(k_pages.shape[1]), int(k_pages.shape[2])
    _buf(row_lse, torch.float32, h.win_rows(n) * Hq, "row_lse")
    if out is None:
        out = torch.empty(h.nb_tot(G), dtype=torch.float32, device=qwin.device)
    _buf(out, torch.float32, h.nb_tot(G), "out")
    need = int(lib().up_block_scores_lse_workspace(h.ptr, h.B, Hq, Hkv, d, n, G))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=qwin.device)
    _buf(workspace, torch.uint8, need, "workspace")
    st = lib().up_block_scores_lse_paged(_ptr(qwin), _ptr(k_pages), num_pages, page_size,
                                         _ptr(block_table), int(block_table.shape[1]),
                                         _ptr(row_lse), _ptr(cu_seqlens), h.ptr, h.B, Hq, Hkv, d,
                                         n, G, float(scale), _ptr(out), _ptr(workspace),
                                         workspace.numel(), _stream(stream))
    _check(st, "up_block_scores_lse_paged")
    return out


def _select(fn, scores, cu_seqlens, cu_h, n, G, arg, keep, cu_out, stream, what):
    _dev(scores, torch.float32, "scores")
    _dev(cu_seqlens, torch.int32, "cu_seqlens")
    h = _HostCu(cu_h)
    _buf(cu_seqlens, torch.int32, h.B + 1, "cu_seqlens")
    nbt = h.nb_tot(G)
    _buf(scores, torch.float32, nbt, "scores")
    if keep is None:
        keep = torch.empty(nbt, dtype=torch.uint8, device=scores.device)
    if cu_out is None:
        cu_out = torch.empty(h.B + 1, dtype=torch.int32, device=scores.device)
    _buf(keep, torch.uint8, nbt, "keep_blocks")
    _buf(cu_out, torch.int32, h.B + 1, "cu_seqlens_out")
    st = fn(_ptr(scores), _ptr(cu_seqlens), h.ptr, h.B, n, G, arg, _ptr(keep), _ptr(cu_out),
            _stream(stream))
    _check(st, what)
    return keep, cu_out


def topp_select(scores, cu_seqlens, cu_h, n, G, p, keep=None, cu_out=None, stream=None):
    """Top-p cut: (keep_blocks uint8 [NB_tot], cu_seqlens_out int32 [B+1])."""
    return _select(lib().up_topp_select, scores, cu_seqlens, cu_h, n, G, ctypes.c_float(p), keep,
                   cu_out, stream, "up_topp_select")


def topk_select(scores, cu_seqlens, cu_h, n, G, topk, keep=None, cu_out=None, stream=None):
    """Top-k cut (fixed block count per request) plus the window blocks."""
    return _select(lib().up_topk_select, scores, cu_seqlens, cu_h, n, G, int(topk), keep, cu_out,
                   stream, "up_topk_select")


def expand_compact(hidden, pos, keep, cu_seqlens, cu_out, cu_h, G, idx_out=None, hidden_out=None,
                   pos_out=None, workspace=None, stream=None, prev_orig=None, orig_out=None):
    """Kept-token rows: (idx_out, hidden_out, pos_out), each with capacity T rows.
    With ``prev_orig`` given, ``orig_out[r] = prev_orig[idx_out[r]]`` is written in the
    same pass (pass ``orig_out`` to choose the buffer)."""
    _dev(hidden, hidden.dtype, "hidden")
    _dev(keep, torch.uint8, "keep_blocks")
    _dev(cu_seqlens, torch.int32, "cu_seqlens")
    _dev(cu_out, torch.int32, "cu_seqlens_out")
    if pos is not None:
        _dev(pos, torch.int32, "pos")
    h = _HostCu(cu_h)
    _buf(cu_seqlens, torch.int32, h.B + 1, "cu_seqlens")
    T = h.T
    _rank(hidden, 2, "hidden")
    if int(hidden.shape[0]) < T:
        raise ValueError(f"hidden has {int(hidden.shape[0])} rows, cu_seqlens needs {T}")
    H = int(hidden.shape[1])
    eb = hidden.element_size()
    dev = hidden.device
    _buf(keep, torch.uint8, h.nb_tot(G), "keep_blocks")
    _buf(cu_out, torch.int32, h.B + 1, "cu_seqlens_out")
    if pos is not None:
        _buf(pos, torch.int32, T, "pos")
    if idx_out is None:
        idx_out = torch.empty(T, dtype=torch.int32, device=dev)
    if hidden_out is None:
        hidden_out = torch.empty((T, H), dtype=hidden.dtype, device=dev)
    if pos_out is None and pos is not None:
        pos_out = torch.empty(T, dtype=torch.int32, device=dev)
    _buf(idx_out, torch.int32, T, "idx_out")
    _buf(hidden_out, hidden.dtype, T * H, "hidden_out")
    if pos_out is not None:
        _buf(pos_out, torch.int32, T, "pos_out")
    if prev_orig is not None:
        _buf(prev_orig, torch.int32, T, "prev_orig")
        if orig_out is None:
            orig_out = torch.empty(T, dtype=torch.int32, device=dev)
        _buf(orig_out, torch.int32, T, "orig_out")
    elif orig_out is not None:
        raise ValueError("orig_out needs prev_orig")
    need = int(lib().up_expand_compact_workspace(h.ptr, h.B, G))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _buf(workspace, torch.uint8, need, "workspace")
    st = lib().up_expand_compact(_ptr(hidden), H, eb, _ptr(pos), _ptr(keep), _ptr(cu_seqlens),
                                 _ptr(cu_out), h.ptr, h.B, G, _ptr(idx_out), _ptr(hidden_out),
                                 _ptr(pos_out), _ptr(prev_orig), _ptr(orig_out), _ptr(workspace),
                                 workspace.numel(), _stream(stream))
    _check(st, "up_expand_compact")
    return idx_out, hidden_out, pos_out


def expand_compact_noalloc(hidden, pos, keep, cu_seqlens, cu_out, cu_h, G, idx_out, hidden_out,
                           pos_out=None, stream=None, prev_orig=None, orig_out=None):
    """up_expand_compact_noalloc: expand_compact with the run table in the library's
    own device array; every output is the caller's (nothing is allocated here or in
    the library).  At most 65,536 blocks per call; calls overlapping on one GPU race."""
    _dev(hidden, hidden.dtype, "hidden")
    _dev(keep, torch.uint8, "keep_blocks")
    _dev(cu_seqlens, torch.int32, "cu_seqlens")
    _dev(cu_out, torch.int32, "cu_seqlens_out")
    h = _HostCu(cu_h)
    _buf(cu_seqlens, torch.int32, h.B + 1, "cu_seqlens")
    T = h.T
    _rank(hidden, 2, "hidden")
    if int(hidden.shape[0]) < T:
        raise ValueError(f"hidden has {int(hidden.shape[0])} rows, cu_seqlens needs {T}")
    H = int(hidden.shape[1])
    _buf(keep, torch.uint8, h.nb_tot(G), "keep_blocks")
    _buf(cu_out, torch.int32, h.B + 1, "cu_seqlens_out")
    _buf(idx_out, torch.int32, T, "idx_out")
    _buf(hidden_out, hidden.dtype, T * H, "hidden_out")
    if pos is not None:
        _buf(pos, torch.int32, T, "pos")
        _buf(pos_out, torch.int32, T, "pos_out")
    elif pos_out is not None:
        raise ValueError("pos_out needs pos")
    if prev_orig is not None:
        _buf(prev_orig, torch.int32, T, "prev_orig")
        _buf(orig_out, torch.int32, T, "orig_out")
    elif orig_out is not None:
        raise ValueError("orig_out needs prev_orig")
    st = lib().up_expand_compact_noalloc(_ptr(hidden), H, hidden.element_size(), _ptr(pos),
                                         _ptr(keep), _ptr(cu_seqlens), _ptr(cu_out), h.ptr, h.B,
                                         G, _ptr(idx_out), _ptr(hidden_out), _ptr(pos_out),
                                         _ptr(prev_orig), _ptr(orig_out), _stream(stream))
    _check(st, "up_expand_compact_noalloc")
    return idx_out, hidden_out, pos_out


def compose_drops(prev_orig, idx, count, capacity=None, out=None, stream=None):
    """orig[r] = prev_orig[idx[r]] for r < *count (count: device int32 scalar view)."""
    _dev(prev_orig, torch.int32, "prev_orig")
    _buf(count, torch.int32, 1, "count")
    cap = int(idx.numel()) if capacity is None else int(capacity)
    _buf(idx, torch.int32, cap, "idx")
    if out is None:
        out = torch.empty(cap, dtype=torch.int32, device=idx.device)
    _buf(out, torch.int32, cap, "out")
    st = lib().up_compose_drops(_ptr(prev_orig), int(prev_orig.numel()), _ptr(idx), _ptr(count),
                                cap, _ptr(out), _stream(stream))
    _check(st, "up_compose_drops")
    return out


def device_error(stream=None) -> int:
    """Read and clear the library's device error word (synchronises)."""
    v = ctypes.c_int32(0)
    _check(lib().up_device_error(ctypes.byref(v), _stream(stream)), "up_device_error")
    return int(v.value)


def profile_enable(on: bool = True):
    _check(lib().up_profile_enable(1 if on else 0), "up_profile_enable")


def profile_reset():
    _check(lib().up_profile_reset(), "up_profile_reset")


def profile_read(name: str):
    """(launches, total milliseconds) recorded for a kernel family."""
    n = ctypes.c_int(0)
    ms = ctypes.c_double(0.0)
    _check(lib().up_profile_read(KERNEL_IDS[name], ctypes.byref(n), ctypes.byref(ms)),
           "up_profile_read")
    return int(n.value), float(ms.value)


class LayerDecision:
    """One full-attention layer decision with every buffer allocated up front.

    ``run()`` issues the calls -- scores, Top-p, expand+compact with the drop
    composition fused into the compaction pass -- on the current stream and
    allocates nothing.  (``up_compose_drops`` is the standalone form of the last
    step.)  For a plain Top-p decision (no given row log-sum-exp, no Top-k) it is one
    ``up_layer_decision`` call; ``separate=True`` issues the three calls instead.
    """

    def __init__(self, qwin, k, cu_seqlens, cu_h, hidden, pos, n, G, p, scale=0.0,
                 prev_orig=None, topk=None, row_lse=None, separate=False):
        self.qwin, self.k, self.cu, self.hidden, self.pos = qwin, k, cu_seqlens, hidden, pos
        self.h = _HostCu(cu_h)
        self.n, self.G, self.p, self.scale, self.topk = n, G, p, scale, topk
        dev = qwin.device
        T, B = self.h.T, self.h.B
        # The one call hands these pointers straight to the library: check them here.
        _dev(qwin, torch.bfloat16, "qwin")
        _dev(k, torch.bfloat16, "k")
        _check_scores_inputs(qwin, _rank(k, 3, "k"), self.h, n)
        if int(k.shape[0]) < T:
            raise ValueError(f"k has {int(k.shape[0])} rows, cu_seqlens needs {T}")
        _buf(cu_seqlens, torch.int32, B + 1, "cu_seqlens")
        _rank(_dev(hidden, hidden.dtype, "hidden"), 2, "hidden")
        if int(hidden.shape[0]) < T:
            raise ValueError(f"hidden has {int(hidden.shape[0])} rows, cu_seqlens needs {T}")
        if pos is not None:
            _buf(pos, torch.int32, T, "pos")
        if prev_orig is not None:
            _buf(prev_orig, torch.int32, T, "prev_orig")
        nbt = self.h.nb_tot(G)
        Hq, d, Hkv = int(qwin.shape[1]), int(qwin.shape[2]), int(k.shape[1])
        self.scores = torch.empty(nbt, dtype=torch.float32, device=dev)
        # With the layer's own row statistics the scores come from the given-lse pass.
        self.row_lse = row_lse
        ws_bytes = (block_scores_lse_workspace_bytes if row_lse is not None
                    else block_scores_workspace_bytes)(self.h.arr, Hq, Hkv, d, n, G)
        self.ws_scores = torch.empty(max(1, ws_bytes), dtype=torch.uint8, device=dev)
        self.keep = torch.empty(nbt, dtype=torch.uint8, device=dev)
        self.cu_out = torch.empty(B + 1, dtype=torch.int32, device=dev)
        self.idx = torch.empty(T, dtype=torch.int32, device=dev)
        self.hidden_out = torch.empty_like(hidden)
        self.pos_out = torch.empty(T, dtype=torch.int32, device=dev)
        self.ws_compact = torch.empty(max(1, expand_compact_workspace_bytes(self.h.arr, G)),
                                      dtype=torch.uint8, device=dev)
        self.prev_orig = prev_orig if prev_orig is not None else torch.arange(
            T, dtype=torch.int32, device=dev)
        self.orig = torch.empty(T, dtype=torch.int32, device=dev)
        self.one_call = not separate and row_lse is None and topk is None and pos is not None
        if self.one_call:
            need = int(lib().up_layer_decision_workspace(self.h.ptr, B, Hq, Hkv, d, n, G))
            self.ws_one = torch.empty(max(1, need), dtype=torch.uint8, device=dev)
            self.dims = (Hq, Hkv, d, int(hidden.shape[1]), hidden.element_size())

    def run(self, stream=None):
        if self.one_call:
            Hq, Hkv, d, H, eb = self.dims
            st = lib().up_layer_decision(
                _ptr(self.qwin), _ptr(self.k), _ptr(self.cu), self.h.ptr, self.h.B, Hq, Hkv, d,
                self.n, self.G, float(self.scale), float(self.p), _ptr(self.hidden), H, eb,
                _ptr(self.pos), _ptr(self.prev_orig), _ptr(self.scores), _ptr(self.keep),
                _ptr(self.cu_out), _ptr(self.idx), _ptr(self.hidden_out), _ptr(self.pos_out),
                _ptr(self.orig), _ptr(self.ws_one), self.ws_one.numel(), _stream(stream))
            _check(st, "up_layer_decision")
            return
        if self.row_lse is None:
            block_scores(self.qwin, self.k, self.cu, self.h.arr, self.n, self.G, self.scale,
                         out=self.scores, workspace=self.ws_scores, stream=stream)
        else:
            block_scores_lse(self.qwin, self.k, self.row_lse, self.cu, self.h.arr, self.n, self.G,
                             self.scale, out=self.scores, workspace=self.ws_scores, stream=stream)
        if self.topk is None:
            topp_select(self.scores, self.cu, self.h.arr, self.n, self.G, self.p, keep=self.keep,
                        cu_out=self.cu_out, stream=stream)
        else:
            topk_select(self.scores, self.cu, self.h.arr, self.n, self.G, self.topk, keep=self.keep,
                        cu_out=self.cu_out, stream=stream)
        expand_compact(self.hidden, self.pos, self.keep, self.cu, self.cu_out, self.h.arr, self.G,
                       idx_out=self.idx, hidden_out=self.hidden_out, pos_out=self.pos_out,
                       workspace=self.ws_compact, stream=stream, prev_orig=self.prev_orig,
                       orig_out=self.orig)


# ---- the layer on the surviving tokens ------------------------------------------

def rope_attention_workspace_bytes(cu_h, Hq, Hkv, d) -> int:
    h = _HostCu(cu_h)
    return int(lib().up_rope_attention_workspace(h.ptr, h.B, Hq, Hkv, d))


def rope_attention(q, k, v, pos, cu_seqlens, cu_h, scale=0.0, rope_theta=500000.0, out=None,
                   workspace=None, stream=None):
    """Rotary embedding at ``pos`` then causal GQA attention per request (bf16 [R, Hq, d]);
    see up_rope_attention.  q [R, Hq, d], k and v [R, Hkv, d] bf16, pos int32 [R]."""
    _dev(q, torch.bfloat16, "q")
    _dev(k, torch.bfloat16, "k")
    _dev(v, torch.bfloat16, "v")
    _dev(pos, torch.int32, "pos")
    _dev(cu_seqlens, torch.int32, "cu_seqlens")
    h = _HostCu(cu_h)
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _rank(t, 3, name)
    Hq, d, Hkv = int(q.shape[1]), int(q.shape[2]), int(k.shape[1])
    R = h.T
    if int(q.shape[0]) < R:
        raise ValueError(f"q has {int(q.shape[0])} rows, cu_seqlens needs {R}")
    if tuple(k.shape) != tuple(v.shape) or int(k.shape[0]) < R or int(k.shape[2]) != d:
        raise ValueError(f"k {tuple(k.shape)} and v {tuple(v.shape)} must both be "
                         f"[>= {R}, Hkv, {d}]")
    _buf(pos, torch.int32, R, "pos")
    _buf(cu_seqlens, torch.int32, h.B + 1, "cu_seqlens")
    if out is None:
        out = torch.empty_like(q)
    _buf(out, torch.bfloat16, R * Hq * d, "out")
    need = int(lib().up_rope_attention_workspace(h.ptr, h.B, Hq, Hkv, d))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _buf(workspace, torch.uint8, need, "workspace")
    st = lib().up_rope_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(pos), _ptr(cu_seqlens), h.ptr, h.B,
                                 Hq, Hkv, d, float(scale), float(rope_theta), _ptr(out),
                                 _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st, "up_rope_attention")
    return out


def rope_attention_scores_workspace_bytes(cu_h, Hq, Hkv, d, n, G) -> int:
    h = _HostCu(cu_h)
    return int(lib().up_rope_attention_scores_workspace(h.ptr, h.B, Hq, Hkv, d, n, G))


def rope_attention_scores(q, k, v, pos, cu_seqlens, cu_h, n, G, scale=0.0, rope_theta=500000.0,
                          out=None, scores=None, row_lse=None, workspace=None, stream=None):
    """The rotary attention of ``rope_attention`` and the block scores of its window rows
    from the same probabilities; see up_rope_attention_scores.  Returns (out, scores)."""
    _dev(q, torch.bfloat16, "q")
    _dev(k, torch.bfloat16, "k")
    _dev(v, torch.bfloat16, "v")
    _dev(pos, torch.int32, "pos")
    _dev(cu_seqlens, torch.int32, "cu_seqlens")
    h = _HostCu(cu_h)
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _rank(t, 3, name)
    Hq, d, Hkv = int(q.shape[1]), int(q.shape[2]), int(k.shape[1])
    R = h.T
    if int(q.shape[0]) < R:
        raise ValueError(f"q has {int(q.shape[0])} rows, cu_seqlens needs {R}")
    if tuple(k.shape) != tuple(v.shape) or int(k.shape[0]) < R or int(k.shape[2]) != d:
        raise ValueError(f"k {tuple(k.shape)} and v {tuple(v.shape)} must both be "
                         f"[>= {R}, Hkv, {d}]")
    _buf(pos, torch.int32, R, "pos")
    _buf(cu_seqlens, torch.int32, h.B + 1, "cu_seqlens")
    nb = h.nb_tot(G)
    if out is None:
        out = torch.empty_like(q)
    _buf(out, torch.bfloat16, R * Hq * d, "out")
    if scores is None:
        scores = torch.empty(max(nb, 1), dtype=torch.float32, device=q.device)
    _buf(scores, torch.float32, nb, "scores")
    if row_lse is not None:
        W = int(sum(min(int(L), n) for L in np.diff(h.arr)))
        _buf(row_lse, torch.float32, W * Hq, "row_lse")
    need = int(lib().up_rope_attention_scores_workspace(h.ptr, h.B, Hq, Hkv, d, n, G))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _buf(workspace, torch.uint8, need, "workspace")
    st = lib().up_rope_attention_scores(
        _ptr(q), _ptr(k), _ptr(v), _ptr(pos), _ptr(cu_seqlens), h.ptr, h.B, Hq, Hkv, d,
        float(scale), float(rope_theta), int(n), int(G), _ptr(out), _ptr(scores),
        _ptr(row_lse) if row_lse is not None else None, _ptr(workspace), workspace.numel(),
        _stream(stream))
    _check(st, "up_rope_attention_scores")
    return out, scores


def linear(x, w, residual=None, out=None, workspace=None, stream=None):
    """x [R, K] . w[N, K]^T (+ residual) in bf16 through hipBLASLt; see up_linear."""
    _rank(_dev(x, torch.bfloat16, "x"), 2, "x")
    _rank(_dev(w, torch.bfloat16, "w"), 2, "w")
    R, K = int(x.shape[0]), int(x.shape[1])
    N = int(w.shape[0])
    if int(w.shape[1]) != K:
        raise ValueError(f"w {tuple(w.shape)} does not match x {tuple(x.shape)}")
    if residual is not None:
        _buf(residual, torch.bfloat16, R * N, "residual")
    if out is None:
        out = torch.empty((R, N), dtype=torch.bfloat16, device=x.device)
    _buf(out, torch.bfloat16, R * N, "out")
    if workspace is not None:
        _dev(workspace, torch.uint8, "workspace")
    nbytes = 0 if workspace is None else workspace.numel()
    st = layer_lib().up_linear(_ptr(x), _ptr(w), _ptr(residual), R, K, N, _ptr(out), _ptr(workspace),
                         nbytes, _stream(stream))
    _check(st, "up_linear")
    return out


def swiglu(gu, out=None, stream=None):
    """silu(gu[:, :F]) * gu[:, F:] in bf16; see up_swiglu."""
    _rank(_dev(gu, torch.bfloat16, "gu"), 2, "gu")
    if int(gu.shape[1]) % 2:
        raise ValueError("gu must hold [gate | up] columns of equal width")
    R, F = int(gu.shape[0]), int(gu.shape[1]) // 2
    if out is None:
        out = torch.empty((R, F), dtype=torch.bfloat16, device=gu.device)
    _buf(out, torch.bfloat16, R * F, "out")
    _check(lib().up_swiglu(_ptr(gu), R, F, _ptr(out), _stream(stream)), "up_swiglu")
    return out


def swiglu_ffn_workspace_bytes(R, H, F) -> int:
    return int(layer_lib().up_swiglu_ffn_workspace(R, H, F))


def swiglu_ffn(x, w_gu, w_down, residual=None, out=None, workspace=None, stream=None):
    """SwiGLU FFN: swiglu(x . w_gu^T) . w_down^T (+ residual); see up_swiglu_ffn."""
    _rank(_dev(x, torch.bfloat16, "x"), 2, "x")
    _rank(_dev(w_gu, torch.bfloat16, "w_gu"), 2, "w_gu")
    _rank(_dev(w_down, torch.bfloat16, "w_down"), 2, "w_down")
    R, H = int(x.shape[0]), int(x.shape[1])
    F = int(w_gu.shape[0]) // 2
    if int(w_gu.shape[0]) != 2 * F or int(w_gu.shape[1]) != H or tuple(w_down.shape) != (H, F):
        raise ValueError(f"w_gu must be [2F, {H}] and w_down [{H}, F]; got "
                         f"{tuple(w_gu.shape)} and {tuple(w_down.shape)}")
    if residual is not None:
        _buf(residual, torch.bfloat16, R * H, "residual")
    if out is None:
        out = torch.empty((R, H), dtype=torch.bfloat16, device=x.device)
    _buf(out, torch.bfloat16, R * H, "out")
    need = int(layer_lib().up_swiglu_ffn_workspace(R, H, F))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _buf(workspace, torch.uint8, need, "workspace")
    st = layer_lib().up_swiglu_ffn(_ptr(x), _ptr(w_gu), _ptr(w_down), _ptr(residual), R, H, F, _ptr(out),
                             _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st, "up_swiglu_ffn")
    return out
