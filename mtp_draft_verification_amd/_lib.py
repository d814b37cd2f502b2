"""ctypes binding of libspecverify: the C ABI of include/specverify.h, same names.

Argument marshalling only.  Tensors are torch tensors that already live on the
GPU (torch is the allocator and the stream provider); every computation happens
in the library's HIP kernels.  There is no fallback: if the shared library is
missing or a call returns an error status, this module raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# SV_LIBRARY: another build of the library to load (e.g. one with host-side sanitizers)
LIB_PATH = os.environ.get("SV_LIBRARY") or os.path.join(HERE, "libspecverify.so")

SV_OK, SV_ERR_ARG, SV_ERR_UNSUPPORTED, SV_ERR_WORKSPACE, SV_ERR_LAUNCH, SV_ERR_DEVICE, SV_ERR_SCRATCH = 0, -1, -2, -3, -4, -5, -6
SV_NOALLOC_SCRATCH_BYTES = 32 << 20
SV_F32, SV_BF16, SV_BF16X2 = 0, 1, 2
SV_SELECT_GREEDY, SV_SELECT_SAMPLE, SV_SELECT_RESIDUAL, SV_SELECT_SAMPLE_RS = 0, 1, 2, 3
SV_EPI_STORE, SV_EPI_ADD_F32, SV_EPI_GEGLU, SV_EPI_SPLIT_F32 = 0, 1, 2, 3
SV_W_ROWMAJOR, SV_W_TILED = 0, 1
SV_DEV_CACHE_OVERFLOW, SV_DEV_BAD_TOKEN, SV_DEV_BAD_LENGTH = 1, 2, 4

EXPORTS = ("sv_status_string", "sv_version", "sv_verify_attn_workspace", "sv_verify_attn", "sv_verify_attn_fp8",
           "sv_lmhead_workspace", "sv_lmhead_select", "sv_accept", "sv_embed", "sv_rmsnorm",
           "sv_add_rmsnorm", "sv_draft_input", "sv_linear_splits", "sv_linear_workspace", "sv_linear",
           "sv_linear_tiled_bytes", "sv_linear_tile_weights",
           "sv_geglu", "sv_cluster_unembed_workspace", "sv_cluster_unembed", "sv_lmhead_select_rs", "sv_accept_rs",
           "sv_verify_attn_noalloc")


class SvError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {msg} ({status})")
        self.status = status


class AttnDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q", ctypes.c_int32), ("n_heads_q", ctypes.c_int32),
                ("n_heads_kv", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("window", ctypes.c_int32),
                ("rope_dims", ctypes.c_int32), ("k_is_v", ctypes.c_int32), ("append", ctypes.c_int32),
                ("q_pos_offset", ctypes.c_int32), ("dtype", ctypes.c_int32), ("in_splits", ctypes.c_int32),
                ("rope_base", ctypes.c_double), ("softmax_scale", ctypes.c_float),
                ("reserved_f", ctypes.c_float), ("cache_capacity", ctypes.c_int64),
                ("q_row_stride", ctypes.c_int64), ("kv_row_stride", ctypes.c_int64),
                ("act_pair", ctypes.c_int32), ("reserved_i", ctypes.c_int32)]


class LMHeadDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("k", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("vocab", ctypes.c_int32), ("mode", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("out_stride", ctypes.c_int32)]


class AcceptDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("k", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("mode", ctypes.c_int32)]


class LinearDesc(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int32), ("in_features", ctypes.c_int32),
                ("out_features", ctypes.c_int32), ("dtype", ctypes.c_int32), ("epilogue", ctypes.c_int32),
                ("act_pair", ctypes.c_int32), ("w_layout", ctypes.c_int32)]


class ClusterDesc(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int32), ("d_model", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("n_clusters", ctypes.c_int32), ("top_clusters", ctypes.c_int32), ("dtype", ctypes.c_int32)]


# host views of the device result structs
ROW_STATS_DTYPE = np.dtype([("top1_id", "<i4"), ("top2_id", "<i4"), ("top1", "<f4"), ("top2", "<f4"),
                            ("lse", "<f4"), ("draft_logit", "<f4"), ("sample_id", "<i4"),
                            ("sample_s1", "<f4"), ("sample_s2", "<f4")])
ACCEPT_OUT_DTYPE = np.dtype([("n_accepted", "<i4"), ("next_token", "<i4"), ("new_len", "<i4"),
                             ("keep_begin", "<i4"), ("keep_end", "<i4"), ("drop_begin", "<i4"),
                             ("drop_end", "<i4"), ("hidden_row", "<i4"), ("residual_row", "<i4"),
                             ("draw_margin", "<f4")])
ROW_STATS_WORDS = ROW_STATS_DTYPE.itemsize // 4   # 9
RS_CAND_DTYPE = np.dtype([("id", "<i4"), ("z", "<f4"), ("s1", "<f4"), ("s2", "<f4"), ("pad", "<i4")])
RS_CAND_WORDS = RS_CAND_DTYPE.itemsize // 4       # 5
RS_CANDIDATES = 4
ACCEPT_OUT_WORDS = ACCEPT_OUT_DTYPE.itemsize // 4  # 10

_lib = None


def load():
    """Load libspecverify.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`")
    L = ctypes.CDLL(LIB_PATH)
    P, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    L.sv_status_string.restype = ctypes.c_char_p
    L.sv_status_string.argtypes = [ctypes.c_int]
    L.sv_version.restype = ctypes.c_char_p
    L.sv_verify_attn_workspace.restype = sz
    L.sv_verify_attn_workspace.argtypes = [ctypes.POINTER(AttnDesc)]
    L.sv_verify_attn.restype = ctypes.c_int
    L.sv_verify_attn.argtypes = [ctypes.POINTER(AttnDesc), P, P, P, P, P, P, P, P, sz, P, P]
    L.sv_verify_attn_noalloc.restype = ctypes.c_int
    L.sv_verify_attn_noalloc.argtypes = [ctypes.POINTER(AttnDesc), P, P, P, P, P, P, P, P, P]
    L.sv_verify_attn_fp8.restype = ctypes.c_int
    L.sv_verify_attn_fp8.argtypes = [ctypes.POINTER(AttnDesc), P, P, P, P, P, P, P, P, P, P, sz, P, P]
    L.sv_lmhead_workspace.restype = sz
    L.sv_lmhead_workspace.argtypes = [ctypes.POINTER(LMHeadDesc)]
    L.sv_lmhead_select.restype = ctypes.c_int
    L.sv_lmhead_select.argtypes = [ctypes.POINTER(LMHeadDesc), P, P, P, P, P, P, P, P, P, sz, P]
    L.sv_accept.restype = ctypes.c_int
    L.sv_accept.argtypes = [ctypes.POINTER(AcceptDesc), P, P, P, P, P, P, P, P, P]
    L.sv_embed.restype = ctypes.c_int
    L.sv_embed.argtypes = [i32, i32, i32, ctypes.c_int, P, P, f32, P, P, P]
    L.sv_rmsnorm.restype = ctypes.c_int
    L.sv_rmsnorm.argtypes = [i32, i32, f32, P, P, P, ctypes.c_int, P]
    L.sv_add_rmsnorm.restype = ctypes.c_int
    L.sv_add_rmsnorm.argtypes = [i32, i32, f32, P, P, i32, P, P, ctypes.c_int, P]
    L.sv_draft_input.restype = ctypes.c_int
    L.sv_draft_input.argtypes = [i32, i32, i32, f32, P, i32, P, i32, P, i32, P, i32, f32, P, i32, P, P, P]
    L.sv_linear_splits.restype = i32
    L.sv_linear_splits.argtypes = [ctypes.POINTER(LinearDesc)]
    L.sv_linear_workspace.restype = sz
    L.sv_linear_workspace.argtypes = [ctypes.POINTER(LinearDesc)]
    L.sv_linear.restype = ctypes.c_int
    L.sv_linear.argtypes = [ctypes.POINTER(LinearDesc), P, P, P, P, sz, P]
    L.sv_linear_tiled_bytes.restype = sz
    L.sv_linear_tiled_bytes.argtypes = [ctypes.POINTER(LinearDesc)]
    L.sv_linear_tile_weights.restype = ctypes.c_int
    L.sv_linear_tile_weights.argtypes = [ctypes.POINTER(LinearDesc), P, P, P]
    L.sv_geglu.restype = ctypes.c_int
    L.sv_geglu.argtypes = [i32, i32, ctypes.c_int, P, P, P]
    u32 = ctypes.c_uint32
    L.sv_lmhead_select_rs.restype = ctypes.c_int
    L.sv_lmhead_select_rs.argtypes = [ctypes.POINTER(LMHeadDesc), P, P, P, P, u32, u32, P, P, P, P, sz, P]
    L.sv_accept_rs.restype = ctypes.c_int
    L.sv_accept_rs.argtypes = [ctypes.POINTER(AcceptDesc), P, P, P, P, P, P, P, P, P, P, P]
    L.sv_cluster_unembed_workspace.restype = sz
    L.sv_cluster_unembed_workspace.argtypes = [ctypes.POINTER(ClusterDesc)]
    L.sv_cluster_unembed.restype = ctypes.c_int
    L.sv_cluster_unembed.argtypes = [ctypes.POINTER(ClusterDesc), P, P, P, P, P, P, P, i32, P, sz, P]
    _lib = L
    return L


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, rc: int):
    if rc != SV_OK:
        raise SvError(fn, rc, sv_status_string(rc))


def _dtype_code(t) -> int:
    import torch
    return {torch.bfloat16: SV_BF16, torch.float32: SV_F32}[t.dtype]


# ---------------------------------------------------------------------------
# the C ABI, one Python function per entry point
# ---------------------------------------------------------------------------

def sv_status_string(status: int) -> str:
    return load().sv_status_string(int(status)).decode()


def sv_version() -> str:
    return load().sv_version().decode()


def sv_verify_attn_workspace(desc: AttnDesc) -> int:
    return int(load().sv_verify_attn_workspace(ctypes.byref(desc)))


def sv_verify_attn(desc: AttnDesc, q, k_new, v_new, k_cache, v_cache, cache_len, out, workspace,
                   dev_status=None, stream=None) -> None:
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = load().sv_verify_attn(ctypes.byref(desc), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                               _ptr(v_cache), _ptr(cache_len), _ptr(out), _ptr(workspace), ws_bytes,
                               _ptr(dev_status), _stream(stream))
    _check("sv_verify_attn", rc)


def sv_verify_attn_noalloc(desc: AttnDesc, q, k_new, v_new, k_cache, v_cache, cache_len, out, dev_status=None,
                           stream=None) -> None:
    rc = load().sv_verify_attn_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                                       _ptr(v_cache), _ptr(cache_len), _ptr(out), _ptr(dev_status), _stream(stream))
    _check("sv_verify_attn_noalloc", rc)


def sv_verify_attn_fp8(desc: AttnDesc, q, k_new, v_new, k_cache, v_cache, k_scale, v_scale, cache_len, out,
                       workspace, dev_status=None, stream=None) -> None:
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = load().sv_verify_attn_fp8(ctypes.byref(desc), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                                   _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(cache_len), _ptr(out),
                                   _ptr(workspace), ws_bytes, _ptr(dev_status), _stream(stream))
    _check("sv_verify_attn_fp8", rc)


def sv_lmhead_workspace(desc: LMHeadDesc) -> int:
    return int(load().sv_lmhead_workspace(ctypes.byref(desc)))


def sv_lmhead_select(desc: LMHeadDesc, hidden, w, drafts, u_tok, q_rows, stats, acc, out_tokens, workspace,
                     stream=None) -> None:
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = load().sv_lmhead_select(ctypes.byref(desc), _ptr(hidden), _ptr(w), _ptr(drafts), _ptr(u_tok),
                                 _ptr(q_rows), _ptr(stats), _ptr(acc), _ptr(out_tokens), _ptr(workspace),
                                 ws_bytes, _stream(stream))
    _check("sv_lmhead_select", rc)


def sv_lmhead_select_rs(desc: LMHeadDesc, hidden, w, drafts, u_tok, key0: int, key1: int, stats, cands, out_tokens,
                        workspace, stream=None) -> None:
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = load().sv_lmhead_select_rs(ctypes.byref(desc), _ptr(hidden), _ptr(w), _ptr(drafts), _ptr(u_tok),
                                    int(key0) & 0xFFFFFFFF, int(key1) & 0xFFFFFFFF, _ptr(stats), _ptr(cands),
                                    _ptr(out_tokens), _ptr(workspace), ws_bytes, _stream(stream))
    _check("sv_lmhead_select_rs", rc)


def sv_accept_rs(desc: AcceptDesc, drafts, stats, cands, q_rows, u_accept, u_rs, cache_len, out_tokens, acc,
                 dev_status=None, stream=None) -> None:
    rc = load().sv_accept_rs(ctypes.byref(desc), _ptr(drafts), _ptr(stats), _ptr(cands), _ptr(q_rows),
                             _ptr(u_accept), _ptr(u_rs), _ptr(cache_len), _ptr(out_tokens), _ptr(acc),
                             _ptr(dev_status), _stream(stream))
    _check("sv_accept_rs", rc)


def decode_rs_cands(t) -> np.ndarray:
    """int32 tensor [..., 5] holding sv_rs_cand -> structured numpy array."""
    a = np.ascontiguousarray(t.detach().cpu().numpy().astype(np.int32, copy=False))
    return a.view(RS_CAND_DTYPE).reshape(a.shape[:-1])


def sv_accept(desc: AcceptDesc, drafts, stats, q_rows, u_accept, cache_len, out_tokens, acc,
              dev_status=None, stream=None) -> None:
    rc = load().sv_accept(ctypes.byref(desc), _ptr(drafts), _ptr(stats), _ptr(q_rows), _ptr(u_accept),
                          _ptr(cache_len), _ptr(out_tokens), _ptr(acc), _ptr(dev_status), _stream(stream))
    _check("sv_accept", rc)


def sv_embed(rows: int, d_model: int, vocab: int, dtype: int, tokens, table, scale: float, x,
             dev_status=None, stream=None) -> None:
    rc = load().sv_embed(rows, d_model, vocab, dtype, _ptr(tokens), _ptr(table), float(scale), _ptr(x),
                         _ptr(dev_status), _stream(stream))
    _check("sv_embed", rc)


def sv_rmsnorm(rows: int, dim: int, eps: float, x, gain, y, out_dtype: int, stream=None) -> None:
    rc = load().sv_rmsnorm(rows, dim, float(eps), _ptr(x), _ptr(gain), _ptr(y), out_dtype, _stream(stream))
    _check("sv_rmsnorm", rc)


def sv_add_rmsnorm(rows: int, dim: int, eps: float, x, parts, splits: int, gain, y, out_dtype: int,
                   stream=None) -> None:
    rc = load().sv_add_rmsnorm(rows, dim, float(eps), _ptr(x), _ptr(parts), int(splits), _ptr(gain), _ptr(y),
                               out_dtype, _stream(stream))
    _check("sv_add_rmsnorm", rc)


def sv_draft_input(batch: int, d_main: int, d_draft: int, eps: float, hidden, rows_h: int, hidden_row,
                   row_stride: int, emb, vocab: int, tokens, tok_stride: int, emb_scale: float, cat,
                   cat_dtype: int, x, dev_status=None, stream=None) -> None:
    rc = load().sv_draft_input(batch, d_main, d_draft, float(eps), _ptr(hidden), rows_h, _ptr(hidden_row),
                               row_stride, _ptr(emb), vocab, _ptr(tokens), tok_stride, float(emb_scale),
                               _ptr(cat), cat_dtype, _ptr(x), _ptr(dev_status), _stream(stream))
    _check("sv_draft_input", rc)


def sv_linear_splits(desc: LinearDesc) -> int:
    return int(load().sv_linear_splits(ctypes.byref(desc)))


def sv_linear_workspace(desc: LinearDesc) -> int:
    return int(load().sv_linear_workspace(ctypes.byref(desc)))


def sv_linear(desc: LinearDesc, x, w, y, workspace=None, stream=None) -> None:
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = load().sv_linear(ctypes.byref(desc), _ptr(x), _ptr(w), _ptr(y), _ptr(workspace), ws_bytes,
                          _stream(stream))
    _check("sv_linear", rc)


def sv_linear_tiled_bytes(desc: LinearDesc) -> int:
    return int(load().sv_linear_tiled_bytes(ctypes.byref(desc)))


def sv_linear_tile_weights(desc: LinearDesc, w, w_tiled, stream=None) -> None:
    rc = load().sv_linear_tile_weights(ctypes.byref(desc), _ptr(w), _ptr(w_tiled), _stream(stream))
    _check("sv_linear_tile_weights", rc)


def tiled_weight(desc: LinearDesc, w, stream=None):
    """A new device tensor holding the tiled copy of w ([N, K] bf16) for desc."""
    import torch
    n = sv_linear_tiled_bytes(desc)
    if n <= 0:
        raise SvError("sv_linear_tiled_bytes", SV_ERR_ARG, "no tiled layout for this descriptor")
    wt = torch.empty(n // 2, dtype=torch.bfloat16, device=w.device)
    sv_linear_tile_weights(desc, w, wt, stream)
    return wt


def sv_geglu(rows: int, d_ff: int, dtype: int, gate_up, out, stream=None) -> None:
    rc = load().sv_geglu(rows, d_ff, dtype, _ptr(gate_up), _ptr(out), _stream(stream))
    _check("sv_geglu", rc)


def sv_cluster_unembed_workspace(desc: ClusterDesc) -> int:
    return int(load().sv_cluster_unembed_workspace(ctypes.byref(desc)))


def sv_cluster_unembed(desc: ClusterDesc, hidden, centroids, w_perm, perm, stats, clusters, out_tokens,
                       out_stride: int, workspace, stream=None) -> None:
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = load().sv_cluster_unembed(ctypes.byref(desc), _ptr(hidden), _ptr(centroids), _ptr(w_perm), _ptr(perm),
                                   _ptr(stats), _ptr(clusters), _ptr(out_tokens), int(out_stride),
                                   _ptr(workspace), ws_bytes, _stream(stream))
    _check("sv_cluster_unembed", rc)


def decode_row_stats(t) -> np.ndarray:
    """int32 tensor [..., 9] holding sv_row_stats -> structured numpy array."""
    a = np.ascontiguousarray(t.detach().cpu().numpy().astype(np.int32, copy=False))
    return a.view(ROW_STATS_DTYPE).reshape(a.shape[:-1])


def decode_accept_out(t) -> np.ndarray:
    a = np.ascontiguousarray(t.detach().cpu().numpy().astype(np.int32, copy=False))
    return a.view(ACCEPT_OUT_DTYPE).reshape(a.shape[:-1])
