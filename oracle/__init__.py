"""CPU oracle for the MTP verify step -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never uses it, shares no
code with it, and the product path fails loudly instead of falling back to it.

The arithmetic lives in ``svoracle.c`` (plain fp64 loops, built with gcc into
``liboracle.so``).  This module only marshals numpy arrays into those loops;
``model.py`` composes them into a whole verify step of a small decoder stack.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "svoracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# another build of svoracle.c to load instead (the sanitizer test's ASan/UBSan build)
_LIB_OVERRIDE = os.environ.get("SVO_ORACLE_LIB")

_lib = None


def build() -> str:
    """Compile liboracle.so with gcc (OpenMP, no fast-math: IEEE fp64)."""
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-std=gnu11", "-Wall", "-shared", "-fPIC",
           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


class AttnArgs(ctypes.Structure):
    _fields_ = [
        ("n_q", ctypes.c_int32), ("group", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("window", ctypes.c_int32), ("rope_dims", ctypes.c_int32), ("k_is_v", ctypes.c_int32),
        ("append", ctypes.c_int32), ("q_pos_offset", ctypes.c_int32),
        ("round_bf16", ctypes.c_int32), ("pad_", ctypes.c_int32),
        ("rope_base", ctypes.c_double), ("scale", ctypes.c_double),
        ("cap", ctypes.c_int64), ("L", ctypes.c_int64),
        ("q", ctypes.c_void_p), ("k_new", ctypes.c_void_p), ("v_new", ctypes.c_void_p),
        ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p), ("out", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
    ]


class Stats(ctypes.Structure):
    _fields_ = [
        ("top1_id", ctypes.c_int32), ("top2_id", ctypes.c_int32),
        ("top1", ctypes.c_double), ("top2", ctypes.c_double),
        ("lse", ctypes.c_double), ("draft_logit", ctypes.c_double),
    ]


def lib():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            L = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
            L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64, i32, f64 = ctypes.c_int64, ctypes.c_int32, ctypes.c_double
        L.svo_num_threads.restype = ctypes.c_int
        L.svo_bf16_round.restype = f64
        L.svo_bf16_round.argtypes = [f64]
        L.svo_bf16_round_array.argtypes = [P, i64]
        L.svo_rope.argtypes = [P, ctypes.c_int, f64, f64]
        L.svo_e4m3_decode.restype = f64
        L.svo_e4m3_decode.argtypes = [ctypes.c_int]
        L.svo_e4m3_encode.restype = ctypes.c_int
        L.svo_e4m3_encode.argtypes = [ctypes.c_float]
        L.svo_attn_group.argtypes = [ctypes.POINTER(AttnArgs)]
        L.svo_attn_group.restype = ctypes.c_int
        L.svo_linear.argtypes = [i64, i64, i64, P, P, ctypes.c_int, P]
        L.svo_rmsnorm.argtypes = [i64, i64, f64, P, P]
        L.svo_gelu_tanh.argtypes = [f64]
        L.svo_gelu_tanh.restype = f64
        L.svo_geglu.argtypes = [i64, P, P, P]
        L.svo_lmhead.argtypes = [i64, i64, i64, P, P, ctypes.c_int, P]
        L.svo_row_stats.argtypes = [i64, P, i32, ctypes.POINTER(Stats)]
        L.svo_accept_greedy.argtypes = [ctypes.c_int, P, P, P]
        L.svo_accept_greedy.restype = ctypes.c_int
        L.svo_accept_sample.argtypes = [ctypes.c_int, P, P, P, P, P]
        L.svo_accept_sample.restype = ctypes.c_int
        L.svo_sample_residual.argtypes = [i64, P, f64, P, P, ctypes.POINTER(f64)]
        L.svo_sample_residual.restype = ctypes.c_int
        L.svo_sample_bonus.argtypes = [i64, P, P, ctypes.POINTER(f64)]
        L.svo_sample_bonus.restype = ctypes.c_int
        L.svo_toy_spec_trials.argtypes = [i64, ctypes.c_int, i64, P, P, P, P, P, P, P]
        u32 = ctypes.c_uint32
        L.svo_philox4x32.argtypes = [P, P, P]
        L.svo_rs_uniform.restype = f64
        L.svo_rs_uniform.argtypes = [u32, u32, ctypes.c_int, ctypes.c_int, i64, ctypes.c_int]
        L.svo_rs_candidates.argtypes = [i64, P, u32, u32, ctypes.c_int, ctypes.c_int, ctypes.c_int, P, P]
        L.svo_rs_accept.restype = ctypes.c_int
        L.svo_rs_accept.argtypes = [ctypes.c_int, P, P, f64, P, P, P]
        L.svo_toy_spec_trials_rs.argtypes = [i64, ctypes.c_int, i64, P, P, P, P, P, u32, u32, ctypes.c_int, P, P, P,
                                             P]
        _lib = L
    return _lib


def num_threads() -> int:
    return int(lib().svo_num_threads())


def set_threads(n: int) -> None:
    """Threads of the oracle's parallel loops from now on (for timing; results do not
    depend on the count)."""
    lib().svo_set_threads(ctypes.c_int(int(n)))


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


def _weight(w: np.ndarray):
    """(array, is_bf16): fp32 arrays pass as they are, uint16 arrays are bf16 bits."""
    if w.dtype == np.uint16:
        return np.ascontiguousarray(w), 1
    return _f32(w), 0


# --------------------------------------------------------------------------
# elementwise pieces
# --------------------------------------------------------------------------

def bf16_round(x) -> np.ndarray:
    y = _f64(x).copy()
    lib().svo_bf16_round_array(_ptr(y), y.size)
    return y


def rope(x, rope_dims: int, base: float, pos: float) -> np.ndarray:
    y = _f64(x).copy()
    lib().svo_rope(_ptr(y), int(rope_dims), float(base), float(pos))
    return y


def e4m3_decode(codes) -> np.ndarray:
    """Values of fp8 E4M3 codes (OCP E4M3FN: bias 7, subnormals m 2^-9, no
    infinities, 0x7F / 0xFF NaN), fp64, same shape as `codes`."""
    table = np.array([lib().svo_e4m3_decode(c) for c in range(256)], dtype=np.float64)
    return table[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x) -> np.ndarray:
    """Nearest E4M3 code of each fp32 value (ties to even, saturating at +-448)."""
    x = np.asarray(x, dtype=np.float32)
    return np.array([lib().svo_e4m3_encode(float(v)) for v in x.ravel()], dtype=np.uint8).reshape(x.shape)


def dequant_cache(codes, scale) -> np.ndarray:
    """An fp8 cache [..., cap, D] with per-channel scales [D] as the fp32 array the
    attention oracle reads: scale * value, rounded once to fp32."""
    return (e4m3_decode(codes) * np.asarray(scale, dtype=np.float64)).astype(np.float32)


def gelu_tanh(x: float) -> float:
    return float(lib().svo_gelu_tanh(float(x)))


def geglu(g, u) -> np.ndarray:
    g, u = _f64(g), _f64(u)
    f = np.empty_like(g)
    lib().svo_geglu(g.size, _ptr(g), _ptr(u), _ptr(f))
    return f


def rmsnorm(x, eps: float) -> np.ndarray:
    x = _f64(x)
    R, d = x.shape
    y = np.empty_like(x)
    lib().svo_rmsnorm(R, d, float(eps), _ptr(x), _ptr(y))
    return y


def linear(x, w: np.ndarray) -> np.ndarray:
    """y = x @ w.T with w [N, K] (fp32 or bf16 bits), x [R, K] -> fp64 [R, N]."""
    x = _f64(x)
    R, K = x.shape
    wa, wb = _weight(w)
    N = wa.shape[0]
    assert wa.shape[1] == K
    y = np.empty((R, N), dtype=np.float64)
    lib().svo_linear(R, K, N, _ptr(x), _ptr(wa), wb, _ptr(y))
    return y


def lmhead(h, w: np.ndarray) -> np.ndarray:
    """Full logits z = h @ w.T, fp64 [R, V]."""
    h = _f64(h)
    R, d = h.shape
    wa, wb = _weight(w)
    V = wa.shape[0]
    assert wa.shape[1] == d
    z = np.empty((R, V), dtype=np.float64)
    lib().svo_lmhead(R, d, V, _ptr(h), _ptr(wa), wb, _ptr(z))
    return z


def row_stats(z_row, draft_id: int = -1) -> dict:
    z = _f64(z_row)
    st = Stats()
    lib().svo_row_stats(z.size, _ptr(z), int(draft_id), ctypes.byref(st))
    return dict(top1_id=st.top1_id, top2_id=st.top2_id, top1=st.top1, top2=st.top2,
                lse=st.lse, draft_logit=st.draft_logit)


def cluster_unembed(h, centroids, w_perm, perm, top: int) -> list:
    """Clustered unembedding ("Gemma 4 拆解" (marsggbo), section 4.3, cheap_unembed),
    fp64: cluster scores s = h . centroid, the `top` best clusters (ties: lowest
    cluster index), the logits h . w of every token of those clusters (w_perm row j
    is token perm[j]; cluster c owns rows [c V / C, (c + 1) V / C)), and per row the
    statistics over those candidates only: top-1 / top-2 token ids and logits (ties:
    lowest token id) and the log-sum-exp.  Returns one dict per row."""
    h = _f64(h)
    C = np.asarray(centroids).shape[0]
    V = np.asarray(perm).shape[0]
    csize = V // C
    out = []
    scores = lmhead(h, centroids)                          # [R, C] = h . centroid_c
    for r in range(h.shape[0]):
        order = sorted(range(C), key=lambda c: (-scores[r, c], c))
        kept = order[:top]
        rows = np.concatenate([np.arange(c * csize, (c + 1) * csize) for c in kept])
        z = lmhead(h[r:r + 1], np.asarray(w_perm)[rows])[0]
        ids = np.asarray(perm)[rows].astype(np.int64)
        o = sorted(range(rows.size), key=lambda k: (-z[k], ids[k]))
        m = z.max()
        out.append(dict(clusters=kept, top1_id=int(ids[o[0]]), top2_id=int(ids[o[1]]) if rows.size > 1 else -1,
                        top1=float(z[o[0]]), top2=float(z[o[1]]) if rows.size > 1 else float("-inf"),
                        lse=float(m + np.log(np.exp(z - m).sum())),
                        scores=scores[r].copy()))
    return out


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------

def attn_group(*, q, k_new, v_new, k_cache, v_cache, L: int, window: int, rope_dims: int,
               rope_base: float, scale: float, k_is_v: bool, append: bool,
               q_pos_offset: int = 0, round_bf16: bool, k_scale=None, v_scale=None) -> np.ndarray:
    """One sequence, one KV head.  q [n_q, group, D]; k_new/v_new [n_q, D];
    k_cache/v_cache [cap, D] float32 (modified in place when append).  With k_scale /
    v_scale [D] the cache is an fp8 one seen through its scales (dequant_cache): an
    appended row is stored as scale * e4m3(row / scale).
    Returns out [n_q, group, D] fp64."""
    q = _f32(q)
    n_q, group, D = q.shape
    assert k_cache.dtype == np.float32 and k_cache.flags["C_CONTIGUOUS"]
    if v_cache is not None:
        assert v_cache.dtype == np.float32 and v_cache.flags["C_CONTIGUOUS"]
    kn = _f32(k_new) if append else None
    vn = _f32(v_new) if (append and not k_is_v) else None
    out = np.zeros((n_q, group, D), dtype=np.float64)
    ks = None if k_scale is None else _f32(k_scale)
    vs = None if (v_scale is None or k_is_v) else _f32(v_scale)
    assert ks is None or ks.shape == (D,)
    assert vs is None or vs.shape == (D,)
    a = AttnArgs(n_q=n_q, group=group, head_dim=D, window=int(window), rope_dims=int(rope_dims),
                 k_is_v=int(bool(k_is_v)), append=int(bool(append)),
                 q_pos_offset=int(q_pos_offset), round_bf16=int(bool(round_bf16)), pad_=0,
                 rope_base=float(rope_base), scale=float(scale), cap=k_cache.shape[0], L=int(L),
                 q=_ptr(q), k_new=_ptr(kn), v_new=_ptr(vn), k_cache=_ptr(k_cache),
                 v_cache=_ptr(v_cache) if not k_is_v else None, out=_ptr(out),
                 k_scale=_ptr(ks), v_scale=_ptr(vs))
    rc = lib().svo_attn_group(ctypes.byref(a))
    if rc != 0:
        raise ValueError("oracle attention: appended rows exceed the cache capacity")
    return out


def verify_attn(*, q, k_new, v_new, k_cache, v_cache, cache_len, window: int, rope_dims: int,
                rope_base: float, scale: float, k_is_v: bool, append: bool = True,
                q_pos_offset: int = 0, round_bf16: bool, k_scale=None, v_scale=None) -> np.ndarray:
    """Whole batch.  q [B, n_q, Hq, D]; k_new/v_new [B, n_q, Hkv, D];
    k_cache/v_cache [B, Hkv, cap, D] float32 (modified in place); k_scale / v_scale
    [Hkv, D] for fp8 caches (see attn_group).
    Returns out [B, n_q, Hq, D] fp64."""
    q = np.asarray(q)
    B, n_q, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, n_q, Hq, D), dtype=np.float64)
    for b in range(B):
        for g in range(Hkv):
            kc = k_cache[b, g]
            vc = None if k_is_v else v_cache[b, g]
            o = attn_group(q=q[b, :, g * G:(g + 1) * G, :],
                           k_new=None if k_new is None else k_new[b, :, g, :],
                           v_new=None if (v_new is None or k_is_v) else v_new[b, :, g, :],
                           k_cache=kc, v_cache=vc, L=int(cache_len[b]), window=window,
                           rope_dims=rope_dims, rope_base=rope_base, scale=scale,
                           k_is_v=k_is_v, append=append, q_pos_offset=q_pos_offset,
                           round_bf16=round_bf16, k_scale=None if k_scale is None else k_scale[g],
                           v_scale=None if v_scale is None else v_scale[g])
            out[b, :, g * G:(g + 1) * G, :] = o
    return out


# --------------------------------------------------------------------------
# acceptance
# --------------------------------------------------------------------------

def accept_greedy(drafts, top1) -> tuple[int, np.ndarray]:
    """One sequence: drafts [k], top1 [k+1] -> (n, tokens[k+1] padded with -1)."""
    d, t = _i32(drafts), _i32(top1)
    k = d.size
    assert t.size == k + 1
    out = np.empty(k + 1, dtype=np.int32)
    n = lib().svo_accept_greedy(k, _ptr(d), _ptr(t), _ptr(out))
    return int(n), out


def accept_sample(lse, draft_logit, q_at_draft, u_accept) -> tuple[int, np.ndarray]:
    """One sequence: lse/draft_logit of rows 0..k-1, q_i(d_i), u_i -> (n, margins[k])."""
    lse, dl = _f64(lse), _f64(draft_logit)
    qd, ua = _f32(q_at_draft), _f32(u_accept)
    k = lse.size
    margin = np.full(k, np.nan, dtype=np.float64)
    n = lib().svo_accept_sample(k, _ptr(lse), _ptr(dl), _ptr(qd), _ptr(ua), _ptr(margin))
    return int(n), margin


def sample_residual(z_row, lse: float, q_row, u_row) -> tuple[int, float]:
    z, q, u = _f64(z_row), _f32(q_row), _f32(u_row)
    m = ctypes.c_double()
    y = lib().svo_sample_residual(z.size, _ptr(z), float(lse), _ptr(q), _ptr(u), ctypes.byref(m))
    return int(y), float(m.value)


def sample_bonus(z_row, u_row) -> tuple[int, float]:
    z, u = _f64(z_row), _f32(u_row)
    m = ctypes.c_double()
    y = lib().svo_sample_bonus(z.size, _ptr(z), _ptr(u), ctypes.byref(m))
    return int(y), float(m.value)


def philox4x32(ctr, key) -> np.ndarray:
    """One Philox4x32-10 block: counter [4] and key [2] uint32 -> 4 uint32."""
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    o = np.zeros(4, dtype=np.uint32)
    lib().svo_philox4x32(_ptr(c), _ptr(k), _ptr(o))
    return o


def rs_uniform(key, b: int, i: int, v: int, r: int) -> float:
    return float(lib().svo_rs_uniform(int(key[0]), int(key[1]), int(b), int(i), int(v), int(r)))


def rs_candidates(z_row, key, b: int, i: int, R: int = 4) -> tuple[np.ndarray, np.ndarray]:
    """R draws from softmax(z_row) for draft row (b, i) under `key` (2 uint32):
    (token ids [R], Gumbel margins [R])."""
    z = _f64(z_row)
    cand = np.empty(R, dtype=np.int32)
    margin = np.empty(R, dtype=np.float64)
    lib().svo_rs_candidates(z.size, _ptr(z), int(key[0]), int(key[1]), int(b), int(i), int(R), _ptr(cand),
                            _ptr(margin))
    return cand, margin


def rs_accept(cand, z_row, lse: float, q_row, u_rs) -> tuple[int, np.ndarray]:
    """Residual by rejection over the candidates: (token or -1, margins [R])."""
    c, z, q, u = _i32(cand), _f64(z_row), _f32(q_row), _f32(u_rs)
    margin = np.full(c.size, np.nan, dtype=np.float64)
    y = lib().svo_rs_accept(c.size, _ptr(c), _ptr(z), float(lse), _ptr(q), _ptr(u), _ptr(margin))
    return int(y), margin


def toy_spec_trials_rs(z, q, drafts, u_acc, u_tok, key, u_rs) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """toy_spec_trials with single-pass sampling (see svo_toy_spec_trials_rs).
    Returns (n [T], y [T], fallback used [T])."""
    z, q = _f64(z), _f32(q)
    d, ua, ut, ur = _i32(drafts), _f32(u_acc), _f32(u_tok), _f32(u_rs)
    T, k = d.shape
    V = z.size
    R = ur.shape[1]
    n = np.empty(T, dtype=np.int32)
    y = np.empty(T, dtype=np.int32)
    fb = np.empty(T, dtype=np.int32)
    lib().svo_toy_spec_trials_rs(T, k, V, _ptr(z), _ptr(q), _ptr(d), _ptr(ua), _ptr(ut), int(key[0]), int(key[1]),
                                 R, _ptr(ur), _ptr(n), _ptr(y), _ptr(fb))
    return n, y, fb


def toy_spec_trials(z, q, drafts, u_acc, u_tok) -> tuple[np.ndarray, np.ndarray]:
    """Many sampling-mode steps of a context-free toy (see svo_toy_spec_trials).
    z [V] logits, q [V] drafter probabilities, drafts [T, k], u_acc [T, k], u_tok [T, V].
    Returns (n [T], y [T])."""
    z, q = _f64(z), _f32(q)
    d, ua, ut = _i32(drafts), _f32(u_acc), _f32(u_tok)
    T, k = d.shape
    V = z.size
    assert ut.shape == (T, V) and ua.shape == (T, k)
    n = np.empty(T, dtype=np.int32)
    y = np.empty(T, dtype=np.int32)
    lib().svo_toy_spec_trials(T, k, V, _ptr(z), _ptr(q), _ptr(d), _ptr(ua), _ptr(ut), _ptr(n), _ptr(y))
    return n, y
