"""Pins of the oracle's compositions against an independent numpy fp64 recomputation.

The oracle computes a verify step with C loops (svoracle.c) strung together by
oracle/model.py.  The tests below recompute the same quantities from their plain
definitions with code that shares nothing with it: RoPE as a complex rotation of
the pairs (x_i, x_{i+r/2}), attention as a dense einsum with a visibility mask and
exp() taken directly (no max shift), the GELU in its logistic form, bf16 rounding
from frexp/rint, the decoder layer written per sequence.  A plausible slip in the
composition (a dropped residual, a norm in the wrong place, a missing sqrt(d) on
the embedding or a missing final norm, a transposed projection, a wrong RoPE
position) changes the result far beyond the 1e-10 these comparisons allow.

The composition itself follows the pages: one target forward over [last committed
token, d_1..d_k] ("Gemma 4 拆解" (marsggbo), section 4.2, speculative_step:
main_model.verify, then accept_longest_prefix), local and global layers in a 5:1
pattern with p-RoPE and value = key on the global ones ("Gemma 4 发布时未包含 MTP
数据" (flowhunt), section "什么是 Gemma 4？"; "Gemma 4 拆解", section 2).
"""
import math

import numpy as np
import pytest
from scipy import special, stats

import oracle
from oracle import model as om
from mtp_draft_verification_amd import configs, inputs


# ---------------------------------------------------------------------------
# independent building blocks (numpy, fp64)
# ---------------------------------------------------------------------------

def bf16_rne(x):
    """Round fp64 values to the nearest bf16 value, ties to even (8 significant
    bits): the quantum of |x| in [2^(e-1), 2^e) is 2^(e-8)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    nz = x != 0
    _, e = np.frexp(x[nz])
    q = np.ldexp(1.0, e - 8)
    out[nz] = np.rint(x[nz] / q) * q
    return out


def f32_rne(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def rope_complex(x, pos, r, base):
    """Rotate the pairs (x_i, x_{i+r/2}), i < r/2, by the angle pos * base^(-2i/r),
    written as a product of complex numbers; dims >= r are left alone.
    x [..., D] fp64, pos broadcastable to x.shape[:-1]."""
    x = np.array(x, dtype=np.float64)
    if r == 0:
        return x
    h = r // 2
    inv_freq = np.power(float(base), -np.arange(h, dtype=np.float64) * 2.0 / r)
    z = (x[..., :h] + 1j * x[..., h:r]) * np.exp(1j * np.asarray(pos, dtype=np.float64)[..., None] * inv_freq)
    x[..., :h] = z.real
    x[..., h:r] = z.imag
    return x


def attn_dense(q, keys, vals, qpos, n_keys, window, scale):
    """q [n, Hq, D] (already rotated), keys/vals [Hkv, T, D]; key t is visible to the
    query at position qpos[j] iff t < n_keys, t <= qpos[j] and (no window or
    t > qpos[j] - window).  Softmax with exp() taken directly."""
    n, Hq, D = q.shape
    Hkv, T, _ = keys.shape
    G = Hq // Hkv
    kh = keys[np.arange(Hq) // G]                 # [Hq, T, D]
    vh = vals[np.arange(Hq) // G]
    t = np.arange(T)
    vis = (t[None, :] < n_keys) & (t[None, :] <= qpos[:, None])
    if window:
        vis &= t[None, :] > qpos[:, None] - window
    s = np.einsum("jhd,htd->jht", q, kh) * scale
    w = np.where(vis[:, None, :], np.exp(s), 0.0)
    den = w.sum(-1, keepdims=True)
    w = np.divide(w, den, out=np.zeros_like(w), where=den > 0)
    return np.einsum("jht,htd->jhd", w, vh)


def rms_norm(x, eps):
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def gelu_logistic(x):
    # 0.5 (1 + tanh(y)) == 1 / (1 + exp(-2y)), y = sqrt(2/pi) (x + 0.044715 x^3)
    y = math.sqrt(2.0 / math.pi) * (x + 0.044715 * x ** 3)
    return x * special.expit(2.0 * y)


def as_f64(w):
    w = np.asarray(w)
    if w.dtype == np.uint16:
        return (w.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return w.astype(np.float64)


class DenseStack:
    """The verify forward of a pre-norm decoder stack, one sequence at a time:
    x = sqrt(d) E[tok]; per layer a = norm(x), q/k/v = a W, RoPE on q and the new
    keys at positions L+j, the new rows appended to the layer's cache, causal
    (sliding-window) attention, x += o Wo; m = norm(x), x += (gelu(m Wg) (m Wu)) Wd;
    h = norm(x); z = h E^T.  Stored values are rounded as the stack stores them:
    activations between the ops in fp32; new cache rows and the final hidden state
    in the stack's type (bf16 or fp32)."""

    def __init__(self, cfg, weights):
        self.cfg = cfg
        self.E = as_f64(weights["E"])
        self.layers = [{k: as_f64(v) for k, v in lw.items()} for lw in weights["layers"]]
        self.store = f32_rne
        self.store_kv = bf16_rne if cfg.dtype == "bf16" else f32_rne

    def forward(self, caches, L, tokens):
        """caches: per layer {"k": [B, Hkv, cap, D], "v": same or None} (fp32, updated);
        L [B]; tokens [B, n].  Returns (h [B*n, d], z [B*n, V])."""
        cfg, st, skv = self.cfg, self.store, self.store_kv
        B, n = tokens.shape
        hs, zs = [], []
        for b in range(B):
            pos = int(L[b]) + np.arange(n)
            x = math.sqrt(cfg.d_model) * self.E[tokens[b]]
            for ly, lw, c in zip(cfg.layers, self.layers, caches):
                H, Hk, D = ly.n_heads_q, ly.n_heads_kv, ly.head_dim
                a = st(rms_norm(x, cfg.eps) if cfg.norm else x)
                wq = lw["wqkv"][:H * D]
                wk = lw["wqkv"][H * D:(H + Hk) * D]
                q = st(a @ wq.T).reshape(n, H, D)
                kn = st(a @ wk.T).reshape(n, Hk, D)
                q = rope_complex(q, pos[:, None], ly.rope_dims, ly.rope_base)
                kn = skv(rope_complex(kn, pos[:, None], ly.rope_dims, ly.rope_base))
                c["k"][b, :, pos[0]:pos[-1] + 1] = kn.transpose(1, 0, 2)
                if not ly.k_is_v:
                    wv = lw["wqkv"][(H + Hk) * D:]
                    vn = skv(st(a @ wv.T)).reshape(n, Hk, D)
                    c["v"][b, :, pos[0]:pos[-1] + 1] = vn.transpose(1, 0, 2)
                keys = c["k"][b].astype(np.float64)
                vals = keys if ly.k_is_v else c["v"][b].astype(np.float64)
                o = attn_dense(q, keys, vals, pos, pos[-1] + 1, ly.window, ly.scale)
                x = x + st(o.reshape(n, H * D)) @ lw["wo"].T
                if cfg.d_ff:
                    m = st(rms_norm(x, cfg.eps) if cfg.norm else x)
                    g = m @ lw["wgu"][:cfg.d_ff].T
                    u = m @ lw["wgu"][cfg.d_ff:].T
                    x = x + st(gelu_logistic(g) * u) @ lw["wd"].T
            h = skv(rms_norm(x, cfg.eps) if cfg.norm else x)
            hs.append(h)
            zs.append(h @ self.E.T)
        return np.concatenate(hs), np.concatenate(zs)


def _host(cfg, seed, extra=16):
    W = inputs.stack_weights(cfg, seed)
    conv = inputs.bf16_bits if cfg.dtype == "bf16" else inputs.host_f32
    host = {"E": conv(W["E"]), "layers": [{k: conv(v) for k, v in lw.items()} for lw in W["layers"]]}
    caches = inputs.stack_caches(cfg, seed, capacity=cfg.ctx + extra)
    hc = [{"k": inputs.host_f32(c["k"]), "v": None if c["v"] is None else inputs.host_f32(c["v"])}
          for c in caches]
    return host, hc


def _copy_caches(hc):
    return [{"k": c["k"].copy(), "v": None if c["v"] is None else c["v"].copy()} for c in hc]


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def _two_layer(dtype):
    # one sliding-window layer (GQA 4:2, full RoPE, window shorter than the context)
    # and one global layer (GQA 4:1, p-RoPE over a quarter of the dims, base 1e6,
    # value = key), pre-norm, GeGLU MLP, tied embedding
    return configs.StackConfig(
        name="two_layer", d_model=48, vocab=131,
        layers=(configs.local_layer(4, 2, 16, 7), configs.global_layer(4, 1, 32)),
        d_ff=80, norm=True, eps=1e-6, dtype=dtype, batch=3, k=4, ctx=23, steps=1)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_stack_forward_equals_dense_recomputation(dtype):
    cfg = _two_layer(dtype)
    host, hc = _host(cfg, seed=5)
    L = np.array([23, 9, 30], dtype=np.int32)            # ragged committed lengths
    tokens = inputs.randint((cfg.batch, cfg.k + 1), 0, cfg.vocab - 1, 5, "tok").numpy()
    ref = DenseStack(cfg, host)
    c_ref = _copy_caches(hc)
    h_ref, z_ref = ref.forward(c_ref, L, tokens)
    st = om.new_state(_copy_caches(hc), L)
    h, z = om.OracleModel(cfg, host).forward(st, tokens)
    assert _rel(h, h_ref) < 1e-10
    assert _rel(z, z_ref) < 1e-10
    # the appended rows: same stored values; every other row untouched
    for c, cr in zip(st["caches"], c_ref):
        np.testing.assert_array_equal(c["k"], cr["k"])
        if c["v"] is not None:
            np.testing.assert_array_equal(c["v"], cr["v"])


def test_stack_greedy_step_equals_dense_recomputation():
    """The whole greedy step: logits, per-row argmax, the longest matching prefix,
    the emitted tokens and the new lengths ("Gemma 4 拆解", section 4.2,
    accept_longest_prefix; one more token of the target's own, "Accelerating
    Gemma 4 ..." (Lighthouse), section 3)."""
    cfg = _two_layer("bf16")
    host, hc = _host(cfg, seed=8)
    L = np.array([15, 31, 20], dtype=np.int32)
    ref = DenseStack(cfg, host)
    first = np.array([3, 77, 120])
    # drafts: the target's own greedy continuation with one wrong token per sequence
    # at a different place (0, 2, none)
    cont = []
    cc = _copy_caches(hc)
    for b in range(cfg.batch):
        toks, cur, Lb = [], int(first[b]), int(L[b])
        for _ in range(cfg.k):
            sub = [{"k": c["k"][b:b + 1], "v": None if c["v"] is None else c["v"][b:b + 1]} for c in cc]
            _, z1 = ref.forward(sub, np.array([Lb]), np.array([[cur]]))
            cur = int(np.argmax(z1[0]))
            toks.append(cur)
            Lb += 1
        cont.append(toks)
    drafts = np.array(cont)
    drafts[0, 0] = (drafts[0, 0] + 1) % cfg.vocab
    drafts[1, 2] = (drafts[1, 2] + 1) % cfg.vocab
    tokens = np.concatenate([first[:, None], drafts], axis=1)
    _, z_ref = ref.forward(_copy_caches(hc), L, tokens)
    st = om.new_state(_copy_caches(hc), L)
    r = om.OracleModel(cfg, host).greedy_step(st, tokens)
    n = cfg.k + 1
    for b in range(cfg.batch):
        top1 = np.argmax(z_ref[b * n:(b + 1) * n], axis=1)   # first maximum = lowest id
        nb = 0
        while nb < cfg.k and drafts[b, nb] == top1[nb]:
            nb += 1
        assert r["n"][b] == nb
        assert list(r["tokens"][b, :nb + 1]) == list(drafts[b, :nb]) + [top1[nb]]
        assert r["new_len"][b] == L[b] + nb + 1
    assert list(r["n"]) == [0, 2, 4]
    assert _rel(r["z"], z_ref) < 1e-10


def test_tiny_fp32_verify_step_equals_dense_recomputation():
    """The tiny fp32 workload (one attention layer, 2 q heads / 1 KV head, head dim
    64, no RoPE / norm / MLP, 64 cached tokens, k = 3, vocab 1024)."""
    cfg = configs.TINY_F32
    host, hc = _host(cfg, seed=0)
    L = np.array([cfg.ctx], dtype=np.int32)
    tokens = np.array([[5, 900, 17, 1023]])
    h_ref, z_ref = DenseStack(cfg, host).forward(_copy_caches(hc), L, tokens)
    st = om.new_state(_copy_caches(hc), L)
    h, z = om.OracleModel(cfg, host).forward(st, tokens)
    assert _rel(h, h_ref) < 1e-10
    assert _rel(z, z_ref) < 1e-10


@pytest.mark.parametrize("kind", ["local", "global", "drafter_read"])
def test_attention_many_keys_brute_force(kind):
    """Many keys, several heads, GQA, RoPE (full or p-RoPE), a window, ragged
    lengths and positions past 10^5: the oracle's attention against the dense
    direct-exp softmax."""
    rng = np.random.default_rng({"local": 1, "global": 2, "drafter_read": 3}[kind])
    B, nq = 3, 5
    if kind == "local":
        Hq, Hkv, D, window, r, base, kv_same = 8, 2, 32, 40, 32, 1e4, False
        L = np.array([37, 260, 123456], dtype=np.int32)
    else:
        Hq, Hkv, D, window, r, base, kv_same = 8, 1, 64, 0, 16, 1e6, True
        L = np.array([1, 300, 200], dtype=np.int32)
    read_only = kind == "drafter_read"
    if read_only:
        nq = 1
    lo = np.maximum(L - (window + 8 if window else 10 ** 9), 0)
    cap = int(L.max()) + nq + 4
    q = rng.standard_normal((B, nq, Hq, D)).astype(np.float32)
    kn = rng.standard_normal((B, nq, Hkv, D)).astype(np.float32)
    vn = None if kv_same else rng.standard_normal((B, nq, Hkv, D)).astype(np.float32)
    kc = np.zeros((B, Hkv, cap, D), dtype=np.float32)
    vc = None if kv_same else np.zeros_like(kc)
    for b in range(B):
        kc[b, :, lo[b]:L[b]] = rng.standard_normal((Hkv, L[b] - lo[b], D))
        if vc is not None:
            vc[b, :, lo[b]:L[b]] = rng.standard_normal((Hkv, L[b] - lo[b], D))
    off = 2 if read_only else 0
    scale = D ** -0.5
    kc_o, vc_o = kc.copy(), None if vc is None else vc.copy()
    out = oracle.verify_attn(q=q, k_new=None if read_only else kn, v_new=None if read_only else vn,
                             k_cache=kc_o, v_cache=vc_o, cache_len=L, window=window, rope_dims=r,
                             rope_base=base, scale=scale, k_is_v=kv_same, append=not read_only,
                             q_pos_offset=off, round_bf16=False)
    for b in range(B):
        pos = L[b] + off + np.arange(nq)
        keys = kc[b].astype(np.float64)
        vals = keys if kv_same else vc[b].astype(np.float64)
        n_keys = L[b] if read_only else L[b] + nq
        if not read_only:
            krot = f32_rne(rope_complex(kn[b].astype(np.float64), pos[:, None], r, base))
            keys[:, L[b]:L[b] + nq] = krot.transpose(1, 0, 2)
            if not kv_same:
                vals[:, L[b]:L[b] + nq] = vn[b].astype(np.float64).transpose(1, 0, 2)
            np.testing.assert_array_equal(kc_o[b].astype(np.float64), keys)
        qr = rope_complex(q[b].astype(np.float64), pos[:, None], r, base)
        want = attn_dense(qr, keys, vals, pos, n_keys, window, scale)
        assert _rel(out[b], want) < 1e-10, b


def test_residual_draw_with_no_residual_mass_falls_back_to_p():
    """With q_v >= p_v for every token the residual max(p - q, 0) is zero
    everywhere; the draw then comes from p itself (the plain sample of the
    target's row).  Empirical frequencies over 2e5 seeded draws against p."""
    rng = np.random.default_rng(4)
    V = 12
    z = rng.standard_normal(V) * 1.3
    lse = float(special.logsumexp(z))
    p = np.exp(z - lse)
    q = p.astype(np.float32)
    q = np.where(q.astype(np.float64) < p, np.nextafter(q, np.float32(2.0)), q).astype(np.float32)
    assert np.all(q.astype(np.float64) >= p)
    T = 200000
    u = rng.random((T, V)).astype(np.float32)
    u = np.maximum(u, np.float32(1e-7))
    counts = np.zeros(V)
    for t in range(T):
        y, _ = oracle.sample_residual(z, lse, q, u[t])
        counts[y] += 1
    chi = stats.chisquare(counts, p * T)
    assert chi.pvalue > 1e-3, chi
    # one token with residual mass: the draw is that token whatever the uniforms
    q2 = q.copy()
    q2[7] = np.float32(0.0)
    for t in range(200):
        y, _ = oracle.sample_residual(z, lse, q2, u[t])
        assert y == 7
