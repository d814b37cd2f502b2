"""Oracle composition of a whole verify step of a small decoder stack.

TEST INFRASTRUCTURE ONLY (see the package docstring).  The arithmetic is the C
oracle's (svoracle.c); this file strings its functions together in the order
of a pre-norm decoder layer and of the speculative step:

  speculative step ("Gemma 4 拆解" (marsggbo), section 4.2, speculative_step):
      the drafter proposes d_1..d_k; ONE target forward scores the rows
      [last committed token, d_1..d_k] at positions L..L+k (verify); the longest
      prefix of drafts that agrees with the target is accepted plus one token of
      the target's own ("Accelerating Gemma 4 ..." (Lighthouse), section 3).
  target layer (a pre-norm decoder layer; the pages give the layer pattern,
      "Gemma 4 发布时未包含 MTP 数据" (flowhunt), section "什么是 Gemma 4？"):
      a = norm(x); q,k,v = a Wq, a Wk, a Wv; x += attn(q,k,v; cache) Wo;
      m = norm(x); x += (gelu_tanh(m Wg) * (m Wu)) Wd;  final h = norm(x);
      logits = h E^T with the embedding E tied to the LM head, x0 = sqrt(d) E[tok].

Values the GPU path stores are rounded here at the same points: activations
between the ops (normed inputs, q/k/v, attention output, GeGLU output) are
stored in fp32; in bf16 mode the appended cache rows and the final hidden state
(the LM head's input) are stored in bf16, in fp32 mode in fp32.  All arithmetic
stays fp64 and the residual stream is never rounded.
"""
from __future__ import annotations

import copy

import numpy as np

from . import (accept_greedy, bf16_round, geglu, lmhead, linear, rmsnorm, row_stats, verify_attn)


def _to_f64(w: np.ndarray) -> np.ndarray:
    if w.dtype == np.uint16:  # bf16 bit patterns
        return (w.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return w.astype(np.float64)


class OracleModel:
    """Geometry (a StackConfig-like object) plus host weights.

    weights: {"E": [V, d], "layers": [{"wqkv", "wo", ("wgu", "wd")}]}, each array
    fp32 or uint16 bf16 bits; wqkv stacks the q, k (and v) projections along the
    output dimension, wgu the gate then the up projection."""

    def __init__(self, cfg, weights: dict):
        self.cfg = cfg
        self.W = weights
        self.bf16 = cfg.dtype == "bf16"

    @staticmethod
    def _r(x):
        """Round an activation to its storage type (fp32)."""
        return np.asarray(x, dtype=np.float32).astype(np.float64)

    def _rh(self, x):
        """Round the final hidden state to the LM head's input type (bf16, or fp32 in
        fp32 mode)."""
        return bf16_round(x) if self.bf16 else self._r(x)

    def embed(self, tokens: np.ndarray) -> np.ndarray:
        E = self.W["E"]
        rows = _to_f64(E[np.asarray(tokens, dtype=np.int64).reshape(-1)])
        return np.sqrt(float(self.cfg.d_model)) * rows

    def forward(self, state: dict, tokens: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
        """Verify forward of tokens [B, n] (row 0 = last committed token) at positions
        L_b..L_b+n-1; appends the n new cache rows of every layer.  Returns
        (final hidden [B*n, d], logits [B*n, V]), both fp64.  Does not commit."""
        cfg = self.cfg
        tokens = np.asarray(tokens, dtype=np.int64)
        B, n = tokens.shape
        x = self.embed(tokens)                      # [B*n, d]
        for ly, lw, cache in zip(cfg.layers, self.W["layers"], state["caches"]):
            a = self._r(rmsnorm(x, cfg.eps) if cfg.norm else x)
            qkv = self._r(linear(a, lw["wqkv"]))
            nq = ly.n_heads_q * ly.head_dim
            nk = ly.n_heads_kv * ly.head_dim
            q = qkv[:, :nq].reshape(B, n, ly.n_heads_q, ly.head_dim)
            k = qkv[:, nq:nq + nk].reshape(B, n, ly.n_heads_kv, ly.head_dim)
            v = None if ly.k_is_v else qkv[:, nq + nk:].reshape(B, n, ly.n_heads_kv, ly.head_dim)
            o = verify_attn(q=q.astype(np.float32),
                            k_new=k.astype(np.float32),
                            v_new=None if v is None else v.astype(np.float32),
                            k_cache=cache["k"], v_cache=cache["v"], cache_len=state["L"],
                            window=ly.window, rope_dims=ly.rope_dims, rope_base=ly.rope_base,
                            scale=ly.scale, k_is_v=ly.k_is_v, append=True,
                            round_bf16=self.bf16)
            o = self._r(o.reshape(B * n, nq))
            x = x + linear(o, lw["wo"])
            if cfg.d_ff:
                m = self._r(rmsnorm(x, cfg.eps) if cfg.norm else x)
                g = linear(m, lw["wgu"][:cfg.d_ff])
                u = linear(m, lw["wgu"][cfg.d_ff:])
                f = self._r(geglu(g, u))
                x = x + linear(f, lw["wd"])
        h = self._rh(rmsnorm(x, cfg.eps) if cfg.norm else x)
        z = lmhead(h, self.W["E"])
        return h, z

    def greedy_step(self, state: dict, tokens: np.ndarray) -> dict:
        """One greedy verify step: forward, per-row statistics, longest-prefix
        acceptance, commit L_b += n_b + 1 (rows beyond are rolled back by simply
        being overwritten by the next append)."""
        tokens = np.asarray(tokens, dtype=np.int64)
        B, n = tokens.shape
        k = n - 1
        h, z = self.forward(state, tokens)
        stats = []
        nacc = np.zeros(B, dtype=np.int32)
        y = np.zeros(B, dtype=np.int32)
        out_tok = np.full((B, n), -1, dtype=np.int32)
        for b in range(B):
            st = [row_stats(z[b * n + i], int(tokens[b, i + 1]) if i < k else -1) for i in range(n)]
            stats.append(st)
            top1 = np.array([s["top1_id"] for s in st], dtype=np.int32)
            nb, toks = accept_greedy(tokens[b, 1:], top1)
            nacc[b] = nb
            y[b] = toks[nb]
            out_tok[b] = toks
        new_len = np.asarray(state["L"], dtype=np.int64) + nacc + 1
        res = dict(n=nacc, y=y, tokens=out_tok, stats=stats, h=h, z=z,
                   old_len=np.asarray(state["L"]).copy(), new_len=new_len)
        state["L"] = new_len.astype(np.int32)
        return res


class OracleDrafter:
    """One step of an MTP drafter that cross-attends the target's caches ("Gemma 4
    拆解" (marsggbo), section 4.2, MTPDrafter.draft_one_step and draft):

        cat = [norm(h_prev), norm(sqrt(d_draft) E_d[token])]   (the target's last
              activation and the drafter's own token embedding)
        x   = cat W_down^T
        per block (reading the cache of the target's last local or global layer,
              committed rows only, as a query at position L + i):
            a = norm(x); q = a Wq^T; x += attn(q; cache) Wo^T
            m = norm(x); x += (gelu_tanh(m Wg^T) * (m Wu^T)) Wd^T
        h   = norm(x) W_up^T           (back to the target's width)
        z   = h E^T with the target's tied unembedding; the draft is argmax z, and
              h is the next step's h_prev.

    The pages' listing leaves norms and RoPE out; here every norm is an RMSNorm of
    unit gain and the queries get the RoPE of the target layer they read.  Values
    the GPU path stores are rounded at the same points as in OracleModel: the
    activations between the ops (cat, normed inputs, q, attention output, GeGLU
    output) to fp32, h -- the unembedding's input, like the target's final hidden
    state -- to bf16."""

    def __init__(self, target_cfg, dcfg, target_E: np.ndarray, weights: dict):
        self.t = target_cfg
        self.d = dcfg
        self.E = target_E
        self.W = weights
        last = {}
        for i, ly in enumerate(target_cfg.layers):
            last[ly.kind] = i
        self.reads = [last[kind] for kind in dcfg.blocks]

    @staticmethod
    def _r(x):
        """Round an activation to its storage type (fp32)."""
        return np.asarray(x, dtype=np.float32).astype(np.float64)

    def step(self, state: dict, h_prev: np.ndarray, tokens, i: int) -> tuple[np.ndarray, np.ndarray]:
        """h_prev [B, d_model] (values as stored), tokens [B]; the step's query sits at
        position L_b + i.  Returns (h [B, d_model] as stored, logits [B, V] fp64)."""
        t, dc = self.t, self.d
        eps = dc.eps
        tokens = np.asarray(tokens, dtype=np.int64)
        B = tokens.shape[0]
        e = np.sqrt(float(dc.d_draft)) * _to_f64(self.W["E"][tokens])
        cat = np.concatenate([self._r(rmsnorm(np.asarray(h_prev, dtype=np.float64), eps)),
                              self._r(rmsnorm(e, eps))], axis=1)
        x = linear(cat, self.W["w_down"])
        for blk, ti in zip(self.W["blocks"], self.reads):
            ly = t.layers[ti]
            cache = state["caches"][ti]
            a = self._r(rmsnorm(x, eps))
            q = self._r(linear(a, blk["wq"])).reshape(B, 1, ly.n_heads_q, ly.head_dim)
            o = verify_attn(q=q.astype(np.float32), k_new=None, v_new=None, k_cache=cache["k"],
                            v_cache=cache["v"], cache_len=state["L"], window=ly.window,
                            rope_dims=ly.rope_dims, rope_base=ly.rope_base, scale=ly.scale,
                            k_is_v=ly.k_is_v, append=False, q_pos_offset=i, round_bf16=True)
            o = self._r(o.reshape(B, ly.n_heads_q * ly.head_dim))
            x = x + linear(o, blk["wo"])
            m = self._r(rmsnorm(x, eps))
            g = linear(m, blk["wgu"][:dc.d_ff])
            u = linear(m, blk["wgu"][dc.d_ff:])
            f = self._r(geglu(g, u))
            x = x + linear(f, blk["wd"])
        h = bf16_round(linear(self._r(rmsnorm(x, eps)), self.W["w_up"]))
        return h, lmhead(h, self.E)


def new_state(caches: list, cache_len) -> dict:
    """caches: per layer {"k": [B, Hkv, cap, D] float32, "v": same or None}."""
    return {"caches": caches, "L": np.asarray(cache_len, dtype=np.int32).copy()}


def clone_state(state: dict) -> dict:
    return copy.deepcopy(state)


def ar_greedy(model: OracleModel, state: dict, first_token: int, n_tokens: int) -> list:
    """Plain autoregressive greedy decoding of one sequence (batch 1): one row per
    forward.  Returns the n_tokens generated tokens."""
    out = []
    cur = int(first_token)
    while len(out) < n_tokens:
        r = model.greedy_step(state, np.array([[cur]]))
        cur = int(r["y"][0])
        out.append(cur)
    return out


def spec_greedy(model: OracleModel, state: dict, first_token: int, n_tokens: int, k: int,
                drafter) -> tuple[list, list]:
    """Speculative greedy decoding of one sequence: drafter(history, k) -> k tokens,
    one verify forward over [last token, drafts], accept the longest agreeing
    prefix plus the target's token.  Returns (tokens, accept lengths)."""
    out = []
    accepts = []
    cur = int(first_token)
    while len(out) < n_tokens:
        drafts = [int(t) for t in drafter([first_token] + out, k)]
        r = model.greedy_step(state, np.array([[cur] + drafts]))
        nb = int(r["n"][0])
        accepts.append(nb)
        out.extend(int(t) for t in r["tokens"][0, :nb + 1])
        cur = int(r["y"][0])
    return out[:n_tokens], accepts
