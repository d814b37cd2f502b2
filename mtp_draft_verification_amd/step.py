"""The verify step of a decoder stack on the GPU, as a sequence of C-ABI calls.

speculative_step ("Gemma 4 拆解" (marsggbo), section 4.2): ONE target forward
over the rows [last committed token, d_1..d_k] of every sequence (main_model.verify),
then accept_longest_prefix.  Here that forward is, per layer,

    a = rmsnorm(x)                 sv_rmsnorm      (x: fp32 residual stream)
    qkv = a Wqkv^T                 sv_linear       (q, k, v in one projection; K-split
                                   partials, summed by the attention call)
    o = attn(q, k, v; cache)       sv_verify_attn  (appends the k+1 new rows)
    x += o Wo^T                    sv_linear (SV_EPI_SPLIT_F32: the K-split partial
                                   products), added into x by the next norm
    m = rmsnorm(x)                 sv_add_rmsnorm  (x += the partials, then the norm)
    f = gelu_tanh(m Wg^T) * (m Wu^T)   sv_linear (SV_EPI_GEGLU: one launch, gate/up
                                   rows interleaved by 16; sv_linear + sv_geglu where
                                   that layout does not apply)
    x += f Wd^T                    sv_linear (SV_EPI_SPLIT_F32), added by the next
                                   layer's (or the final) sv_add_rmsnorm

then h = rmsnorm(x), sv_lmhead_select over the tied embedding and sv_accept.  The
fp32 stack (no norms) adds into x with SV_EPI_ADD_F32 instead.

In the bf16 stack the weights and the caches are bf16 and the activations between
the calls keep fp32 precision: q / k / v are fp32 K-split partial sums, and the norm
outputs, the attention output and the GeGLU output -- the inputs of the projections
-- are bf16 pairs (act_pair: hi = bf16(v) and lo = bf16(v - hi) in two planes,
within 2^-16 |v|, multiplied as two bf16 MFMA operands).  Only the new cache rows
and the final hidden state that the LM head reads are rounded to bf16.

Every call is enqueued on one stream with no host synchronisation; all buffers
are allocated once up front, so a step allocates nothing.  This module only
marshals arguments: the arithmetic is the library's.
"""
from __future__ import annotations

import math

import torch

from . import _lib as L


def attn_desc(layer, batch: int, n_q: int, cap: int, dtype: str, append: bool = True,
              q_pos_offset: int = 0, q_row_stride: int = 0, kv_row_stride: int = 0,
              in_splits: int = 0, act_pair: bool = False) -> L.AttnDesc:
    return L.AttnDesc(batch=batch, n_q=n_q, n_heads_q=layer.n_heads_q, n_heads_kv=layer.n_heads_kv,
                      head_dim=layer.head_dim, window=layer.window, rope_dims=layer.rope_dims,
                      k_is_v=int(layer.k_is_v), append=int(append), q_pos_offset=q_pos_offset,
                      dtype=L.SV_BF16 if dtype == "bf16" else L.SV_F32, in_splits=int(in_splits),
                      rope_base=float(layer.rope_base), softmax_scale=float(layer.scale), reserved_f=0.0,
                      cache_capacity=int(cap), q_row_stride=int(q_row_stride),
                      kv_row_stride=int(kv_row_stride), act_pair=int(bool(act_pair)), reserved_i=0)


def interleave_gate_up(wgu: torch.Tensor) -> torch.Tensor:
    """[2*d_ff, d] (gate rows, then up rows) -> the same rows interleaved by 16 (gate
    16j..16j+15, up 16j..16j+15, ...), the layout SV_EPI_GEGLU reads.  A one-time
    copy of the weights (layout only)."""
    two_dff, d = wgu.shape
    dff = two_dff // 2
    return wgu.view(2, dff // 16, 16, d).permute(1, 0, 2, 3).contiguous().view(two_dff, d)


class VerifyStack:
    """Device-resident state of a stack: weights, caches, committed lengths, buffers."""

    def __init__(self, cfg, weights: dict, caches: list, cache_len: torch.Tensor, device="cuda",
                 tiled_weights: bool = True):
        self.cfg = cfg
        self.W = weights
        self.caches = caches
        self.cache_len = cache_len
        self.dev = torch.device(device)
        self.bf16 = cfg.dtype == "bf16"
        self.dt = L.SV_BF16 if self.bf16 else L.SV_F32
        self.act = int(self.bf16)  # bf16 weights and caches, pair activations
        if not cfg.norm and self.bf16:
            raise ValueError("a bf16 stack needs its final RMSNorm to produce the bf16 hidden state "
                             "the LM head reads")
        B, k, d = cfg.batch, cfg.k, cfg.d_model
        self.R = R = B * (k + 1)
        self.cap = caches[0]["k"].shape[2]
        # fused GeGLU projection where the layout applies (bf16, 2*d_ff a multiple of 128); the
        # bf16 stack's pair activations come only from the fused one
        self.fused_geglu = bool(self.bf16 and cfg.d_ff and (2 * cfg.d_ff) % 128 == 0)
        if self.bf16 and cfg.d_ff and not self.fused_geglu:
            raise ValueError("a bf16 stack needs d_ff to be a multiple of 64 (the fused GeGLU projection)")
        self.wgu_il = ([interleave_gate_up(lw["wgu"]) for lw in weights["layers"]]
                       if self.fused_geglu else None)
        dev = self.dev
        z = lambda *s, dtype=torch.float32: torch.zeros(*s, dtype=dtype, device=dev)
        # projection inputs: bf16 pairs [2, R, n] (bf16 stack) or fp32 [R, n]
        act = (lambda n: z(2, R, n, dtype=torch.bfloat16)) if self.bf16 else (lambda n: z(R, n))
        self.act_dt = L.SV_BF16X2 if self.bf16 else L.SV_F32
        self.x = z(R, d)
        self.a = act(d)
        nout = max(ly.n_heads_q * ly.head_dim + (1 if ly.k_is_v else 2) * ly.n_heads_kv * ly.head_dim
                   for ly in cfg.layers)
        self.qkv = z(R, nout)
        self.hd_max = max(ly.n_heads_q * ly.head_dim for ly in cfg.layers)
        self.o = act(self.hd_max)
        self.gu = z(R, 2 * cfg.d_ff) if cfg.d_ff and not self.fused_geglu else None
        self.f = act(cfg.d_ff) if cfg.d_ff else None
        # the final hidden state, in the LM head's dtype
        self.h = z(R, d, dtype=torch.bfloat16) if self.bf16 else self.a
        # residual projections leave K-split partials that the next norm adds into x
        self.split = {}
        if self.bf16:
            for ly in cfg.layers:
                for K in (ly.n_heads_q * ly.head_dim, cfg.d_ff):
                    if K:
                        S = L.sv_linear_splits(L.LinearDesc(rows=R, in_features=K, out_features=d, dtype=self.dt,
                                                            epilogue=L.SV_EPI_SPLIT_F32, act_pair=self.act))
                        if S > 0:
                            self.split[K] = S
        self.parts = z(max(self.split.values()) * R * d, dtype=torch.float32) if self.split else None
        # the q/k/v projection also leaves K-split partials, summed by the attention's rope/append
        self.qkv_split = []
        for ly in cfg.layers:
            S = 0
            if self.bf16:
                S = max(0, L.sv_linear_splits(L.LinearDesc(rows=R, in_features=d, out_features=self._nout(ly),
                                                           dtype=self.dt, epilogue=L.SV_EPI_SPLIT_F32,
                                                           act_pair=self.act)))
            self.qkv_split.append(S)
        nout_max = max(self._nout(ly) for ly in cfg.layers)
        self.qkv_parts = (z(max(self.qkv_split) * R * nout_max, dtype=torch.float32) if max(self.qkv_split) else None)
        ws = max(L.sv_verify_attn_workspace(attn_desc(ly, B, k + 1, self.cap, cfg.dtype)) for ly in cfg.layers)
        self.attn_ws = torch.empty(max(ws, 256), dtype=torch.uint8, device=dev)
        self.lin_ws = torch.zeros(max([self._lin_ws(*s) for s in self._lin_shapes()] + [256]),
                                  dtype=torch.uint8, device=dev)
        # bf16 projections read tiled copies of their weights (made once here, for the
        # epilogue each call uses): the weight stream then reads whole DRAM pages
        self.tiled = {}
        if self.bf16 and tiled_weights:
            for i, (ly, lw) in enumerate(zip(cfg.layers, weights["layers"])):
                self._tile(lw["wqkv"], L.SV_EPI_SPLIT_F32 if self.qkv_split[i] else L.SV_EPI_STORE)
                self._tile(lw["wo"], self._residual_epi(lw["wo"].shape[1]))
                if cfg.d_ff:
                    self._tile(self.wgu_il[i], L.SV_EPI_GEGLU)
                    self._tile(lw["wd"], self._residual_epi(cfg.d_ff))
        self.lm_desc = L.LMHeadDesc(batch=B, k=k, d_model=d, vocab=cfg.vocab, mode=L.SV_SELECT_GREEDY,
                                    dtype=self.dt)
        self.lm_ws = torch.zeros(max(L.sv_lmhead_workspace(self.lm_desc), 256), dtype=torch.uint8, device=dev)
        self.stats = torch.zeros(R, L.ROW_STATS_WORDS, dtype=torch.int32, device=dev)
        self.acc = torch.zeros(B, L.ACCEPT_OUT_WORDS, dtype=torch.int32, device=dev)
        self.out_tokens = torch.zeros(B, k + 1, dtype=torch.int32, device=dev)
        self.dev_status = torch.zeros(1, dtype=torch.int32, device=dev)
        self.acc_desc = L.AcceptDesc(batch=B, k=k, vocab=cfg.vocab, mode=L.SV_SELECT_GREEDY)
        self.timers = None   # {call name: [(start event, end event), ...]} when timing
        self.attn_descs = [
            attn_desc(ly, B, k + 1, self.cap, cfg.dtype, q_row_stride=self._nout(ly), kv_row_stride=self._nout(ly),
                      in_splits=S, act_pair=self.act) for ly, S in zip(cfg.layers, self.qkv_split)]

    def _ev(self, name: str, stream):
        """Record a HIP event pair around a named call when that call is being timed."""
        if self.timers is None or name not in self.timers:
            return None
        st = stream if stream is not None else torch.cuda.current_stream()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(st)
        self.timers[name].append((e0, e1))
        return e1, st

    @staticmethod
    def _end(tok):
        if tok is not None:
            tok[0].record(tok[1])

    @staticmethod
    def _nout(ly) -> int:
        return ly.n_heads_q * ly.head_dim + (1 if ly.k_is_v else 2) * ly.n_heads_kv * ly.head_dim

    def _lin_shapes(self):
        cfg, R = self.cfg, self.R
        for ly in cfg.layers:
            yield R, cfg.d_model, self._nout(ly), L.SV_EPI_STORE
            yield R, ly.n_heads_q * ly.head_dim, cfg.d_model, L.SV_EPI_ADD_F32
            if cfg.d_ff:
                yield R, cfg.d_model, 2 * cfg.d_ff, (L.SV_EPI_GEGLU if self.fused_geglu else L.SV_EPI_STORE)
                yield R, cfg.d_ff, cfg.d_model, L.SV_EPI_ADD_F32

    def _lin_ws(self, R, K, N, epi) -> int:
        return L.sv_linear_workspace(L.LinearDesc(rows=R, in_features=K, out_features=N, dtype=self.dt,
                                                  epilogue=epi, act_pair=self.act))

    def _tile(self, w, epi):
        N, K = w.shape
        desc = L.LinearDesc(rows=self.R, in_features=K, out_features=N, dtype=self.dt, epilogue=epi,
                            act_pair=self.act)
        self.tiled[(w.data_ptr(), epi)] = L.tiled_weight(desc, w)

    def _residual_epi(self, K: int) -> int:
        return L.SV_EPI_SPLIT_F32 if self.split.get(K, 0) else L.SV_EPI_ADD_F32

    def _linear(self, x, w, y, epi, stream):
        R, K = self.R, w.shape[1]
        N = w.shape[0]
        wt = self.tiled.get((w.data_ptr(), epi))
        desc = L.LinearDesc(rows=R, in_features=K, out_features=N, dtype=self.dt, epilogue=epi, act_pair=self.act,
                            w_layout=L.SV_W_ROWMAJOR if wt is None else L.SV_W_TILED)
        L.sv_linear(desc, x, w if wt is None else wt, y, self.lin_ws, stream)

    def _residual(self, inp, w, stream):
        """x += inp W^T: K-split partials left for the next norm (returned as
        (parts, S)) where the split applies, else added into x now (None)."""
        K = w.shape[1]
        S = self.split.get(K, 0)
        if S:
            self._linear(inp, w, self.parts, L.SV_EPI_SPLIT_F32, stream)
            return (self.parts, S)
        self._linear(inp, w, self.x, L.SV_EPI_ADD_F32, stream)
        return None

    def _norm(self, x, y, stream, pending=None, odt=None):
        if self.cfg.norm:
            odt = self.act_dt if odt is None else odt
            if pending is not None:
                L.sv_add_rmsnorm(self.R, x.shape[1], self.cfg.eps, x, pending[0], pending[1], None, y, odt, stream)
            else:
                L.sv_rmsnorm(self.R, x.shape[1], self.cfg.eps, x, None, y, odt, stream)
            return y
        assert pending is None
        return x  # fp32 stack without norms feeds the residual stream directly

    def _act_view(self, buf, n):
        """The first n columns of a projection-input buffer, densely packed (rows of n)."""
        if self.bf16:
            return buf.view(-1)[:2 * self.R * n].view(2, self.R, n)
        return buf.view(-1)[:self.R * n].view(self.R, n)

    # ------------------------------------------------------------------
    def forward(self, tokens: torch.Tensor, stream=None) -> torch.Tensor:
        """Verify forward of tokens [B, k+1] int32 (device); appends the k+1 new
        rows of every layer's cache; returns the final hidden states [R, d].
        Call names for timing: embed, L{i}.qkv, L{i}.attn, L{i}.o, L{i}.gu (with the
        GeGLU gate when fused), L{i}.geglu (otherwise), L{i}.down, final_norm."""
        cfg = self.cfg
        d = cfg.d_model
        t = self._ev("embed", stream)
        L.sv_embed(self.R, d, cfg.vocab, self.dt, tokens, self.W["E"], math.sqrt(d), self.x,
                   self.dev_status, stream)
        self._end(t)
        pending = None  # partials of the last residual projection, not yet in x
        for i, (ly, lw, cache, desc) in enumerate(zip(cfg.layers, self.W["layers"], self.caches,
                                                      self.attn_descs)):
            a = self._norm(self.x, self.a, stream, pending)
            nq_f = ly.n_heads_q * ly.head_dim
            nk_f = ly.n_heads_kv * ly.head_dim
            nout = self._nout(ly)
            S = self.qkv_split[i]
            t = self._ev(f"L{i}.qkv", stream)
            if S:
                qkv = self.qkv_parts.view(-1)[:S * self.R * nout].view(S * self.R, nout)
                self._linear(a, lw["wqkv"], qkv, L.SV_EPI_SPLIT_F32, stream)
            else:
                qkv = self.qkv.view(-1)[:self.R * nout].view(self.R, nout)
                self._linear(a, lw["wqkv"], qkv, L.SV_EPI_STORE, stream)
            self._end(t)
            esz = qkv.element_size()
            base = qkv.data_ptr()
            k_ptr = base + nq_f * esz
            v_ptr = None if ly.k_is_v else base + (nq_f + nk_f) * esz
            o = self._act_view(self.o, nq_f)
            t = self._ev(f"L{i}.attn", stream)
            L.sv_verify_attn(desc, base, k_ptr, v_ptr, cache["k"], cache["v"], self.cache_len, o,
                             self.attn_ws, self.dev_status, stream)
            self._end(t)
            t = self._ev(f"L{i}.o", stream)
            pending = self._residual(o, lw["wo"], stream)
            self._end(t)
            if cfg.d_ff:
                m = self._norm(self.x, self.a, stream, pending)
                t = self._ev(f"L{i}.gu", stream)
                if self.fused_geglu:
                    self._linear(m, self.wgu_il[i], self.f, L.SV_EPI_GEGLU, stream)
                    self._end(t)
                else:
                    self._linear(m, lw["wgu"], self.gu, L.SV_EPI_STORE, stream)
                    self._end(t)
                    t = self._ev(f"L{i}.geglu", stream)
                    L.sv_geglu(self.R, cfg.d_ff, L.SV_F32, self.gu, self.f, stream)
                    self._end(t)
                t = self._ev(f"L{i}.down", stream)
                pending = self._residual(self.f, lw["wd"], stream)
                self._end(t)
        t = self._ev("final_norm", stream)
        h = self._norm(self.x, self.h, stream, pending, odt=self.dt)
        self._end(t)
        return h

    def select(self, h: torch.Tensor, drafts: torch.Tensor, stream=None) -> None:
        t = self._ev("lmhead", stream)
        L.sv_lmhead_select(self.lm_desc, h, self.W["E"], drafts, None, None, self.stats, None, None,
                           self.lm_ws, stream)
        self._end(t)

    def accept(self, drafts: torch.Tensor, stream=None) -> None:
        t = self._ev("accept", stream)
        L.sv_accept(self.acc_desc, drafts, self.stats, None, None, self.cache_len, self.out_tokens, self.acc,
                    self.dev_status, stream)
        self._end(t)

    def step(self, tokens: torch.Tensor, drafts: torch.Tensor, stream=None) -> None:
        """One greedy verify step: forward, LM-head select, accept (commits on device)."""
        h = self.forward(tokens, stream)
        self.select(h, drafts, stream)
        self.accept(drafts, stream)

    def capture(self, tokens: torch.Tensor, drafts: torch.Tensor):
        """Record one verify step on the input buffers `tokens` [B, k+1] and `drafts`
        [B, k] into a HIP graph and return it (torch.cuda.CUDAGraph).  The step
        allocates nothing, never waits on the host and clears nothing with a memset,
        so every launch of it is captured as it is; each replay() runs the step on
        whatever the two buffers hold at that time and commits on device like step()."""
        if self.timers is not None:
            raise RuntimeError("capture with per-call timers set")
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.step(tokens, drafts)
        return g
