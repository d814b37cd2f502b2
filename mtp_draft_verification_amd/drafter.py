"""A drafter step over the target's shared caches on the GPU, as C-ABI calls.

The drafter ("Gemma 4 拆解" (marsggbo), section 4.2: MTPDrafter.draft_one_step and
draft) proposes k tokens one at a time.  Step i, for every sequence b:

    cat = [norm(h_prev), norm(sqrt(d_draft) E_d[token])]   sv_draft_input (x := 0)
    x  += cat W_down^T                                      sv_linear (K-split partials)
    per block, reading the cache of the target's last local / global layer
    (committed rows only; the query sits at position L_b + i):
        a = norm(x)                                         sv_add_rmsnorm
        q = a Wq^T                                          sv_linear (K-split partials)
        o = attn(q; target cache)                           sv_verify_attn (read-only, n_q = 1)
        x += o Wo^T                                         sv_linear (K-split partials)
        m = norm(x)                                         sv_add_rmsnorm
        x += (gelu_tanh(m Wg^T) * (m Wu^T)) Wd^T            sv_linear (GeGLU), sv_linear
    h  = norm(x) W_up^T                                     sv_add_rmsnorm, sv_linear (stored bf16)
    d_{b,i+1} = argmax h E^T                                sv_lmhead_select (greedy; the
                                                            token goes to drafts[b][i])
    or, with a clustering of E given (section 4.3, cheap_unembed), the argmax over
    the tokens of the clusters whose centroids score highest   sv_cluster_unembed

As in the target's verify step, the activations between the calls keep fp32
precision: the residual stream x is fp32, q is a K-split fp32 partial sum, and the
projections' inputs (cat, the norm outputs, the attention output and the GeGLU
output) are bf16 pairs (hi = bf16(v), lo = bf16(v - hi), within 2^-16 |v|).  Only
h, which the unembedding reads and the next step normalises, is stored in bf16, as
the target's final hidden state is.

The target's caches may be fp8 E4M3 codes with per-channel scales (kv_scales given
for the layers the drafter reads): the blocks then read them with
sv_verify_attn_fp8.

h_prev and the token of step 0 are the verify step's final hidden state at the
accepted row and its next token (both read through sv_accept_out); later steps use
the previous step's h and draft.  Everything runs on one stream, nothing is
allocated per step, and this module only marshals arguments."""
from __future__ import annotations

import math

import torch

from . import _lib as L
from .step import attn_desc, interleave_gate_up


class Drafter:
    """Device-resident drafter: weights, buffers and descriptors for batch B."""

    def __init__(self, target_cfg, dcfg, target_E: torch.Tensor, weights: dict, caches: list,
                 cache_len: torch.Tensor, device="cuda", clusters: dict | None = None,
                 kv_scales: dict | None = None):
        if target_cfg.dtype != "bf16":
            raise ValueError("the drafter path is bf16")
        self.t = target_cfg
        self.cfg = dcfg
        self.E = target_E
        self.W = weights
        self.caches = caches
        self.cache_len = cache_len
        # fp8 caches: {target layer: (k_scale [Hkv, D], v_scale or None)}
        self.kv_scales = kv_scales or {}
        self.dev = torch.device(device)
        B, d, dd = target_cfg.batch, target_cfg.d_model, dcfg.d_draft
        self.B = B
        self.reads = dcfg.target_layers(target_cfg)
        dev = self.dev
        z = lambda *s, dtype=torch.bfloat16: torch.zeros(*s, dtype=dtype, device=dev)
        # projection inputs as bf16 pairs [2, B, n]
        self.cat = z(2, B, d + dd)
        self.x = z(B, dd, dtype=torch.float32)
        self.a = z(2, B, dd)
        self.f = z(2, B, dcfg.d_ff)
        self.h = z(B, d)
        self.rows = torch.arange(B, dtype=torch.int32, device=dev)
        self.wgu_il = [interleave_gate_up(bw["wgu"]) for bw in weights["blocks"]]
        self.stats = torch.zeros(B, L.ROW_STATS_WORDS, dtype=torch.int32, device=dev)
        self.dev_status = torch.zeros(1, dtype=torch.int32, device=dev)
        self.timers = None

        def lin(K, N, epi, pair=1):
            # pair inputs; pair=2: a plain store writes bf16 (h), otherwise fp32
            return L.LinearDesc(rows=B, in_features=K, out_features=N, dtype=L.SV_BF16, epilogue=epi,
                                act_pair=pair)
        self._lin = lin
        # K-split partial buffers: residual projections (added by the next norm) and queries
        self.split = {}
        q_split = []
        nq_max = 0
        for ti in self.reads:
            ly = target_cfg.layers[ti]
            nq = ly.n_heads_q * ly.head_dim
            nq_max = max(nq_max, nq)
            q_split.append(L.sv_linear_splits(lin(dd, nq, L.SV_EPI_SPLIT_F32)))
            for K in (nq, dcfg.d_ff):
                self.split[K] = L.sv_linear_splits(lin(K, dd, L.SV_EPI_SPLIT_F32))
        self.split[d + dd] = L.sv_linear_splits(lin(d + dd, dd, L.SV_EPI_SPLIT_F32))
        if min(self.split.values()) <= 0 or min(q_split) <= 0:
            raise ValueError("drafter projections too large for a K split on this device")
        self.q_split = q_split
        self.parts = z(max(self.split.values()) * B * dd, dtype=torch.float32)
        self.q_parts = z(max(q_split) * B * nq_max, dtype=torch.float32)
        self.o = z(2, B, nq_max)
        self.lin_ws = torch.zeros(max(256, L.sv_linear_workspace(lin(dd, d, L.SV_EPI_STORE, 2)),
                                      L.sv_linear_workspace(lin(dd, 2 * dcfg.d_ff, L.SV_EPI_GEGLU))),
                                  dtype=torch.uint8, device=dev)
        cap = caches[0]["k"].shape[2]
        self.cap = cap
        # one attention descriptor per (block, step): the query position offset is the step
        self._attn = {}
        ws = max(L.sv_verify_attn_workspace(self._attn_desc(j, 0)) for j in range(len(self.reads)))
        self.attn_ws = torch.empty(max(ws, 256), dtype=torch.uint8, device=dev)
        # the greedy unembed's workspace (its size does not depend on out_stride)
        lm_desc = L.LMHeadDesc(batch=B, k=0, d_model=d, vocab=target_cfg.vocab, mode=L.SV_SELECT_GREEDY,
                               dtype=L.SV_BF16, out_stride=1)
        self.lm_ws = torch.zeros(max(256, L.sv_lmhead_workspace(lm_desc)), dtype=torch.uint8, device=dev)
        self.drafts = None
        # clustered unembedding: {"perm", "w_perm", "centroids", "top"} (None: full vocabulary)
        self.clusters = clusters
        if clusters is not None:
            C = clusters["centroids"].shape[0]
            self.cl_desc = L.ClusterDesc(rows=B, d_model=d, vocab=target_cfg.vocab, n_clusters=C,
                                         top_clusters=clusters["top"], dtype=L.SV_BF16)
            self.cl_ws = torch.zeros(max(256, L.sv_cluster_unembed_workspace(self.cl_desc)), dtype=torch.uint8,
                                     device=dev)
            self.kept = torch.zeros(B, clusters["top"], dtype=torch.int32, device=dev)

    def _attn_desc(self, j: int, i: int) -> L.AttnDesc:
        key = (j, i)
        if key not in self._attn:
            ly = self.t.layers[self.reads[j]]
            self._attn[key] = attn_desc(ly, self.B, 1, self.cap, "bf16", append=False, q_pos_offset=i,
                                        in_splits=self.q_split[j], act_pair=True)
        return self._attn[key]

    def _ev(self, name: str, stream):
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

    def _norm(self, pending, stream):
        parts, S = pending if pending is not None else (None, 0)
        L.sv_add_rmsnorm(self.B, self.cfg.d_draft, self.cfg.eps, self.x, parts, S, None, self.a, L.SV_BF16X2,
                         stream)
        return self.a

    def _residual(self, inp, w, stream):
        K = w.shape[1]
        L.sv_linear(self._lin(K, self.cfg.d_draft, L.SV_EPI_SPLIT_F32), inp, w, self.parts, None, stream)
        return (self.parts, self.split[K])

    def step(self, i: int, k: int, h_src, rows_h: int, hidden_row, row_stride: int, tokens, tok_stride: int,
             drafts: torch.Tensor, stream=None) -> None:
        """Draft step i of k: writes the argmax token of every sequence to drafts[b][i]
        and leaves h (the next step's h_prev) in self.h.  hidden_row / tokens are int32
        device pointers (or tensors) read with the given strides."""
        t, dc = self.t, self.cfg
        B, d, dd = self.B, t.d_model, dc.d_draft
        tok = self._ev("draft_input", stream)
        L.sv_draft_input(B, d, dd, dc.eps, h_src, rows_h, hidden_row, row_stride, self.W["E"], t.vocab, tokens,
                         tok_stride, math.sqrt(dd), self.cat, L.SV_BF16X2, self.x, self.dev_status, stream)
        pending = self._residual(self.cat, self.W["w_down"], stream)
        self._end(tok)
        for j, (bw, ti) in enumerate(zip(self.W["blocks"], self.reads)):
            ly = t.layers[ti]
            nq = ly.n_heads_q * ly.head_dim
            a = self._norm(pending, stream)
            tok = self._ev(f"D{j}.attn", stream)
            S = self.q_split[j]
            qp = self.q_parts.view(-1)[:S * B * nq]
            L.sv_linear(self._lin(dd, nq, L.SV_EPI_SPLIT_F32), a, bw["wq"], qp, None, stream)
            o = self.o.view(-1)[:2 * B * nq].view(2, B, nq)
            kc = self.caches[ti]
            if ti in self.kv_scales:
                ks, vs = self.kv_scales[ti]
                L.sv_verify_attn_fp8(self._attn_desc(j, i), qp, None, None, kc["k"], kc["v"], ks, vs, self.cache_len,
                                     o, self.attn_ws, self.dev_status, stream)
            else:
                L.sv_verify_attn(self._attn_desc(j, i), qp, None, None, kc["k"], kc["v"], self.cache_len, o,
                                 self.attn_ws, self.dev_status, stream)
            pending = self._residual(o, bw["wo"], stream)
            self._end(tok)
            tok = self._ev(f"D{j}.mlp", stream)
            m = self._norm(pending, stream)
            L.sv_linear(self._lin(dd, 2 * dc.d_ff, L.SV_EPI_GEGLU), m, self.wgu_il[j], self.f, self.lin_ws, stream)
            pending = self._residual(self.f, bw["wd"], stream)
            self._end(tok)
        tok = self._ev("unembed", stream)
        u = self._norm(pending, stream)
        L.sv_linear(self._lin(dd, d, L.SV_EPI_STORE, 2), u, self.W["w_up"], self.h, self.lin_ws, stream)
        if self.clusters is not None:
            c = self.clusters
            L.sv_cluster_unembed(self.cl_desc, self.h, c["centroids"], c["w_perm"], c["perm"], self.stats, self.kept,
                                 drafts.data_ptr() + 4 * i, k, self.cl_ws, stream)
            self._end(tok)
            return
        desc = L.LMHeadDesc(batch=B, k=0, d_model=d, vocab=t.vocab, mode=L.SV_SELECT_GREEDY, dtype=L.SV_BF16,
                            out_stride=k)
        L.sv_lmhead_select(desc, self.h, self.E, None, None, None, self.stats, None, drafts.data_ptr() + 4 * i,
                           self.lm_ws, stream)
        self._end(tok)

    def draft(self, k: int, h_verify: torch.Tensor, acc: torch.Tensor, drafts: torch.Tensor, stream=None) -> None:
        """k draft steps after a verify step: h_verify [B*(k'+1), d] final hidden states,
        acc [B, ACCEPT_OUT_WORDS] (hidden_row and next_token are read); drafts [B, k]
        int32 receives the proposals."""
        words = L.ACCEPT_OUT_WORDS
        hr = acc.data_ptr() + 4 * 7   # sv_accept_out.hidden_row
        nt = acc.data_ptr() + 4 * 1   # sv_accept_out.next_token
        self.step(0, k, h_verify, h_verify.shape[0], hr, words, nt, words, drafts, stream)
        for i in range(1, k):
            self.step(i, k, self.h, self.B, self.rows, 1, drafts.data_ptr() + 4 * (i - 1), k, drafts, stream)
