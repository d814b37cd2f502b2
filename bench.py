#!/usr/bin/env python3
"""Verify-step throughput of libspecverify on one MI355X.

Workload: the full verify step of a synthetic random-init decoder stack
(6 layers, 5 sliding-window : 1 global, d = 3840, d_ff = 15360 GeGLU, RMSNorm,
tied 262,144-token LM head, committed context 131,072, k = 4 drafts), batch 8 by
default (batch 1 is measured in the same run as a sweep point).

A step is one pass of the whole hot path: embedding, every layer's
projections, verify attention with KV append (local window and global K=V
p-RoPE layers), the fused LM-head select and the accept kernel with KV
commit/rollback.  Drafts follow the workload recipe: the target's own greedy
continuation with each draft replaced by a random token with probability 0.2.
They are recorded in an untimed pass (k single-row passes per step produce the
continuation) and the recorded steps are then replayed back to back in the
timed region from the same starting state, which reproduces the same
trajectory (the kernels are deterministic; this is checked).

value = committed tokens (sum over steps and sequences of n_b + 1) / time.
roofline: the kernel call that takes the most time per step, its algorithmic
bytes / its mean duration (HIP events on the step's stream, timed region).
cpu_baseline: the fp64 oracle on one sequence of the same step (host cores).
"""
from __future__ import annotations

import argparse
import dataclasses
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "verify-step tokens/s (k=4, batch 1/8) + attn/LM-head HBM GB/s as % of peak"
PEAK_HBM_GBS = 8000.0


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--batch", type=int, default=8)
    ap.add_argument("--k", type=int, default=4)
    ap.add_argument("--ctx", type=int, default=131072)
    ap.add_argument("--sweep", default="1,2,4,8", help="batch sizes of the sweep, comma separated ('' for none)")
    ap.add_argument("--sweep-k", default="3,4", help="draft counts of the sweep, comma separated")
    ap.add_argument("--no-configs", action="store_true", help="skip the standalone workload lines")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile", action="store_true", help="short run for profilers: no sweep, no oracle")
    ap.add_argument("--no-drafter", action="store_true", help="skip the drafter measurement")
    ap.add_argument("--only", default=None,
                    help="time calls of the step in isolation at the workload's shapes; comma-separated "
                         f"from {', '.join(ONLY_CALLS)}")
    ap.add_argument("--iters", type=int, default=100, help="iterations of --only and of the workload lines")
    return ap.parse_args()


ONLY_CALLS = ("attn_global", "attn_local", "attn_global_fp8", "attn_local_fp8", "lmhead", "lmhead_sample",
              "lmhead_sample_rs", "cluster_unembed",
              "qkv_local", "qkv_global", "o_local", "o_global", "gu", "down", "hbm_copy")
COPY_BYTES = 1 << 30  # hbm_copy: a plain 1 GiB device-to-device copy (counter calibration)


def bench_only(args):
    for name in args.only.split(","):
        if name not in ONLY_CALLS:
            raise SystemExit(f"unknown --only call {name!r}; choose from {', '.join(ONLY_CALLS)}")
    for name in args.only.split(","):
        bench_one(args, name)


def bench_one(args, only):
    print(json.dumps(time_one(args, only)), flush=True)


def time_one(args, only) -> dict:
    """One call of the verify step, timed alone at the workload's shapes (batch,
    k, context): the global-layer attention (16q/4kv, D=512, K=V, p-RoPE), a local
    layer's attention (16q/8kv, D=256, window 1024), either over an fp8 cache
    (suffix _fp8), the LM-head select, or one of a layer's projections (fused
    q/k/v, output, gate/up, down)."""
    import torch

    from mtp_draft_verification_amd import _lib as L
    from mtp_draft_verification_amd import configs, inputs
    from mtp_draft_verification_amd.step import attn_desc

    dev = torch.device("cuda:0")
    cfg = dataclasses.replace(configs.STACK, batch=args.batch, k=args.k, ctx=args.ctx)
    B, nq = cfg.batch, cfg.k + 1
    stream = torch.cuda.current_stream()
    if only.startswith("attn"):
        fp8 = only.endswith("_fp8")
        ly = cfg.layers[-1] if only.startswith("attn_global") else cfg.layers[0]
        cap = cfg.ctx + nq + 8
        lo = 0 if ly.window == 0 else max(0, cfg.ctx - ly.window - 8)
        if fp8:
            ks = inputs.channel_scales((ly.n_heads_kv, ly.head_dim), 1.0, 0, "ks", dev)
            kc = torch.zeros((B, ly.n_heads_kv, cap, ly.head_dim), dtype=torch.uint8, device=dev)
            kc[:, :, lo:cfg.ctx] = inputs.fp8_codes((B, ly.n_heads_kv, cfg.ctx - lo, ly.head_dim), 1.0, ks, 0, "kc8", dev)
        else:
            kc = torch.zeros((B, ly.n_heads_kv, cap, ly.head_dim), dtype=torch.bfloat16, device=dev)
            kc[:, :, lo:cfg.ctx] = inputs.normal((B, ly.n_heads_kv, cfg.ctx - lo, ly.head_dim), 1.0, 0, "kc", dev)
        vc = None if ly.k_is_v else kc.clone()
        # as in the stack: fp32 queries and new rows, a bf16-pair output; bf16 (or fp8) caches
        q = inputs.normal((B, nq, ly.n_heads_q, ly.head_dim), 1.0, 0, "q", dev, "f32")
        kn = inputs.normal((B, nq, ly.n_heads_kv, ly.head_dim), 1.0, 0, "kn", dev, "f32")
        vn = None if ly.k_is_v else kn.clone()
        cl = torch.full((B,), cfg.ctx, dtype=torch.int32, device=dev)
        out = torch.empty((2,) + tuple(q.shape), dtype=torch.bfloat16, device=dev)
        desc = attn_desc(ly, B, nq, cap, "bf16", act_pair=True)
        ws = torch.empty(L.sv_verify_attn_workspace(desc), dtype=torch.uint8, device=dev)
        if fp8:
            vs = None if ly.k_is_v else ks.clone()
            call = lambda: L.sv_verify_attn_fp8(desc, q, kn, vn, kc, vc, ks, vs, cl, out, ws, None, stream)
        else:
            call = lambda: L.sv_verify_attn(desc, q, kn, vn, kc, vc, cl, out, ws, None, stream)
        lens = [cfg.ctx] * B
        byts = call_bytes(cfg, lens, 1 if fp8 else 2)["L5.attn" if ly.window == 0 else "L0.attn"]
    elif only.startswith("lmhead"):
        mode = {"lmhead": L.SV_SELECT_GREEDY, "lmhead_sample": L.SV_SELECT_SAMPLE,
                "lmhead_sample_rs": L.SV_SELECT_SAMPLE_RS}[only]
        R = B * nq
        h = inputs.normal((R, cfg.d_model), 1.0, 0, "h", dev)
        W = inputs.normal((cfg.vocab, cfg.d_model), cfg.d_model ** -0.5, 0, "E", dev)
        drafts = torch.randint(0, cfg.vocab, (B, cfg.k), dtype=torch.int32, device=dev)
        u_tok = torch.rand((B, cfg.vocab), device=dev) if mode != L.SV_SELECT_GREEDY else None
        desc = L.LMHeadDesc(batch=B, k=cfg.k, d_model=cfg.d_model, vocab=cfg.vocab, mode=mode, dtype=L.SV_BF16)
        ws = torch.zeros(L.sv_lmhead_workspace(desc), dtype=torch.uint8, device=dev)
        stats = torch.empty((R, L.ROW_STATS_WORDS), dtype=torch.int32, device=dev)
        if mode == L.SV_SELECT_SAMPLE_RS:
            cands = torch.empty((B * cfg.k * L.RS_CANDIDATES, L.RS_CAND_WORDS), dtype=torch.int32, device=dev)
            call = lambda: L.sv_lmhead_select_rs(desc, h, W, drafts, u_tok, 1, 2, stats, cands, None, ws, stream)
        else:
            call = lambda: L.sv_lmhead_select(desc, h, W, drafts, u_tok, None, stats, None, None, ws, stream)
        byts = call_bytes(cfg, [cfg.ctx] * B)["lmhead"]
    elif only == "cluster_unembed":
        # the drafter's clustered unembedding at its shape: one row per sequence over
        # 2048 clusters of 128 tokens, the best 32 kept (4096 candidates per row)
        C, top = 2048, 32
        E = inputs.normal((cfg.vocab, cfg.d_model), cfg.d_model ** -0.5, 0, "E", dev)
        cu = inputs.clusters_of(E, C, top, 0)
        del E
        h = inputs.normal((B, cfg.d_model), 1.0, 0, "h", dev)
        cdesc = L.ClusterDesc(rows=B, d_model=cfg.d_model, vocab=cfg.vocab, n_clusters=C, top_clusters=top,
                              dtype=L.SV_BF16)
        ws = torch.zeros(L.sv_cluster_unembed_workspace(cdesc), dtype=torch.uint8, device=dev)
        stats = torch.empty((B, L.ROW_STATS_WORDS), dtype=torch.int32, device=dev)
        call = lambda: L.sv_cluster_unembed(cdesc, h, cu["centroids"], cu["w_perm"], cu["perm"], stats, None, None,
                                            1, ws, stream)
        cand = (cfg.vocab // C) * top
        byts = C * cfg.d_model * 2 + B * (cand * cfg.d_model * 2 + cand * 4)
    elif only == "hbm_copy":
        src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        call = lambda: dst.copy_(src)
        byts = 2 * COPY_BYTES
    else:
        R = B * nq
        loc, glo = cfg.layers[0], cfg.layers[-1]
        nout = lambda ly: ly.n_heads_q * ly.head_dim + (1 if ly.k_is_v else 2) * ly.n_heads_kv * ly.head_dim
        K, N, add = {"qkv_local": (cfg.d_model, nout(loc), False),
                     "qkv_global": (cfg.d_model, nout(glo), False),
                     "o_local": (loc.n_heads_q * loc.head_dim, cfg.d_model, True),
                     "o_global": (glo.n_heads_q * glo.head_dim, cfg.d_model, True),
                     "gu": (cfg.d_model, 2 * cfg.d_ff, False),
                     "down": (cfg.d_ff, cfg.d_model, True)}[only]
        # as in the stack: bf16-pair activations, bf16 weights, and the stack's epilogue:
        # the fused GeGLU, else K-split fp32 partials (summed by the next call) where
        # the split applies, else a plain fp32 store / add
        x = inputs.normal((2, R, K), 1.0, 0, "x", dev)
        W = inputs.normal((N, K), K ** -0.5, 0, "W", dev)
        if only == "gu":
            epi, S = L.SV_EPI_GEGLU, 0
        else:
            S = max(0, L.sv_linear_splits(L.LinearDesc(rows=R, in_features=K, out_features=N, dtype=L.SV_BF16,
                                                       epilogue=L.SV_EPI_SPLIT_F32, act_pair=1)))
            epi = L.SV_EPI_SPLIT_F32 if S else (L.SV_EPI_ADD_F32 if add else L.SV_EPI_STORE)
        y = (torch.zeros((2, R, N // 2), dtype=torch.bfloat16, device=dev) if epi == L.SV_EPI_GEGLU
             else torch.zeros((max(S, 1) * R, N), dtype=torch.float32, device=dev))
        desc = L.LinearDesc(rows=R, in_features=K, out_features=N, dtype=L.SV_BF16, epilogue=epi, act_pair=1)
        ws = torch.zeros(max(L.sv_linear_workspace(desc), 256), dtype=torch.uint8, device=dev)
        # rotate over copies of W (1 GiB in all) so that, as inside the step, no call
        # finds its weights in the last-level cache; tiled as the step's weights are
        Ws = [L.tiled_weight(desc, W)]
        Ws += [Ws[0].clone() for _ in range(max(0, -(-(1 << 30) // (2 * N * K)) - 1))]
        desc.w_layout = L.SV_W_TILED
        turn = [0]

        def call():
            turn[0] += 1
            L.sv_linear(desc, x, Ws[turn[0] % len(Ws)], y, ws, stream)
        byts = 2 * N * K + 4 * R * K + R * N * (8 if add else 2 if epi == L.SV_EPI_GEGLU else 4)
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.iters):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / args.iters
    gbs = byts / (us * 1e-6) / 1e9
    return {"call": only, "batch": B, "k": cfg.k, "ctx": cfg.ctx, "us_per_call": round(us, 2),
            "alg_bytes": int(byts), "GB/s": round(gbs, 1), "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4),
            # verified positions per second (attention, LM head): the B (k+1) rows one call serves
            "positions_per_s": round(B * nq / (us * 1e-6), 1) if only.startswith(("attn", "lmhead")) else None,
            "source_digest": source_digest()}


def bench_fp8_kv(args) -> dict:
    """The attention calls of the step over fp8 E4M3 caches (per-channel scales)
    next to the same calls over bf16 caches, each timed alone (context, batch and
    k of the workload)."""
    res = {}
    for layer in ("global", "local"):
        a = time_one(args, f"attn_{layer}_fp8")
        b = time_one(args, f"attn_{layer}")
        res[layer] = {"us": a["us_per_call"], "alg_bytes": a["alg_bytes"], "GB/s": a["GB/s"],
                      "frac": a["frac_of_peak"], "bf16_us": b["us_per_call"],
                      "speedup_vs_bf16": round(b["us_per_call"] / a["us_per_call"], 3)}
    return res


def source_digest() -> str:
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "mtp_draft_verification_amd", "csrc", "*"))):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------------
# algorithmic bytes of the calls of one step (what the method must move)
# ---------------------------------------------------------------------------
def call_bytes(cfg, lens, kv_bytes: int = 2) -> dict:
    """Bytes each named call must move once, for committed lengths `lens` (per
    sequence); kv_bytes per cache element (2 bf16, 1 fp8)."""
    B, k, d, R = cfg.batch, cfg.k, cfg.d_model, cfg.batch * (cfg.k + 1)
    nq = k + 1
    e = 2  # bf16 weights and cache rows
    a = 4  # activations between the ops: fp32, or bf16 pairs (the final hidden state is bf16)
    out = {"lmhead": cfg.vocab * d * e + R * d * e}
    for i, ly in enumerate(cfg.layers):
        H, Hk, D = ly.n_heads_q, ly.n_heads_kv, ly.head_dim
        tensors = 1 if ly.k_is_v else 2
        keys = 0
        for L in lens:
            n = L + nq
            keys += min(n, ly.window + k) if ly.window else n
        kv = keys * Hk * D * kv_bytes * tensors
        qio = B * nq * H * D * a * 2 + B * nq * Hk * D * a * tensors
        out[f"L{i}.attn"] = kv + qio
        nout = H * D + Hk * D * tensors
        out[f"L{i}.qkv"] = nout * d * e + R * d * a + R * nout * a
        out[f"L{i}.o"] = d * H * D * e + R * H * D * a + R * d * 4 * 2
        if cfg.d_ff:
            out[f"L{i}.gu"] = 2 * cfg.d_ff * d * e + R * d * a + R * cfg.d_ff * a  # fused GeGLU output
            out[f"L{i}.down"] = d * cfg.d_ff * e + R * cfg.d_ff * a + R * d * 4 * 2
    return out


def only_call(cfg, name: str) -> str | None:
    """The standalone (--only) call that times step call `name` at the step's shape."""
    if name == "lmhead":
        return "lmhead"
    layer, _, op = name.partition(".")
    if not layer.startswith("L") or op not in ("attn", "qkv", "o", "gu", "down"):
        return None
    ly = cfg.layers[int(layer[1:])]
    kind = "global" if ly.window == 0 else "local"
    return op if op in ("gu", "down") else f"{op}_{kind}"


def load_traffic(call: str | None) -> float | None:
    """HBM bytes per launch of standalone call `call` from the committed counter
    summary, if it was taken on the current kernel sources (otherwise None)."""
    p = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if call is None or not os.path.exists(p):
        return None
    try:
        with open(p) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    ent = t.get("calls", {}).get(call)
    if not ent or t.get("source_digest") != source_digest():
        return None
    return float(ent["bytes_per_call"])


# ---------------------------------------------------------------------------
def run_workload(cfg, W, steps, warmup, seed, dev, time_calls=None):
    import numpy as np
    import torch

    from mtp_draft_verification_amd import _lib as L
    from mtp_draft_verification_amd import inputs
    from mtp_draft_verification_amd.step import VerifyStack

    B, k = cfg.batch, cfg.k
    cap = cfg.ctx + (k + 1) * (steps + 2) + 16
    log(f"B={B}: caches (capacity {cap})")
    caches = inputs.stack_caches(cfg, seed, dev, capacity=cap, fill_from=0)
    cl = torch.full((B,), cfg.ctx, dtype=torch.int32, device=dev)
    vs = VerifyStack(cfg, W, caches, cl, dev)
    cfg0 = dataclasses.replace(cfg, k=0)
    cl_ar = torch.empty_like(cl)
    ar = VerifyStack(cfg0, W, caches, cl_ar, dev)
    no_drafts = torch.empty((B, 0), dtype=torch.int32, device=dev)
    rng = np.random.default_rng(seed)

    # warm-up: random drafts, then back to the starting state
    for _ in range(warmup):
        tok = torch.randint(0, cfg.vocab, (B, k + 1), dtype=torch.int32, device=dev)
        vs.step(tok, tok[:, 1:].contiguous())
    torch.cuda.synchronize()
    cl.fill_(cfg.ctx)

    # record the trajectory (untimed)
    last = torch.randint(0, cfg.vocab, (B,), dtype=torch.int32, device=dev)
    rec_tok, rec_dr, rec_n, rec_len = [], [], [], []
    for s in range(steps):
        cl_ar.copy_(cl)
        cont = torch.empty((B, k), dtype=torch.int32, device=dev)
        cur = last.view(B, 1).clone()
        for i in range(k):
            ar.step(cur, no_drafts)
            cur = ar.out_tokens[:, :1].clone()
            cont[:, i] = cur[:, 0]
        keep = torch.from_numpy(rng.random((B, k)) < cfg.draft_match).to(dev)
        other = torch.from_numpy(rng.integers(0, cfg.vocab - 1, (B, k)).astype(np.int32)).to(dev)
        other = torch.where(other >= cont, other + 1, other)
        drafts = torch.where(keep, cont, other).contiguous()
        tokens = torch.cat([last.view(B, 1), drafts], dim=1).contiguous()
        rec_len.append(cl.cpu().numpy().copy())
        vs.step(tokens, drafts)
        acc = L.decode_accept_out(vs.acc)
        rec_tok.append(tokens)
        rec_dr.append(drafts)
        rec_n.append(acc["n_accepted"].copy())
        last = vs.acc[:, 1].clone()
    torch.cuda.synchronize()
    assert int(vs.dev_status.item()) == 0, "device status set while recording"
    committed = int(sum(int((n + 1).sum()) for n in rec_n))
    mean_lens = np.mean(np.stack(rec_len), axis=0)

    def replay(timers):
        cl.fill_(cfg.ctx)
        vs.timers = timers
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for s in range(steps):
            vs.step(rec_tok[s], rec_dr[s])
        e1.record(stream)
        torch.cuda.synchronize()
        vs.timers = None
        return e0.elapsed_time(e1)

    # per-call durations (instrumented replay, all calls)
    names = ["embed", "lmhead", "accept", "final_norm"]
    for i, _ in enumerate(cfg.layers):
        names += [f"L{i}.{c}" for c in ("qkv", "attn", "o", "gu", "geglu", "down")]
    timers = {n: [] for n in names}
    replay(timers)
    # median: a call's time in the instrumented pass can include an occasional host-side stall
    call_ms = {n: float(np.median([a.elapsed_time(b) for a, b in v])) for n, v in timers.items() if v}
    byts = call_bytes(cfg, mean_lens)
    dominant = max((n for n in call_ms if n in byts), key=lambda n: call_ms[n])
    if time_calls:
        dominant = time_calls

    # eager replay of the whole step, with events around the dominant call only
    dom_t = {dominant: []}
    ms_eager = replay(dom_t)
    ok = all(np.array_equal(L.decode_accept_out(vs.acc)["n_accepted"], rec_n[-1]) for _ in [0])
    assert ok, "replay diverged from the recorded trajectory"
    dom_ms = float(np.mean([a.elapsed_time(b) for a, b in dom_t[dominant]]))

    # timed replay: the step's launches captured once in a HIP graph, one replay per
    # step on input buffers that take each step's tokens and drafts (no launch gaps
    # from the host); then once more with events around every step for the spread
    tok_buf = torch.empty_like(rec_tok[0])
    dr_buf = torch.empty_like(rec_dr[0])
    cl.fill_(cfg.ctx)
    torch.cuda.synchronize()
    try:
        graph = vs.capture(tok_buf, dr_buf)
    except Exception as e:  # keep the measurement: time the step call by call instead
        log(f"graph capture failed ({e!r}); timing the step call by call")
        graph = None

    def replay_graph(step_ev=None):
        cl.fill_(cfg.ctx)
        torch.cuda.synchronize()
        st = torch.cuda.current_stream()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for s in range(steps):
            tok_buf.copy_(rec_tok[s])
            dr_buf.copy_(rec_dr[s])
            if step_ev is not None:
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record(st)
                graph.replay()
                b.record(st)
                step_ev.append((a, b))
            else:
                graph.replay()
        e1.record(st)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    if graph is not None:
        replay_graph()  # untimed: the first launch of a new graph also uploads it
        ms = replay_graph()
        ok = all(np.array_equal(L.decode_accept_out(vs.acc)["n_accepted"], rec_n[-1]) for _ in [0])
        assert ok, "graph replay diverged from the recorded trajectory"
        step_ev = []
        replay_graph(step_ev)
        step_pct = np.percentile([a.elapsed_time(b) for a, b in step_ev], [10, 50, 90])
        launch = "one HIP graph replay per step (the step's launches captured once)"
    else:
        ms = ms_eager
        step_pct = None
        launch = "call by call (graph capture failed)"
    res = dict(B=B, steps=steps, ms_total=ms, ms_per_step=ms / steps, committed=committed,
               ms_per_step_eager=ms_eager / steps, step_launch=launch,
               step_ms_p10_p50_p90=None if step_pct is None else [round(float(x), 4) for x in step_pct],
               tokens_per_s=committed / (ms / 1e3), mean_accepted=float(np.mean(np.stack(rec_n))),
               call_ms=call_ms, call_bytes=byts, dominant=dominant, dominant_ms=dom_ms,
               first_tokens=rec_tok[0], first_len=rec_len[0], caches=caches)
    return res


def bench_drafter(cfg, W, caches, lens, dev, cycles: int = 10, warmup: int = 2) -> dict:
    """Time k draft steps of the MTP drafter (3 local + 1 global cross-attention
    blocks of width 1024) over the same caches, after the verify replay: reported
    apart from the verify step.  Inputs: synthetic final hidden states and accept
    records (row b(k+1), a random next token); random-init drafter weights."""
    import numpy as np
    import torch

    from mtp_draft_verification_amd import _lib as L
    from mtp_draft_verification_amd import configs, inputs
    from mtp_draft_verification_amd.drafter import Drafter

    dcfg = configs.DRAFTER
    B, k = cfg.batch, cfg.k
    log(f"drafter: d_draft={dcfg.d_draft}, blocks {','.join(dcfg.blocks)}, k={k}")
    dw = inputs.drafter_weights(cfg, dcfg, 1, dev)
    cl = torch.tensor(np.asarray(lens, dtype=np.int64).round().astype(np.int32), device=dev)
    dr = Drafter(cfg, dcfg, W["E"], dw, caches, cl, dev)
    R = B * (k + 1)
    h = inputs.normal((R, cfg.d_model), 1.0, 1, "h_verify", dev)
    acc = torch.zeros(B, L.ACCEPT_OUT_WORDS, dtype=torch.int32, device=dev)
    acc[:, 7] = torch.arange(B, dtype=torch.int32, device=dev) * (k + 1)
    acc[:, 1] = inputs.randint((B,), 0, cfg.vocab - 1, 1, "next_tok", dev)
    drafts = torch.zeros(B, k, dtype=torch.int32, device=dev)
    for _ in range(warmup):
        dr.draft(k, h, acc, drafts)
    torch.cuda.synchronize()
    names = ["draft_input", "unembed"] + [f"D{j}.{c}" for j in range(len(dcfg.blocks)) for c in ("attn", "mlp")]
    dr.timers = {n: [] for n in names}
    dr.draft(k, h, acc, drafts)
    torch.cuda.synchronize()
    call_us = {n: round(float(np.median([a.elapsed_time(b) for a, b in v])) * 1e3, 2) for n, v in dr.timers.items()}
    dr.timers = None
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(cycles):
        dr.draft(k, h, acc, drafts)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / cycles
    assert int(dr.dev_status.item()) == 0
    gi = dcfg.blocks.index("global")
    ly = cfg.layers[dr.reads[gi]]
    g_bytes = float(sum(int(x) for x in cl.tolist())) * ly.n_heads_kv * ly.head_dim * 2
    g_us = call_us[f"D{gi}.attn"]
    out = {"k": k, "ms_per_k_steps": round(ms, 4), "ms_per_step": round(ms / k, 4),
           "global_block_read_bytes_per_step": int(g_bytes),
           "global_block_us": g_us, "global_block_GB/s": round(g_bytes / (g_us * 1e-6) / 1e9, 1),
           "calls_us": call_us,
           "config": f"{dcfg.name}: d_draft {dcfg.d_draft}, d_ff {dcfg.d_ff}, blocks {'/'.join(dcfg.blocks)} "
                     f"reading the target's last local and global caches, batch {B}"}
    # the same drafter with the clustered unembedding: 2048 clusters of 128 tokens, the
    # best 32 kept (4096 candidate rows per sequence)
    C, top = 2048, 32
    log(f"drafter: clustered unembedding, {C} clusters, {top} kept")
    cu = inputs.clusters_of(W["E"], C, top, 1)
    drc = Drafter(cfg, dcfg, W["E"], dw, caches, cl, dev, clusters=cu)
    for _ in range(warmup):
        drc.draft(k, h, acc, drafts)
    torch.cuda.synchronize()
    drc.timers = {"unembed": []}
    drc.draft(k, h, acc, drafts)
    torch.cuda.synchronize()
    un_us = round(float(np.median([a.elapsed_time(b) for a, b in drc.timers["unembed"]])) * 1e3, 2)
    drc.timers = None
    e0.record()
    for _ in range(cycles):
        drc.draft(k, h, acc, drafts)
    e1.record()
    torch.cuda.synchronize()
    msc = e0.elapsed_time(e1) / cycles
    assert int(drc.dev_status.item()) == 0
    d = cfg.d_model
    cand = (cfg.vocab // C) * top
    cl_bytes = C * d * 2 + B * (cand * d * 2 + cand * 4)
    out["clustered_unembed"] = {
        "n_clusters": C, "top_clusters": top, "candidates_per_row": cand,
        "ms_per_k_steps": round(msc, 4), "ms_per_step": round(msc / k, 4),
        "unembed_us": un_us, "unembed_read_bytes": int(cl_bytes),
        "note": "unembed_us includes the final norm and W_up projection, as calls_us.unembed does"}
    del drc, cu
    torch.cuda.empty_cache()
    # the same drafter reading fp8 E4M3 copies (per-channel scales) of the caches of
    # the two target layers it reads
    log("drafter: fp8 caches of the layers it reads")
    caches8 = list(caches)
    scales = {}
    for ti in sorted(set(dr.reads)):
        ly = cfg.layers[ti]
        ks = inputs.channel_scales((ly.n_heads_kv, ly.head_dim), 1.0, 1, f"ks{ti}", dev)
        vs = None if ly.k_is_v else inputs.channel_scales((ly.n_heads_kv, ly.head_dim), 1.0, 1, f"vs{ti}", dev)
        caches8[ti] = {"k": inputs.fp8_codes(caches[ti]["k"].shape, 1.0, ks, 1, f"k8{ti}", dev),
                       "v": None if vs is None else inputs.fp8_codes(caches[ti]["v"].shape, 1.0, vs, 1, f"v8{ti}", dev)}
        scales[ti] = (ks, vs)
    dr8 = Drafter(cfg, dcfg, W["E"], dw, caches8, cl, dev, kv_scales=scales)
    for _ in range(warmup):
        dr8.draft(k, h, acc, drafts)
    torch.cuda.synchronize()
    dr8.timers = {f"D{gi}.attn": []}
    dr8.draft(k, h, acc, drafts)
    torch.cuda.synchronize()
    g8_us = round(float(np.median([a.elapsed_time(b) for a, b in dr8.timers[f"D{gi}.attn"]])) * 1e3, 2)
    dr8.timers = None
    e0.record()
    for _ in range(cycles):
        dr8.draft(k, h, acc, drafts)
    e1.record()
    torch.cuda.synchronize()
    ms8 = e0.elapsed_time(e1) / cycles
    assert int(dr8.dev_status.item()) == 0
    out["fp8_kv"] = {"ms_per_k_steps": round(ms8, 4), "ms_per_step": round(ms8 / k, 4), "global_block_us": g8_us,
                     "global_block_read_bytes_per_step": int(g_bytes // 2),
                     "global_block_GB/s": round(g_bytes / 2 / (g8_us * 1e-6) / 1e9, 1)}
    del dr8, caches8
    return out


def host_cpu() -> str:
    """The host CPU's model name (from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _timed(call, iters, warm=3) -> float:
    """Mean microseconds per call over `iters` back-to-back calls on the current
    stream (HIP events), after `warm` untimed calls."""
    import torch
    for _ in range(warm):
        call()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(iters):
        call()
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / iters


def _rate(byts, us):
    gbs = byts / (us * 1e-6) / 1e9
    return {"GB/s": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4)}


def bench_configs(args) -> dict:
    """Standalone lines for the other workloads, each call timed alone (`iters`
    back-to-back calls after warm-up, HIP events), inputs generated as the parity
    tests generate them:
      tiny_f32_verify    -- the one-layer fp32 step (d=128, 2q/1kv, D=64, 64 cached
                            tokens, k=3, vocab 1024): latency only;
      local_attn_verify  -- B=1, 16q/8kv, D=256, L=4096, W=1024, k=4 (bf16);
      global_attn_verify -- B=8, 32q/4kv, D=512, K=V, p-RoPE, L ~ U[8192, 32768],
                            k=4, over a bf16 and over an fp8 cache;
      lmhead_select_b1 / _b8 -- V=262,144, d=3840, k=4: the greedy select; a
                            sampling step done two ways: two-pass (pass 1 with the
                            bonus draw, accept, the residual pass) and single-pass
                            (pass 1 with four candidates per draft row, accept,
                            and the residual pass only for a sequence that refuses
                            all four), drafter rows q ~ Dirichlet(0.1)."""
    import numpy as np
    import torch

    from mtp_draft_verification_amd import _lib as L
    from mtp_draft_verification_amd import configs, inputs
    from mtp_draft_verification_amd.step import VerifyStack, attn_desc

    dev = torch.device("cuda:0")
    it = args.iters
    out = {}

    # tiny fp32 step
    cfg = configs.TINY_F32
    W = inputs.stack_weights(cfg, 0, dev)
    caches = inputs.stack_caches(cfg, 0, dev, capacity=cfg.ctx + 16)
    cl = torch.full((1,), cfg.ctx, dtype=torch.int32, device=dev)
    vs = VerifyStack(cfg, W, caches, cl, dev)
    tok = inputs.randint((1, cfg.k + 1), 0, cfg.vocab - 1, 0, "tok", dev)
    dr = tok[:, 1:].contiguous()

    def tiny():
        cl.fill_(cfg.ctx)
        vs.step(tok, dr)
    out["tiny_f32_verify"] = {"us_per_step": round(_timed(tiny, it), 2),
                              "note": "one verify step (embedding, attention with append, output projection, "
                                      "LM head, accept) launched call by call; latency only"}
    del vs, W, caches

    # verify attention workloads
    def attn_line(acfg, fp8):
        ly = acfg.layer
        B, nq = acfg.batch, acfg.k + 1
        a = inputs.attn_inputs(acfg, 0, dev)
        cap = a["cap"]
        desc = attn_desc(ly, B, nq, cap, "bf16")
        ws = torch.empty(L.sv_verify_attn_workspace(desc), dtype=torch.uint8, device=dev)
        out_t = torch.empty_like(a["q"])
        lens = a["cache_len"].cpu().numpy()
        keys = sum(min(int(l) + nq, ly.window + acfg.k) if ly.window else int(l) + nq for l in lens)
        tensors = 1 if ly.k_is_v else 2
        qio = B * nq * ly.n_heads_q * ly.head_dim * 2 * 2 + B * nq * ly.n_heads_kv * ly.head_dim * 2 * tensors
        if fp8:
            ks = inputs.channel_scales((ly.n_heads_kv, ly.head_dim), acfg.std, 0, "ks", dev)
            kc = inputs.fp8_codes(tuple(a["k_cache"].shape), acfg.std, ks, 0, "kc8", dev)
            vsc = None if ly.k_is_v else ks.clone()
            vc = None if ly.k_is_v else kc.clone()
            call = lambda: L.sv_verify_attn_fp8(desc, a["q"], a["k_new"], a["v_new"], kc, vc, ks, vsc,
                                                a["cache_len"], out_t, ws)
            byts = keys * ly.n_heads_kv * ly.head_dim * 1 * tensors + qio
        else:
            call = lambda: L.sv_verify_attn(desc, a["q"], a["k_new"], a["v_new"], a["k_cache"], a["v_cache"],
                                            a["cache_len"], out_t, ws)
            byts = keys * ly.n_heads_kv * ly.head_dim * 2 * tensors + qio
        us = _timed(call, it)
        res = {"us_per_call": round(us, 2), "alg_bytes": int(byts), **_rate(byts, us),
               "positions_per_s": round(B * nq / (us * 1e-6), 1)}
        del a
        return res

    out["local_attn_verify"] = attn_line(configs.LOCAL_ATTN, False)
    out["local_attn_verify"]["note"] = ("8.42 MB per call is below what one launch can stream at peak "
                                        "(bandwidth x latency): latency-bound")
    out["global_attn_verify"] = attn_line(configs.GLOBAL_ATTN, False)
    out["global_attn_verify_fp8"] = attn_line(configs.GLOBAL_ATTN, True)
    torch.cuda.empty_cache()

    # LM head select, greedy and sampling
    for lcfg in (configs.LMHEAD_B1, configs.LMHEAD_B8):
        B, k, d, V = lcfg.batch, lcfg.k, lcfg.d_model, lcfg.vocab
        R = B * (k + 1)
        h = inputs.normal((R, d), 1.0, 0, "h", dev)
        Wt = inputs.normal((V, d), d ** -0.5, 0, "W", dev)
        wbytes = V * d * 2 + R * d * 2
        drafts_g = inputs.randint((B, k), 0, V - 1, 0, "drafts", dev)
        gdesc = L.LMHeadDesc(batch=B, k=k, d_model=d, vocab=V, mode=L.SV_SELECT_GREEDY, dtype=L.SV_BF16)
        ws = torch.zeros(max(L.sv_lmhead_workspace(gdesc),
                             L.sv_lmhead_workspace(L.LMHeadDesc(batch=B, k=k, d_model=d, vocab=V,
                                                                mode=L.SV_SELECT_SAMPLE_RS, dtype=L.SV_BF16))),
                         dtype=torch.uint8, device=dev)
        stats = torch.empty((R, L.ROW_STATS_WORDS), dtype=torch.int32, device=dev)
        us_g = _timed(lambda: L.sv_lmhead_select(gdesc, h, Wt, drafts_g, None, None, stats, None, None, ws), it)
        line = {"greedy": {"us_per_call": round(us_g, 2), "alg_bytes": int(wbytes), **_rate(wbytes, us_g),
                           "positions_per_s": round(R / (us_g * 1e-6), 1)}}
        # sampling inputs: drafter rows q ~ Dirichlet(0.1), drafts ~ q, uniforms
        q_rows = inputs.dirichlet_rows(B * k, V, lcfg.dirichlet_alpha, 0, "q", dev).view(B, k, V)
        drafts = inputs.categorical(q_rows.view(B * k, V), 0, "drafts").view(B, k)
        u_acc = inputs.uniform((B, k), 0, "u_acc", dev)
        u_tok = inputs.uniform((B, V), 0, "u_tok", dev)
        u_rs = inputs.uniform((B, L.RS_CANDIDATES), 0, "u_rs", dev)
        sdesc = L.LMHeadDesc(batch=B, k=k, d_model=d, vocab=V, mode=L.SV_SELECT_SAMPLE, dtype=L.SV_BF16)
        rdesc = L.LMHeadDesc(batch=B, k=k, d_model=d, vocab=V, mode=L.SV_SELECT_RESIDUAL, dtype=L.SV_BF16)
        xdesc = L.LMHeadDesc(batch=B, k=k, d_model=d, vocab=V, mode=L.SV_SELECT_SAMPLE_RS, dtype=L.SV_BF16)
        adesc = L.AcceptDesc(batch=B, k=k, vocab=V, mode=L.SV_SELECT_SAMPLE)
        xadesc = L.AcceptDesc(batch=B, k=k, vocab=V, mode=L.SV_SELECT_SAMPLE_RS)
        cl = torch.zeros((B,), dtype=torch.int32, device=dev)
        toks = torch.empty((B, k + 1), dtype=torch.int32, device=dev)
        acc = torch.zeros((B, L.ACCEPT_OUT_WORDS), dtype=torch.int32, device=dev)
        cands = torch.empty((B * k * L.RS_CANDIDATES, L.RS_CAND_WORDS), dtype=torch.int32, device=dev)

        def two_pass():
            L.sv_lmhead_select(sdesc, h, Wt, drafts, u_tok, None, stats, None, None, ws)
            L.sv_accept(adesc, drafts, stats, q_rows, u_acc, cl, toks, acc)
            L.sv_lmhead_select(rdesc, h, Wt, drafts, u_tok, q_rows, stats, acc, toks, ws)
        us_two = _timed(two_pass, it)
        n_two = L.decode_accept_out(acc)["n_accepted"]
        key = [0]

        def one_pass():
            key[0] += 1
            L.sv_lmhead_select_rs(xdesc, h, Wt, drafts, u_tok, key[0], 7, stats, cands, None, ws)
            L.sv_accept_rs(xadesc, drafts, stats, cands, q_rows, u_acc, u_rs, cl, toks, acc)
        us_one = _timed(one_pass, it)
        us_res = _timed(lambda: L.sv_lmhead_select(rdesc, h, Wt, drafts, u_tok, q_rows, stats, acc, toks, ws), it)
        # the standard mode's per-step uniforms (u_tok [B, V], u_accept [B, k], u_rs) drawn on
        # the device, as a decode loop would before each step
        u_gen = torch.Generator(device=dev)
        u_gen.manual_seed(1)
        us_unif = _timed(lambda: (torch.rand((B, V), generator=u_gen, device=dev, out=u_tok),
                                  torch.rand((B, k), generator=u_gen, device=dev, out=u_acc)), it)
        # how often a rejecting sequence refuses all four candidates (new key per step)
        rej = fb = 0
        for _ in range(32):
            one_pass()
            a = L.decode_accept_out(acc)
            rej += int((a["n_accepted"] < k).sum())
            fb += int((a["residual_row"] >= 0).sum())
        p_step = 1.0 - (1.0 - fb / max(rej, 1)) ** max(1, int(round(rej / 32)))  # a step needs pass 2
        line["sampling"] = {
            "two_pass_us_per_step": round(us_two, 2),
            "single_pass_us_first_pass_and_accept": round(us_one, 2),
            "residual_pass_us": round(us_res, 2),
            "rejecting_sequences_per_step": round(rej / 32, 2),
            "candidates_all_refused_fraction": round(fb / max(rej, 1), 4),
            "single_pass_expected_us_per_step": round(us_one + p_step * us_res, 2),
            "two_pass_n_accepted": n_two.tolist(),
            "uniforms_us_per_step": round(us_unif, 2),
            "uniforms_bytes_per_step": int(4 * (B * V + B * k)),
            "note": "two-pass always launches the residual pass (graph-friendly); the single-pass step "
                    "launches it only when some rejecting sequence refused all four candidates, with the "
                    "probability measured over 32 steps; uniforms_us_per_step: drawing the step's "
                    "uniform inputs on the device (torch.rand), not included in the step times"}
        out[lcfg.name] = line
        del h, Wt, q_rows, ws
        torch.cuda.empty_cache()
    return out


def cpu_baseline(cfg, W, caches, tokens, lens, dev):
    """Time the oracle on a bounded sample: the first recorded verify step of
    sequences 0..2 (three single-sequence steps, one batched oracle call) on all
    host threads, and the step of sequence 0 on one thread."""
    import numpy as np

    import oracle
    from oracle import model as om
    from mtp_draft_verification_amd import inputs

    nseq = min(3, cfg.batch)
    log(f"cpu baseline: host copies for sequences 0..{nseq - 1}")
    hw = {"E": inputs.bf16_bits(W["E"]),
          "layers": [{k: inputs.bf16_bits(v) for k, v in lw.items()} for lw in W["layers"]]}
    cap = caches[0]["k"].shape[2]
    Ls = [int(x) for x in lens[:nseq]]

    def host_state(n):
        hc = []
        for ly, c in zip(cfg.layers, caches):
            ent = {}
            for nm in ("k", "v"):
                t = c[nm]
                if t is None:
                    ent[nm] = None
                    continue
                a = np.zeros((n, t.shape[1], cap, t.shape[3]), dtype=np.float32)
                for b in range(n):
                    lo = max(0, Ls[b] - ly.window - 8) if ly.window else 0
                    a[b, :, lo:Ls[b]] = t[b, :, lo:Ls[b]].float().cpu().numpy()
                ent[nm] = a
            hc.append(ent)
        return om.new_state(hc, Ls[:n])

    model = om.OracleModel(dataclasses.replace(cfg, batch=nseq), hw)
    state = host_state(nseq)
    tok = tokens[:nseq].cpu().numpy()
    cores = oracle.num_threads()
    log(f"cpu baseline: oracle steps on {cores} threads")
    t0 = time.perf_counter()
    r = model.greedy_step(state, tok)
    dt = time.perf_counter() - t0
    n = int(np.sum(r["n"])) + nseq
    # sequence 0's step on one thread (from the same starting state)
    log("cpu baseline: oracle step on 1 thread")
    model1 = om.OracleModel(dataclasses.replace(cfg, batch=1), hw)
    state1 = host_state(1)
    oracle.set_threads(1)
    t0 = time.perf_counter()
    r1 = model1.greedy_step(state1, tok[:1])
    dt1 = time.perf_counter() - t0
    oracle.set_threads(cores)
    n1 = int(r1["n"][0]) + 1
    return dict(value=n / dt, unit="tokens/s", cores=cores, kind="oracle",
                single_thread_value=n1 / dt1, cpu_model=host_cpu(), host_threads=os.cpu_count(),
                sample=f"the first recorded verify step of sequences 0..{nseq - 1} ({cfg.k + 1} rows each, all 6 "
                       f"layers, LM head, accept) of the same workload: {n} tokens committed in {dt:.1f} s on "
                       f"{cores} threads ({dt / nseq:.2f} s per step); sequence 0's step on one thread: "
                       f"{n1} tokens in {dt1:.1f} s")


def pmc_summary(roots, out_path=None):
    """Write profiles/hbm_traffic.json from rocprofv3 --pmc runs (csv output) of
    `bench.py --only <call> --iters 3`, one run per call and counter:
    roots[0]/<call>/ holds the FETCH_SIZE run, roots[1]/<call>/ the WRITE_SIZE run,
    and <root>/<call>.json that run's own output line (for the algorithmic bytes).
    A call's bytes: its library kernels' counter values summed over the run and
    divided by the number of calls made (the dispatch count of its most frequent
    kernel), each counter scaled by what it reads for the plain 1 GiB copy.  The
    weight tiling that sets up a projection call runs once and is left out."""
    import csv
    from collections import Counter

    def dispatches(d, counter):
        rows = []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                rows += [r for r in csv.DictReader(fh) if r["Counter_Name"] == counter]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        return [(r["Kernel_Name"], float(r["Counter_Value"])) for r in rows]

    def ours(name):
        # the library's kernels of the call itself: the one-time weight tiling that sets
        # up a projection call is not part of it
        return name.startswith(("sv::", "void sv::")) and "tile_weights_kernel" not in name

    out = {"source_digest": source_digest(), "counters": "FETCH_SIZE, WRITE_SIZE (KiB per dispatch)",
           "method": "one rocprofv3 --pmc run per call and counter of bench.py --only <call> --iters 3; "
                     "library kernels summed, divided by the calls made, scaled by the 1 GiB copy",
           "copy_scale": {}, "calls": {}}
    for key, root in (("FETCH_SIZE", roots[0]), ("WRITE_SIZE", roots[1])):
        cp = [v for n, v in dispatches(os.path.join(root, "hbm_copy"), key) if not ours(n)]
        cp = sorted(cp)[-3:]  # the copy's own dispatches are the largest
        out["copy_scale"][key] = round((COPY_BYTES / 1024) / (sum(cp) / len(cp)), 4)
    calls = sorted(os.path.basename(d) for d in glob.glob(os.path.join(roots[0], "*"))
                   if os.path.isdir(d) and os.path.basename(d) != "hbm_copy")
    for call in calls:
        ent = {}
        tot = 0.0
        for key, root in (("FETCH_SIZE", roots[0]), ("WRITE_SIZE", roots[1])):
            ds = [(n, v) for n, v in dispatches(os.path.join(root, call), key) if ours(n)]
            if not ds:
                break
            ncalls = max(Counter(n for n, _ in ds).values())
            kib = sum(v for _, v in ds) / ncalls
            ent[key + "_KiB_per_call_raw"] = round(kib, 1)
            ent["calls_counted"] = ncalls
            tot += kib * 1024 * out["copy_scale"][key]
        else:
            ent["bytes_per_call"] = round(tot)
            try:
                with open(os.path.join(roots[0], call + ".json")) as f:
                    alg = json.loads(f.read().strip().splitlines()[-1])["alg_bytes"]
                ent["alg_bytes"] = alg
                ent["traffic_over_alg"] = round(tot / alg, 4)
            except (OSError, ValueError, KeyError, IndexError):
                pass
            out["calls"][call] = ent
    with open(out_path or os.path.join(ROOT, "profiles", "hbm_traffic.json"), "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))
    return out


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--pmc-summary":
        pmc_summary(sys.argv[2:4])
        return
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the library implements the "
              f"one-GPU path; across GPUs the verify step would shard by sequence, with no exchange.",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from mtp_draft_verification_amd import _lib as L
    from mtp_draft_verification_amd import configs, inputs

    L.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.only:
        bench_only(args)
        return
    dev = torch.device("cuda:0")
    if args.profile:
        args.sweep = ""
        args.no_cpu_baseline = True
    cfg = dataclasses.replace(configs.STACK, batch=args.batch, k=args.k, ctx=args.ctx, steps=args.steps)
    log(f"weights (d={cfg.d_model}, d_ff={cfg.d_ff}, vocab={cfg.vocab})")
    W = inputs.stack_weights(cfg, args.seed, dev)
    main_res = run_workload(cfg, W, args.steps, args.warmup, args.seed, dev)
    log(f"B={cfg.batch}: {main_res['tokens_per_s']:.1f} tokens/s, {main_res['ms_per_step']:.3f} ms/step, "
        f"mean accepted {main_res['mean_accepted']:.2f}")

    # the sweep: k x batch, each point the same protocol as the main line
    sweep = {}
    for kk in [int(x) for x in args.sweep_k.split(",") if x.strip()]:
        row = {}
        for b in [int(x) for x in args.sweep.split(",") if x.strip()]:
            if (kk, b) == (cfg.k, cfg.batch):
                row[f"B{b}"] = {"tokens_per_s": round(main_res["tokens_per_s"], 1),
                                "ms_per_step": round(main_res["ms_per_step"], 4),
                                "mean_accepted": round(main_res["mean_accepted"], 3)}
                continue
            c2 = dataclasses.replace(cfg, batch=b, k=kk)
            r = run_workload(c2, W, args.steps, args.warmup, args.seed, dev)
            row[f"B{b}"] = {"tokens_per_s": round(r["tokens_per_s"], 1), "ms_per_step": round(r["ms_per_step"], 4),
                            "mean_accepted": round(r["mean_accepted"], 3)}
            log(f"k={kk} B={b}: {r['tokens_per_s']:.1f} tokens/s, {r['ms_per_step']:.3f} ms/step")
            del r
            torch.cuda.empty_cache()
        sweep[f"k{kk}"] = row

    config_lines = None
    if not args.no_configs and not args.profile:
        config_lines = bench_configs(args)
        log("workload lines: " + ", ".join(config_lines))

    dom = main_res["dominant"]
    dom_bytes = main_res["call_bytes"][dom]
    ach = dom_bytes / (main_res["dominant_ms"] * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": load_traffic(only_call(cfg, dom)), "kernel": dom,
            "alg_bytes_per_launch": int(dom_bytes), "mean_launch_us": round(main_res["dominant_ms"] * 1e3, 2)}
    kern = {}
    for n, ms in sorted(main_res["call_ms"].items(), key=lambda kv: -kv[1]):
        b = main_res["call_bytes"].get(n)
        kern[n] = {"us": round(ms * 1e3, 2)}
        if b:
            kern[n]["GB/s"] = round(b / (ms * 1e-3) / 1e9, 1)
            kern[n]["frac"] = round(b / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 3)
            tr = load_traffic(only_call(cfg, n))
            if tr:
                kern[n]["traffic_over_alg"] = round(tr / b, 3)

    drafter = None
    if not args.no_drafter and not args.profile:
        drafter = bench_drafter(cfg, W, main_res["caches"], main_res["first_len"], dev)
        log(f"drafter: {drafter['ms_per_k_steps']:.3f} ms per {cfg.k} steps")

    fp8_kv = None
    if not args.profile:
        fp8_kv = bench_fp8_kv(args)
        log(f"fp8 KV: global attention {fp8_kv['global']['us']} us (bf16 {fp8_kv['global']['bf16_us']} us)")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, W, main_res["caches"], main_res["first_tokens"], main_res["first_len"], dev)
        log(f"cpu baseline: {cpu['value']:.4f} tokens/s on {cpu['cores']} threads")

    out = {
        "metric": METRIC, "value": round(main_res["tokens_per_s"], 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(main_res["ms_per_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded random-init weights and caches; drafts = the target's greedy "
                "continuation kept with probability 0.8)",
        "config": {"workload": f"stack_verify: 6-layer 5:1 local/global decoder stack, d={cfg.d_model}, "
                               f"d_ff={cfg.d_ff}, vocab {cfg.vocab}, committed context {cfg.ctx}, k={cfg.k}, "
                               f"batch {cfg.batch}, greedy verify with KV append/rollback",
                   "batch": cfg.batch, "k": cfg.k, "ctx": cfg.ctx, "d_model": cfg.d_model,
                   "vocab": cfg.vocab, "layers": "LLLLLG"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "sweep": sweep,
        "workload_lines": config_lines,
        "mean_accepted": round(main_res["mean_accepted"], 3),
        "step_ms_p10_p50_p90": main_res["step_ms_p10_p50_p90"],
        "step_launch": main_res["step_launch"],
        "ms_per_step_eager": round(main_res["ms_per_step_eager"], 4),
        "kernels": kern,
        "drafter": drafter,
        "fp8_kv_attention": fp8_kv,
        "source_digest": source_digest(),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
