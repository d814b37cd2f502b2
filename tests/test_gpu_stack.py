"""GPU parity of a whole verify step (embedding, layers, LM head, accept) against
the oracle, in lockstep over many steps.

Drafts follow the workloads' recipe: the target's own greedy continuation
(computed by the oracle) with each draft replaced by a uniform random token with
probability 1 - draft_match.  Per step the GPU's row statistics must match the
oracle's within 2e-2, and accept lengths / emitted tokens bit for bit wherever
the oracle's deciding top-2 margin exceeds 1e-2.  Where the margin rule excuses
a difference both sides commit the oracle's decision (lockstep)."""
import numpy as np
import pytest
import torch

import oracle
from oracle import model as om
import mtp_draft_verification_amd._lib as L
from mtp_draft_verification_amd import configs, inputs
from mtp_draft_verification_amd.step import VerifyStack, attn_desc
from gpu_util import gpu, host, need_gpu, rel_l2, say

ATOL = 2e-2
MARGIN = 1e-2


def host_weights(W, bf16):
    conv = inputs.bf16_bits if bf16 else inputs.host_f32
    return {"E": conv(W["E"]), "layers": [{k: conv(v) for k, v in lw.items()} for lw in W["layers"]]}


def host_caches(caches, seqs, cfg, cap, only_window=False):
    """fp32 host copies of the caches of the given sequences.  With only_window,
    local layers copy just the rows their window can still see (np.zeros is lazy,
    so the untouched rows cost no memory)."""
    out = []
    for ly, c in zip(cfg.layers, caches):
        ent = {}
        for nm in ("k", "v"):
            t = c[nm]
            if t is None:
                ent[nm] = None
                continue
            if only_window and ly.window > 0:
                a = np.zeros((len(seqs), t.shape[1], cap, t.shape[3]), dtype=np.float32)
                lo = max(0, cfg.ctx - ly.window - 8)
                for i, b in enumerate(seqs):
                    a[i, :, lo:cfg.ctx] = host(t[b, :, lo:cfg.ctx])
            else:
                a = np.ascontiguousarray(np.stack([host(t[b]) for b in seqs]))
            ent[nm] = a
        out.append(ent)
    return out


def make_drafts(model, state, last_tokens, k, match, vocab, rng):
    """Greedy continuation of each sequence (oracle, batch 1 per sequence) with each
    draft replaced by a random other token with probability 1 - match."""
    B = len(last_tokens)
    drafts = np.zeros((B, k), dtype=np.int32)
    for b in range(B):
        st = {"caches": [{"k": c["k"][b:b + 1].copy(), "v": None if c["v"] is None else c["v"][b:b + 1].copy()}
                         for c in state["caches"]],
              "L": state["L"][b:b + 1].copy()}
        cont = om.ar_greedy(model, st, int(last_tokens[b]), k)
        for i in range(k):
            if rng.random() < match:
                drafts[b, i] = cont[i]
            else:
                t = int(rng.integers(0, vocab - 1))
                drafts[b, i] = t if t < cont[i] else t + 1
    return drafts


def compare_step(vs, ref, k, B, seqs, tag):
    """Returns the per-sequence (n, y) the step must commit (oracle's on excused rows)."""
    gs = L.decode_row_stats(vs.stats)
    ga = L.decode_accept_out(vs.acc)
    commit = []
    for bi, b in enumerate(seqs):
        st = ref["stats"][bi]
        for i in range(k + 1):
            g, o = gs[b * (k + 1) + i], st[i]
            assert abs(float(g["top1"]) - o["top1"]) <= ATOL, (tag, b, i, g, o)
            assert abs(float(g["lse"]) - o["lse"]) <= ATOL, (tag, b, i, g, o)
            if not np.isnan(o["draft_logit"]):
                assert abs(float(g["draft_logit"]) - o["draft_logit"]) <= ATOL, (tag, b, i, g, o)
        n = int(ref["n"][bi])
        deciding = [st[i]["top1"] - st[i]["top2"] for i in range(n + 1)]
        if min(deciding) > MARGIN:
            assert int(ga[b]["n_accepted"]) == n, (tag, b, ga[b], n)
            assert int(ga[b]["next_token"]) == int(ref["y"][bi]), (tag, b)
            assert int(ga[b]["new_len"]) == int(ref["new_len"][bi])
            assert int(ga[b]["hidden_row"]) == b * (k + 1) + n
        commit.append((n, int(ref["y"][bi])))
    return commit


def lockstep(cfg, steps, seed=0, check_drafter=False):
    dev = need_gpu()
    B, k = cfg.batch, cfg.k
    cap = cfg.ctx + (k + 1) * (steps + 1) + 8
    say(f"[stack] {cfg.name}: d={cfg.d_model} layers={len(cfg.layers)} V={cfg.vocab} B={B} k={k} "
        f"ctx={cfg.ctx} steps={steps} seed={seed}")
    W = inputs.stack_weights(cfg, seed, dev)
    caches = inputs.stack_caches(cfg, seed, dev, capacity=cap)
    model = om.OracleModel(cfg, host_weights(W, cfg.dtype == "bf16"))
    state = om.new_state(host_caches(caches, range(B), cfg, cap), [cfg.ctx] * B)
    cl = torch.full((B,), cfg.ctx, dtype=torch.int32, device=dev)
    vs = VerifyStack(cfg, W, caches, cl, dev)
    rng = np.random.default_rng(seed)
    last = inputs.randint((B,), 0, cfg.vocab - 1, seed, "first_tokens", "cpu").numpy()
    accepted = []
    worst_h = 0.0
    for s in range(steps):
        drafts = make_drafts(model, state, last, k, cfg.draft_match, cfg.vocab, rng)
        tokens = np.concatenate([last[:, None], drafts], axis=1).astype(np.int32)
        tok_d = torch.from_numpy(tokens).to(dev)
        dr_d = torch.from_numpy(drafts).to(dev)
        old = state["L"].copy()
        ref = model.greedy_step(state, tokens)
        vs.step(tok_d, dr_d)
        torch.cuda.synchronize()
        hg = host(vs.h if cfg.norm else vs.x)
        e = rel_l2(hg, ref["h"])
        worst_h = max(worst_h, e)
        assert e <= (1e-2 if cfg.dtype == "bf16" else 1e-5), f"step {s}: final hidden rel L2 {e:.2e}"
        commit = compare_step(vs, ref, k, B, range(B), f"step {s} (final hidden rel L2 {e:.2e})")
        # lockstep: both sides continue from the oracle's decision
        new_len = np.array([old[b] + commit[b][0] + 1 for b in range(B)], dtype=np.int32)
        state["L"] = new_len.copy()
        cl.copy_(torch.from_numpy(new_len))
        last = np.array([c[1] for c in commit], dtype=np.int32)
        accepted.extend(c[0] for c in commit)
        assert int(vs.dev_status.item()) == 0
    say(f"[stack] {cfg.name}: worst final-hidden rel L2 {worst_h:.2e}; mean accepted "
        f"{np.mean(accepted):.2f} (tokens/step/seq {np.mean(accepted) + 1:.2f})")
    if check_drafter:
        drafter_reads(cfg, vs, state, seed, dev)
    return accepted


def drafter_reads(cfg, vs, state, seed, dev):
    """Read-only single-query calls (the drafter's cross-attention) on the last
    local and the last global layer caches, against the committed lengths."""
    B = cfg.batch
    for li in (max(i for i, l in enumerate(cfg.layers) if l.kind == "local"),
               max(i for i, l in enumerate(cfg.layers) if l.kind == "global")):
        ly = cfg.layers[li]
        for step in range(cfg.k):
            q = inputs.normal((B, 1, ly.n_heads_q, ly.head_dim), 1.0, seed + step, f"drafter_q{li}", dev)
            out = torch.empty_like(q)
            desc = attn_desc(ly, B, 1, vs.cap, cfg.dtype, append=False, q_pos_offset=step)
            ws = torch.empty(L.sv_verify_attn_workspace(desc), dtype=torch.uint8, device=dev)
            L.sv_verify_attn(desc, q, None, None, vs.caches[li]["k"], vs.caches[li]["v"], vs.cache_len, out, ws)
            torch.cuda.synchronize()
            G = ly.group
            qh = host(q)
            for b in range(B):
                ref = np.zeros((1, ly.n_heads_q, ly.head_dim))
                for g in range(ly.n_heads_kv):
                    kc = host(vs.caches[li]["k"][b, g])
                    vc = None if ly.k_is_v else host(vs.caches[li]["v"][b, g])
                    ref[:, g * G:(g + 1) * G] = oracle.attn_group(
                        q=qh[b, :, g * G:(g + 1) * G], k_new=None, v_new=None, k_cache=kc, v_cache=vc,
                        L=int(state["L"][b]), window=ly.window, rope_dims=ly.rope_dims, rope_base=ly.rope_base,
                        scale=ly.scale, k_is_v=ly.k_is_v, append=False, q_pos_offset=step, round_bf16=True)
                e = rel_l2(host(out[b]), ref)
                assert e <= 1e-2, (li, step, b, e)
    say(f"[stack] {cfg.name}: drafter reads of the last local / global caches ok")


@gpu
def test_tiny_f32_verify_steps():
    """One-layer fp32 model, d=128, 2q/1kv, D=64, 64-token cache, k=3, vocab 1024."""
    acc = lockstep(configs.TINY_F32, steps=8)
    assert len(acc) == 8


@gpu
def test_scaled_stack_lockstep():
    """The 6-layer 5:1 local/global stack at sizes the oracle finishes in seconds,
    16 verify steps with drafts matching the target at rate 0.8."""
    cfg = configs.scaled_stack(steps=16)
    acc = lockstep(cfg, steps=16, check_drafter=True)
    assert np.mean(acc) > 1.0        # drafts at rate 0.8 are mostly accepted


@gpu
def test_full_size_stack_step_one_sequence():
    """The full stack (d=3840, d_ff=15360, 6 layers, vocab 262,144, context 131,072,
    B=4, k=4): one verify step on the GPU, checked against the oracle on sequence 0
    (sequences are independent), with random drafts."""
    dev = need_gpu()
    cfg = configs.STACK
    B, k = cfg.batch, cfg.k
    cap = cfg.ctx + 2 * (k + 1) + 8
    say(f"[stack-full] generating weights and caches (cap={cap})")
    W = inputs.stack_weights(cfg, 0, dev)
    caches = inputs.stack_caches(cfg, 0, dev, capacity=cap, fill_from=0)
    cl = torch.full((B,), cfg.ctx, dtype=torch.int32, device=dev)
    tokens = inputs.randint((B, k + 1), 0, cfg.vocab - 1, 0, "full_tokens", dev)
    drafts = tokens[:, 1:].contiguous()
    say("[stack-full] host copies for sequence 0")
    model = om.OracleModel(cfg, host_weights(W, True))
    state = om.new_state(host_caches(caches, [0], cfg, cap, only_window=True), [cfg.ctx])
    vs = VerifyStack(cfg, W, caches, cl, dev)
    vs.step(tokens, drafts)
    torch.cuda.synchronize()
    say("[stack-full] oracle step for sequence 0")
    ref = model.greedy_step(state, tokens[:1].cpu().numpy())
    e = rel_l2(host(vs.h[:k + 1]), ref["h"])
    say(f"[stack-full] final hidden rel L2 {e:.2e}")
    assert e <= 1e-2
    compare_step(vs, ref, k, B, [0], "full")
    assert int(vs.dev_status.item()) == 0
