"""A verify step captured in a HIP graph (VerifyStack.capture) against the same steps run
eagerly: every replay must give bit for bit the eager step's tokens, accept records,
committed lengths, final hidden states and appended cache rows.  Replays are separated
by eager work and synchronisations, and each is checked on its own."""
import torch

from mtp_draft_verification_amd import configs, inputs
from mtp_draft_verification_amd.step import VerifyStack
from gpu_util import gpu, need_gpu, say


@gpu
def test_graph_replay_matches_eager():
    dev = need_gpu()
    cfg = configs.scaled_stack(steps=4)
    B, k, steps, seed = cfg.batch, cfg.k, 5, 5
    cap = cfg.ctx + (k + 1) * (steps + 1) + 8
    say(f"[graph] {cfg.name}: B={B} k={k} ctx={cfg.ctx} steps={steps} seed={seed}")
    W = inputs.stack_weights(cfg, seed, dev)
    caches = inputs.stack_caches(cfg, seed, dev, capacity=cap)
    start = [{n: (None if t is None else t.clone()) for n, t in c.items()} for c in caches]
    cl = torch.full((B,), cfg.ctx, dtype=torch.int32, device=dev)
    vs = VerifyStack(cfg, W, caches, cl, dev)
    toks = [inputs.randint((B, k + 1), 0, cfg.vocab - 1, seed + s, "graph_tokens", dev) for s in range(steps)]
    drs = [t[:, 1:].contiguous() for t in toks]

    def snap():
        return [vs.out_tokens.clone(), vs.acc.clone(), cl.clone(), vs.h.clone()]

    def reset():
        cl.fill_(cfg.ctx)
        for c, c0 in zip(caches, start):
            for n, t in c.items():
                if t is not None:
                    t.copy_(c0[n])
        torch.cuda.synchronize()

    eager = []
    for s in range(steps):
        vs.step(toks[s], drs[s])
        torch.cuda.synchronize()
        eager.append(snap())
    eager_caches = [{n: (None if t is None else t.clone()) for n, t in c.items()} for c in caches]

    reset()
    tok_buf = torch.empty_like(toks[0])
    dr_buf = torch.empty_like(drs[0])
    g = vs.capture(tok_buf, dr_buf)
    torch.cuda.synchronize()
    # capturing records the launches without running them
    assert torch.equal(cl, torch.full_like(cl, cfg.ctx))
    for s in range(steps):
        tok_buf.copy_(toks[s])
        dr_buf.copy_(drs[s])
        g.replay()
        torch.cuda.synchronize()
        got = snap()
        for name, a, b in zip(("out_tokens", "acc", "cache_len", "hidden"), got, eager[s]):
            assert torch.equal(a, b), f"replay {s}: {name} differs from the eager step"
        # eager work of the program's own between replays
        float(vs.h.float().abs().sum())
        torch.cuda.synchronize()
    for li, (c, ce) in enumerate(zip(caches, eager_caches)):
        for n, t in c.items():
            if t is not None:
                assert torch.equal(t, ce[n]), f"layer {li} cache {n} differs after the replays"
    say(f"[graph] {steps} replays equal the eager steps (tokens, accept records, lengths, "
        f"hidden states, caches)")
