"""Seeded synthetic inputs shared by the GPU path's tests/benchmark and the oracle.

This module draws random tensors and nothing else: it holds none of the verify
step's arithmetic (no RoPE, attention, logits, softmax or acceptance).  Every
tensor has its own generator, seeded from (seed, tensor name, chunk index), so a
tensor does not change when another one is added or resized.  Values are drawn
in fp32 and rounded once to bf16 (round-to-nearest-even, torch's conversion)
for bf16 workloads; both sides then consume identical bits.

Tensors can be generated on the CPU (small workloads, CPU-only tests) or
directly on the GPU (workloads of several GB); the two devices give different
streams for the same seed, so a test always feeds the oracle host copies of the
very tensors the GPU consumed.
"""
from __future__ import annotations

import hashlib

import numpy as np
import torch

_CHUNK = 1 << 26  # elements per generator chunk (bounds the fp32 temporary)


def _seed_of(seed: int, name: str, chunk: int = 0) -> int:
    h = hashlib.sha256(f"{int(seed)}/{name}/{int(chunk)}".encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def generator(seed: int, name: str, device="cpu", chunk: int = 0) -> torch.Generator:
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(_seed_of(seed, name, chunk))
    return g


def torch_dtype(dtype: str) -> torch.dtype:
    return {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]


def normal(shape, std: float, seed: int, name: str, device="cpu", dtype: str = "bf16") -> torch.Tensor:
    """N(0, std^2) entries, drawn in fp32 chunks along the first dimension."""
    shape = tuple(int(s) for s in shape)
    out = torch.empty(shape, dtype=torch_dtype(dtype), device=device)
    if out.numel() == 0:
        return out
    flat = out.view(-1)
    n = flat.numel()
    for c, start in enumerate(range(0, n, _CHUNK)):
        m = min(_CHUNK, n - start)
        g = generator(seed, name, device, c)
        x = torch.randn(m, generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        flat[start:start + m].copy_(x)
    return out


def uniform(shape, seed: int, name: str, device="cpu") -> torch.Tensor:
    """U[0,1) fp32 entries (the random numbers a sampling step consumes)."""
    g = generator(seed, name, device)
    return torch.rand(tuple(shape), generator=g, device=device, dtype=torch.float32)


def randint(shape, lo: int, hi_inclusive: int, seed: int, name: str, device="cpu") -> torch.Tensor:
    g = generator(seed, name, device)
    return torch.randint(int(lo), int(hi_inclusive) + 1, tuple(shape), generator=g, device=device,
                         dtype=torch.int64).to(torch.int32)


def bernoulli(shape, p: float, seed: int, name: str, device="cpu") -> torch.Tensor:
    return uniform(shape, seed, name, device) < p


def dirichlet_rows(rows: int, vocab: int, alpha: float, seed: int, name: str, device="cpu") -> torch.Tensor:
    """Rows of Dirichlet(alpha) probabilities over the vocabulary, fp32 [rows, vocab]."""
    g = generator(seed, name, device)
    conc = torch.full((rows, vocab), float(alpha), dtype=torch.float32, device=device)
    x = torch._standard_gamma(conc, generator=g)
    x = x / x.sum(dim=1, keepdim=True)
    return x.to(torch.float32)


def categorical(probs: torch.Tensor, seed: int, name: str) -> torch.Tensor:
    """One draw per row of a probability matrix [rows, vocab] -> int32 [rows]."""
    g = generator(seed, name, probs.device)
    return torch.multinomial(probs, 1, replacement=True, generator=g)[:, 0].to(torch.int32)


def channel_scales(shape, std: float, seed: int, name: str, device="cpu") -> torch.Tensor:
    """Per-channel fp32 scales of an fp8 cache whose entries are about N(0, std^2):
    a 4-sigma value lands near the largest E4M3 magnitude (448), times a seeded
    per-channel factor in [0.75, 1.25)."""
    return (std * 4.0 / 448.0) * (0.75 + 0.5 * uniform(shape, seed, name, device))


def fp8_codes(shape, std: float, scales: torch.Tensor, seed: int, name: str, device="cpu") -> torch.Tensor:
    """uint8 fp8 E4M3 codes of N(0, std^2) entries divided by per-channel `scales`
    ([Hkv, D] for a [B, Hkv, cap, D] cache), clipped to +-448 and rounded to nearest
    even by torch's fp8 cast."""
    x = normal(shape, std, seed, name, device, "f32")
    s = scales.view(1, scales.shape[0], 1, scales.shape[1]) if x.dim() == 4 else scales
    x.div_(s).clamp_(-448.0, 448.0)
    return x.to(torch.float8_e4m3fn).view(torch.uint8)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Host uint16 array holding the bit patterns of a bf16 tensor."""
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def host_f32(t: torch.Tensor) -> np.ndarray:
    """Host fp32 copy (exact for bf16 and fp32 tensors)."""
    return t.detach().float().contiguous().cpu().numpy()


# --------------------------------------------------------------------------
# workload builders (shapes from configs.py)
# --------------------------------------------------------------------------

def attn_inputs(cfg, seed: int = 0, device="cpu", capacity_extra: int = 0) -> dict:
    """Inputs of one verify-attention call: committed lengths, a cache filled with
    rotated-key-like rows below them, and the pre-RoPE queries / new rows."""
    ly = cfg.layer
    B, nq = cfg.batch, cfg.k + 1
    lens = randint((B,), cfg.ctx_lo, cfg.ctx_hi, seed, "cache_len", "cpu")
    cap = int(lens.max()) + nq + capacity_extra
    dt = cfg.dtype
    k_cache = normal((B, ly.n_heads_kv, cap, ly.head_dim), cfg.std, seed, "k_cache", device, dt)
    v_cache = None if ly.k_is_v else normal((B, ly.n_heads_kv, cap, ly.head_dim), cfg.std, seed,
                                            "v_cache", device, dt)
    q = normal((B, nq, ly.n_heads_q, ly.head_dim), cfg.std, seed, "q", device, dt)
    k_new = normal((B, nq, ly.n_heads_kv, ly.head_dim), cfg.std, seed, "k_new", device, dt)
    v_new = None if ly.k_is_v else normal((B, nq, ly.n_heads_kv, ly.head_dim), cfg.std, seed,
                                          "v_new", device, dt)
    return dict(cache_len=lens.to(device), cap=cap, k_cache=k_cache, v_cache=v_cache, q=q,
                k_new=k_new, v_new=v_new)


def stack_weights(cfg, seed: int = 0, device="cpu") -> dict:
    """Random-init weights of a decoder stack, N(0, 1/fan_in) entries.

    Per layer: wqkv [Hq*D + Hkv*D (+ Hkv*D for V), d] (q, k, v projections stacked
    along the output dimension), wo [d, Hq*D], and with an MLP wgu [2*d_ff, d]
    (gate projection rows, then up projection rows) and wd [d, d_ff].  The
    embedding table E [vocab, d] is tied to the LM head."""
    dt = cfg.dtype
    d = cfg.d_model
    W = {"E": normal((cfg.vocab, d), d ** -0.5, seed, "E", device, dt), "layers": []}
    for i, ly in enumerate(cfg.layers):
        nq = ly.n_heads_q * ly.head_dim
        nk = ly.n_heads_kv * ly.head_dim
        nout = nq + nk + (0 if ly.k_is_v else nk)
        lw = {"wqkv": normal((nout, d), d ** -0.5, seed, f"L{i}.wqkv", device, dt),
              "wo": normal((d, nq), nq ** -0.5, seed, f"L{i}.wo", device, dt)}
        if cfg.d_ff:
            lw["wgu"] = normal((2 * cfg.d_ff, d), d ** -0.5, seed, f"L{i}.wgu", device, dt)
            lw["wd"] = normal((d, cfg.d_ff), cfg.d_ff ** -0.5, seed, f"L{i}.wd", device, dt)
        W["layers"].append(lw)
    return W


def drafter_weights(target, dcfg, seed: int = 0, device="cpu") -> dict:
    """Random-init drafter weights, N(0, 1/fan_in) entries: its embedder E [vocab,
    d_draft]; w_down [d_draft, d_model + d_draft] over [target activation, token
    embedding]; per block wq [Hq*D, d_draft], wo [d_draft, Hq*D] (the heads of the
    target layer it reads), wgu [2*d_ff, d_draft] (gate rows, then up rows), wd
    [d_draft, d_ff]; w_up [d_model, d_draft]."""
    dt = target.dtype
    d, dd, dff = target.d_model, dcfg.d_draft, dcfg.d_ff
    W = {"E": normal((target.vocab, dd), dd ** -0.5, seed, "D.E", device, dt),
         "w_down": normal((dd, d + dd), (d + dd) ** -0.5, seed, "D.w_down", device, dt),
         "w_up": normal((d, dd), dd ** -0.5, seed, "D.w_up", device, dt), "blocks": []}
    for j, ti in enumerate(dcfg.target_layers(target)):
        ly = target.layers[ti]
        nq = ly.n_heads_q * ly.head_dim
        W["blocks"].append({"wq": normal((nq, dd), dd ** -0.5, seed, f"D{j}.wq", device, dt),
                            "wo": normal((dd, nq), nq ** -0.5, seed, f"D{j}.wo", device, dt),
                            "wgu": normal((2 * dff, dd), dd ** -0.5, seed, f"D{j}.wgu", device, dt),
                            "wd": normal((dd, dff), dff ** -0.5, seed, f"D{j}.wd", device, dt)})
    return W


def clustered_unembedding(vocab: int, d: int, n_clusters: int, seed: int = 0, device="cpu",
                           dtype: str = "bf16", center_std: float | None = None,
                           spread: float = 0.5) -> dict:
    """A vocabulary with cluster structure, for the clustered unembedding.

    perm: a seeded random permutation of the token ids (int32 [V]); cluster c owns
    the V / C consecutive rows [c V / C, (c + 1) V / C) of w_perm, row j holding
    token perm[j].  Each cluster has a centre drawn N(0, center_std^2) (default
    1/sqrt(d)); its rows are the centre plus N(0, (spread * center_std)^2) noise.
    centroids are the centres.  E is the same unembedding in token order
    (E[perm[j]] = w_perm[j]), for comparisons against the full vocabulary."""
    assert vocab % n_clusters == 0
    std = d ** -0.5 if center_std is None else float(center_std)
    csize = vocab // n_clusters
    g = generator(seed, "C.perm", device)
    perm = torch.randperm(vocab, generator=g, device=device).to(torch.int32)
    centers = normal((n_clusters, d), std, seed, "C.centers", device, "f32")
    w = normal((vocab, d), std * spread, seed, "C.noise", device, "f32")
    w.view(n_clusters, csize, d).add_(centers.view(n_clusters, 1, d))
    w_perm = w.to(torch_dtype(dtype))
    del w
    E = torch.empty_like(w_perm)
    E[perm.long()] = w_perm
    return {"perm": perm, "w_perm": w_perm, "centroids": centers.to(torch_dtype(dtype)), "E": E}


def clusters_of(E: torch.Tensor, n_clusters: int, top: int, seed: int = 0) -> dict:
    """A clustering of an existing unembedding E [V, d] for the clustered unembed:
    a seeded random permutation cut into n_clusters equal clusters, w_perm = E[perm]
    and, standing in for trained centroids, the mean of each cluster's rows."""
    V, d = E.shape
    assert V % n_clusters == 0
    g = generator(seed, "C.perm", E.device)
    perm = torch.randperm(V, generator=g, device=E.device).to(torch.int32)
    w_perm = E[perm.long()].contiguous()
    cent = w_perm.view(n_clusters, V // n_clusters, d).float().mean(dim=1).to(E.dtype)
    return {"perm": perm, "w_perm": w_perm, "centroids": cent, "top": int(top)}


def stack_caches(cfg, seed: int = 0, device="cpu", capacity: int | None = None,
                 fill_from: int | None = None) -> list:
    """Per layer: k [B, Hkv, cap, D] (and v unless K = V), rows [fill_lo, ctx) ~ N(0,1),
    all other rows zero.  fill_from=None fills every committed row; a sliding-window
    layer reads only its last `window` rows, so large workloads fill only those."""
    B = cfg.batch
    cap = capacity if capacity is not None else cfg.ctx + (cfg.k + 1) * max(cfg.steps, 1) + 8
    dt = cfg.dtype
    caches = []
    for i, ly in enumerate(cfg.layers):
        lo = 0
        if fill_from is not None:
            lo = fill_from if ly.window == 0 else max(0, cfg.ctx - ly.window - 8)
        shape = (B, ly.n_heads_kv, cap, ly.head_dim)
        ent = {}
        for nm in (("k",) if ly.k_is_v else ("k", "v")):
            t = torch.zeros(shape, dtype=torch_dtype(dt), device=device)
            if cfg.ctx > lo:
                t[:, :, lo:cfg.ctx, :] = normal((B, ly.n_heads_kv, cfg.ctx - lo, ly.head_dim), 1.0,
                                                seed, f"L{i}.cache_{nm}", device, dt)
            ent[nm] = t
        ent["v"] = ent.get("v")
        caches.append(ent)
    return caches
