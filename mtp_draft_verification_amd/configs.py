"""Workload geometry of the verify step: shapes and constants only, no arithmetic.

Architecture facts come from the pages:
  * alternating sliding-window (local) and global attention layers, p-RoPE and
    key-equals-value on global layers: "Gemma 4 发布时未包含 MTP 数据——为什么这很重要"
    (flowhunt), section "什么是 Gemma 4？"; "Gemma 4 拆解" (marsggbo), section 2
    (p = 0.25, value reuses key on global layers, 262k vocabulary);
  * k drafts plus one bonus position verified in one target pass: "Gemma 4 拆解",
    section 4.2; "Accelerating Gemma 4 ..." (Lighthouse), section 3.
The concrete sizes (heads, head dims, window, context, batch, k) are the five
synthetic workloads the library is measured on.
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class AttnLayer:
    kind: str              # "local" (sliding window) or "global"
    n_heads_q: int
    n_heads_kv: int
    head_dim: int
    window: int            # 0 for global layers
    rope_dims: int         # 0: none, head_dim: full RoPE, head_dim/4: p-RoPE p=0.25
    rope_base: float
    k_is_v: bool           # global layers store one tensor used as key and value

    @property
    def group(self) -> int:
        return self.n_heads_q // self.n_heads_kv

    @property
    def scale(self) -> float:
        return self.head_dim ** -0.5


def local_layer(hq=16, hkv=8, d=256, window=1024, base=1.0e4) -> AttnLayer:
    return AttnLayer("local", hq, hkv, d, window, d, base, False)


def global_layer(hq=16, hkv=4, d=512, base=1.0e6) -> AttnLayer:
    return AttnLayer("global", hq, hkv, d, 0, d // 4, base, True)


@dataclass(frozen=True)
class StackConfig:
    """A decoder stack verified k drafts at a time (embedding tied to the LM head)."""
    name: str
    d_model: int
    vocab: int
    layers: tuple
    d_ff: int              # 0: no MLP block
    norm: bool             # pre-norm RMSNorm before attention / MLP and a final norm
    eps: float
    dtype: str             # "f32" or "bf16"
    batch: int
    k: int
    ctx: int               # committed cache length before the first verify step
    steps: int = 1
    draft_match: float = 0.8


@dataclass(frozen=True)
class AttnConfig:
    """A single verify-attention call."""
    name: str
    layer: AttnLayer
    batch: int
    k: int
    ctx_lo: int            # committed length drawn uniformly from [ctx_lo, ctx_hi]
    ctx_hi: int
    std: float             # standard deviation of q, k, v entries
    dtype: str = "bf16"


@dataclass(frozen=True)
class LMHeadConfig:
    name: str
    d_model: int
    vocab: int
    batch: int
    k: int
    draft_match: float = 0.8
    dirichlet_alpha: float = 0.1
    dtype: str = "bf16"

    @property
    def rows(self) -> int:
        return self.batch * (self.k + 1)


# 1. tiny fp32 verify step: one attention layer (2 q heads / 1 kv head, head dim 64,
#    no RoPE, no norm, no MLP), cache of 64 tokens, k = 3, vocab 1024.
TINY_F32 = StackConfig(
    name="tiny_f32_verify", d_model=128, vocab=1024,
    layers=(AttnLayer("global", 2, 1, 64, 0, 0, 1.0e4, False),),
    d_ff=0, norm=False, eps=1e-6, dtype="f32", batch=1, k=3, ctx=64, steps=1,
    draft_match=0.7)

# 2. sliding-window verify attention, bf16: 16q/8kv, head dim 256, cache 4096,
#    window 1024, full RoPE, batch 1, k = 4; entries ~ N(0,1)/sqrt(head_dim).
LOCAL_ATTN = AttnConfig(
    name="local_attn_verify", layer=local_layer(16, 8, 256, 1024), batch=1, k=4,
    ctx_lo=4096, ctx_hi=4096, std=256 ** -0.5)

# 3. global verify attention, bf16: 32q/4kv, head dim 512, K = V, p-RoPE on 128
#    dims with base 1e6, committed lengths ~ U[8192, 32768], batch 8, k = 4.
GLOBAL_ATTN = AttnConfig(
    name="global_attn_verify", layer=global_layer(32, 4, 512), batch=8, k=4,
    ctx_lo=8192, ctx_hi=32768, std=1.0)

# 4. LM-head select over a 262,144-token vocabulary, d = 3840, k = 4,
#    batch 1 or 8, greedy and rejection-sampling modes.
LMHEAD_B1 = LMHeadConfig(name="lmhead_select_b1", d_model=3840, vocab=262144, batch=1, k=4)
LMHEAD_B8 = LMHeadConfig(name="lmhead_select_b8", d_model=3840, vocab=262144, batch=8, k=4)

# 5. full verify step of a synthetic 6-layer stack (5 local : 1 global),
#    d = 3840, d_ff = 15360 GeGLU, RMSNorm, context 131,072, batch 4, k = 4.
STACK = StackConfig(
    name="stack_verify", d_model=3840, vocab=262144,
    layers=(local_layer(),) * 5 + (global_layer(),),
    d_ff=15360, norm=True, eps=1e-6, dtype="bf16", batch=4, k=4, ctx=131072, steps=64,
    draft_match=0.8)


def scaled_stack(base: StackConfig = STACK, *, name: str = "stack_small", d_model=256,
                 vocab=4096, d_ff=512, ctx=2048, batch=2, k=4, steps=16, window=64,
                 local_heads=(4, 2, 128), global_heads=(4, 1, 256)) -> StackConfig:
    """The same layer pattern at sizes the oracle finishes in seconds."""
    hq, hkv, d = local_heads
    gq, gkv, gd = global_heads
    layers = tuple(local_layer(hq, hkv, d, window) if L.kind == "local" else global_layer(gq, gkv, gd)
                   for L in base.layers)
    return StackConfig(name=name, d_model=d_model, vocab=vocab, layers=layers, d_ff=d_ff,
                       norm=base.norm, eps=base.eps, dtype=base.dtype, batch=batch, k=k,
                       ctx=ctx, steps=steps, draft_match=base.draft_match)


@dataclass(frozen=True)
class DrafterConfig:
    """An MTP drafter that cross-attends the target's caches ("Gemma 4 拆解"
    (marsggbo), section 4.2): its own embedder and width d_draft, the target's last
    activation and the token embedding concatenated and projected down, blocks of
    cross-attention into the target's last local (or global) layer cache plus a
    GeGLU MLP, a projection back up to d_model, and the target's unembedding.
    `blocks` names, per drafter block, the kind of target layer whose cache it
    reads; its query heads match that layer (same heads, head dim, RoPE)."""
    name: str
    d_draft: int
    d_ff: int
    blocks: tuple = ("local", "local", "local", "global")
    eps: float = 1e-6

    def target_layers(self, target: StackConfig) -> list:
        """Index of the target layer each block attends: the last of its kind."""
        last = {}
        for i, ly in enumerate(target.layers):
            last[ly.kind] = i
        return [last[kind] for kind in self.blocks]


# 3 local + 1 global blocks at the larger drafter width the pages give (1024)
DRAFTER = DrafterConfig(name="drafter_1024", d_draft=1024, d_ff=4096)


def scaled_drafter(name: str = "drafter_small", d_draft=128, d_ff=256) -> DrafterConfig:
    return DrafterConfig(name=name, d_draft=d_draft, d_ff=d_ff)
