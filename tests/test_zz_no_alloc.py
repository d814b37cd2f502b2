"""sv_verify_attn_noalloc (the verify attention for callers that cannot allocate)
against sv_verify_attn with a caller-owned workspace.

Both run the same kernels over the same work split, so the outputs and the cache
rows each call appends must be identical bit for bit.  Two calls in a row on the
library's one static scratch array: first the global-layer attention workload
(batch 8, 32 q / 4 KV heads, head dim 512, keys reused as values, p-RoPE, cache
lengths ~ U[8192, 32768]), then a smaller sliding-window call (batch 1, 16 q / 8 KV
heads, head dim 256, window 1024, context 4096).  A descriptor that needs more
scratch than the array holds is refused with nothing launched."""
import torch

import mtp_draft_verification_amd._lib as L
from mtp_draft_verification_amd import configs, inputs
from mtp_draft_verification_amd.step import attn_desc
from gpu_util import gpu, need_gpu, say


def _compare(cfg, seed):
    dev = need_gpu()
    ly = cfg.layer
    B, nq = cfg.batch, cfg.k + 1
    a = inputs.attn_inputs(cfg, seed, dev)
    cap = a["cap"]
    say(f"[noalloc] {cfg.name} B={B} Hq={ly.n_heads_q} Hkv={ly.n_heads_kv} D={ly.head_dim} "
        f"lens={a['cache_len'].tolist()} cap={cap}")
    desc = attn_desc(ly, B, nq, cap, "bf16")
    k_ref, k_got = a["k_cache"].clone(), a["k_cache"].clone()
    v_ref = None if a["v_cache"] is None else a["v_cache"].clone()
    v_got = None if a["v_cache"] is None else a["v_cache"].clone()
    out_ref = torch.full_like(a["q"], float("nan"))
    out_got = torch.full_like(a["q"], float("nan"))
    st_ref = torch.zeros(1, dtype=torch.int32, device=dev)
    st_got = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = torch.empty(L.sv_verify_attn_workspace(desc), dtype=torch.uint8, device=dev)
    L.sv_verify_attn(desc, a["q"], a["k_new"], a["v_new"], k_ref, v_ref, a["cache_len"], out_ref, ws, st_ref)
    L.sv_verify_attn_noalloc(desc, a["q"], a["k_new"], a["v_new"], k_got, v_got, a["cache_len"], out_got, st_got)
    torch.cuda.synchronize()
    assert int(st_ref.item()) == 0 and int(st_got.item()) == 0
    assert not torch.isnan(out_got.float()).any()
    assert torch.equal(out_got, out_ref)
    assert torch.equal(k_got, k_ref)
    if v_got is not None:
        assert torch.equal(v_got, v_ref)
    say(f"[noalloc] {cfg.name} ok")


@gpu
def test_noalloc_equals_workspace_call_twice_then_smaller():
    _compare(configs.GLOBAL_ATTN, seed=11)
    _compare(configs.LOCAL_ATTN, seed=12)
    # and the large one again after the small one: nothing the small call left matters
    _compare(configs.GLOBAL_ATTN, seed=13)


@gpu
def test_noalloc_refuses_more_than_its_scratch():
    dev = need_gpu()
    ly = configs.global_layer(32, 4, 512)
    desc = attn_desc(ly, 256, 5, 1024, "bf16")          # ~ (CUs + 1024) * 40 * 514 * 4 bytes
    fake = torch.zeros(16, dtype=torch.bfloat16, device=dev)
    cl = torch.zeros(256, dtype=torch.int32, device=dev)
    try:
        L.sv_verify_attn_noalloc(desc, fake, fake, None, fake, None, cl, fake)
    except L.SvError as e:
        assert e.status == L.SV_ERR_SCRATCH
    else:
        raise AssertionError("an oversized descriptor was accepted")
