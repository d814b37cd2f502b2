"""GPU parity of sv_verify_attn_fp8 (verify attention over an fp8 E4M3 KV cache
with per-channel scales) against the oracle.

The oracle reads the same codes through the same scales (oracle.dequant_cache)
and quantizes its appended rows the same way.  Tolerance: relative L2 per
sequence <= 1e-2, as for bf16 caches (the GPU folds the key scales into the
queries with one bf16 rounding; products of codes are exact).  Appended value
codes must equal the oracle's; appended key codes may differ by one code step,
since the bf16 rotated key may differ by one bf16 ulp (fp32 against fp64 RoPE)
before quantization.  Every other cache byte must be left untouched."""
import numpy as np
import pytest
import torch

import oracle
import mtp_draft_verification_amd._lib as L
from mtp_draft_verification_amd import configs, inputs
from mtp_draft_verification_amd.step import attn_desc
from gpu_util import gpu, host, need_gpu, rel_l2, say

TOL = 1e-2


def e4m3_step(x):
    """Quantum of the E4M3 grid at magnitude |x| (2^-9 below the normal range)."""
    a = np.maximum(np.abs(x), 2.0 ** -6)
    return 2.0 ** (np.floor(np.log2(a)) - 3)


def run_case(layer, B, nq, lens, cap, seed, std=1.0, append=True, qoff=0, check_groups=None, tag=""):
    dev = need_gpu()
    say(f"[attn-fp8] {tag} D={layer.head_dim} Hq={layer.n_heads_q} Hkv={layer.n_heads_kv} W={layer.window} "
        f"B={B} nq={nq} lens={list(lens)[:8]} cap={cap} append={append} qoff={qoff} seed={seed}")
    Hq, Hkv, D = layer.n_heads_q, layer.n_heads_kv, layer.head_dim
    ks = inputs.channel_scales((Hkv, D), std, seed, "ks", dev)
    vs = None if layer.k_is_v else inputs.channel_scales((Hkv, D), std, seed, "vs", dev)
    kc = inputs.fp8_codes((B, Hkv, cap, D), std, ks, seed, "kc8", dev)
    vc = None if layer.k_is_v else inputs.fp8_codes((B, Hkv, cap, D), std, vs, seed, "vc8", dev)
    q = inputs.normal((B, nq, Hq, D), std, seed, "q", dev)
    kn = inputs.normal((B, nq, Hkv, D), std, seed, "kn", dev) if append else None
    vn = inputs.normal((B, nq, Hkv, D), std, seed, "vn", dev) if (append and not layer.k_is_v) else None
    cl = torch.tensor(list(lens), dtype=torch.int32, device=dev)
    kc0 = kc.clone()
    vc0 = None if vc is None else vc.clone()
    out = torch.full((B, nq, Hq, D), float("nan"), dtype=torch.bfloat16, device=dev)
    desc = attn_desc(layer, B, nq, cap, "bf16", append=append, q_pos_offset=qoff)
    ws = torch.empty(L.sv_verify_attn_workspace(desc), dtype=torch.uint8, device=dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    L.sv_verify_attn_fp8(desc, q, kn, vn, kc, vc, ks, vs, cl, out, ws, st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    G = Hq // Hkv
    groups = check_groups if check_groups is not None else [(b, g) for b in range(B) for g in range(Hkv)]
    qh = host(q)
    knh = None if kn is None else host(kn)
    vnh = None if vn is None else host(vn)
    ksh = ks.cpu().numpy()
    vsh = None if vs is None else vs.cpu().numpy()
    outh = host(out)
    per_seq = {}
    n_key, n_key_exact = 0, 0
    for (b, g) in groups:
        kcg = oracle.dequant_cache(kc0[b, g].cpu().numpy(), ksh[g])
        vcg = None if vc0 is None else oracle.dequant_cache(vc0[b, g].cpu().numpy(), vsh[g])
        o = oracle.attn_group(q=qh[b, :, g * G:(g + 1) * G], k_new=None if knh is None else knh[b, :, g],
                              v_new=None if vnh is None else vnh[b, :, g], k_cache=kcg, v_cache=vcg,
                              L=int(lens[b]), window=layer.window, rope_dims=layer.rope_dims,
                              rope_base=layer.rope_base, scale=layer.scale, k_is_v=layer.k_is_v,
                              append=append, q_pos_offset=qoff, round_bf16=True, k_scale=ksh[g],
                              v_scale=None if vsh is None else vsh[g])
        per_seq.setdefault(b, ([], []))
        per_seq[b][0].append(outh[b, :, g * G:(g + 1) * G])
        per_seq[b][1].append(o)
        if append:
            Lb = int(lens[b])
            got = oracle.dequant_cache(kc[b, g, Lb:Lb + nq].cpu().numpy(), ksh[g]).astype(np.float64)
            ref = kcg[Lb:Lb + nq].astype(np.float64)
            exact = got == ref
            n_key += got.size
            n_key_exact += int(exact.sum())
            step = e4m3_step(ref / ksh[g]) * ksh[g]
            assert np.all(np.abs(got - ref) <= step * 1.0001), f"appended key codes differ by more than a step (b={b}, g={g})"
            if vc is not None:
                gv = oracle.dequant_cache(vc[b, g, Lb:Lb + nq].cpu().numpy(), vsh[g])
                np.testing.assert_array_equal(gv, vcg[Lb:Lb + nq])
    if n_key:
        assert n_key_exact >= 0.99 * n_key, f"only {n_key_exact} of {n_key} appended key codes equal"
    worst = 0.0
    for b, (gs, os_) in per_seq.items():
        e = rel_l2(np.stack(gs), np.stack(os_))
        worst = max(worst, e)
        assert e <= TOL, f"sequence {b}: rel L2 {e:.3e}"
    for b in range(B):
        Lb = int(lens[b])
        n_new = nq if append else 0
        for t, t0 in ((kc, kc0), (vc, vc0)):
            if t is None:
                continue
            assert torch.equal(t[b, :, :Lb], t0[b, :, :Lb])
            assert torch.equal(t[b, :, Lb + n_new:], t0[b, :, Lb + n_new:])
    say(f"[attn-fp8] {tag} ok worst rel L2 {worst:.2e}, appended key codes equal {n_key_exact}/{n_key}")
    return worst


@gpu
def test_fp8_local_window_small_ragged():
    ly = configs.local_layer(16, 8, 256, 100)
    run_case(ly, 3, 5, [0, 37, 333], 400, 1, std=1 / 16, tag="local-small")


@gpu
def test_fp8_global_kv_same_small_ragged():
    ly = configs.global_layer(32, 4, 512)
    run_case(ly, 4, 5, [1, 70, 129, 1000], 1100, 2, tag="global-small")


@gpu
@pytest.mark.parametrize("D", [128, 256, 512])
def test_fp8_head_dims_and_row_tiles(D):
    for (hq, hkv, nq) in ((4, 4, 5), (8, 2, 5), (16, 2, 5), (16, 2, 8)):
        ly = configs.AttnLayer("global", hq, hkv, D, 0, D // 4, 1e6, True)
        run_case(ly, 2, nq, [45, 300], 320, 3, tag=f"tiles-{D}-{hq}/{hkv}x{nq}")
        if D == 512:
            continue
        ly = configs.AttnLayer("local", hq, hkv, D, 77, D, 1e4, False)
        run_case(ly, 2, nq, [45, 300], 320, 4, tag=f"tiles-local-{D}-{hq}/{hkv}x{nq}")


@gpu
def test_fp8_many_sequences_work_split():
    ly = configs.AttnLayer("local", 8, 4, 128, 40, 128, 1e4, False)
    lens = inputs.randint((70,), 0, 300, 13, "lens", "cpu").tolist()
    lens[3] = 0
    lens[66] = 0
    run_case(ly, 70, 3, lens, 310, 13, std=0.2, tag="many-seqs")


@gpu
def test_fp8_two_workgroups_per_cu_work_split():
    """512-dim heads with one row tile (2 q heads per KV head x 5 rows) run two workgroups
    per compute unit, so the keys are cut into twice as many pieces: fewer segments than
    pieces (70 x 4) and more (150 x 4, one piece per segment), ragged and empty
    sequences, with appends."""
    ly = configs.global_layer(8, 4, 512)
    for B, seed in ((70, 21), (150, 22)):
        lens = inputs.randint((B,), 0, 600, seed, "lens", "cpu").tolist()
        lens[1] = 0
        run_case(ly, B, 5, lens, 610, seed, std=0.5, tag=f"two-per-cu-B{B}")


@gpu
def test_fp8_read_only_drafter_queries():
    ly = configs.global_layer(16, 4, 512)
    run_case(ly, 3, 1, [50, 0, 777], 800, 5, append=False, qoff=0, tag="read-only-global")
    ly = configs.local_layer(16, 8, 256, 64)
    run_case(ly, 2, 1, [500, 31], 600, 6, append=False, qoff=2, std=1 / 16, tag="read-only-local")


@gpu
def test_fp8_full_size_global_config():
    """The global workload at full size over an fp8 cache; all 32 (sequence, KV head)
    groups recomputed by the oracle."""
    cfg = configs.GLOBAL_ATTN
    lens = inputs.randint((cfg.batch,), cfg.ctx_lo, cfg.ctx_hi, 0, "cache_len", "cpu").tolist()
    cap = max(lens) + cfg.k + 1
    run_case(cfg.layer, cfg.batch, cfg.k + 1, lens, cap, 0, std=cfg.std, tag="global-full")
