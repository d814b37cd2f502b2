"""The C-ABI library loads, exports every symbol the header declares, and
rejects bad arguments on the host (no GPU needed: nothing is launched)."""
import ctypes
import os
import re

import pytest

import mtp_draft_verification_amd._lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    src = open(os.path.join(ROOT, "include", "specverify.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sv_\w+)\s*\(", src)))


def test_header_symbols_are_exported():
    lib = L.load()
    syms = declared_symbols()
    assert len(syms) >= 12
    for s in syms:
        assert hasattr(lib, s), s
    assert set(syms) == set(L.EXPORTS)


def test_version_and_status_strings():
    assert "gfx950" in L.sv_version()
    for st in (L.SV_OK, L.SV_ERR_ARG, L.SV_ERR_UNSUPPORTED, L.SV_ERR_WORKSPACE, L.SV_ERR_LAUNCH,
               L.SV_ERR_DEVICE):
        assert L.sv_status_string(st).startswith("SV_")


def _desc(**kw):
    base = dict(batch=2, n_q=5, n_heads_q=16, n_heads_kv=8, head_dim=256, window=1024, rope_dims=256,
                k_is_v=0, append=1, q_pos_offset=0, dtype=L.SV_BF16, in_splits=0, rope_base=1e4,
                softmax_scale=1 / 16, reserved_f=0.0, cache_capacity=5000, q_row_stride=0, kv_row_stride=0)
    base.update(kw)
    return L.AttnDesc(**base)


def test_attention_descriptor_validation():
    lib = L.load()
    fake = ctypes.c_void_p(4096)
    big = 1 << 40

    def call(d, **ptrs):
        p = dict(q=fake, kn=fake, vn=fake, kc=fake, vc=fake, cl=fake, out=fake, ws=fake)
        p.update(ptrs)
        return lib.sv_verify_attn(ctypes.byref(d), p["q"], p["kn"], p["vn"], p["kc"], p["vc"], p["cl"],
                                  p["out"], p["ws"], big, None, None)

    assert L.sv_verify_attn_workspace(_desc()) > 0
    bad = [dict(batch=0), dict(n_q=0), dict(n_heads_q=12, n_heads_kv=8), dict(head_dim=200, rope_dims=200),
           dict(rope_dims=300), dict(rope_dims=7), dict(window=-1), dict(k_is_v=2), dict(append=1, q_pos_offset=3),
           dict(in_splits=-1), dict(in_splits=2, dtype=L.SV_F32), dict(cache_capacity=0), dict(softmax_scale=0.0), dict(dtype=7),
           dict(q_row_stride=100), dict(rope_base=0.5)]
    for kw in bad:
        assert call(_desc(**kw)) in (L.SV_ERR_ARG, L.SV_ERR_UNSUPPORTED), kw
        assert L.sv_verify_attn_workspace(_desc(**kw)) == 0, kw
    assert call(_desc(head_dim=64, rope_dims=64)) == L.SV_ERR_UNSUPPORTED      # no bf16 kernel for D=64
    assert call(_desc(head_dim=512, rope_dims=128)) == L.SV_ERR_UNSUPPORTED    # D=512 needs K = V
    assert call(_desc(n_q=9, n_heads_q=64, n_heads_kv=8)) == L.SV_ERR_UNSUPPORTED  # 72 rows > 64
    assert call(_desc(), q=None) == L.SV_ERR_ARG
    assert call(_desc(), vn=None) == L.SV_ERR_ARG                            # V needed on local layers
    assert call(_desc(k_is_v=1)) == L.SV_ERR_ARG                             # V given on a K=V layer
    assert call(_desc(append=0)) == L.SV_ERR_ARG                             # new rows given read-only
    assert call(_desc(), ws=None) == L.SV_ERR_WORKSPACE
    d = _desc()
    small = L.sv_verify_attn_workspace(d) - 1
    assert lib.sv_verify_attn(ctypes.byref(d), fake, fake, fake, fake, fake, fake, fake, fake, small,
                              None, None) == L.SV_ERR_WORKSPACE
    assert call(_desc(dtype=L.SV_F32, cache_capacity=100000)) == L.SV_ERR_UNSUPPORTED


def test_other_entry_points_reject_bad_arguments():
    lib = L.load()
    fake = ctypes.c_void_p(4096)
    lm = L.LMHeadDesc(batch=8, k=4, d_model=3840, vocab=262144, mode=L.SV_SELECT_GREEDY, dtype=L.SV_BF16)
    assert L.sv_lmhead_workspace(lm) > 0
    for kw in (dict(vocab=1000), dict(d_model=100), dict(batch=16), dict(mode=9), dict(batch=0)):
        d = L.LMHeadDesc(**{**dict(batch=8, k=4, d_model=3840, vocab=262144, mode=0, dtype=1), **kw})
        assert lib.sv_lmhead_select(ctypes.byref(d), fake, fake, fake, None, None, fake, None, None, fake,
                                    1 << 40, None) in (L.SV_ERR_ARG, L.SV_ERR_UNSUPPORTED), kw
    samp = L.LMHeadDesc(batch=8, k=4, d_model=3840, vocab=262144, mode=L.SV_SELECT_SAMPLE, dtype=L.SV_BF16)
    assert lib.sv_lmhead_select(ctypes.byref(samp), fake, fake, fake, None, None, fake, None, None, fake,
                                1 << 40, None) == L.SV_ERR_ARG            # no uniforms
    assert lib.sv_lmhead_select(ctypes.byref(lm), fake, fake, fake, None, None, fake, None, None, fake,
                                16, None) == L.SV_ERR_WORKSPACE
    ad = L.AcceptDesc(batch=4, k=4, vocab=1000, mode=L.SV_SELECT_SAMPLE)
    assert lib.sv_accept(ctypes.byref(ad), fake, fake, None, None, fake, fake, fake, None, None) == L.SV_ERR_ARG
    ld = L.LinearDesc(rows=20, in_features=3840, out_features=100, dtype=L.SV_BF16, epilogue=0)
    assert lib.sv_linear(ctypes.byref(ld), fake, fake, fake, fake, 1 << 40, None) == L.SV_ERR_ARG
    ld = L.LinearDesc(rows=80, in_features=3840, out_features=128, dtype=L.SV_BF16, epilogue=0)
    assert lib.sv_linear(ctypes.byref(ld), fake, fake, fake, fake, 1 << 40, None) == L.SV_ERR_UNSUPPORTED
    assert lib.sv_embed(0, 128, 10, L.SV_BF16, fake, fake, 1.0, fake, None, None) == L.SV_ERR_ARG
    assert lib.sv_rmsnorm(4, 128, -1.0, fake, None, fake, L.SV_BF16, None) == L.SV_ERR_ARG
    assert lib.sv_geglu(4, 128, 5, fake, fake, None) == L.SV_ERR_ARG
    for pair in (-1, 3):
        ld = L.LinearDesc(rows=20, in_features=3840, out_features=128, dtype=L.SV_BF16, epilogue=0, act_pair=pair)
        assert lib.sv_linear(ctypes.byref(ld), fake, fake, fake, fake, 1 << 40, None) == L.SV_ERR_ARG
    for cat_dtype in (L.SV_F32, 7):
        assert lib.sv_draft_input(4, 3840, 1024, 1e-6, fake, 40, fake, 1, fake, 1000, fake, 1, 32.0, fake,
                                  cat_dtype, fake, None, None) == L.SV_ERR_ARG


def test_tiled_weights_sizes_and_validation():
    lib = L.load()
    fake = ctypes.c_void_p(4096)
    base = dict(rows=40, in_features=3840, out_features=30720, dtype=L.SV_BF16, epilogue=L.SV_EPI_GEGLU,
                act_pair=1)
    # GeGLU and K-split use two 64-feature tiles per wave (blocks of 128 features)
    assert L.sv_linear_tiled_bytes(L.LinearDesc(**base)) == 240 * 60 * 128 * 128
    split = dict(base, in_features=4096 + 32, out_features=704, epilogue=L.SV_EPI_SPLIT_F32)
    assert L.sv_linear_tiled_bytes(L.LinearDesc(**split)) == 6 * 65 * 128 * 128   # ragged N and K padded
    small = dict(base, in_features=96, out_features=192, epilogue=L.SV_EPI_STORE)
    assert L.sv_linear_tiled_bytes(L.LinearDesc(**small)) == 3 * 2 * 64 * 128       # one tile per wave
    assert L.sv_linear_tiled_bytes(L.LinearDesc(**dict(base, dtype=L.SV_F32, act_pair=0,
                                                         epilogue=L.SV_EPI_STORE))) == 0
    for bad in (dict(w_layout=2), dict(w_layout=-1), dict(w_layout=L.SV_W_TILED, dtype=L.SV_F32, act_pair=0,
                                                        epilogue=L.SV_EPI_STORE)):
        d = L.LinearDesc(**{**base, **bad})
        assert lib.sv_linear(ctypes.byref(d), fake, fake, fake, fake, 1 << 40, None) == L.SV_ERR_ARG, bad
    d = L.LinearDesc(**base)
    assert lib.sv_linear_tile_weights(ctypes.byref(d), None, fake, None) == L.SV_ERR_ARG
    assert lib.sv_linear_tile_weights(ctypes.byref(d), fake, None, None) == L.SV_ERR_ARG
    assert lib.sv_linear_tile_weights(ctypes.byref(d), ctypes.c_void_p(4104), fake, None) == L.SV_ERR_ARG
    d32 = L.LinearDesc(**dict(base, dtype=L.SV_F32, act_pair=0, epilogue=L.SV_EPI_STORE))
    assert lib.sv_linear_tile_weights(ctypes.byref(d32), fake, fake, None) == L.SV_ERR_ARG
    dt = L.LinearDesc(**dict(base, w_layout=L.SV_W_TILED))
    assert lib.sv_linear(ctypes.byref(dt), fake, ctypes.c_void_p(4104), fake, fake, 1 << 40, None) == L.SV_ERR_ARG


def test_cluster_unembed_rejects_bad_arguments():
    lib = L.load()
    fake = ctypes.c_void_p(4096)
    base = dict(rows=8, d_model=2560, vocab=262144, n_clusters=2048, top_clusters=32, dtype=L.SV_BF16)
    assert L.sv_cluster_unembed_workspace(L.ClusterDesc(**base)) > 0

    def call(d, hidden=fake, ws_bytes=1 << 40, out_stride=1):
        return lib.sv_cluster_unembed(ctypes.byref(d), hidden, fake, fake, fake, fake, None, None, out_stride,
                                      fake, ws_bytes, None)

    for kw, want in ((dict(rows=0), L.SV_ERR_ARG), (dict(d_model=100), L.SV_ERR_ARG),
                     (dict(vocab=1000), L.SV_ERR_ARG), (dict(top_clusters=0), L.SV_ERR_ARG),
                     (dict(n_clusters=16, top_clusters=17, vocab=4096), L.SV_ERR_ARG),
                     (dict(dtype=L.SV_F32), L.SV_ERR_ARG), (dict(rows=65), L.SV_ERR_UNSUPPORTED),
                     (dict(n_clusters=8192, vocab=8192 * 32), L.SV_ERR_UNSUPPORTED),
                     (dict(top_clusters=65), L.SV_ERR_UNSUPPORTED)):
        d = L.ClusterDesc(**{**base, **kw})
        assert call(d) == want, kw
        assert L.sv_cluster_unembed_workspace(d) == 0, kw
    d = L.ClusterDesc(**base)
    assert call(d, hidden=ctypes.c_void_p(4096 + 8)) == L.SV_ERR_ARG      # misaligned rows
    assert call(d, hidden=None) == L.SV_ERR_ARG
    assert call(d, out_stride=-1) == L.SV_ERR_ARG
    assert call(d, ws_bytes=L.sv_cluster_unembed_workspace(d) - 1) == L.SV_ERR_WORKSPACE


def test_fp8_attention_and_single_pass_sampling_reject_bad_arguments():
    lib = L.load()
    fake = ctypes.c_void_p(4096)
    big = 1 << 40

    def fp8(d, ks=fake, vs=fake, **ptrs):
        p = dict(q=fake, kn=fake, vn=fake, kc=fake, vc=fake, cl=fake, out=fake, ws=fake)
        p.update(ptrs)
        return lib.sv_verify_attn_fp8(ctypes.byref(d), p["q"], p["kn"], p["vn"], p["kc"], p["vc"], ks, vs, p["cl"],
                                      p["out"], p["ws"], big, None, None)

    assert fp8(_desc(dtype=L.SV_F32, cache_capacity=1000)) == L.SV_ERR_ARG      # fp8 caches need bf16 rows
    assert fp8(_desc(), ks=None) == L.SV_ERR_ARG                                  # key scales missing
    assert fp8(_desc(), ks=ctypes.c_void_p(4096 + 4)) == L.SV_ERR_ARG             # misaligned scales
    assert fp8(_desc(), vs=None) == L.SV_ERR_ARG                                  # value scales missing (K != V)
    gl = _desc(k_is_v=1, head_dim=512, rope_dims=128)
    assert fp8(gl, vn=None, vc=None) == L.SV_ERR_ARG                              # K = V takes no value scales
    assert fp8(_desc(batch=0)) == L.SV_ERR_ARG

    rs = L.LMHeadDesc(batch=8, k=4, d_model=3840, vocab=262144, mode=L.SV_SELECT_SAMPLE_RS, dtype=L.SV_BF16)
    assert L.sv_lmhead_workspace(rs) > L.sv_lmhead_workspace(
        L.LMHeadDesc(batch=8, k=4, d_model=3840, vocab=262144, mode=L.SV_SELECT_SAMPLE, dtype=L.SV_BF16))
    # the RS mode only through its own entry point, and the entry point only in RS mode
    assert lib.sv_lmhead_select(ctypes.byref(rs), fake, fake, fake, fake, None, fake, None, None, fake, big,
                                None) == L.SV_ERR_ARG
    smp = L.LMHeadDesc(batch=8, k=4, d_model=3840, vocab=262144, mode=L.SV_SELECT_SAMPLE, dtype=L.SV_BF16)
    assert lib.sv_lmhead_select_rs(ctypes.byref(smp), fake, fake, fake, fake, 1, 2, fake, fake, None, fake, big,
                                   None) == L.SV_ERR_ARG
    assert lib.sv_lmhead_select_rs(ctypes.byref(rs), fake, fake, fake, fake, 1, 2, fake, None, None, fake, big,
                                   None) == L.SV_ERR_ARG                             # candidates missing
    f32 = L.LMHeadDesc(batch=2, k=4, d_model=64, vocab=1024, mode=L.SV_SELECT_SAMPLE_RS, dtype=L.SV_F32)
    assert L.sv_lmhead_workspace(f32) == 0                                          # bf16 only
    ad = L.AcceptDesc(batch=4, k=4, vocab=1000, mode=L.SV_SELECT_SAMPLE_RS)
    assert lib.sv_accept(ctypes.byref(ad), fake, fake, fake, fake, fake, fake, fake, None, None) == L.SV_ERR_ARG
    assert lib.sv_accept_rs(ctypes.byref(ad), fake, fake, None, fake, fake, fake, fake, fake, fake, None,
                            None) == L.SV_ERR_ARG                                   # candidates missing
    ad2 = L.AcceptDesc(batch=4, k=4, vocab=1000, mode=L.SV_SELECT_SAMPLE)
    assert lib.sv_accept_rs(ctypes.byref(ad2), fake, fake, fake, fake, fake, fake, fake, fake, fake, None,
                            None) == L.SV_ERR_ARG                                   # wrong mode


def test_valid_call_without_gpu_reports_device_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    lib = L.load()
    fake = ctypes.c_void_p(4096)
    d = _desc()
    assert lib.sv_verify_attn(ctypes.byref(d), fake, fake, fake, fake, fake, fake, fake, fake, 1 << 40,
                              None, None) == L.SV_ERR_DEVICE
