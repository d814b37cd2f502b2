"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

None of these re-types the oracle's formulas: each checks a closed form, an
invariant, a special case that reduces to a library routine, or a statistical
property, chosen so that a plausible slip in the oracle (a dropped term, a wrong
sign or index, a transposed operand, an off-by-one mask) fails at least one.
"""
import math

import numpy as np
import pytest
import torch
from scipy import special, stats

import oracle
from oracle import model as om
from mtp_draft_verification_amd import configs, inputs


# ---------------------------------------------------------------------------
# bf16 storage rounding
# ---------------------------------------------------------------------------

def test_bf16_round_halfway_cases():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties go to the even significand.
    assert oracle.bf16_round([1 + 2 ** -8])[0] == 1.0
    assert oracle.bf16_round([1 + 3 * 2 ** -8])[0] == 1 + 2 ** -6
    assert oracle.bf16_round([-(1 + 3 * 2 ** -8)])[0] == -(1 + 2 ** -6)
    assert oracle.bf16_round([1 + 2 ** -8 + 2 ** -20])[0] == 1 + 2 ** -7
    # largest finite bf16 and overflow
    assert oracle.bf16_round([3.3895313892515355e38])[0] == 3.3895313892515355e38
    assert np.isinf(oracle.bf16_round([3.4e38])[0])


def test_bf16_round_matches_torch_conversion():
    g = torch.Generator().manual_seed(3)
    x = torch.randn(20000, generator=g) * torch.exp(torch.randn(20000, generator=g) * 8)
    ref = x.to(torch.bfloat16).double().numpy()
    got = oracle.bf16_round(x.double().numpy())
    np.testing.assert_array_equal(got, ref)


# ---------------------------------------------------------------------------
# RoPE / p-RoPE
# ---------------------------------------------------------------------------

def test_rope_pairing_and_frequency_closed_form():
    # rope_dims = 4, base 1e4: pair (0, 2) turns at rate 1, pair (1, 3) at rate 1e4^(-1/2).
    e1 = np.zeros(6); e1[1] = 1.0
    y = oracle.rope(e1, 4, 1.0e4, 100.0)           # angle 100 * 0.01 = 1 rad
    np.testing.assert_allclose(y, [0, math.cos(1.0), 0, math.sin(1.0), 0, 0], atol=1e-13)
    e0 = np.zeros(6); e0[0] = 1.0
    y = oracle.rope(e0, 4, 1.0e4, 0.5)              # angle 0.5 rad on pair (0, 2)
    np.testing.assert_allclose(y, [math.cos(0.5), 0, math.sin(0.5), 0, 0, 0], atol=1e-15)
    e2 = np.zeros(6); e2[2] = 1.0                   # second half turns towards -first half
    y = oracle.rope(e2, 4, 1.0e4, 0.5)
    np.testing.assert_allclose(y, [-math.sin(0.5), 0, math.cos(0.5), 0, 0, 0], atol=1e-15)


def test_rope_invariants():
    rng = np.random.default_rng(0)
    for D, r, base in [(256, 256, 1e4), (512, 128, 1e6), (64, 0, 1e4)]:
        x = rng.standard_normal(D)
        y = oracle.rope(x, r, base, 12345.0)
        assert abs(np.linalg.norm(y) - np.linalg.norm(x)) < 1e-12 * np.linalg.norm(x)
        np.testing.assert_array_equal(y[r:], x[r:])            # p-RoPE leaves the tail alone
        np.testing.assert_array_equal(oracle.rope(x, r, base, 0.0), x)
        # rotations compose: R(p1) R(p2) = R(p1 + p2)
        np.testing.assert_allclose(oracle.rope(oracle.rope(x, r, base, 300.0), r, base, 77.0),
                                   oracle.rope(x, r, base, 377.0), atol=1e-11)
        # relative position: <R(m) q, R(n) k> depends on m - n only
        q, k = rng.standard_normal(D), rng.standard_normal(D)
        a = oracle.rope(q, r, base, 1000.0) @ oracle.rope(k, r, base, 990.0)
        b = oracle.rope(q, r, base, 131000.0) @ oracle.rope(k, r, base, 130990.0)
        assert abs(a - b) < 1e-9 * (1 + abs(a))


# ---------------------------------------------------------------------------
# verify attention
# ---------------------------------------------------------------------------

def _attn_case(rng, B=2, nq=3, Hq=4, Hkv=2, D=16, L=(7, 11), cap=24, k_is_v=False):
    q = rng.standard_normal((B, nq, Hq, D)).astype(np.float32)
    kn = rng.standard_normal((B, nq, Hkv, D)).astype(np.float32)
    vn = None if k_is_v else rng.standard_normal((B, nq, Hkv, D)).astype(np.float32)
    kc = rng.standard_normal((B, Hkv, cap, D)).astype(np.float32)
    vc = None if k_is_v else rng.standard_normal((B, Hkv, cap, D)).astype(np.float32)
    return q, kn, vn, kc, vc, np.array(L, dtype=np.int32)


def _run(q, kn, vn, kc, vc, L, **kw):
    kc = kc.copy()
    vc = None if vc is None else vc.copy()
    base = dict(window=0, rope_dims=0, rope_base=1e4, scale=0.25, k_is_v=vc is None,
                round_bf16=False)
    base.update(kw)
    out = oracle.verify_attn(q=q, k_new=kn, v_new=vn, k_cache=kc, v_cache=vc, cache_len=L, **base)
    return out, kc, vc


def test_attn_single_visible_key_returns_its_value():
    rng = np.random.default_rng(1)
    q, kn, vn, kc, vc, L = _attn_case(rng)
    out, kc2, _ = _run(q, kn, vn, kc, vc, L, window=1)          # each row sees only itself
    for b in range(2):
        for j in range(3):
            for h in range(4):
                np.testing.assert_array_equal(out[b, j, h], vn[b, j, h // 2].astype(np.float64))
    # K = V with RoPE: the output is the stored (rotated, bf16-rounded) key of the row
    q, kn, _, kc, _, L = _attn_case(rng, k_is_v=True)
    out, kc2, _ = _run(q, kn, None, kc, None, L, window=1, rope_dims=8, round_bf16=True)
    for b in range(2):
        for j in range(3):
            row = kc2[b, 0, L[b] + j].astype(np.float64)
            np.testing.assert_array_equal(out[b, j, 0], row)
            assert np.all(oracle.bf16_round(row) == row)


def test_attn_identical_keys_give_mean_of_visible_values():
    rng = np.random.default_rng(2)
    q, kn, vn, kc, vc, L = _attn_case(rng, B=1, L=(9,), cap=16)
    kc[:] = kc[0, 0, 0]
    kn[:] = kc[0, 0, 0]
    out, _, vc2 = _run(q, kn, vn, kc, vc, L)
    for j in range(3):
        for h in range(4):
            g = h // 2
            ref = vc2[0, g, :L[0] + j + 1].astype(np.float64).mean(axis=0)
            np.testing.assert_allclose(out[0, j, h], ref, rtol=1e-12, atol=1e-13)


def test_attn_two_keys_sigmoid_closed_form():
    rng = np.random.default_rng(3)
    D = 8
    q = rng.standard_normal((1, 1, 1, D)).astype(np.float32)
    kn = rng.standard_normal((1, 1, 1, D)).astype(np.float32)
    vn = rng.standard_normal((1, 1, 1, D)).astype(np.float32)
    kc = rng.standard_normal((1, 1, 4, D)).astype(np.float32)
    vc = rng.standard_normal((1, 1, 4, D)).astype(np.float32)
    scale = 1 / math.sqrt(D)
    out, _, _ = _run(q, kn, vn, kc, vc, np.array([1], np.int32), scale=scale)
    s0 = scale * float(q[0, 0, 0].astype(np.float64) @ kc[0, 0, 0].astype(np.float64))
    s1 = scale * float(q[0, 0, 0].astype(np.float64) @ kn[0, 0, 0].astype(np.float64))
    w0 = special.expit(s0 - s1)
    ref = w0 * vc[0, 0, 0].astype(np.float64) + (1 - w0) * vn[0, 0, 0].astype(np.float64)
    np.testing.assert_allclose(out[0, 0, 0], ref, rtol=1e-12, atol=1e-14)


def test_attn_wide_window_equals_global():
    rng = np.random.default_rng(4)
    args = _attn_case(rng, L=(7, 11))
    g, _, _ = _run(*args, window=0, rope_dims=16)
    w, _, _ = _run(*args, window=11 + 3 + 1, rope_dims=16)
    np.testing.assert_array_equal(g, w)


def test_attn_gqa_equals_mha_with_repeated_kv():
    rng = np.random.default_rng(5)
    q, kn, vn, kc, vc, L = _attn_case(rng, Hq=6, Hkv=2)
    gqa, _, _ = _run(q, kn, vn, kc, vc, L, rope_dims=16, window=5)
    rep = lambda a, ax: np.repeat(a, 3, axis=ax)
    mha, _, _ = _run(q, rep(kn, 2), rep(vn, 2), rep(kc, 1), rep(vc, 1), L, rope_dims=16, window=5)
    np.testing.assert_array_equal(gqa, mha)


def test_attn_permuting_committed_rows_leaves_global_output():
    rng = np.random.default_rng(6)
    q, kn, vn, kc, vc, L = _attn_case(rng, L=(10, 10))
    a, _, _ = _run(q, kn, vn, kc, vc, L, rope_dims=16)
    perm = rng.permutation(10)
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[:, :, :10] = kc[:, :, perm]
    vc2[:, :, :10] = vc[:, :, perm]
    b, _, _ = _run(q, kn, vn, kc2, vc2, L, rope_dims=16)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


def test_attn_causality_and_window_boundary():
    rng = np.random.default_rng(7)
    q, kn, vn, kc, vc, L = _attn_case(rng, L=(12, 12))
    base, _, _ = _run(q, kn, vn, kc, vc, L, window=6, rope_dims=16)
    # later new rows never influence earlier rows
    kn2, vn2 = kn.copy(), vn.copy()
    kn2[:, 2] += 5.0
    vn2[:, 2] -= 3.0
    o, _, _ = _run(q, kn2, vn2, kc, vc, L, window=6, rope_dims=16)
    np.testing.assert_array_equal(o[:, :2], base[:, :2])
    assert np.abs(o[:, 2] - base[:, 2]).max() > 1e-3
    # row j at position p = 12 + j sees exactly keys p-5 .. p
    for j in range(3):
        p = 12 + j
        kc_out, vc_out = kc.copy(), vc.copy()
        vc_out[:, :, p - 6] += 10.0           # just outside the window
        o, _, _ = _run(q, kn, vn, kc_out, vc_out, L, window=6, rope_dims=16)
        np.testing.assert_array_equal(o[:, j], base[:, j])
        if p - 5 < 12:                          # first visible key is a committed row
            vc_in = vc.copy()
            vc_in[:, :, p - 5] += 10.0
            o, _, _ = _run(q, kn, vn, kc, vc_in, L, window=6, rope_dims=16)
            assert np.abs(o[:, j] - base[:, j]).max() > 1e-6


def test_attn_value_shift_and_scale_equivariance():
    rng = np.random.default_rng(8)
    q, kn, vn, kc, vc, L = _attn_case(rng)
    a, _, _ = _run(q, kn, vn, kc, vc, L, window=4, rope_dims=8)
    c = rng.standard_normal(16).astype(np.float32)
    b, _, _ = _run(q, kn, vn + c, kc, vc + c, L, window=4, rope_dims=8)
    np.testing.assert_allclose(b, a + c.astype(np.float64), rtol=1e-6, atol=1e-5)
    b2, _, _ = _run(q, kn, 2 * vn, kc, 2 * vc, L, window=4, rope_dims=8)
    np.testing.assert_allclose(b2, 2 * a, rtol=1e-12, atol=1e-12)


def test_attn_read_only_query_matches_verify_row():
    """A read-only query at position L against the cache after the append sees the
    same keys as verify row 0 (which sees the committed rows plus its own)."""
    rng = np.random.default_rng(9)
    q, kn, vn, kc, vc, L = _attn_case(rng, nq=1, L=(8, 13))
    o_verify, kc2, vc2 = _run(q, kn, vn, kc, vc, L, window=5, rope_dims=16)
    o_read, _, _ = _run(q, None, None, kc2, vc2, L + 1, window=5, rope_dims=16, append=False,
                        q_pos_offset=-1)
    np.testing.assert_array_equal(o_read, o_verify)


def test_attn_capacity_overflow_raises():
    rng = np.random.default_rng(10)
    q, kn, vn, kc, vc, _ = _attn_case(rng, cap=12)
    with pytest.raises(ValueError):
        _run(q, kn, vn, kc, vc, np.array([5, 10], np.int32))


# ---------------------------------------------------------------------------
# LM head and row statistics
# ---------------------------------------------------------------------------

def test_lmhead_equals_matmul_and_stats_equal_library_routines():
    rng = np.random.default_rng(11)
    h = rng.standard_normal((5, 64))
    W = rng.standard_normal((300, 64)).astype(np.float32)
    z = oracle.lmhead(h, W)
    np.testing.assert_allclose(z, h @ W.astype(np.float64).T, rtol=1e-12, atol=1e-12)
    Wb = torch.from_numpy(W).to(torch.bfloat16)
    zb = oracle.lmhead(h, inputs.bf16_bits(Wb))
    np.testing.assert_allclose(zb, h @ Wb.double().numpy().T, rtol=1e-12, atol=1e-12)
    for r in range(5):
        st = oracle.row_stats(z[r], draft_id=17)
        order = np.argsort(-z[r], kind="stable")
        assert st["top1_id"] == order[0] and st["top2_id"] == order[1]
        assert st["top1"] == z[r, order[0]] and st["top2"] == z[r, order[1]]
        assert abs(st["lse"] - special.logsumexp(z[r])) < 1e-12
        assert st["draft_logit"] == z[r, 17]
    assert math.isnan(oracle.row_stats(z[0], -1)["draft_logit"])


def test_row_stats_ties_go_to_lowest_id():
    z = np.array([0.5, 2.0, -1.0, 2.0, 2.0, 1.0])
    st = oracle.row_stats(z)
    assert (st["top1_id"], st["top2_id"]) == (1, 3)
    W = np.random.default_rng(12).standard_normal((8, 16)).astype(np.float32)
    W[6] = W[2]                                   # duplicate vocabulary rows
    h = W[2:3].astype(np.float64)                 # makes rows 2 and 6 the argmax
    st = oracle.row_stats(oracle.lmhead(h, W)[0])
    assert (st["top1_id"], st["top2_id"]) == (2, 6)


def test_lse_is_stable_for_large_logits():
    z = np.array([1000.0, 999.0, -1000.0])
    st = oracle.row_stats(z)
    assert abs(st["lse"] - (1000.0 + math.log1p(math.exp(-1.0)))) < 1e-12


def test_cluster_unembed_keeping_every_cluster_is_the_full_vocabulary():
    # With every cluster kept, the candidates are the whole vocabulary: the result
    # must be the plain argmax / logsumexp over E in token order, whatever perm is.
    V, C, d = 96, 8, 32
    cu = inputs.clustered_unembedding(V, d, C, seed=3, dtype="f32")
    h = np.random.default_rng(13).standard_normal((4, d))
    E = cu["E"].double().numpy()
    res = oracle.cluster_unembed(h, cu["centroids"].numpy(), cu["w_perm"].numpy(), cu["perm"].numpy(), top=C)
    for r in range(4):
        z = h[r] @ E.T
        order = np.argsort(-z, kind="stable")
        assert (res[r]["top1_id"], res[r]["top2_id"]) == (order[0], order[1])
        assert abs(res[r]["top1"] - z[order[0]]) < 1e-12 and abs(res[r]["lse"] - special.logsumexp(z)) < 1e-12
        sc = h[r] @ cu["centroids"].double().numpy().T
        assert list(res[r]["clusters"]) == list(np.argsort(-sc, kind="stable"))


def test_cluster_unembed_restricts_to_kept_clusters_and_maps_ids():
    # Three clusters of two tokens, centroids on the axes.  h scores cluster 1
    # highest, but the largest logit overall belongs to a token of cluster 0: with
    # one cluster kept the answer is cluster 1's best token, named by perm.
    cent = np.array([[1, 0, 0, 0], [0, 1, 0, 0], [0, 0, 1, 0]], dtype=np.float32)
    w_perm = np.array([[8, 0, 0, 0], [0, 0, 0, 1],        # cluster 0: rows 0, 1
                       [0, 2, 0, 0], [0, 3, 0, 0],        # cluster 1: rows 2, 3
                       [0, 0, 1, 0], [0, 0, 0, 0]], dtype=np.float32)
    perm = np.array([5, 0, 3, 1, 4, 2], dtype=np.int32)
    h = np.array([[0.5, 1.0, 0.0, 0.0]])
    r = oracle.cluster_unembed(h, cent, w_perm, perm, top=1)[0]
    assert r["clusters"] == [1]
    assert (r["top1_id"], r["top2_id"]) == (1, 3)          # rows 3 then 2
    assert (r["top1"], r["top2"]) == (3.0, 2.0)
    assert abs(r["lse"] - special.logsumexp([2.0, 3.0])) < 1e-12
    r2 = oracle.cluster_unembed(h, cent, w_perm, perm, top=2)[0]
    assert r2["clusters"] == [1, 0] and (r2["top1_id"], r2["top1"]) == (5, 4.0)
    # equal cluster scores: the lower cluster index is kept; equal logits: lower token id
    h = np.array([[1.0, 1.0, 0.0, 0.0]])
    w_tie = w_perm.copy()
    w_tie[0] = [0, 0, 0, 0]                                # cluster 0 logits 0, 0
    r3 = oracle.cluster_unembed(h, cent, w_tie, perm, top=1)[0]
    assert r3["clusters"] == [0] and (r3["top1_id"], r3["top2_id"]) == (0, 5)


# ---------------------------------------------------------------------------
# fp8 E4M3 cache codes
# ---------------------------------------------------------------------------

def test_e4m3_decode_fixed_points_of_the_format():
    # OCP E4M3FN: largest finite 448 (S.1111.110), smallest normal 2^-6, smallest
    # subnormal 2^-9, 1.0 = 0.0111.000, NaN at S.1111.111 and no infinity
    d = oracle.e4m3_decode(np.arange(256))
    assert d[0x7E] == 448.0 and d[0xFE] == -448.0
    assert d[0x08] == 2.0 ** -6 and d[0x01] == 2.0 ** -9 and d[0x38] == 1.0 and d[0x39] == 1.125
    assert np.isnan(d[0x7F]) and np.isnan(d[0xFF]) and np.isfinite(np.delete(d, [0x7F, 0xFF])).all()
    assert (np.diff(d[:0x7F]) > 0).all()                        # magnitudes increase with the code
    np.testing.assert_array_equal(d[0x80:0xFF], -d[:0x7F])
    # the library's fp8 type agrees on every finite code
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    fin = np.isfinite(d)
    np.testing.assert_array_equal(d[fin], lib[fin])


def test_e4m3_encode_round_to_nearest_even_and_saturation():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    np.testing.assert_array_equal(oracle.e4m3_encode(oracle.e4m3_decode(codes)), codes)
    # exact midpoints go to the even code, including across a binade and into zero
    mids = np.array([1.0625, 1.1875, 1.9375, 2.0 ** -10, 3 * 2.0 ** -10, 432.0], dtype=np.float32)
    np.testing.assert_array_equal(oracle.e4m3_encode(mids), [0x38, 0x3A, 0x40, 0x00, 0x02, 0x7E])
    # beyond the largest finite value: saturate, never NaN
    np.testing.assert_array_equal(oracle.e4m3_encode([449.0, 1e30, -5000.0]), [0x7E, 0x7E, 0xFE])
    # random in-range values: the library's round-to-nearest-even cast
    x = (np.random.default_rng(21).standard_normal(4000) * 60).clip(-448, 448).astype(np.float32)
    lib = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(oracle.e4m3_encode(x), lib)


def test_attn_quantized_append_stores_scaled_codes():
    # appended rows of an fp8 cache = scale * e4m3(bf16 row / scale); checked against
    # the unquantized append of the same rows and the library's fp8 cast
    rng = np.random.default_rng(22)
    D, cap, L, nq = 64, 40, 30, 3
    q = rng.standard_normal((nq, 2, D)).astype(np.float32)
    kn = rng.standard_normal((nq, D)).astype(np.float32)
    vn = rng.standard_normal((nq, D)).astype(np.float32)
    ks = (0.01 + 0.02 * rng.random(D)).astype(np.float32)
    vs = (0.01 + 0.02 * rng.random(D)).astype(np.float32)
    kc = np.zeros((cap, D), np.float32); vc = np.zeros((cap, D), np.float32)
    args = dict(L=L, window=0, rope_dims=D, rope_base=1e4, scale=0.125, k_is_v=False, append=True,
                round_bf16=True)
    oracle.attn_group(q=q, k_new=kn, v_new=vn, k_cache=kc, v_cache=vc, **args)
    kq = np.zeros_like(kc); vq = np.zeros_like(vc)
    o = oracle.attn_group(q=q, k_new=kn, v_new=vn, k_cache=kq, v_cache=vq, k_scale=ks, v_scale=vs, **args)

    def lib_q(x, s):
        c = torch.from_numpy((x / s).astype(np.float32)).to(torch.float8_e4m3fn)
        return (c.double().numpy() * s.astype(np.float64)).astype(np.float32)
    np.testing.assert_array_equal(kq[L:L + nq], lib_q(kc[L:L + nq], ks))
    np.testing.assert_array_equal(vq[L:L + nq], lib_q(vc[L:L + nq], vs))
    # and the output is plain attention over the stored (dequantized) rows
    kq2, vq2 = kq.copy(), vq.copy()
    o2 = oracle.attn_group(q=q, k_new=None, v_new=None, k_cache=kq2, v_cache=vq2,
                           **{**args, "append": False, "L": L + nq, "q_pos_offset": -nq})
    np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# greedy acceptance
# ---------------------------------------------------------------------------

def test_accept_greedy_all_right_all_wrong_first_mismatch():
    top1 = np.array([5, 6, 7, 8, 9])
    n, t = oracle.accept_greedy([5, 6, 7, 8], top1)          # all right: k accepted, k+1 tokens
    assert n == 4 and list(t) == [5, 6, 7, 8, 9]
    n, t = oracle.accept_greedy([1, 6, 7, 8], top1)          # first wrong: 0 accepted
    assert n == 0 and list(t) == [5, -1, -1, -1, -1]
    n, t = oracle.accept_greedy([5, 6, 0, 8], top1)          # truncated at the first mismatch
    assert n == 2 and list(t) == [5, 6, 7, -1, -1]
    n, t = oracle.accept_greedy([], np.array([3]))           # k = 0 is plain decoding
    assert n == 0 and list(t) == [3]


def _tiny_stack(dtype="bf16", seed=0):
    cfg = configs.StackConfig(
        name="tiny_stack", d_model=32, vocab=97,
        layers=(configs.local_layer(4, 2, 8, 5), configs.global_layer(4, 1, 16)),
        d_ff=48, norm=True, eps=1e-6, dtype=dtype, batch=1, k=4, ctx=9, steps=1)
    return cfg


def _host_model(cfg, seed=0):
    W = inputs.stack_weights(cfg, seed)
    conv = (inputs.bf16_bits if cfg.dtype == "bf16" else inputs.host_f32)
    host = {"E": conv(W["E"]), "layers": [{k: conv(v) for k, v in lw.items()} for lw in W["layers"]]}
    caches = inputs.stack_caches(cfg, seed, capacity=cfg.ctx + 400)
    hc = [{"k": inputs.host_f32(c["k"]), "v": None if c["v"] is None else inputs.host_f32(c["v"])}
          for c in caches]
    return om.OracleModel(cfg, host), om.new_state(hc, [cfg.ctx] * cfg.batch)


@pytest.mark.parametrize("which", ["tiny_f32", "stack_bf16", "stack_f32"])
def test_spec_greedy_equals_ar_greedy(which):
    """Greedy speculative decoding emits exactly the autoregressive greedy stream,
    whatever the drafter proposes ("Gemma 4 拆解", section 4.2: only drafts the
    target agrees with are kept; every emitted token is the target's argmax)."""
    if which == "tiny_f32":
        cfg = configs.TINY_F32
        cfg = configs.StackConfig(**{**cfg.__dict__, "vocab": 97})
    else:
        cfg = _tiny_stack("bf16" if which == "stack_bf16" else "f32")
    model, st0 = _host_model(cfg)
    N = 256 if which != "stack_f32" else 96
    ref = om.ar_greedy(model, om.clone_state(st0), 3, N)
    k = cfg.k
    rng = np.random.default_rng(13)

    def random_drafter(hist, k):
        return rng.integers(0, cfg.vocab, k)

    def const_drafter(hist, k):
        return [0] * k

    def oracle_drafter(hist, k):
        n = len(hist) - 1
        return (ref + [0] * k)[n:n + k]

    def noisy_drafter(hist, k):
        good = oracle_drafter(hist, k)
        return [g if rng.random() < 0.7 else int(rng.integers(0, cfg.vocab)) for g in good]

    for drafter in (random_drafter, const_drafter, oracle_drafter, noisy_drafter):
        got, acc = om.spec_greedy(model, om.clone_state(st0), 3, N, k, drafter)
        assert got == ref, drafter.__name__
        if drafter is oracle_drafter:
            # every draft right: k accepted and k + 1 tokens per target pass
            assert all(a == k for a in acc[:-1])


def test_batch_rows_are_independent():
    cfg = _tiny_stack("bf16")
    cfg2 = configs.StackConfig(**{**cfg.__dict__, "batch": 2})
    model, st = _host_model(cfg2)
    toks = np.array([[3, 5, 8, 13, 21], [1, 2, 3, 4, 5]])
    single = om.clone_state(st)
    single["caches"] = [{"k": c["k"][:1].copy(), "v": None if c["v"] is None else c["v"][:1].copy()}
                        for c in st["caches"]]
    single["L"] = st["L"][:1].copy()
    r2 = model.greedy_step(om.clone_state(st), toks)
    r1 = model.greedy_step(single, toks[:1])
    np.testing.assert_array_equal(r2["z"][:5], r1["z"])


# ---------------------------------------------------------------------------
# rejection sampling
# ---------------------------------------------------------------------------

def _toy_pq(V=16, seed=0):
    rng = np.random.default_rng(seed)
    z = rng.standard_normal(V) * 1.5
    q = rng.dirichlet(np.full(V, 0.7))
    return z, q.astype(np.float32)


def _draws(q, shape, rng):
    cdf = np.cumsum(q.astype(np.float64))
    cdf /= cdf[-1]
    return np.minimum(np.searchsorted(cdf, rng.random(shape), side="right"), q.size - 1)


@pytest.mark.parametrize("k", [1, 4])
def test_rejection_sampling_reproduces_target_distribution(k):
    """Chi-square over 10^6 seeded trials on a vocab-16 toy: every emitted token is
    distributed as the target's softmax p ("Gemma 4 与 Gemini Nano" (kongchang),
    section "草稿模型": speculative decoding leaves the output distribution unchanged)."""
    V, T = 16, 1_000_000
    z, q = _toy_pq(V)
    p = special.softmax(z)
    rng = np.random.default_rng(100 + k)
    drafts = _draws(q, (T, k), rng).astype(np.int32)
    u_acc = rng.random((T, k), dtype=np.float32)
    u_tok = rng.random((T, V), dtype=np.float32)
    n, y = oracle.toy_spec_trials(z, q, drafts, u_acc, u_tok)
    # first emitted token of every step: d_1 if accepted, else the target's own draw
    first = np.where(n >= 1, drafts[:, 0], y)
    cnt = np.bincount(first, minlength=V)
    chi2, pval = stats.chisquare(cnt, T * p)
    assert pval > 0.01, (chi2, pval)
    # the whole emitted stream (accepted drafts, then the target's token) is iid p
    idx = np.arange(k)[None, :] < n[:, None]
    stream = np.concatenate([drafts[idx], y])
    cnt = np.bincount(stream, minlength=V)
    chi2, pval = stats.chisquare(cnt, cnt.sum() * p)
    assert pval > 0.01, (chi2, pval)
    # acceptance rate of the first draft equals sum_v min(p_v, q_v)
    rate = (n >= 1).mean()
    expect = np.minimum(p, q.astype(np.float64)).sum()
    assert abs(rate - expect) < 5 * math.sqrt(expect * (1 - expect) / T)


def test_philox4x32_known_answers():
    # the known-answer vectors published with the generator's reference
    # implementation (Random123, Salmon et al. SC 2011) for Philox4x32-10
    kat = [((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
           ((0xFFFFFFFF,) * 4, (0xFFFFFFFF,) * 2, (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
           ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
            (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1))]
    for ctr, key, want in kat:
        np.testing.assert_array_equal(oracle.philox4x32(ctr, key), np.array(want, dtype=np.uint32))


def test_rs_uniform_layout():
    # token v of draft row (b, i): word r of block (v, i, b, 0); ((x >> 9) + 1/2) 2^-23
    key = (0x1234, 0xABCD)
    for (b, i, v, r) in ((0, 0, 0, 0), (3, 2, 7, 1), (1, 3, 262143, 2), (5, 0, 1000, 3)):
        x = int(oracle.philox4x32((v, i, b, 0), key)[r])
        assert oracle.rs_uniform(key, b, i, v, r) == ((x >> 9) + 0.5) * 2.0 ** -23
    # uniforms are open-interval and fill [0, 1) evenly
    u = np.array([oracle.rs_uniform(key, 0, 0, v, r) for v in range(2000) for r in range(4)])
    assert u.min() > 0 and u.max() < 1
    assert stats.kstest(u, "uniform").pvalue > 0.001


def test_rs_candidates_are_draws_from_p():
    """Each candidate is an exact draw from softmax(z): chi-square over many keys,
    per candidate slot, and the four slots of one key are independent draws."""
    V = 8
    z = np.array([1.0, 0.2, -0.5, 2.0, 0.0, -1.5, 0.7, 1.2])
    p = special.softmax(z)
    T = 20000
    cands = np.array([oracle.rs_candidates(z, (7 + t, 99), 0, 1, 4)[0] for t in range(T)])
    for r in range(4):
        cnt = np.bincount(cands[:, r], minlength=V)
        chi2, pval = stats.chisquare(cnt, T * p)
        assert pval > 0.001, (r, chi2, pval)
    same = (cands[:, 0] == cands[:, 1]).mean()
    assert abs(same - (p ** 2).sum()) < 5 * math.sqrt((p ** 2).sum() / T)


@pytest.mark.parametrize("k", [1, 4])
def test_single_pass_sampling_reproduces_target_distribution(k):
    """Residual by rejection over first-pass candidates, with the direct residual draw
    as fallback, emits exactly p: chi-square on a vocab-16 toy; the fallback rate is
    (1 - alpha)^R with alpha = sum_v max(0, p_v - q_v)."""
    V, T, R = 16, 200_000, 4
    z, q = _toy_pq(V)
    p = special.softmax(z)
    rng = np.random.default_rng(200 + k)
    drafts = _draws(q, (T, k), rng).astype(np.int32)
    u_acc = rng.random((T, k), dtype=np.float32)
    u_tok = rng.random((T, V), dtype=np.float32)
    u_rs = rng.random((T, R), dtype=np.float32)
    n, y, fb = oracle.toy_spec_trials_rs(z, q, drafts, u_acc, u_tok, (1000 * k, 5), u_rs)
    first = np.where(n >= 1, drafts[:, 0], y)
    cnt = np.bincount(first, minlength=V)
    chi2, pval = stats.chisquare(cnt, T * p)
    assert pval > 0.01, (chi2, pval)
    # the target's own token after a rejection follows the residual max(p - q, 0)
    res = np.maximum(p - q.astype(np.float64), 0.0)
    res /= res.sum()
    rej = n < k
    cnt = np.bincount(y[rej], minlength=V)
    keep = res > 0
    assert cnt[~keep].sum() == 0
    chi2, pval = stats.chisquare(cnt[keep], rej.sum() * res[keep])
    assert pval > 0.01, (chi2, pval)
    alpha = np.maximum(p - q.astype(np.float64), 0.0).sum()
    rate = fb[rej].mean()
    expect = (1 - alpha) ** R
    assert abs(rate - expect) < 5 * math.sqrt(expect * (1 - expect) / rej.sum())


def test_sampling_special_cases():
    V, T = 16, 20000
    z, _ = _toy_pq(V, 1)
    p = special.softmax(z)
    rng = np.random.default_rng(5)
    # q = p: every draft accepted (u < 1 gives u q < p)
    q = p.astype(np.float32)
    drafts = _draws(q, (T, 4), rng).astype(np.int32)
    n, _ = oracle.toy_spec_trials(z, q, drafts, rng.random((T, 4), dtype=np.float32),
                                  rng.random((T, V), dtype=np.float32))
    assert np.all(n == 4)
    # disjoint supports: q puts all mass where p is ~0; every draft rejected and the
    # residual max(p - q, 0) is p itself
    z2 = z.copy()
    z2[8:] = -1e4
    p2 = special.softmax(z2)
    q2 = np.zeros(V, np.float32)
    q2[8:] = 1.0 / 8
    T2 = 200000
    drafts = _draws(q2, (T2, 2), rng).astype(np.int32)
    n, y = oracle.toy_spec_trials(z2, q2, drafts, rng.random((T2, 2), dtype=np.float32),
                                  rng.random((T2, V), dtype=np.float32))
    assert np.all(n == 0)
    cnt = np.bincount(y, minlength=V)
    assert cnt[8:].sum() == 0
    chi2, pval = stats.chisquare(cnt[:8], T2 * p2[:8] / p2[:8].sum())
    assert pval > 0.01


def test_gumbel_max_bonus_is_a_softmax_sample():
    V, T = 12, 200000
    z = np.random.default_rng(2).standard_normal(V)
    rng = np.random.default_rng(3)
    u = rng.random((T, V), dtype=np.float32)
    ys = np.array([oracle.sample_bonus(z, u[t])[0] for t in range(0, T, 10)])
    cnt = np.bincount(ys, minlength=V)
    chi2, pval = stats.chisquare(cnt, cnt.sum() * special.softmax(z))
    assert pval > 0.01


def test_accept_sample_margin_sign_is_decision():
    lse = np.array([0.0, 0.0])
    dl = np.log(np.array([0.3, 0.2]))
    n, m = oracle.accept_sample(lse, dl, np.array([0.5, 0.5], np.float32),
                                np.array([0.5, 0.9], np.float32))
    # draft 1: u q = 0.25 < p = 0.3 accepted; draft 2: u q = 0.45 >= 0.2 rejected
    assert n == 1
    assert m[0] > 0 and m[1] < 0
    assert abs(m[0] - math.log(0.3 / 0.25)) < 1e-6


# ---------------------------------------------------------------------------
# dense layer pieces
# ---------------------------------------------------------------------------

def test_rmsnorm_unit_rms_and_gelu_identities():
    x = np.random.default_rng(4).standard_normal((3, 100)) * 7
    y = oracle.rmsnorm(x, 1e-6)
    np.testing.assert_allclose(np.sqrt((y ** 2).mean(axis=1)), 1.0, rtol=1e-7)
    np.testing.assert_allclose(y / x, (y / x)[:, :1].repeat(100, axis=1), rtol=1e-12)
    for v in np.linspace(-6, 6, 49):
        # gelu(x) - gelu(-x) = x for any function of the form 0.5 x (1 + odd(x))
        assert abs(oracle.gelu_tanh(v) - oracle.gelu_tanh(-v) - v) < 1e-12
        # the tanh form stays within 1e-3 of the exact erf GELU
        exact = 0.5 * v * (1 + math.erf(v / math.sqrt(2)))
        assert abs(oracle.gelu_tanh(v) - exact) < 1e-3
    assert oracle.gelu_tanh(0.0) == 0.0
    g = np.array([0.0, 1.0, -2.0])
    u = np.array([3.0, 2.0, 0.5])
    np.testing.assert_allclose(oracle.geglu(g, u), [0.0, 2 * oracle.gelu_tanh(1.0),
                                                    0.5 * oracle.gelu_tanh(-2.0)])


# ---------------------------------------------------------------------------
# drafter step
# ---------------------------------------------------------------------------

def test_drafter_step_closed_form():
    """A drafter step where the attention has a closed form: the local blocks read a
    cache of two committed rows with a window of 3, so the query at position L + 1
    sees only row 1 (its output is v_1) and the query at L + 2 sees no row (zero
    output); the global block's two rows are equal keys (output: that key, the value
    on a K = V layer).  Everything else is written out with numpy in fp64; the oracle
    stores the activations in fp32 and h in bf16, hence the tolerance (one bf16
    rounding of h, 2^-8 relative).  A swapped concatenation, a
    block reading the wrong layer's cache, a dropped residual or a wrong query
    position changes the logits by far more."""
    rng = np.random.default_rng(7)
    loc = configs.AttnLayer("local", 4, 2, 8, 3, 8, 1e4, False)
    glo = configs.AttnLayer("global", 4, 1, 16, 0, 4, 1e6, True)
    tcfg = configs.StackConfig(name="pin", d_model=16, vocab=32, layers=(loc, loc, glo), d_ff=0, norm=True,
                               eps=1e-6, dtype="bf16", batch=2, k=2, ctx=2)
    dcfg = configs.DrafterConfig(name="pin_drafter", d_draft=8, d_ff=8, blocks=("local", "global"))
    bf = lambda *s, sc=1.0: oracle.bf16_round(rng.standard_normal(s) * sc)
    bits = lambda a: (np.asarray(a, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    d, dd, dff, V, B = 16, 8, 8, 32, 2
    E = bf(V, d, sc=0.3)
    W = {"E": bf(V, dd, sc=0.5), "w_down": bf(dd, d + dd, sc=0.2), "w_up": bf(d, dd, sc=0.3),
         "blocks": [{"wq": bf(loc.n_heads_q * loc.head_dim, dd), "wo": bf(dd, 32, sc=0.2),
                     "wgu": bf(2 * dff, dd, sc=0.3), "wd": bf(dd, dff, sc=0.3)},
                    {"wq": bf(glo.n_heads_q * glo.head_dim, dd), "wo": bf(dd, 64, sc=0.2),
                     "wgu": bf(2 * dff, dd, sc=0.3), "wd": bf(dd, dff, sc=0.3)}]}
    cap = 4
    caches = []
    for ly in tcfg.layers:
        kc = bf(B, ly.n_heads_kv, cap, ly.head_dim).astype(np.float32)
        vc = None if ly.k_is_v else bf(B, ly.n_heads_kv, cap, ly.head_dim).astype(np.float32)
        if ly.k_is_v:
            kc[:, :, 1] = kc[:, :, 0]
        caches.append({"k": kc, "v": vc})
    o = om.OracleDrafter(tcfg, dcfg, bits(E), {"E": bits(W["E"]), "w_down": bits(W["w_down"]),
                                               "w_up": bits(W["w_up"]),
                                               "blocks": [{k: bits(v) for k, v in b.items()} for b in W["blocks"]]})
    h_prev = bf(B, d)
    tok = np.array([3, 30])

    def rms(v):
        return v / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + 1e-6)

    def gelu(v):
        return 0.5 * v * (1 + np.tanh(np.sqrt(2 / np.pi) * (v + 0.044715 * v ** 3)))

    for i in (1, 2):
        st = om.new_state([{k: (None if a is None else a.copy()) for k, a in c.items()} for c in caches], [2, 2])
        h, z = o.step(st, h_prev, tok, i)
        x = np.concatenate([rms(h_prev), rms(np.sqrt(dd) * W["E"][tok])], axis=1) @ W["w_down"].T
        # blocks read the last local layer (index 1) and the global layer (index 2)
        for blk, ly, c in ((W["blocks"][0], loc, caches[1]), (W["blocks"][1], glo, caches[2])):
            G = ly.n_heads_q // ly.n_heads_kv
            if ly.k_is_v:
                src = c["k"][:, :, 0]                       # both rows equal
            else:
                src = c["v"][:, :, 1] if i == 1 else np.zeros_like(c["v"][:, :, 0])
            att = np.repeat(src, G, axis=1).reshape(B, -1).astype(np.float64)
            x = x + att @ blk["wo"].T
            m = rms(x)
            x = x + (gelu(m @ blk["wgu"][:dff].T) * (m @ blk["wgu"][dff:].T)) @ blk["wd"].T
        href = rms(x) @ W["w_up"].T
        zref = href @ E.T
        assert np.all(np.abs(h - href) <= 2.0 ** -8 * np.abs(href) + 1e-6 * np.abs(href).max()), i
        assert np.abs(z - zref).max() < 1e-2 * np.abs(zref).max(), i
        # the same check fails if the step reads the other query position
        _, z_wrong = o.step(st, h_prev, tok, 0)
        assert np.abs(z_wrong - zref).max() > 0.1 * np.abs(zref).max()
