"""GPU parity of sv_linear (bf16 skinny projections) against the oracle.

The bound is derived from the arithmetic: products of two bf16 values are exact
in fp32, and any summation order of K terms is within gamma_K * sum |x_k w_k|
(gamma_K = K * 2^-24) of the exact sum, which the oracle computes in fp64 (with
sum |x_k w_k| from the oracle on |x|, |W|).  A stored bf16 output adds one unit
roundoff, 2^-8 |y|.  Blocks split across workgroups are summed in a fixed order,
so two calls give identical bits."""
import numpy as np
import pytest
import torch

import oracle
import mtp_draft_verification_amd._lib as L
from mtp_draft_verification_amd import inputs
from gpu_util import gpu, host, need_gpu, say


def linear_case(R, K, N, epi, seed, ws=None, check_repeat=False):
    dev = need_gpu()
    say(f"[linear] R={R} K={K} N={N} epi={'add' if epi else 'store'} seed={seed}")
    x = inputs.normal((R, K), 1.0, seed, "x", dev)
    W = inputs.normal((N, K), K ** -0.5, seed, "W", dev)
    desc = L.LinearDesc(rows=R, in_features=K, out_features=N, dtype=L.SV_BF16, epilogue=epi)
    if ws is None:
        ws = torch.zeros(L.sv_linear_workspace(desc), dtype=torch.uint8, device=dev)
    if epi == L.SV_EPI_ADD_F32:
        y0 = inputs.normal((R, N), 1.0, seed, "y0", dev, "f32")
        y = y0.clone()
    else:
        y0 = None
        y = torch.full((R, N), float("nan"), dtype=torch.bfloat16, device=dev)
    L.sv_linear(desc, x, W, y, ws)
    torch.cuda.synchronize()
    ref = oracle.linear(host(x), inputs.bf16_bits(W))
    mag = oracle.linear(np.abs(host(x)), np.abs(host(W)))
    bound = K * 2.0 ** -24 * mag + 1e-30
    got = host(y)
    if y0 is not None:
        ref = ref + host(y0).astype(np.float64)
        bound = bound + 2.0 ** -24 * np.abs(ref)      # the final add into fp32
    else:
        bound = bound * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(ref)
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got))
    bad = err > bound
    assert not bad.any(), f"{bad.sum()} outputs beyond the bound; worst excess {(err - bound).max():.3e}"
    if check_repeat:
        y2 = y0.clone() if y0 is not None else torch.empty_like(y)
        L.sv_linear(desc, x, W, y2, ws)
        torch.cuda.synchronize()
        assert torch.equal(y, y2), "repeat call differs"
    say(f"[linear] ok, max err/bound {float((err / bound).max()):.3f}")
    return ws


@gpu
def test_projection_shapes():
    # fused q/k/v of a sliding-window layer, 40 rows (three row tiles)
    linear_case(40, 3840, 8192, L.SV_EPI_STORE, 1, check_repeat=True)
    # down projection into the residual stream: K = 15360, each block spans many workgroups
    linear_case(20, 15360, 3840, L.SV_EPI_ADD_F32, 2, check_repeat=True)


@gpu
def test_ragged_and_tiny_shapes():
    linear_case(5, 96, 192, L.SV_EPI_STORE, 3)          # K % 64 == 32, N not a multiple of 128
    linear_case(64, 4096 + 32, 320, L.SV_EPI_ADD_F32, 4)  # four row tiles, ragged K
    linear_case(1, 64, 64, L.SV_EPI_STORE, 5)           # one unit of work
    linear_case(17, 256, 1024, L.SV_EPI_ADD_F32, 6)     # two row tiles, 17 rows


@gpu
def test_shared_workspace_across_shapes():
    """The arrival counters are left zero, so one workspace serves calls of any shape."""
    dev = need_gpu()
    big = max(L.sv_linear_workspace(L.LinearDesc(rows=r, in_features=k, out_features=n, dtype=L.SV_BF16,
                                                 epilogue=0))
              for (r, k, n) in ((40, 3840, 8192), (40, 8192, 3840), (33, 512, 640)))
    ws = torch.zeros(big, dtype=torch.uint8, device=dev)
    for (r, k, n, e, sd) in ((40, 8192, 3840, 1, 7), (33, 512, 640, 0, 8), (40, 3840, 8192, 0, 9),
                             (40, 8192, 3840, 1, 10)):
        linear_case(r, k, n, e, sd, ws=ws)
    # the counter region (the first 256 KiB) is back to zero after the calls
    assert int(torch.count_nonzero(ws[:1 << 18]).item()) == 0


@gpu
@pytest.mark.parametrize("R,K,dff", [(40, 3840, 15360), (20, 256, 512), (7, 96, 64)])
def test_fused_geglu(R, K, dff):
    """SV_EPI_GEGLU against the oracle's gelu_tanh(bf16(x Wg)) * bf16(x Wu).  Bound:
    the fp32 sums are within gamma_K sum|x w| of the exact ones, bf16 rounding of g and
    u adds at most 2^-8 relative each, gelu_tanh has slope below 1.13, and the stored
    f adds 2^-8 relative."""
    dev = need_gpu()
    from mtp_draft_verification_amd.step import interleave_gate_up
    say(f"[linear geglu] R={R} K={K} d_ff={dff}")
    x = inputs.normal((R, K), 1.0, 11, "x", dev)
    Wgu = inputs.normal((2 * dff, K), K ** -0.5, 11, "Wgu", dev)
    desc = L.LinearDesc(rows=R, in_features=K, out_features=2 * dff, dtype=L.SV_BF16, epilogue=L.SV_EPI_GEGLU)
    ws = torch.zeros(L.sv_linear_workspace(desc), dtype=torch.uint8, device=dev)
    f = torch.full((R, dff), float("nan"), dtype=torch.bfloat16, device=dev)
    L.sv_linear(desc, x, interleave_gate_up(Wgu), f, ws)
    torch.cuda.synchronize()
    xh, wh = host(x), inputs.bf16_bits(Wgu)
    GU = oracle.linear(xh, wh)
    mag = oracle.linear(np.abs(xh), np.abs(host(Wgu)))
    e_acc = K * 2.0 ** -24 * mag
    G, U = GU[:, :dff], GU[:, dff:]
    g, u = oracle.bf16_round(G), oracle.bf16_round(U)
    ref = oracle.bf16_round(oracle.geglu(g, u))
    dg = e_acc[:, :dff] + 2.0 ** -8 * np.abs(G) + 1e-30
    du = e_acc[:, dff:] + 2.0 ** -8 * np.abs(U) + 1e-30
    gel = np.abs(oracle.geglu(g, np.ones_like(g)))
    bound = 1.13 * dg * (np.abs(u) + du) + gel * du + 2.0 ** -7 * np.abs(ref) + 1e-30
    got = host(f)
    assert np.all(np.isfinite(got))
    err = np.abs(got - ref)
    assert np.all(err <= bound), f"worst excess {(err - bound).max():.3e}"
    say(f"[linear geglu] ok, max err/bound {float((err / bound).max()):.3f}")


@gpu
@pytest.mark.parametrize("R,K,N", [(40, 15360, 3840), (40, 4096, 3840), (7, 96, 192), (33, 8192 + 32, 640)])
def test_split_partials(R, K, N):
    """SV_EPI_SPLIT_F32: every slice written, their sum in slice order within
    (K + S) 2^-24 sum |x w| of the exact product."""
    dev = need_gpu()
    desc = L.LinearDesc(rows=R, in_features=K, out_features=N, dtype=L.SV_BF16, epilogue=L.SV_EPI_SPLIT_F32)
    S = L.sv_linear_splits(desc)
    say(f"[linear split] R={R} K={K} N={N} S={S}")
    assert S >= 1
    assert L.sv_linear_workspace(desc) == 0
    x = inputs.normal((R, K), 1.0, 12, "x", dev)
    W = inputs.normal((N, K), K ** -0.5, 12, "W", dev)
    y = torch.full((S, R, N), float("nan"), dtype=torch.float32, device=dev)
    L.sv_linear(desc, x, W, y, None)
    torch.cuda.synchronize()
    got = host(y)
    assert np.all(np.isfinite(got)), "a slice was left unwritten"
    total = got[0].astype(np.float64)
    for s in range(1, S):
        total = (total.astype(np.float32) + got[s]).astype(np.float64)
    ref = oracle.linear(host(x), inputs.bf16_bits(W))
    mag = oracle.linear(np.abs(host(x)), np.abs(host(W)))
    bound = (K + S) * 2.0 ** -24 * mag + 1e-30
    err = np.abs(total - ref)
    assert np.all(err <= bound), f"worst excess {(err - bound).max():.3e}"
    y2 = torch.empty_like(y)
    L.sv_linear(desc, x, W, y2, None)
    torch.cuda.synchronize()
    assert torch.equal(y, y2), "repeat call differs"
