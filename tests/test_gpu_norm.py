"""GPU parity of sv_rmsnorm and sv_add_rmsnorm against the oracle.

Bounds from the arithmetic: the fp32 sum of squares over d terms is within
d 2^-24 (relative) of the exact one, so the scale 1/sqrt(mean + eps) is within
(d/2 + 2) 2^-24 and the product with x and the gain within (d/2 + 4) 2^-24; a
bf16 store adds 2^-8.  The residual add of S slices (summed in slice order, then
added to x) is within (S + 1) 2^-24 (|x| + sum |p_s|) of the exact sum."""
import numpy as np
import pytest
import torch

import oracle
import mtp_draft_verification_amd._lib as L
from mtp_draft_verification_amd import inputs
from gpu_util import gpu, host, need_gpu, say

EPS = 1e-6


def norm_bound(ref, d, bf16):
    rel = (d / 2 + 4) * 2.0 ** -24 + (2.0 ** -8 if bf16 else 0.0)
    return rel * np.abs(ref) + 1e-30


@gpu
@pytest.mark.parametrize("R,d,bf16", [(40, 3840, True), (3, 100, False), (5, 8192, True)])
def test_rmsnorm(R, d, bf16):
    dev = need_gpu()
    say(f"[norm] R={R} d={d} bf16={bf16}")
    x = inputs.normal((R, d), 2.0, 1, "x", dev, "f32")
    g = inputs.normal((d,), 1.0, 1, "g", dev, "f32")
    y = torch.full((R, d), float("nan"), dtype=torch.bfloat16 if bf16 else torch.float32, device=dev)
    L.sv_rmsnorm(R, d, EPS, x, g, y, L.SV_BF16 if bf16 else L.SV_F32)
    torch.cuda.synchronize()
    ref = oracle.rmsnorm(host(x), EPS) * host(g).astype(np.float64)
    err = np.abs(host(y) - ref)
    assert np.all(err <= norm_bound(ref, d, bf16)), f"worst excess {(err - norm_bound(ref, d, bf16)).max():.3e}"


@gpu
@pytest.mark.parametrize("R,d,S,gain", [(40, 3840, 8, False), (7, 256, 3, True), (5, 96, 0, True),
                                        (2, 8192, 5, False)])
def test_add_rmsnorm(R, d, S, gain):
    dev = need_gpu()
    say(f"[add_norm] R={R} d={d} S={S} gain={gain}")
    x = inputs.normal((R, d), 1.0, 2, "x", dev, "f32")
    x0 = host(x).astype(np.float64)
    parts = inputs.normal((S, R, d), 0.5, 2, "parts", dev, "f32") if S else None
    g = inputs.normal((d,), 1.0, 2, "g", dev, "f32") if gain else None
    y = torch.full((R, d), float("nan"), dtype=torch.bfloat16, device=dev)
    L.sv_add_rmsnorm(R, d, EPS, x, parts, S, g, y, L.SV_BF16)
    torch.cuda.synchronize()
    ph = host(parts).astype(np.float64) if S else np.zeros((0, R, d))
    xs = x0 + ph.sum(axis=0)
    xb = (S + 1) * 2.0 ** -24 * (np.abs(x0) + np.abs(ph).sum(axis=0)) + 1e-30
    xe = np.abs(host(x) - xs)
    assert np.all(xe <= xb), f"residual: worst excess {(xe - xb).max():.3e}"
    # the norm of the stored residual (what the kernel normalises)
    ref = oracle.rmsnorm(host(x), EPS)
    if gain:
        ref = ref * host(g).astype(np.float64)
    err = np.abs(host(y) - ref)
    bnd = norm_bound(ref, d, True)
    assert np.all(err <= bnd), f"norm: worst excess {(err - bnd).max():.3e}"
    say(f"[add_norm] ok, max err/bound {float((err / bnd).max()):.3f}")


def pair_value(y):
    """The value a bf16 pair [2, ...] holds: hi + lo (exact in fp64)."""
    return host(y[0]).astype(np.float64) + host(y[1]).astype(np.float64)


@gpu
@pytest.mark.parametrize("R,d,S", [(40, 3840, 8), (5, 100, 0), (3, 8192, 2)])
def test_norms_pair_output(R, d, S):
    """SV_BF16X2 output: plane 0 holds bf16(y), plane 1 bf16(y - plane 0); their sum is
    within 2^-16 |y| of the fp32 result, so the bound is the fp32 one plus 2^-16."""
    dev = need_gpu()
    say(f"[norm pair] R={R} d={d} S={S}")
    x = inputs.normal((R, d), 1.5, 3, "x", dev, "f32")
    if d % 4 == 0:
        parts = inputs.normal((S, R, d), 0.5, 3, "parts", dev, "f32") if S else None
        y = torch.full((2, R, d), float("nan"), dtype=torch.bfloat16, device=dev)
        L.sv_add_rmsnorm(R, d, EPS, x, parts, S, None, y, L.SV_BF16X2)
    else:
        y = torch.full((2, R, d), float("nan"), dtype=torch.bfloat16, device=dev)
        L.sv_rmsnorm(R, d, EPS, x, None, y, L.SV_BF16X2)
    torch.cuda.synchronize()
    ref = oracle.rmsnorm(host(x), EPS)
    got = pair_value(y)
    bnd = ((d / 2 + 4) * 2.0 ** -24 + 2.0 ** -16) * np.abs(ref) + 1e-30
    err = np.abs(got - ref)
    assert np.all(err <= bnd), f"worst excess {(err - bnd).max():.3e}"
    # plane 0 is the bf16 rounding of the fp32 result: |hi - y| <= 2^-8 |y|
    hi = host(y[0]).astype(np.float64)
    assert np.all(np.abs(hi - ref) <= (2.0 ** -8 + d * 2.0 ** -24) * np.abs(ref) + 1e-30)
