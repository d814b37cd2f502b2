"""Helpers of the GPU parity tests (host copies, error measures)."""
import numpy as np
import pytest
import torch

gpu = pytest.mark.gpu


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU in this container")
    return torch.device("cuda:0")


def rel_l2(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def host(t):
    """fp32 host copy of a device tensor (exact for bf16 / fp32)."""
    return t.detach().float().contiguous().cpu().numpy()


def say(*a):
    print(*a, flush=True)
