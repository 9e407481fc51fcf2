"""Shared helpers of the GPU parity tests (argument plumbing only)."""
import numpy as np
import pytest

U32 = 2.0 ** -24


def torch_or_skip():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    return torch


def dev(a):
    """numpy -> contiguous CUDA tensor (float32 or int32 kept)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def host(t):
    return t.detach().cpu().numpy()


def logits_close(got, ref, rel=1e-4):
    """The parity bar of the decode step: max |d logit| <= rel * max |logit|."""
    err = float(np.max(np.abs(got.astype(np.float64) - ref)))
    tol = rel * float(np.max(np.abs(ref)))
    return err <= tol and np.all(np.isfinite(got)), err, tol


def tie_tolerance(ref_logits, rel=1e-4):
    return rel * float(np.max(np.abs(ref_logits)))


def acceptable_token(tok, ref_logits, rel=1e-4):
    """A greedy token is right if the oracle's logit for it is within the parity
    tolerance of the oracle's maximum (several tokens qualify at a near-tie)."""
    return ref_logits[tok] >= ref_logits.max() - tie_tolerance(ref_logits, rel)


def top2_gap(ref_logits):
    s = np.sort(ref_logits.astype(np.float64))
    return s[-1] - s[-2]
