"""Shared comparison helpers for the GPU parity tests."""
import numpy as np
import torch

# Attention tolerance for bf16 outputs against the float64 oracle, over each
# call's whole output: max-abs error and relative L2 error.
ATTN_MAX_ABS = 2e-2
ATTN_REL_L2 = 5e-3
# lse: fp32 running sums over at most ~131k keys; 1e-3 absolute in natural log
LSE_MAX_ABS = 1e-3


def attn_errors(got: torch.Tensor, ref: np.ndarray):
    g = got.detach().to("cpu", torch.float64).numpy()
    diff = g - ref
    max_abs = float(np.abs(diff).max()) if diff.size else 0.0
    denom = float(np.linalg.norm(ref.ravel()))
    rel_l2 = float(np.linalg.norm(diff.ravel()) / denom) if denom > 0 else float(np.linalg.norm(diff.ravel()))
    return max_abs, rel_l2


def assert_attn_close(got, ref, what=""):
    max_abs, rel_l2 = attn_errors(got, ref)
    assert np.isfinite(max_abs), f"{what}: non-finite output"
    assert max_abs <= ATTN_MAX_ABS and rel_l2 <= ATTN_REL_L2, \
        f"{what}: max_abs={max_abs:.3e} rel_l2={rel_l2:.3e}"
    return max_abs, rel_l2


def assert_lse_close(got, ref, what=""):
    g = got.detach().to("cpu", torch.float64).numpy()
    err = float(np.abs(g - ref).max())
    assert err <= LSE_MAX_ABS, f"{what}: lse max_abs={err:.3e}"
    return err
