"""GPU parity of the fused forward KL(P_AR || P_Diff) and its gradient.

Compared with the fp64 oracle on the same inputs (fp32 or bf16 logits).
Tolerances, from the fp32 arithmetic of the kernels:
* KL: |err| <= 1e-4 + 2e-5 |KL|.  Sums of up to 151936 fp32 terms (relative
  error ~1e-6) scaled by |a - b| and by log-sum-exps of up to ~30.
* gradient: |err| <= scale * (2e-5 (p + q) + 1e-10) for fp32 output -- each of
  e^(b-B) and e^(a-A) carries a relative error of a few 1e-6 from the
  argument's rounding and the exponential -- plus 2^-8 |grad| when the
  gradient is stored in bf16 (one rounding of the result).
"""
import numpy as np
import pytest
import torch

import dual_view_block_amd as dvb
import oracle
from oracle.kl import log_softmax_row
from synth import kl_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _check(a, b, what, scale=1.0, rows=None):
    kl, grad = dvb.orthrus_forward_kl(a, b, want_grad=True, grad_scale=scale)
    kl_only, none = dvb.orthrus_forward_kl(a, b)
    torch.cuda.synchronize()
    assert none is None
    assert torch.equal(kl, kl_only), "the loss must not depend on whether a gradient is asked for"
    rows = list(range(a.shape[0])) if rows is None else rows
    idx = torch.tensor(rows, device=a.device)
    a_s, b_s = a[idx].cpu(), b[idx].cpu()   # only the checked rows leave the device
    ref_kl, ref_g = oracle.forward_kl(a_s, b_s, grad_scale=scale)
    got_kl = kl[idx].cpu().double().numpy()
    err = np.abs(got_kl - ref_kl)
    assert np.all(err <= 1e-4 + 2e-5 * np.abs(ref_kl)), f"{what}: kl err {err.max():.3e}"
    g = grad[idx].cpu().double().numpy()
    a64 = a_s.double().numpy()
    b64 = b_s.double().numpy()
    worst = 0.0
    for i, r in enumerate(rows):
        p = np.exp(log_softmax_row(a64[i]))
        q = np.exp(log_softmax_row(b64[i]))
        tol = abs(scale) * (2e-5 * (p + q) + 1e-10)
        if grad.dtype == torch.bfloat16:
            tol = tol + 2.0 ** -8 * np.abs(ref_g[i])
        d = np.abs(g[i] - ref_g[i])
        assert np.all(d <= tol), f"{what}: row {r} grad err {d.max():.3e} at {int(d.argmax())}"
        worst = max(worst, float((d / tol).max()))
    print(f"{what}: kl max err {err.max():.2e} (kl ~ {np.abs(ref_kl).mean():.3g}); grad err/tol {worst:.2f}",
          flush=True)
    return kl, grad


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_tiny_vocab_1000(dtype):
    a, b = kl_inputs(4, 1000, 4.0, dtype, seed=1, device=DEV)
    _check(a, b, f"tiny/{dtype}")


@pytest.mark.parametrize("dtype,V", [(torch.float32, 1001), (torch.bfloat16, 1003), (torch.float32, 4099),
                                     (torch.bfloat16, 8), (torch.float32, 1), (torch.bfloat16, 12289)])
def test_odd_and_small_vocabularies(dtype, V):
    """Row lengths whose rows are not 16-byte aligned take the scalar-load path;
    V = 1 gives KL = 0 and a zero gradient."""
    a, b = kl_inputs(5, V, 3.0, dtype, seed=V, device=DEV)
    kl, grad = _check(a, b, f"V{V}/{dtype}", scale=0.5)
    if V == 1:
        assert torch.all(kl.abs() <= 1e-6) and torch.all(grad == 0)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("noise", [None, 0.5])
def test_qwen_vocab(dtype, noise):
    """V = 151936 (Qwen3), 48 rows, independent and close drafts, mean-loss scale."""
    a, b = kl_inputs(48, 151936, 3.0, dtype, seed=7, draft_noise=noise, device=DEV)
    _check(a, b, f"qwen/{dtype}/noise{noise}", scale=1.0 / 48)


def test_identical_rows_and_shifted_rows():
    a, _ = kl_inputs(6, 151936, 3.0, torch.float32, seed=3, device=DEV)
    kl, grad = dvb.orthrus_forward_kl(a, a.clone(), want_grad=True)
    torch.cuda.synchronize()
    assert torch.all(kl.abs() <= 2e-5), kl
    assert float(grad.abs().max()) <= 1e-9
    # a constant added to a row changes neither the loss nor the gradient (beyond rounding)
    kl2, grad2 = dvb.orthrus_forward_kl(a, a + 3.0, want_grad=True)
    torch.cuda.synchronize()
    assert torch.all(kl2.abs() <= 1e-4)


def test_large_logits_and_peaked_rows():
    """sigma 20 logits (nearly one-hot softmaxes) and rows with a planted spike."""
    a, b = kl_inputs(8, 32768, 20.0, torch.float32, seed=11, device=DEV)
    a[0, 123] = 250.0
    b[1, 7] = -250.0
    _check(a, b, "sigma20")


def test_training_shape_sampled_rows_and_determinism():
    """8192 rows (256 blocks x K = 32 diffusion positions) x 151936, bf16, the
    benchmark launch: 12 sampled rows against the oracle, every loss finite
    and non-negative up to rounding, and two calls bit-identical."""
    a, b = kl_inputs(8192, 151936, 3.0, torch.bfloat16, seed=5, device=DEV)
    kl, grad = _check(a, b, "train8192", scale=1.0 / 8192, rows=[0, 1, 77, 1000, 2047, 2048, 4095, 4096, 5555,
                                                                  8000, 8190, 8191])
    assert torch.isfinite(kl).all() and float(kl.min()) > -1e-4
    kl2, grad2 = dvb.orthrus_forward_kl(a, b, want_grad=True, grad_scale=1.0 / 8192)
    torch.cuda.synchronize()
    assert torch.equal(kl, kl2) and torch.equal(grad, grad2)
