"""Oracle for the training objective's hot op: forward KL over the vocabulary.

TEST INFRASTRUCTURE ONLY -- never imported by the product path.

Sources (the Orthrus pages):

* Paper notes on Orthrus (zhangshuibai.github.io paper-notes), §3.1 and §3.3:
  the diffusion head is distilled against the frozen AR model's full softmax
  at every masked position, with the forward KL divergence
  KL(P_AR || P_Diff) as the loss (soft labels rather than hard tokens, §3.4).
* zhichai.net forum topic on Orthrus (English and Chinese versions) and the
  hotdry.top blog post (training-strategy section): the same objective,
  written D_KL(P_AR || P_Diff).

Readings of points the pages leave open:

* R19 -- both distributions are softmaxes of logit rows over the whole
  vocabulary (no temperature: the caller scales logits if it wants one); the
  loss of one position is
      KL = sum_v p_v (ln p_v - ln q_v),  p = softmax(target row), q = softmax(draft row),
  and its gradient with respect to the draft logits is q - p (the target is
  frozen, so no gradient flows into it).  A caller-given scale multiplies the
  gradient (for example 1 / number of positions for a mean loss).
* Logits are finite.

Everything is float64 and runs one row at a time: explicit max shift,
``numpy.exp``, ``numpy.log`` and sums.
"""
from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def log_softmax_row(z: np.ndarray) -> np.ndarray:
    """ln softmax(z) of one row: z - (max + ln sum exp(z - max))."""
    m = np.max(z)
    return z - (m + np.log(np.sum(np.exp(z - m))))


def forward_kl(target_logits, draft_logits, grad_scale: float = 1.0):
    """Forward KL(P_target || P_draft) per row, and its draft-logit gradient.

    target_logits, draft_logits: [N, V] (any float type; widened to float64).
    Returns (kl [N], grad [N, V]) in float64 with
      kl[n]      = sum_v p[n,v] * (ln p[n,v] - ln q[n,v])
      grad[n, v] = grad_scale * (q[n,v] - p[n,v])   (d kl[n] / d draft_logits[n,v])
    """
    a = _f64(target_logits)
    b = _f64(draft_logits)
    if a.shape != b.shape or a.ndim != 2:
        raise ValueError("logits must both be [N, V]")
    n_rows = a.shape[0]
    kl = np.zeros(n_rows)
    grad = np.zeros_like(a)
    for n in range(n_rows):
        lp = log_softmax_row(a[n])
        lq = log_softmax_row(b[n])
        p = np.exp(lp)
        q = np.exp(lq)
        kl[n] = np.sum(p * (lp - lq))
        grad[n] = float(grad_scale) * (q - p)
    return kl, grad


def forward_kl_rows(target_logits, draft_logits, rows, grad_scale: float = 1.0):
    """The same definition at selected rows only (for very large inputs)."""
    rows = [int(r) for r in rows]
    a = np.stack([_f64(target_logits[r]) for r in rows])
    b = np.stack([_f64(draft_logits[r]) for r in rows])
    return forward_kl(a, b, grad_scale)
