"""Oracle for the training-time dual-pass block-mask attention (forward and
backward).

TEST INFRASTRUCTURE ONLY -- never imported by the product path.

Sources (the Orthrus pages):

* Paper notes on Orthrus (zhangshuibai.github.io paper-notes), §3.1 (a packed
  training sequence of L = 2048 tokens carries 256 randomly placed anchor
  blocks of K = 32 positions: the anchor kept, K-1 positions masked), §3.2
  (one block mask over the packed sequence: the AR path processes the clean
  context; every diffusion position attends causally to the clean context
  before its block's anchor and bidirectionally to the positions of its own
  block; different blocks never see each other), §2.1-2.2 (the diffusion view
  has its own projections; the AR backbone is frozen).
* hotdry.top blog post on Orthrus (training-strategy section) and the
  zhichai.net forum topic: the same mask.

Readings of points the pages leave open:

* R20 -- key set of every row.  AR row i (clean position i) attends to clean
  keys j <= i.  Diffusion row (block n, position p) attends to clean keys
  j < a_n (strictly before the block's anchor position a_n, as at inference,
  R1) and to the K diffusion keys of block n (its own K_diff/V_diff), in one
  softmax.
* R21 -- gradients.  The AR path is frozen, so the backward pass returns the
  gradients of the diffusion rows' outputs with respect to the diffusion
  queries, keys and values only (dQ_diff, dK_diff, dV_diff); the clean K/V are
  not differentiated and the AR rows need no backward.
* GQA as at inference: q head h reads KV head h // (Hq / Hkv); scale
  1/sqrt(D) unless given.

Layouts (head-major, one packed sequence): q_ar [Hq, L, D], k_ar / v_ar
[Hkv, L, D]; q_diff [Hq, N*K, D], k_diff / v_diff [Hkv, N*K, D] (block n
holds positions n*K .. n*K+K-1); anchors [N].

Everything is float64, one row (forward) or one block (backward) at a time,
with explicit key lists; ``numpy.matmul`` and ``numpy.exp`` are the only
library steps.
"""
from __future__ import annotations

import math

import numpy as np

from .attention import _as_f64, _as_int


def _softmax_rows(s: np.ndarray):
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=-1, keepdims=True)
    return e / z, (m + np.log(z))[..., 0]


def dual_pass_forward(q_ar, k_ar, v_ar, q_diff, k_diff, v_diff, anchors, block_k: int, scale=None):
    """Forward of the dual-pass attention.

    Returns (out_ar [Hq,L,D], lse_ar [Hq,L], out_diff [Hq,N*K,D], lse_diff
    [Hq,N*K]) in float64; lse is the natural-log normaliser of each row.
    """
    qa, ka, va = _as_f64(q_ar), _as_f64(k_ar), _as_f64(v_ar)
    qd, kd, vd = _as_f64(q_diff), _as_f64(k_diff), _as_f64(v_diff)
    anc = _as_int(anchors)
    Hq, L, D = qa.shape
    Hkv = ka.shape[0]
    K = int(block_k)
    N = anc.shape[0]
    G = Hq // Hkv
    sc = 1.0 / math.sqrt(D) if not scale else float(scale)
    out_ar = np.zeros_like(qa)
    lse_ar = np.zeros((Hq, L))
    out_d = np.zeros_like(qd)
    lse_d = np.zeros((Hq, N * K))
    for h in range(Hq):
        g = h // G
        for i in range(L):                      # AR row i: clean keys 0..i
            s = sc * (ka[g, :i + 1] @ qa[h, i])
            p, lse = _softmax_rows(s[None, :])
            out_ar[h, i] = p[0] @ va[g, :i + 1]
            lse_ar[h, i] = lse[0]
        for n in range(N):                      # block n: clean keys < a_n, own block
            a_n = int(anc[n])
            keys = np.concatenate([ka[g, :a_n], kd[g, n * K:(n + 1) * K]])
            vals = np.concatenate([va[g, :a_n], vd[g, n * K:(n + 1) * K]])
            rows = qd[h, n * K:(n + 1) * K]
            p, lse = _softmax_rows(sc * rows @ keys.T)
            out_d[h, n * K:(n + 1) * K] = p @ vals
            lse_d[h, n * K:(n + 1) * K] = lse
    return out_ar, lse_ar, out_d, lse_d


def dual_pass_backward(k_ar, v_ar, q_diff, k_diff, v_diff, anchors, block_k: int, d_out_diff, scale=None):
    """Backward of the diffusion rows (R21).

    With S = scale Q K^T over a row's keys, P = softmax(S), O = P V and the
    upstream gradient dO:  dV = P^T dO,  dP = dO V^T,
    dS = P * (dP - rowsum(dO * O)),  dQ = scale dS K,  dK = scale dS^T Q,
    where dK and dV are kept for the block's own diffusion keys (summed over
    the q heads that share a KV head).
    Returns (dq_diff [Hq,N*K,D], dk_diff [Hkv,N*K,D], dv_diff [Hkv,N*K,D]).
    """
    ka, va = _as_f64(k_ar), _as_f64(v_ar)
    qd, kd, vd = _as_f64(q_diff), _as_f64(k_diff), _as_f64(v_diff)
    do = _as_f64(d_out_diff)
    anc = _as_int(anchors)
    Hq, NK, D = qd.shape
    Hkv = ka.shape[0]
    K = int(block_k)
    N = anc.shape[0]
    G = Hq // Hkv
    sc = 1.0 / math.sqrt(D) if not scale else float(scale)
    dq = np.zeros_like(qd)
    dk = np.zeros_like(kd)
    dv = np.zeros_like(vd)
    for h in range(Hq):
        g = h // G
        for n in range(N):
            a_n = int(anc[n])
            blk = slice(n * K, (n + 1) * K)
            keys = np.concatenate([ka[g, :a_n], kd[g, blk]])
            vals = np.concatenate([va[g, :a_n], vd[g, blk]])
            q = qd[h, blk]
            p, _ = _softmax_rows(sc * q @ keys.T)
            o = p @ vals
            g_o = do[h, blk]
            dp = g_o @ vals.T
            ds = p * (dp - np.sum(g_o * o, axis=1, keepdims=True))
            dq[h, blk] = sc * ds @ keys
            dk[g, blk] += sc * ds[:, a_n:].T @ q
            dv[g, blk] += p[:, a_n:].T @ g_o
    return dq, dk, dv


def training_attention_flops(seq_len: int, anchors, block_k: int, n_q_heads: int, head_dim: int):
    """Matrix flops of the dual-pass forward (QK^T and PV over every allowed
    key of every row): AR rows see i+1 keys, diffusion rows a_n + K."""
    anc = _as_int(anchors)
    ar_keys = seq_len * (seq_len + 1) // 2
    diff_keys = int(sum(int(a) + block_k for a in anc)) * block_k
    return 4 * n_q_heads * head_dim * (ar_keys + diff_keys)
