"""Pins for the dual-pass training attention oracle (CPU only).

* The forward against torch's scaled_dot_product_attention (fp64) over the
  whole packed sequence [clean L | diffusion N*K] with the full boolean block
  mask built independently, in vectorised form, from block ids and positions.
* The backward against torch autograd through that same library attention,
  with the clean keys and values frozen (detached).
* AR rows against plain causal attention (is_causal), and block rows with the
  anchor at 0 against bidirectional attention over the block alone.
* Isolation: perturbing another block, or clean keys at or after a block's
  anchor, leaves that block's outputs unchanged.
* Central finite differences for dQ, dK, dV on a tiny case.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle.train_attn import dual_pass_backward, dual_pass_forward, training_attention_flops


def _inputs(Hq, Hkv, L, N, K, D, seed, anchors=None):
    g = torch.Generator().manual_seed(seed)
    r = lambda *s: torch.randn(s, generator=g, dtype=torch.float64)
    if anchors is None:
        anchors = torch.randint(0, L - K + 1, (N,), generator=g)
    return dict(q_ar=r(Hq, L, D), k_ar=r(Hkv, L, D), v_ar=r(Hkv, L, D), q_diff=r(Hq, N * K, D),
                k_diff=r(Hkv, N * K, D), v_diff=r(Hkv, N * K, D), anchors=torch.as_tensor(anchors), K=K)


def _full_mask(L, N, K, anchors):
    """[L+N*K, L+N*K] bool: True = may attend.  Rows/cols 0..L-1 are clean
    positions, L + n*K + p is position p of block n."""
    T = L + N * K
    idx = torch.arange(T)
    is_clean = idx < L
    blk = torch.where(is_clean, torch.full_like(idx, -1), (idx - L) // K)
    anc = torch.where(is_clean, idx, anchors[blk.clamp(min=0)])
    qi, kj = idx[:, None], idx[None, :]
    clean_q, clean_k = is_clean[:, None], is_clean[None, :]
    ar_part = clean_q & clean_k & (kj <= qi)
    ctx_part = ~clean_q & clean_k & (kj < anc[:, None])
    own_block = ~clean_q & ~clean_k & (blk[:, None] == blk[None, :])
    return ar_part | ctx_part | own_block


def _library_forward(x, requires_grad=False):
    Hq, L, D = x["q_ar"].shape
    Hkv = x["k_ar"].shape[0]
    N, K = len(x["anchors"]), x["K"]
    q = torch.cat([x["q_ar"], x["q_diff"]], dim=1)
    k = torch.cat([x["k_ar"], x["k_diff"]], dim=1)
    v = torch.cat([x["v_ar"], x["v_diff"]], dim=1)
    rep = Hq // Hkv
    k = k.repeat_interleave(rep, dim=0)
    v = v.repeat_interleave(rep, dim=0)
    mask = _full_mask(L, N, K, x["anchors"])
    out = F.scaled_dot_product_attention(q[None], k[None], v[None], attn_mask=mask[None, None])[0]
    return out[:, :L], out[:, L:]


@pytest.mark.parametrize("Hq,Hkv,L,N,K,D", [(2, 1, 40, 3, 4, 8), (4, 2, 64, 5, 8, 16), (8, 2, 96, 6, 32, 32)])
def test_forward_matches_library_attention_with_full_block_mask(Hq, Hkv, L, N, K, D):
    x = _inputs(Hq, Hkv, L, N, K, D, seed=L + N)
    out_ar, lse_ar, out_d, lse_d = dual_pass_forward(x["q_ar"], x["k_ar"], x["v_ar"], x["q_diff"], x["k_diff"],
                                                     x["v_diff"], x["anchors"], K)
    ref_ar, ref_d = _library_forward(x)
    np.testing.assert_allclose(out_ar, ref_ar.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(out_d, ref_d.numpy(), rtol=0, atol=1e-12)
    # lse: the log normaliser of each row, checked on row 0 of block 0 of head 0
    a0 = int(x["anchors"][0])
    keys = torch.cat([x["k_ar"][0, :a0], x["k_diff"][0, :K]])
    s = (keys @ x["q_diff"][0, 0]) / math.sqrt(D)
    assert math.isclose(lse_d[0, 0], torch.logsumexp(s, 0).item(), rel_tol=1e-12)
    s = (x["k_ar"][0, :1] @ x["q_ar"][0, 0]) / math.sqrt(D)
    assert math.isclose(lse_ar[0, 0], s[0].item(), rel_tol=1e-12)


@pytest.mark.parametrize("Hq,Hkv,L,N,K,D", [(2, 1, 40, 3, 4, 8), (4, 2, 48, 4, 8, 16)])
def test_backward_matches_autograd_with_frozen_clean_path(Hq, Hkv, L, N, K, D):
    x = _inputs(Hq, Hkv, L, N, K, D, seed=7 * L)
    g = torch.Generator().manual_seed(99)
    d_out = torch.randn((Hq, N * K, D), generator=g, dtype=torch.float64)
    xr = dict(x)
    for name in ("q_diff", "k_diff", "v_diff"):
        xr[name] = x[name].clone().requires_grad_(True)
    _, out_d = _library_forward(xr)
    (out_d * d_out).sum().backward()
    dq, dk, dv = dual_pass_backward(x["k_ar"], x["v_ar"], x["q_diff"], x["k_diff"], x["v_diff"], x["anchors"], K,
                                    d_out)
    np.testing.assert_allclose(dq, xr["q_diff"].grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dk, xr["k_diff"].grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv, xr["v_diff"].grad.numpy(), rtol=0, atol=1e-11)


def test_ar_rows_are_causal_attention_and_anchor_zero_is_block_only():
    Hq, Hkv, L, N, K, D = 4, 2, 50, 3, 6, 8
    x = _inputs(Hq, Hkv, L, N, K, D, seed=3, anchors=[0, 17, 44])
    out_ar, _, out_d, _ = dual_pass_forward(x["q_ar"], x["k_ar"], x["v_ar"], x["q_diff"], x["k_diff"],
                                            x["v_diff"], x["anchors"], K)
    k = x["k_ar"].repeat_interleave(2, dim=0)
    v = x["v_ar"].repeat_interleave(2, dim=0)
    causal = F.scaled_dot_product_attention(x["q_ar"][None], k[None], v[None], is_causal=True)[0]
    np.testing.assert_allclose(out_ar, causal.numpy(), rtol=0, atol=1e-12)
    kb = x["k_diff"][:, :K].repeat_interleave(2, dim=0)
    vb = x["v_diff"][:, :K].repeat_interleave(2, dim=0)
    bidir = F.scaled_dot_product_attention(x["q_diff"][None, :, :K], kb[None], vb[None])[0]
    np.testing.assert_allclose(out_d[:, :K], bidir.numpy(), rtol=0, atol=1e-12)


def test_blocks_are_isolated_and_see_only_context_before_their_anchor():
    Hq, Hkv, L, N, K, D = 2, 1, 60, 4, 5, 8
    x = _inputs(Hq, Hkv, L, N, K, D, seed=5, anchors=[10, 30, 30, 55])
    base = dual_pass_forward(x["q_ar"], x["k_ar"], x["v_ar"], x["q_diff"], x["k_diff"], x["v_diff"],
                             x["anchors"], K)[2]
    y = {k: (v.clone() if torch.is_tensor(v) else v) for k, v in x.items()}
    y["k_diff"][:, 2 * K:3 * K] += 5.0          # block 2 only
    y["v_ar"][:, 30:] -= 3.0                    # clean positions >= 30
    y["k_ar"][:, 30:] *= 2.0
    out = dual_pass_forward(y["q_ar"], y["k_ar"], y["v_ar"], y["q_diff"], y["k_diff"], y["v_diff"],
                            y["anchors"], K)[2]
    for n in (0, 1):   # anchors 10 and 30: unaffected by either change
        np.testing.assert_array_equal(out[:, n * K:(n + 1) * K], base[:, n * K:(n + 1) * K])
    assert not np.allclose(out[:, 2 * K:3 * K], base[:, 2 * K:3 * K])   # its own keys moved
    assert not np.allclose(out[:, 3 * K:], base[:, 3 * K:])             # anchor 55 sees 30..54


def test_backward_finite_differences():
    Hq, Hkv, L, N, K, D = 2, 1, 12, 2, 3, 4
    x = _inputs(Hq, Hkv, L, N, K, D, seed=11, anchors=[4, 9])
    g = torch.Generator().manual_seed(5)
    d_out = torch.randn((Hq, N * K, D), generator=g, dtype=torch.float64)
    dq, dk, dv = dual_pass_backward(x["k_ar"], x["v_ar"], x["q_diff"], x["k_diff"], x["v_diff"], x["anchors"], K,
                                    d_out)

    def loss(q, k, v):
        o = dual_pass_forward(x["q_ar"], x["k_ar"], x["v_ar"], q, k, v, x["anchors"], K)[2]
        return float((o * d_out.numpy()).sum())

    h = 1e-6
    for name, grad in (("q_diff", dq), ("k_diff", dk), ("v_diff", dv)):
        t = x[name].numpy()
        for idx in [(0, 0, 0), (0, 4, 3), (t.shape[0] - 1, t.shape[1] - 1, 1)]:
            args = {n: x[n].numpy().copy() for n in ("q_diff", "k_diff", "v_diff")}
            args[name][idx] += h
            up = loss(args["q_diff"], args["k_diff"], args["v_diff"])
            args[name][idx] -= 2 * h
            dn = loss(args["q_diff"], args["k_diff"], args["v_diff"])
            assert math.isclose(grad[idx], (up - dn) / (2 * h), rel_tol=1e-5, abs_tol=1e-8), (name, idx)


def test_flops_closed_form():
    # AR: sum_{i<L} (i+1) = L(L+1)/2 keys; diffusion: K rows x (a_n + K) keys per block
    assert training_attention_flops(4, [0, 2], 2, 1, 1) == 4 * (10 + 2 * (0 + 2) + 2 * (2 + 2))
    f = training_attention_flops(2048, [1024] * 256, 32, 32, 128)
    assert f == 4 * 32 * 128 * (2048 * 2049 // 2 + 256 * 32 * (1024 + 32))
