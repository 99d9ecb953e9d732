"""GPU parity of the training dual-pass block-mask attention (forward).

The HIP path (orthrus_train_attn_fwd) against the fp64 oracle on the same
bf16 inputs: outputs within max-abs 2e-2 and relative L2 5e-3 (the bar of
the inference attention, same kernel and arithmetic), lse within 1e-3.
Cases: several shapes (D 64 / 128, K 8..32, GQA 1..8, rows per KV head past
128), anchors at 0, at L - K and past L (clamped), AR rows only, and the
full packed-sequence shape (L 2048, 256 blocks of 32, Qwen3-8B heads) on
sampled heads.
"""
import numpy as np
import pytest
import torch

import dual_view_block_amd as dvb
import oracle
from synth import train_attn_inputs
from tests._parity import assert_attn_close

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _run(x, **kw):
    res = dvb.orthrus_train_attn_fwd(x["q_ar"], x["k_ar"], x["v_ar"], x["q_diff"], x["k_diff"], x["v_diff"],
                                     x["anchors"], x["block_k"], **kw)
    torch.cuda.synchronize()
    return res


def _ref(x, heads=None):
    """Oracle on selected q heads (with their KV heads)."""
    Hq, Hkv = x["q_ar"].shape[0], x["k_ar"].shape[0]
    G = Hq // Hkv
    heads = list(range(Hq)) if heads is None else heads
    outs = []
    for h in heads:
        g = h // G
        sl = lambda t, i: t[i:i + 1].cpu()
        outs.append(oracle.dual_pass_forward(sl(x["q_ar"], h), sl(x["k_ar"], g), sl(x["v_ar"], g),
                                             sl(x["q_diff"], h), sl(x["k_diff"], g), sl(x["v_diff"], g),
                                             x["anchors"].cpu().clamp(0, x["q_ar"].shape[1]), x["block_k"]))
    cat = lambda i: np.concatenate([o[i] for o in outs], axis=0)
    return cat(0), cat(1), cat(2), cat(3), heads


def _check(x, what, heads=None):
    out_ar, lse_ar, out_d, lse_d = _run(x)
    r_ar, rl_ar, r_d, rl_d, heads = _ref(x, heads)
    idx = torch.tensor(heads, device=DEV)
    e1 = assert_attn_close(out_ar[idx], r_ar, f"{what}/ar")
    e2 = assert_attn_close(out_d[idx], r_d, f"{what}/diff")
    for got, ref, nm in ((lse_ar[idx], rl_ar, "ar"), (lse_d[idx], rl_d, "diff")):
        err = float(np.abs(got.cpu().double().numpy() - ref).max())
        assert err <= 1e-3, f"{what}/{nm} lse err {err:.3e}"
    print(f"{what}: ar max_abs={e1[0]:.2e} rel_l2={e1[1]:.2e}; diff max_abs={e2[0]:.2e} rel_l2={e2[1]:.2e}",
          flush=True)


@pytest.mark.parametrize("shape", [
    # (Hq, Hkv, L, N, K, D)
    (4, 2, 256, 8, 32, 128),
    (2, 1, 128, 5, 16, 64),
    (16, 2, 192, 6, 32, 128),   # GQA 8: 256 rows per KV head -> two row groups
    (8, 8, 96, 7, 8, 64),       # GQA 1
])
def test_forward_matches_oracle(shape):
    Hq, Hkv, L, N, K, D = shape
    _check(train_attn_inputs(Hq, Hkv, L, N, K, D, seed=sum(shape), device=DEV), f"train{shape}")


def test_anchor_edges():
    """Anchors at 0 (block sees only itself), at L - K, at L and past L (clamped)."""
    x = train_attn_inputs(4, 1, 128, 5, 32, 128, seed=3, device=DEV, anchors=[0, 96, 128, 5000, 1])
    _check(x, "anchors")


def test_ar_rows_only():
    x = train_attn_inputs(4, 2, 160, 0, 32, 128, seed=4, device=DEV)
    out_ar, lse_ar, out_d, lse_d = dvb.orthrus_train_attn_fwd(x["q_ar"], x["k_ar"], x["v_ar"])
    torch.cuda.synchronize()
    assert out_d is None and lse_d is None
    r_ar = oracle.dual_pass_forward(x["q_ar"].cpu(), x["k_ar"].cpu(), x["v_ar"].cpu(), x["q_diff"].cpu(),
                                    x["k_diff"].cpu(), x["v_diff"].cpu(), x["anchors"].cpu(), 32)[0]
    assert_attn_close(out_ar, r_ar, "ar-only")


def test_packed_sequence_full_shape_sampled_heads():
    """L 2048, 256 anchor blocks of K 32, 32 q heads / 8 KV heads, D 128: the
    benchmark launch, checked on q heads 0, 13 and 31 (every row of each)."""
    x = train_attn_inputs(32, 8, 2048, 256, 32, 128, seed=5, device=DEV)
    _check(x, "packed2048", heads=[0, 13, 31])


# ------------------------------------------------------------ backward ----
def _rel_l2(got, ref):
    g = got.detach().cpu().double().numpy()
    return float(np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-30)), float(np.abs(g - ref).max())


def _check_bwd(x, what, seed, blocks=None, kv_head=None):
    """GPU forward + backward against the fp64 oracle backward (optionally on
    selected blocks of one KV head).  The bar: relative L2 <= 1e-2 per
    gradient -- bf16 P and dS as MFMA operands (2^-9 each), bf16 O in the row
    sums and bf16 outputs give ~4e-3 -- and max-abs <= 2e-2 of the gradient's
    largest magnitude."""
    K = x["block_k"]
    _, _, out_d, lse_d = _run(x)
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    d_out = torch.randn(x["q_diff"].shape, generator=g, device=DEV).to(torch.bfloat16)
    dq, dk, dv = dvb.orthrus_train_attn_bwd(x["k_ar"], x["v_ar"], x["q_diff"], x["k_diff"], x["v_diff"],
                                            x["anchors"], K, out_d, lse_d, d_out)
    torch.cuda.synchronize()
    Hq, Hkv = x["q_ar"].shape[0], x["k_ar"].shape[0]
    G = Hq // Hkv
    N = x["anchors"].shape[0]
    blocks = list(range(N)) if blocks is None else blocks
    heads = list(range(Hkv)) if kv_head is None else [kv_head]
    rows = torch.cat([torch.arange(b * K, (b + 1) * K) for b in blocks]).to(DEV)
    qh = torch.cat([torch.arange(h * G, (h + 1) * G) for h in heads]).to(DEV)
    kh = torch.tensor(heads, device=DEV)
    sel = lambda t, hs: t[hs][:, rows].cpu()
    ref = oracle.dual_pass_backward(x["k_ar"][kh].cpu(), x["v_ar"][kh].cpu(), sel(x["q_diff"], qh),
                                    sel(x["k_diff"], kh), sel(x["v_diff"], kh),
                                    x["anchors"].cpu()[torch.tensor(blocks)].clamp(0, x["k_ar"].shape[1]), K,
                                    sel(d_out, qh))
    worst = []
    for name, got, r in (("dq", dq[qh][:, rows], ref[0]), ("dk", dk[kh][:, rows], ref[1]),
                         ("dv", dv[kh][:, rows], ref[2])):
        rl2, mabs = _rel_l2(got, r)
        bound = 2e-2 * float(np.abs(r).max())
        assert rl2 <= 1e-2 and mabs <= bound, f"{what}/{name}: rel_l2 {rl2:.2e} max_abs {mabs:.2e} (bound {bound:.2e})"
        worst.append(f"{name} rel_l2={rl2:.2e} max_abs={mabs:.2e}")
    print(f"{what}: " + "; ".join(worst), flush=True)


@pytest.mark.parametrize("shape", [
    (4, 2, 256, 8, 32, 128),
    (2, 1, 128, 5, 16, 64),
    (8, 8, 96, 7, 8, 64),
    (4, 1, 320, 6, 32, 128),
])
def test_backward_matches_oracle(shape):
    Hq, Hkv, L, N, K, D = shape
    x = train_attn_inputs(Hq, Hkv, L, N, K, D, seed=100 + sum(shape), device=DEV)
    _check_bwd(x, f"bwd{shape}", seed=sum(shape))


def test_backward_anchor_edges():
    x = train_attn_inputs(4, 1, 128, 5, 32, 128, seed=13, device=DEV, anchors=[0, 96, 128, 5000, 1])
    _check_bwd(x, "bwd-anchors", seed=13)


def test_backward_rejects_groups_past_128_rows():
    x = train_attn_inputs(8, 1, 64, 2, 32, 128, seed=1, device=DEV)
    _, _, out_d, lse_d = _run(x)
    with pytest.raises(dvb.OrthrusError) as e:
        dvb.orthrus_train_attn_bwd(x["k_ar"], x["v_ar"], x["q_diff"], x["k_diff"], x["v_diff"], x["anchors"], 32,
                                   out_d, lse_d, out_d)
    assert e.value.status == 3


def test_backward_packed_sequence_full_shape_sampled():
    """L 2048, 256 blocks of 32, 32 / 8 heads, D 128: KV heads 0 and 7 on six
    blocks each (every row, key and head_dim of them)."""
    x = train_attn_inputs(32, 8, 2048, 256, 32, 128, seed=6, device=DEV)
    for kvh in (0, 7):
        _check_bwd(x, f"bwd-packed2048-g{kvh}", seed=6, blocks=[0, 1, 100, 128, 200, 255], kv_head=kvh)
