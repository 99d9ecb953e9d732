"""Pins for the attention oracle (CPU only).

Each test checks the oracle against something other than itself: a
hand-derived closed form, torch's float64 scaled_dot_product_attention (a
library routine with its own GQA and causal handling), invariants the pages fix
(verify = K sequential decode steps, the diffusion block never sees cache rows
at or after its anchor), and closed forms (q = 0 averages the visible values).
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle.attention import MASK_DIFF_BIDIR as DIFF, MASK_VERIFY_CAUSAL as VERIFY
from synth import Workload, attention_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _val(x):
    """Fixture literal: a number, "ln<a>" or "<c>*ln<a>"."""
    if isinstance(x, str):
        coef, _, arg = x.rpartition("ln")
        c = float(coef.rstrip("*")) if coef else 1.0
        return c * math.log(float(arg))
    return float(x)


def _arr(rows):
    return np.array([[_val(v) for v in r] for r in rows], dtype=np.float64)


def test_hand_derived_closed_form():
    fx = json.load(open(os.path.join(GOLDEN, "attention_hand.json")))
    q = _arr(fx["q"])[None, None]                      # [1,1,2,4]
    kc = _arr(fx["k_cache"])[None, None]               # [1,1,1,4]
    vc = _arr(fx["v_cache"])[None, None]
    kb = _arr(fx["k_blk_first_coord_log"])[None, None]  # [1,1,2,4]
    vb = _arr(fx["v_blk"])[None, None]
    for name, mode in (("verify", VERIFY), ("diff", DIFF)):
        out, lse = oracle.block_attention(q, kb, vb, kc, vc, [1], mode)
        exp_out = _arr(fx["expected"][name]["out"])
        exp_lse = np.array([_val(v) for v in fx["expected"][name]["lse"]])
        np.testing.assert_allclose(out[0, 0], exp_out, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[0, 0], exp_lse, rtol=0, atol=1e-12)


def _rand_case(B=2, Hq=4, Hkv=2, K=5, D=16, max_len=40, lens=(33, 17), seed=0):
    w = Workload("t", 1, B, Hq, Hkv, D, max_len, K, 10, 1.0, seed)
    x = attention_inputs(w, seed_offset=seed)
    x["cache_len"] = torch.tensor(lens[:B], dtype=torch.int32)
    return x


def _sdpa(q, keys, vals, mask=None, causal=False, gqa=True):
    return F.scaled_dot_product_attention(q, keys, vals, attn_mask=mask, is_causal=causal,
                                          enable_gqa=gqa)


@pytest.mark.parametrize("mode", [DIFF, VERIFY])
def test_k1_is_single_token_decode(mode):
    """K = 1: both views reduce to ordinary decode attention over L + 1 keys."""
    x = _rand_case(K=1, lens=(33, 17))
    out, _ = oracle.block_attention(x["q"], x["k_blk"], x["v_blk"], x["k_cache"], x["v_cache"],
                                    x["cache_len"], mode)
    for b, L in enumerate(x["cache_len"].tolist()):
        keys = torch.cat([x["k_cache"][b, :, :L], x["k_blk"][b]], dim=1).double()
        vals = torch.cat([x["v_cache"][b, :, :L], x["v_blk"][b]], dim=1).double()
        ref = _sdpa(x["q"][b].double(), keys, vals)
        np.testing.assert_allclose(out[b], ref.numpy(), rtol=1e-12, atol=1e-12)


def test_empty_cache_reduces_to_plain_block_attention():
    """L = 0: diffusion = non-causal attention over the block, verify = causal."""
    x = _rand_case(lens=(0, 0))
    for mode, causal in ((DIFF, False), (VERIFY, True)):
        out, _ = oracle.block_attention(x["q"], x["k_blk"], x["v_blk"], x["k_cache"],
                                        x["v_cache"], x["cache_len"], mode)
        ref = _sdpa(x["q"].double(), x["k_blk"].double(), x["v_blk"].double(), causal=causal)
        np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_verify_equals_sequential_decode():
    """Verify row i == one decode step with the cache extended by block keys < i."""
    x = _rand_case(K=6, lens=(21, 9))
    out, lse = oracle.block_attention(x["q"], x["k_blk"], x["v_blk"], x["k_cache"], x["v_cache"],
                                      x["cache_len"], VERIFY)
    for b, L in enumerate(x["cache_len"].tolist()):
        for i in range(6):
            kc = torch.cat([x["k_cache"][b:b + 1, :, :L], x["k_blk"][b:b + 1, :, :i]], dim=2)
            vc = torch.cat([x["v_cache"][b:b + 1, :, :L], x["v_blk"][b:b + 1, :, :i]], dim=2)
            o1, l1 = oracle.block_attention(x["q"][b:b + 1, :, i:i + 1], x["k_blk"][b:b + 1, :, i:i + 1],
                                            x["v_blk"][b:b + 1, :, i:i + 1], kc, vc, [L + i], DIFF)
            np.testing.assert_allclose(out[b, :, i], o1[0, :, 0], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(lse[b, :, i], l1[0, :, 0], rtol=1e-12, atol=1e-12)


def test_later_block_keys_reach_diffusion_rows_only():
    """Changing block key j > i moves diffusion row i, never verify row i."""
    x = _rand_case(K=5, lens=(12, 30))
    base = {m: oracle.block_attention(x["q"], x["k_blk"], x["v_blk"], x["k_cache"], x["v_cache"],
                                      x["cache_len"], m)[0] for m in (DIFF, VERIFY)}
    y = dict(x)
    y["k_blk"] = x["k_blk"].clone()
    y["v_blk"] = x["v_blk"].clone()
    y["k_blk"][:, :, 3] += 1.0
    y["v_blk"][:, :, 3] -= 2.0
    pert = {m: oracle.block_attention(y["q"], y["k_blk"], y["v_blk"], y["k_cache"], y["v_cache"],
                                      y["cache_len"], m)[0] for m in (DIFF, VERIFY)}
    for i in range(5):
        same_v = np.array_equal(base[VERIFY][:, :, i], pert[VERIFY][:, :, i])
        assert same_v == (i < 3), i
        assert not np.allclose(base[DIFF][:, :, i], pert[DIFF][:, :, i])


def test_zero_query_averages_visible_values():
    """q = 0: uniform weights, so out = mean of the visible V rows, lse = ln(count)."""
    x = _rand_case(K=4, lens=(10, 0))
    x["q"] = torch.zeros_like(x["q"])
    G = 2
    for mode in (DIFF, VERIFY):
        out, lse = oracle.block_attention(x["q"], x["k_blk"], x["v_blk"], x["k_cache"],
                                          x["v_cache"], x["cache_len"], mode)
        for b, L in enumerate(x["cache_len"].tolist()):
            for h in range(4):
                g = h // G
                for i in range(4):
                    nblk = 4 if mode == DIFF else i + 1
                    vis = torch.cat([x["v_cache"][b, g, :L], x["v_blk"][b, g, :nblk]]).double()
                    np.testing.assert_allclose(out[b, h, i], vis.mean(0).numpy(), atol=1e-12)
                    assert abs(lse[b, h, i] - math.log(L + nblk)) < 1e-12


def test_cache_rows_at_or_after_len_are_never_read():
    """NaN poison in cache[L_b:] leaves every output unchanged (bitwise)."""
    x = _rand_case(K=3, lens=(25, 7))
    ref = oracle.block_attention(x["q"], x["k_blk"], x["v_blk"], x["k_cache"], x["v_cache"],
                                 x["cache_len"], DIFF)
    kc, vc = x["k_cache"].clone(), x["v_cache"].clone()
    for b, L in enumerate(x["cache_len"].tolist()):
        kc[b, :, L:] = float("nan")
        vc[b, :, L:] = float("nan")
    got = oracle.block_attention(x["q"], x["k_blk"], x["v_blk"], kc, vc, x["cache_len"], DIFF)
    assert np.array_equal(ref[0], got[0]) and np.array_equal(ref[1], got[1])


def test_general_shape_matches_sdpa_with_explicit_mask():
    """Ragged batch, GQA 2, general L and K, against float64 SDPA."""
    x = _rand_case(B=2, Hq=4, Hkv=2, K=5, lens=(33, 17))
    for mode in (DIFF, VERIFY):
        out, lse = oracle.block_attention(x["q"], x["k_blk"], x["v_blk"], x["k_cache"],
                                          x["v_cache"], x["cache_len"], mode)
        for b, L in enumerate(x["cache_len"].tolist()):
            keys = torch.cat([x["k_cache"][b, :, :L], x["k_blk"][b]], dim=1).double()
            vals = torch.cat([x["v_cache"][b, :, :L], x["v_blk"][b]], dim=1).double()
            blk = torch.ones(5, 5, dtype=torch.bool)
            if mode == VERIFY:
                blk = torch.tril(blk)
            mask = torch.cat([torch.ones(5, L, dtype=torch.bool), blk], dim=1)
            ref = _sdpa(x["q"][b].double(), keys, vals, mask=mask)
            np.testing.assert_allclose(out[b], ref.numpy(), rtol=1e-12, atol=1e-12)
            # lse against torch.logsumexp of the masked scores
            s = (x["q"][b].double() @ keys.repeat_interleave(2, 0).transpose(1, 2)) / math.sqrt(16)
            s = s.masked_fill(~mask, float("-inf"))
            np.testing.assert_allclose(lse[b], torch.logsumexp(s, -1).numpy(), rtol=0, atol=1e-12)


def test_row_sampler_matches_full_evaluation():
    x = _rand_case(K=5, lens=(33, 17))
    rows = [(0, 0, 0), (1, 3, 4), (0, 2, 2), (1, 1, 0)]
    for mode in (DIFF, VERIFY):
        out, lse = oracle.block_attention(x["q"], x["k_blk"], x["v_blk"], x["k_cache"],
                                          x["v_cache"], x["cache_len"], mode)
        o2, l2 = oracle.block_attention_rows(x["q"], x["k_blk"], x["v_blk"], x["k_cache"],
                                             x["v_cache"], x["cache_len"], mode, rows)
        for n, (b, h, i) in enumerate(rows):
            np.testing.assert_allclose(o2[n], out[b, h, i], rtol=0, atol=1e-13)
            assert abs(l2[n] - lse[b, h, i]) < 1e-13


def test_transient_kv_is_4p5_mib_and_has_no_length_argument():
    """Qwen3-8B shape, K = 32: 36 x 8 x 32 x 128 x 2 (K,V) x 2 B = 4.5 MiB exactly."""
    assert oracle.transient_kv_bytes(36, 8, 128, 32) == 4718592 == int(4.5 * 2 ** 20)
    import inspect
    params = inspect.signature(oracle.transient_kv_bytes).parameters
    assert not any("len" in p for p in params)
