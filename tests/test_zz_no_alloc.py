"""GPU test of orthrus_block_attn_noalloc (the entry point that allocates
nothing and runs on the library's per-device scratch): two calls in a row,
the second on a smaller problem, each bit-identical to orthrus_block_attn
with a caller workspace on the same inputs, and both within the oracle bar."""
import pytest
import torch

import dual_view_block_amd as dvb
import oracle
from synth import WORKLOADS, Workload, attention_inputs
from tests._parity import assert_attn_close, assert_lse_close

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _both(x, mode):
    ref_out, ref_lse = dvb.orthrus_block_attn(x["q"], x["k_blk"], x["v_blk"], x["k_cache"], x["v_cache"],
                                              x["cache_len"], mode)
    out = torch.full_like(x["q"], float("nan"))
    lse = torch.full(x["q"].shape[:3], float("nan"), dtype=torch.float32, device=DEV)
    dvb.orthrus_block_attn_noalloc(x["q"], x["k_blk"], x["v_blk"], x["k_cache"], x["v_cache"], x["cache_len"],
                                   mode, out, lse)
    torch.cuda.synchronize()
    return ref_out, ref_lse, out, lse


def test_noalloc_matches_the_workspace_entry_point_twice():
    cases = [
        # Qwen3-8B heads, L 8192, K 32, diffusion view: 32 splits per KV head
        (WORKLOADS["qwen3_8b_8k"], dvb.ORTHRUS_MASK_DIFF_BIDIR, oracle.MASK_DIFF_BIDIR),
        # then a smaller problem on the same scratch: 16 / 8 heads, ragged B 2, L <= 1000, K 7, verify
        (Workload("small", 1, 2, 16, 8, 128, 1000, 7, 10, 1.0, 5, max_len=1024), dvb.ORTHRUS_MASK_VERIFY_CAUSAL,
         oracle.MASK_VERIFY_CAUSAL),
    ]
    for n, (w, mode, omode) in enumerate(cases):
        x = attention_inputs(w, device=DEV)
        if w.batch > 1:
            x["cache_len"] = torch.tensor([1000, 333], dtype=torch.int32, device=DEV)
        ref_out, ref_lse, out, lse = _both(x, mode)
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), f"call {n}: differs from orthrus_block_attn"
        r, rl = oracle.block_attention(x["q"], x["k_blk"], x["v_blk"], x["k_cache"], x["v_cache"], x["cache_len"],
                                       omode)
        e = assert_attn_close(out, r, f"noalloc call {n}")
        assert_lse_close(lse, rl, f"noalloc call {n}")
        print(f"noalloc call {n} ({w.name}): bit-identical; max_abs={e[0]:.2e} rel_l2={e[1]:.2e}", flush=True)


def test_noalloc_wide_row_groups():
    """K = 64 at Qwen3-8B heads (256-row work-groups, 32 splits: 17.3 MB of
    partials) fits the scratch and matches the workspace entry point bit for bit."""
    w = WORKLOADS["qwen3_8b_8k"].replace(block_k=64)
    x = attention_inputs(w, device=DEV)
    assert dvb.orthrus_attn_workspace_size(dvb.attn_desc(x["q"], x["k_cache"])) > 16 << 20
    ref_out, ref_lse, out, lse = _both(x, dvb.ORTHRUS_MASK_VERIFY_CAUSAL)
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
    r, rl = oracle.block_attention(x["q"], x["k_blk"], x["v_blk"], x["k_cache"], x["v_cache"], x["cache_len"],
                                   oracle.MASK_VERIFY_CAUSAL)
    e = assert_attn_close(out, r, "noalloc K64")
    assert_lse_close(lse, rl, "noalloc K64")
    print(f"noalloc K64: bit-identical; max_abs={e[0]:.2e} rel_l2={e[1]:.2e}", flush=True)


def test_noalloc_refuses_a_workspace_past_the_scratch():
    w = WORKLOADS["qwen3_8b_8k"].replace(batch=256, cache_len=64)
    x = attention_inputs(w, device=DEV)
    out = torch.empty_like(x["q"])
    with pytest.raises(dvb.OrthrusError) as e:
        dvb.orthrus_block_attn_noalloc(x["q"], x["k_blk"], x["v_blk"], x["k_cache"], x["v_cache"], x["cache_len"],
                                       dvb.ORTHRUS_MASK_DIFF_BIDIR, out)
    assert e.value.status == 3
