"""GPU parity of the block attention (both views) against the fp64 oracle.

Every case calls the HIP path through the C ABI (via the ctypes binding) and
compares the whole output with the oracle on the same seeded bf16 inputs:
max-abs <= 2e-2 and relative L2 <= 5e-3 (bf16 outputs), lse within 1e-3.
Sizes span several tiles and splits, ragged tails, empty caches, K = 1..32,
GQA 1..8, more than 128 query rows per KV head, a ragged batch, and the full
long-context shapes (L = 32768 and 131072) of the benchmark launch.
"""
import math

import numpy as np
import pytest
import torch

import dual_view_block_amd as dvb
import oracle
from synth import WORKLOADS, Workload, attention_inputs
from tests._parity import assert_attn_close, assert_lse_close

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
MODES = {"diff": oracle.MASK_DIFF_BIDIR, "verify": oracle.MASK_VERIFY_CAUSAL}


def _run(x, mode, **kw):
    fn = dvb.orthrus_block_attn_diff if mode == "diff" else dvb.orthrus_block_attn_verify
    out, lse = fn(x["q"], x["k_blk"], x["v_blk"], x["k_cache"], x["v_cache"], x["cache_len"], **kw)
    torch.cuda.synchronize()
    return out, lse


def _check(x, mode, what, scale=None):
    kw = {"softmax_scale": scale} if scale else {}
    out, lse = _run(x, mode, **kw)
    ref, ref_lse = oracle.block_attention(x["q"], x["k_blk"], x["v_blk"], x["k_cache"], x["v_cache"],
                                          x["cache_len"], MODES[mode], scale=scale)
    errs = assert_attn_close(out, ref, f"{what}/{mode}")
    assert_lse_close(lse, ref_lse, f"{what}/{mode}")
    print(f"{what}/{mode}: max_abs={errs[0]:.2e} rel_l2={errs[1]:.2e}", flush=True)
    return out


def _inputs(w, **kw):
    return attention_inputs(w, device=DEV, **kw)


@pytest.mark.parametrize("mode", ["diff", "verify"])
def test_tiny_config(mode):
    """1 layer, 2 q heads / 1 KV head, D=64, L=256, K=4."""
    _check(_inputs(WORKLOADS["tiny"]), mode, "tiny")


@pytest.mark.parametrize("mode", ["diff", "verify"])
def test_qwen3_1p7b_layer(mode):
    """16 q heads / 8 KV heads (GQA 2), D=128, L=2048, K=32."""
    _check(_inputs(WORKLOADS["qwen3_1p7b_layer"]), mode, "qwen3_1p7b")


@pytest.mark.parametrize("layer", [0, 35])
@pytest.mark.parametrize("mode", ["diff", "verify"])
def test_qwen3_8b_8k_layers(mode, layer):
    """Qwen3-8B heads (GQA 4), D=128, L=8192, K=32: first and last layer inputs."""
    _check(_inputs(WORKLOADS["qwen3_8b_8k"], layer=layer), mode, f"qwen3_8b_8k[l{layer}]")


@pytest.mark.parametrize("K", [1, 4, 8, 16, 32])
@pytest.mark.parametrize("mode", ["diff", "verify"])
def test_long_context_32k_k_sweep(mode, K):
    """L=32768 at every block size of the K sweep, in the benchmark's launch shape."""
    w = WORKLOADS["qwen3_8b_32k"].replace(block_k=K)
    _check(_inputs(w), mode, f"32k/K{K}")


@pytest.mark.parametrize("L", [33000, 33918])
@pytest.mark.parametrize("mode", ["diff", "verify"])
def test_long_context_past_32k(mode, L):
    """Lengths the decode cycles reach past 32768: 32 splits of ceil(L/32) keys,
    each ending with a short tile (capacity 36864, as in the cycles)."""
    w = WORKLOADS["qwen3_8b_32k"].replace(cache_len=L, max_len=36864)
    _check(_inputs(w), mode, f"L{L}")


@pytest.mark.parametrize("K", [1, 4, 8, 16, 32])
@pytest.mark.parametrize("mode", ["diff", "verify"])
def test_long_context_128k(mode, K):
    """L=131072 at every block size of the K sweep."""
    w = WORKLOADS["qwen3_8b_128k"].replace(block_k=K)
    _check(_inputs(w), mode, f"128k/K{K}")


@pytest.mark.parametrize("K", [64, 128])
@pytest.mark.parametrize("mode", ["diff", "verify"])
def test_large_blocks_32k(mode, K):
    """K = 64 and 128 at L=32768, Qwen3-8B heads: 256 and 512 query rows per
    KV head, the shapes the block-size sweep times past K = 32."""
    w = WORKLOADS["qwen3_8b_32k"].replace(block_k=K)
    _check(_inputs(w), mode, f"32k/K{K}")


@pytest.mark.parametrize("mode", ["diff", "verify"])
def test_large_blocks_32k_rows128(mode, monkeypatch):
    """K = 64 at L=32768 with work-groups capped at 128 rows (two row groups,
    each streaming the cache): the tuning switch keeps that path exact too."""
    monkeypatch.setenv("ORTHRUS_ROWS128", "1")
    w = WORKLOADS["qwen3_8b_32k"].replace(block_k=64)
    _check(_inputs(w), mode, "32k/K64/rows128")


@pytest.mark.parametrize("mode", ["diff", "verify"])
@pytest.mark.parametrize("shape", [
    # (B, Hq, Hkv, D, L, max_len, K): 256-row work-groups, partly live
    (1, 32, 8, 128, 3000, 3008, 40),   # R = 160: five of eight query blocks live
    (2, 16, 2, 64, 1500, 1600, 33),    # GQA 8, D = 64: R = 264 -> two row groups, the second 8 rows
    (1, 32, 8, 128, 0, 64, 100),       # empty cache: two block tiles only
    (3, 8, 2, 128, 257, 300, 128),     # R = 512, ragged lengths
])
def test_wide_row_groups(mode, shape):
    B, Hq, Hkv, D, L, max_len, K = shape
    w = Workload("wide", 1, B, Hq, Hkv, D, L, K, 10, 1.0, 123, max_len=max_len)
    x = _inputs(w)
    if B > 1 and L > 1:
        x["cache_len"] = torch.tensor([L - 5 * b for b in range(B)], dtype=torch.int32, device=DEV)
    _check(x, mode, f"wide{shape}")


@pytest.mark.parametrize("mode", ["diff", "verify"])
def test_ragged_batch_of_16(mode):
    """16 sequences, L_b ~ U{1024..16384}, capacity 16384, Qwen3-8B heads."""
    w = WORKLOADS["ragged_b16"]
    x = _inputs(w)
    print("lens", x["cache_len"].tolist(), flush=True)
    _check(x, mode, "ragged_b16")


@pytest.mark.parametrize("mode", ["diff", "verify"])
@pytest.mark.parametrize("shape", [
    # (B, Hq, Hkv, D, L, max_len, K)
    (2, 8, 2, 128, 1000, 1100, 5),     # ragged tail, R = 20 rows
    (1, 4, 4, 128, 77, 128, 3),        # GQA 1, L below one tile
    (3, 6, 2, 64, 333, 400, 7),        # D = 64, R = 21
    (1, 64, 8, 128, 700, 704, 32),     # GQA 8: R = 256 rows -> 2 row groups
    (1, 12, 4, 128, 4095, 4096, 17),   # R = 51 rows, L one short of a tile multiple
    (2, 2, 1, 128, 0, 64, 6),          # empty cache: block only
    (2, 8, 8, 128, 1, 64, 1),          # one cached row, K = 1
])
def test_general_shapes(mode, shape):
    B, Hq, Hkv, D, L, max_len, K = shape
    w = Workload("gen", 1, B, Hq, Hkv, D, L, K, 10, 1.0, 99, max_len=max_len)
    x = _inputs(w)
    if B > 1 and L > 1:  # make the batch ragged
        x["cache_len"] = torch.tensor([L - 3 * b for b in range(B)], dtype=torch.int32, device=DEV)
    _check(x, mode, f"shape{shape}")


def test_custom_softmax_scale():
    w = Workload("sc", 1, 1, 8, 2, 128, 500, 8, 10, 1.0, 7)
    _check(_inputs(w), "verify", "scale0.05", scale=0.05)


def test_empty_cache_k1_verify_returns_block_value():
    """L = 0, K = 1: the only visible key is block key 0, so out = v_blk[0]."""
    w = Workload("e", 1, 1, 4, 2, 128, 0, 1, 10, 1.0, 8, max_len=64)
    x = _inputs(w)
    out, lse = _run(x, "verify")
    expect = x["v_blk"].repeat_interleave(2, dim=1)
    assert torch.equal(out, expect)
    assert torch.allclose(lse, (x["q"].float() * x["k_blk"].repeat_interleave(2, dim=1).float()).sum(-1)
                          / math.sqrt(128), atol=1e-3)


def test_rows_beyond_length_and_other_sequences_are_never_read():
    """NaN poison in cache[L_b:]: output bitwise equal to the clean run."""
    w = Workload("p", 1, 3, 8, 2, 128, 900, 6, 10, 1.0, 9, max_len=1024)
    x = _inputs(w)
    x["cache_len"] = torch.tensor([900, 129, 64], dtype=torch.int32, device=DEV)
    for mode in ("diff", "verify"):
        clean, clean_lse = _run(x, mode)
        y = dict(x)
        y["k_cache"], y["v_cache"] = x["k_cache"].clone(), x["v_cache"].clone()
        for b, L in enumerate(x["cache_len"].tolist()):
            y["k_cache"][b, :, L:] = float("nan")
            y["v_cache"][b, :, L:] = float("nan")
        got, got_lse = _run(y, mode)
        assert torch.isfinite(got.float()).all()
        assert torch.equal(clean, got) and torch.equal(clean_lse, got_lse)


def test_block_isolation_and_causality():
    """Perturbing block key j moves diffusion rows i < j but not verify rows i < j."""
    w = Workload("c", 1, 1, 8, 2, 128, 300, 8, 10, 1.0, 10)
    x = _inputs(w)
    base = {m: _run(x, m)[0].clone() for m in MODES}
    y = dict(x)
    y["k_blk"], y["v_blk"] = x["k_blk"].clone(), x["v_blk"].clone()
    y["k_blk"][:, :, 5] += 0.5
    y["v_blk"][:, :, 5] += 1.0
    pert = {m: _run(y, m)[0] for m in MODES}
    for i in range(8):
        assert torch.equal(base["verify"][:, :, i], pert["verify"][:, :, i]) == (i < 5), i
        assert not torch.equal(base["diff"][:, :, i], pert["diff"][:, :, i])


def test_verify_matches_sequential_decode_steps():
    """Verify row i == a K=1 decode call with the cache extended by block rows < i."""
    K, L = 6, 517
    w = Workload("s", 1, 1, 8, 2, 128, L, K, 10, 1.0, 11, max_len=L + K)
    x = _inputs(w)
    out, _ = _run(x, "verify")
    for i in range(K):
        kc, vc = x["k_cache"].clone(), x["v_cache"].clone()
        kc[:, :, L:L + i] = x["k_blk"][:, :, :i]
        vc[:, :, L:L + i] = x["v_blk"][:, :, :i]
        one = {"q": x["q"][:, :, i:i + 1].contiguous(), "k_blk": x["k_blk"][:, :, i:i + 1].contiguous(),
               "v_blk": x["v_blk"][:, :, i:i + 1].contiguous(), "k_cache": kc, "v_cache": vc,
               "cache_len": torch.tensor([L + i], dtype=torch.int32, device=DEV)}
        step, _ = _run(one, "diff")
        d = (out[:, :, i:i + 1].float() - step.float()).abs().max().item()
        assert d <= 1e-2, (i, d)


def test_cache_is_never_written_and_runs_are_deterministic():
    w = WORKLOADS["qwen3_1p7b_layer"]
    x = _inputs(w)
    ksum = x["k_cache"].view(torch.int16).sum(dtype=torch.int64).item()
    vsum = x["v_cache"].view(torch.int16).sum(dtype=torch.int64).item()
    for mode in MODES:
        a, la = _run(x, mode)
        a, la = a.clone(), la.clone()
        b, lb = _run(x, mode)
        assert torch.equal(a, b) and torch.equal(la, lb)
    assert x["k_cache"].view(torch.int16).sum(dtype=torch.int64).item() == ksum
    assert x["v_cache"].view(torch.int16).sum(dtype=torch.int64).item() == vsum


def test_workspace_is_independent_of_cached_length():
    """One workspace serves every L: same size query, and reusing it across
    different lengths gives the same results as fresh workspaces."""
    w = Workload("ws", 1, 1, 32, 8, 128, 4096, 32, 10, 1.0, 12)
    x = _inputs(w)
    desc = dvb.attn_desc(x["q"], x["k_cache"])
    ws = torch.zeros(dvb.orthrus_attn_workspace_size(desc), dtype=torch.uint8, device=DEV)
    for L in (4096, 100, 2500):
        x["cache_len"].fill_(L)
        shared, _ = _run(x, "diff", workspace=ws)
        shared = shared.clone()
        fresh, _ = _run(x, "diff")
        assert torch.equal(shared, fresh)


@pytest.mark.parametrize("mode", ["diff", "verify"])
def test_partial_merge_entry_points_agree_bitwise(mode):
    """orthrus_block_attn_partial followed by orthrus_block_attn_merge gives
    the bits of the one-call entry point, and neither needs an initialised
    workspace (it is filled with NaN bytes first)."""
    w = WORKLOADS["qwen3_8b_8k"]
    x = _inputs(w)
    ref, ref_lse = (t.clone() for t in _run(x, mode))
    desc = dvb.attn_desc(x["q"], x["k_cache"])
    assert dvb.orthrus_attn_num_splits(desc) > 1
    ws = torch.full((dvb.orthrus_attn_workspace_size(desc),), 0xFF, dtype=torch.uint8, device=DEV)
    out = torch.empty_like(x["q"])
    lse = torch.empty(x["q"].shape[:3], dtype=torch.float32, device=DEV)
    m = dvb.ORTHRUS_MASK_DIFF_BIDIR if mode == "diff" else dvb.ORTHRUS_MASK_VERIFY_CAUSAL
    call = dvb.PreparedAttention(m, x["q"], x["k_blk"], x["v_blk"], x["k_cache"], x["v_cache"],
                                 x["cache_len"], out, lse, ws)
    s = torch.cuda.current_stream().cuda_stream
    call.partial(s)
    call.merge(s)
    torch.cuda.synchronize()
    assert torch.equal(ref, out) and torch.equal(ref_lse, lse)
    ws.fill_(0xFF)
    call(s)
    torch.cuda.synchronize()
    assert torch.equal(ref, out) and torch.equal(ref_lse, lse)


@pytest.mark.parametrize("mode", ["diff", "verify"])
def test_single_split_direct_output(mode, monkeypatch):
    """With the split count capped at one the streaming kernel writes the
    output itself (no merge launch); it must meet the same oracle bar."""
    monkeypatch.setenv("ORTHRUS_MAX_SPLITS", "1")
    _check(_inputs(WORKLOADS["qwen3_1p7b_layer"]), mode, "one_split")


@pytest.mark.parametrize("mode", ["diff", "verify"])
@pytest.mark.parametrize("lens", [
    [16384, 1024, 1024, 1024],          # one long sequence takes most of the work-groups
    [0, 5000, 64, 16383],               # an empty cache, a one-tile cache, ragged tails
    [3000, 3000, 3000, 3000, 3000, 3000],
])
def test_ragged_batches_shared_by_length(mode, lens):
    """Several sequences: the launch's work-groups are shared out by cache
    length on the device (a long sequence gets more splits per KV head)."""
    B = len(lens)
    w = Workload("rag", 1, B, 32, 8, 128, max(lens), 32, 10, 1.0, 41 + B, max_len=16384)
    x = _inputs(w)
    x["cache_len"] = torch.tensor(lens, dtype=torch.int32, device=DEV)
    _check(x, mode, f"ragged{lens}")
