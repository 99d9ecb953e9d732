"""GPU parity of the balanced placement for batches of several sequences.

With B > 1 the launch's work-groups share one list of work: per (sequence,
KV-head group) a segment of cost units and tiles, divided evenly, so one
group's partials can come from many work-groups and a work-group can hold
pieces of several groups.  The cases below are built so that a group is cut
into more pieces than the merge folds in one step, so that a piece starts
inside the block-key tiles (K = 128: two block tiles), so that there are
fewer units of work than work-groups, and so that a batch of 100 sequences
spans two lanes' worth of sequence slots.  Each case is checked against the
fp64 oracle (max-abs 2e-2, relative L2 5e-3, lse 1e-3).  `_pieces` restates
the placement arithmetic so that each test can assert that its case has the
property it is there for.
"""
import numpy as np
import pytest
import torch

import dual_view_block_amd as dvb
import oracle
from synth import Workload, attention_inputs
from tests._parity import assert_attn_close, assert_lse_close

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
MODES = {"diff": oracle.MASK_DIFF_BIDIR, "verify": oracle.MASK_VERIFY_CAUSAL}
PIECE_COST = 6  # cost units at the head of every segment


def _cdiv(a, b):
    return -(-a // b)


def _pieces(lens, K, H, N):
    """(work-group, segment, first tile, end tile) of every piece, W, n."""
    nb = _cdiv(K, 64)
    seg_units = [PIECE_COST + nb + _cdiv(L, 64) for L in lens]
    base, acc = [], 0
    for s in seg_units:
        base.append(acc)
        acc += H * s
    W = acc
    n = min(N, W)
    out = []
    for w in range(n):
        T, T1 = W * w // n, W * (w + 1) // n
        while T < T1:
            b = max(i for i in range(len(lens)) if base[i] <= T)
            off = T - base[b]
            h, u0 = divmod(off, seg_units[b])
            u1 = min(seg_units[b], T1 - (base[b] + h * seg_units[b]))
            T += u1 - u0
            p0, p1 = max(u0 - PIECE_COST, 0), max(u1 - PIECE_COST, 0)
            if p0 < p1:
                out.append((w, b * H + h, p0, p1))
    return out, W, n


def _case(lens, Hq, Hkv, D, K, seed):
    B = len(lens)
    w = Workload("bal", 1, B, Hq, Hkv, D, max(max(lens), 1), K, 10, 1.0, seed, max_len=max(max(lens), 4096))
    x = attention_inputs(w, device=DEV)
    x["cache_len"] = torch.tensor(lens, dtype=torch.int32, device=DEV)
    desc = dvb.attn_desc(x["q"], x["k_cache"])
    splits = dvb.orthrus_attn_num_splits(desc)
    rows = (Hq // Hkv) * K
    qblocks = 1 if rows <= 32 else (2 if rows <= 64 else 4)
    row_groups = _cdiv(rows, 32 * qblocks)
    H = Hkv * row_groups
    assert splits > 1, "the balanced placement needs more than one split"
    pieces, W, n = _pieces(lens, K, H, B * H * splits)
    return x, pieces, W, n


def _check(x, mode, what):
    fn = dvb.orthrus_block_attn_diff if mode == "diff" else dvb.orthrus_block_attn_verify
    out, lse = fn(x["q"], x["k_blk"], x["v_blk"], x["k_cache"], x["v_cache"], x["cache_len"])
    torch.cuda.synchronize()
    ref, ref_lse = oracle.block_attention(x["q"], x["k_blk"], x["v_blk"], x["k_cache"], x["v_cache"],
                                          x["cache_len"], MODES[mode])
    errs = assert_attn_close(out, ref, f"{what}/{mode}")
    assert_lse_close(lse, ref_lse, f"{what}/{mode}")
    print(f"{what}/{mode}: max_abs={errs[0]:.2e} rel_l2={errs[1]:.2e}", flush=True)


@pytest.mark.parametrize("mode", ["diff", "verify"])
@pytest.mark.parametrize("D", [128, 64])
def test_one_long_sequence_among_short_ones(mode, D):
    """One 16000-key sequence among 15 of 0..1000 keys: each of the long
    sequence's groups is cut into more than 16 pieces (the merge folds four
    at a time), and short groups share work-groups."""
    lens = [16000, 37, 0, 150, 1, 64, 65, 2, 300, 0, 5, 128, 129, 1000, 7, 63]
    Hq = 32 if D == 128 else 16
    x, pieces, _, _ = _case(lens, Hq, 8, D, 32, seed=71 + D)
    per_seg = np.bincount([p[1] for p in pieces])
    assert per_seg.max() > 16, per_seg.max()
    assert max(np.bincount([p[0] for p in pieces])) >= 2  # a work-group with several pieces
    _check(x, mode, f"long-among-short D{D}")


@pytest.mark.parametrize("mode", ["diff", "verify"])
def test_piece_starting_inside_the_block_tiles(mode):
    """K = 128 (two block-key tiles per segment): lengths chosen (by a seeded
    search over the placement) so that some piece starts at the second block
    tile, and another one ends after the first."""
    K, Hq, Hkv = 128, 8, 8
    rng = np.random.default_rng(5)
    for _ in range(2000):
        lens = [int(v) for v in rng.integers(0, 3000, size=4)]
        pieces, _, _ = _pieces(lens, K, Hkv, 4 * Hkv * (256 // (4 * Hkv)))
        if any(p[2] == 1 for p in pieces) and any(p[3] == 1 for p in pieces):
            break
    else:
        pytest.fail("no length set puts a piece boundary between the block tiles")
    x, pieces, _, _ = _case(lens, Hq, Hkv, 128, K, seed=17)
    assert any(p[2] == 1 for p in pieces) and any(p[3] == 1 for p in pieces), lens
    _check(x, mode, f"block-tile boundary {lens}")


@pytest.mark.parametrize("mode", ["diff", "verify"])
@pytest.mark.parametrize("lens", [[0, 0], [0, 70], [3, 1]])
def test_fewer_units_than_work_groups(mode, lens):
    """Two short sequences: fewer units of work than work-groups, so each
    used work-group takes one unit and most hold no tile at all."""
    x, pieces, W, n = _case(lens, 32, 8, 128, 8, seed=23)
    assert W == n  # one unit per used work-group
    _check(x, mode, f"few units {lens}")


@pytest.mark.parametrize("mode", ["diff", "verify"])
def test_hundred_sequences(mode):
    """100 sequences of 0..3000 keys with one KV head (two splits each): the
    sequence scan covers two 64-sequence lane slots."""
    rng = np.random.default_rng(9)
    lens = [int(v) for v in rng.integers(0, 3000, size=100)]
    x, pieces, _, _ = _case(lens, 2, 1, 128, 4, seed=31)
    assert len({p[1] for p in pieces}) == 100
    _check(x, mode, "100 sequences")


@pytest.mark.parametrize("mode", ["diff", "verify"])
def test_unsplit_batch_taken_longest_first(mode):
    """40 sequences of 0..4000 keys with 8 KV heads: 320 groups, so one
    work-group per group and no split; the work-groups take the sequences
    longest first (ranked on the device from the lengths)."""
    rng = np.random.default_rng(13)
    lens = [int(v) for v in rng.integers(0, 4000, size=40)]
    w = Workload("unsplit", 1, 40, 32, 8, 128, max(lens), 32, 10, 1.0, 43, max_len=4096)
    x = attention_inputs(w, device=DEV)
    x["cache_len"] = torch.tensor(lens, dtype=torch.int32, device=DEV)
    assert dvb.orthrus_attn_num_splits(dvb.attn_desc(x["q"], x["k_cache"])) == 1
    _check(x, mode, "unsplit batch of 40")

