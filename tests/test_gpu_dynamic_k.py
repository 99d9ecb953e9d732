"""GPU parity of dynamic block sizes (a block length per sequence).

Every entry point with a per-sequence block length k_b is checked against
``oracle.dynamic`` on the same seeded inputs:

* attention (``orthrus_block_attn_dyn``): the rows of each sequence's first
  k_b positions within max-abs 2e-2 / relative L2 5e-3 (lse 1e-3), and every
  row past k_b left exactly as it was (out and lse are pre-filled with a
  marker).  The cases cover the one-sequence split launch (query blocks past
  G k_b idle), the balanced launch of several sequences, K = 128 with row
  groups that hold no live row, the single-split launch that writes the
  output directly, head_dim 64, and k_b = 1 and k_b = K.
* greedy and T>0 consensus, the commit with its block-length rule, and whole
  decode cycles: bit-exact integers and cache bytes.
"""
import numpy as np
import pytest
import torch

import dual_view_block_amd as dvb
import oracle
from dual_view_block_amd.cycle import DecodeCycles
from oracle.cycle import bits_to_bf16
from synth import Workload, attention_inputs, cycle_inputs, greedy_inputs, sample_inputs
from tests._parity import assert_attn_close, assert_lse_close

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
MODES = {"diff": oracle.MASK_DIFF_BIDIR, "verify": oracle.MASK_VERIFY_CAUSAL}
MARK_OUT = 3.0      # bf16-exact marker for rows that must stay untouched
MARK_LSE = -7.0


def _inputs(B, Hq, Hkv, D, K, lens, max_len, seed):
    w = Workload("dyn", 1, B, Hq, Hkv, D, max(max(lens), 1), K, 10, 1.0, seed, max_len=max_len)
    x = attention_inputs(w, device=DEV)
    x["cache_len"] = torch.tensor(lens, dtype=torch.int32, device=DEV)
    return x


def _check_attn(x, kl, mode, what):
    B, Hq, K, D = x["q"].shape
    blk = torch.tensor(kl, dtype=torch.int32, device=DEV)
    out = torch.full_like(x["q"], MARK_OUT)
    lse = torch.full(x["q"].shape[:3], MARK_LSE, dtype=torch.float32, device=DEV)
    dvb.orthrus_block_attn_dyn(x["q"], x["k_blk"], x["v_blk"], x["k_cache"], x["v_cache"], x["cache_len"], blk,
                               MODES[mode], out=out, lse=lse)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.block_attention_dyn(x["q"], x["k_blk"], x["v_blk"], x["k_cache"], x["v_cache"],
                                              x["cache_len"], kl, MODES[mode])
    live_g = torch.cat([out[b, :, :k].reshape(-1, D) for b, k in enumerate(kl)])
    live_r = np.concatenate([ref[b, :, :k].reshape(-1, D) for b, k in enumerate(kl)])
    errs = assert_attn_close(live_g, live_r, f"{what}/{mode}")
    assert_lse_close(torch.cat([lse[b, :, :k].reshape(-1) for b, k in enumerate(kl)]),
                     np.concatenate([ref_lse[b, :, :k].reshape(-1) for b, k in enumerate(kl)]), f"{what}/{mode}")
    for b, k in enumerate(kl):
        assert bool((out[b, :, k:] == MARK_OUT).all()), f"{what}/{mode}: row past k_b={k} written (b={b})"
        assert bool((lse[b, :, k:] == MARK_LSE).all()), f"{what}/{mode}: lse past k_b={k} written (b={b})"
    print(f"{what}/{mode} k={kl}: max_abs={errs[0]:.2e} rel_l2={errs[1]:.2e}", flush=True)


@pytest.mark.parametrize("mode", ["diff", "verify"])
@pytest.mark.parametrize("k", [1, 5, 20, 31, 32])
def test_one_sequence_qwen3_8b_heads(mode, k):
    """Qwen3-8B heads, K = 32, L = 3000 (32 splits): the 4 k rows of each KV
    head fill ceil(4k / 32) of the work-group's 4 query blocks."""
    x = _inputs(1, 32, 8, 128, 32, [3000], 4096, seed=100 + k)
    _check_attn(x, [k], mode, "one sequence")


@pytest.mark.parametrize("mode", ["diff", "verify"])
def test_balanced_batch(mode):
    """Four sequences of 0..5000 keys (the balanced placement) with block
    lengths 1, 32, 7 and 17."""
    x = _inputs(4, 32, 8, 128, 32, [0, 5000, 130, 2048], 5120, seed=7)
    _check_attn(x, [1, 32, 7, 17], mode, "balanced")


@pytest.mark.parametrize("mode", ["diff", "verify"])
@pytest.mark.parametrize("lens,kl", [([700], [5]), ([700], [64]), ([700], [72]), ([700], [100]), ([700], [128]),
                                     ([700, 0, 300], [5, 128, 64]), ([2500, 40], [20, 33])])
def test_large_block_row_groups(mode, lens, kl):
    """K = 128 with G = 4: 512 rows in 4 row groups of 128.  With k_b = 5 three
    of them hold no live row, and the head's 32 work-groups are dealt to the
    live one as 32 splits; k_b = 72 leaves 3 live row groups, dealt 11, 11
    and 10 splits.  The batches take the balanced placement, where a short
    block's dead row groups get no segment."""
    x = _inputs(len(lens), 32, 8, 128, 128, lens, 1024, seed=sum(kl))
    _check_attn(x, kl, mode, "K=128")


@pytest.mark.parametrize("mode", ["diff", "verify"])
@pytest.mark.parametrize("D,Hq", [(128, 32), (64, 16)])
def test_single_split_direct_write(mode, D, Hq):
    """Capacity 64: one split, so the streaming kernel writes the rows itself."""
    x = _inputs(1, Hq, 8, D, 16, [40], 64, seed=D)
    _check_attn(x, [9], mode, f"direct D{D}")


@pytest.mark.parametrize("mode", ["diff", "verify"])
def test_head_dim_64_batch(mode):
    x = _inputs(2, 16, 8, 64, 32, [1000, 77], 1024, seed=64)
    _check_attn(x, [13, 32], mode, "D64")


def test_greedy_consensus():
    """Six sequences, K = 32, V = 151936, block lengths 1..32 with first
    mismatches before, at and after the block end."""
    w = Workload("g", 1, 6, 32, 8, 128, 1, 32, 151936, 3.0, 51)
    js = torch.tensor([0, 3, 20, 32, 5, 8])
    kl = [1, 5, 16, 32, 32, 8]
    logits, cand, _ = greedy_inputs(w, first_mismatch=js)
    ref_a, ref_am, ref_c = oracle.greedy_consensus_dyn(logits, cand, kl)
    am = torch.full((6, 32), 12345, dtype=torch.int32, device=DEV)
    a, am, c = dvb.orthrus_consensus_greedy_dyn(logits.to(DEV), cand.to(DEV),
                                                torch.tensor(kl, dtype=torch.int32, device=DEV), row_argmax=am)
    torch.cuda.synchronize()
    assert a.cpu().tolist() == ref_a.tolist() == [0, 3, 16, 32, 5, 8]
    assert c.cpu().tolist() == ref_c.tolist()
    assert np.array_equal(am.cpu().numpy(), ref_am)
    print(f"greedy dyn: a={a.cpu().tolist()} corr={c.cpu().tolist()}", flush=True)


@pytest.mark.parametrize("noise", [None, 0.3])
def test_sample_consensus(noise):
    """T>0 over block lengths 1..16 of K = 16, V = 8192; with a draft close to
    the target (noise 0.3) acceptance runs to the block end."""
    w = Workload("s", 1, 6, 32, 8, 128, 1, 16, 8192, 3.0, 52)
    p, q, cand, u = sample_inputs(w, draft_noise=noise)
    kl = [1, 2, 5, 16, 9, 16]
    ref_a, ref_c = oracle.sample_consensus_dyn(p, q, cand, u, kl)
    a, c = dvb.orthrus_consensus_sample_dyn(p.to(DEV), q.to(DEV), cand.to(DEV), u.to(DEV),
                                            torch.tensor(kl, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    assert a.cpu().tolist() == ref_a.tolist()
    assert c.cpu().tolist() == ref_c.tolist()
    print(f"sample dyn noise={noise}: a={a.cpu().tolist()} corr={c.cpu().tolist()}", flush=True)


def _bf16(shape, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=DEV).to(torch.bfloat16)


def test_commit_and_block_length_rule():
    """Three layers, eight sequences: whole blocks, early mismatches, a = k_b
    at k_b = 1, a > k_b (refused), a cache that fills exactly and one that
    overflows (refused), k_b out of range (clamped); then the next lengths."""
    n_layers, B, Hkv, D, K, max_len = 3, 8, 8, 128, 32, 300
    kc, vc = _bf16((n_layers, B, Hkv, max_len, D), 1), _bf16((n_layers, B, Hkv, max_len, D), 2)
    kb, vb = _bf16((n_layers, B, Hkv, K, D), 3), _bf16((n_layers, B, Hkv, K, D), 4)
    lens = [10, 10, 0, 290, 291, 5, 100, 50]
    kl = [8, 32, 1, 10, 10, 4, 0, 40]
    acc = [8, 3, 1, 9, 10, 5, 0, 31]
    g = torch.Generator().manual_seed(9)
    cand = torch.randint(0, 151936, (B, K), generator=g, dtype=torch.int32)
    corr = torch.randint(0, 151936, (B,), generator=g, dtype=torch.int32)
    # statistics: none yet, a long history of matches, A above N (read as N), saturated fields
    stat = [0, (3000 << 16) | 3100, (200 << 16) | 400, (90 << 16) | 60, 0, 17, -1, (1000 << 16) | 65535]
    ref = oracle.commit_block_dyn(kc, vc, kb, vb, lens, acc, corr, cand, kl, stat, k_min=2)
    dlen = torch.tensor(lens, dtype=torch.int32, device=DEV)
    dblk = torch.tensor(kl, dtype=torch.int32, device=DEV)
    dstat = torch.tensor(stat, dtype=torch.int32, device=DEV)
    anchor, toks, ntok = dvb.orthrus_cache_commit_dyn(kc, vc, kb, vb, dlen, torch.tensor(acc, dtype=torch.int32,
                                                                                           device=DEV),
                                                      corr.to(DEV), cand.to(DEV), dblk, dstat, k_min=2)
    torch.cuda.synchronize()
    assert dlen.cpu().tolist() == ref["cache_len"].tolist()
    assert dblk.cpu().tolist() == ref["blk_len"].tolist()
    assert [x & 0xFFFFFFFF for x in dstat.cpu().tolist()] == [int(x) & 0xFFFFFFFF for x in ref["accept_stat"]]
    assert ntok.cpu().tolist() == ref["n_tokens"].tolist()
    assert anchor.cpu().tolist() == ref["next_anchor"].tolist()
    assert toks.cpu().tolist() == ref["tokens"].tolist()
    assert torch.equal(kc.cpu(), bits_to_bf16(ref["k_cache"]))
    assert torch.equal(vc.cpu(), bits_to_bf16(ref["v_cache"]))
    print(f"commit dyn: lens={dlen.cpu().tolist()} blk_len={dblk.cpu().tolist()}", flush=True)


def _to_dev(sets):
    out = []
    for s in sets:
        d = {"diff": [tuple(t.to(DEV) for t in v) for v in s["diff"]],
             "verify": [tuple(t.to(DEV) for t in v) for v in s["verify"]]}
        d.update({k: s[k].to(DEV) for k in ("logits", "cand", "p", "q", "uniforms") if k in s})
        out.append(d)
    return out


def _cycle_case(w, n, rate, seed):
    sets = cycle_inputs(w, n, accept_rate=rate, seed_offset=seed)
    shape = (w.layers, w.batch, w.n_kv_heads, w.capacity, w.head_dim)
    kc = torch.randn(shape, generator=torch.Generator().manual_seed(seed + 1)).to(torch.bfloat16)
    vc = torch.randn(shape, generator=torch.Generator().manual_seed(seed + 2)).to(torch.bfloat16)
    return sets, kc, vc


def test_decode_cycles_with_adaptive_block_lengths():
    """Six cycles of three sequences (two layers, GQA 4, D 128, K 32) whose
    block lengths start at 32, 4 and 9 and then follow the rule on the
    device; every cycle's integers, attention rows and the final cache match
    the oracle's cycles."""
    w = Workload("dcyc", 2, 3, 8, 2, 128, 700, 32, 4096, 3.0, 24, max_len=700 + 6 * 32)
    sets, kc, vc = _cycle_case(w, 6, 0.75, 5)
    lens, kl, k_min = [700, 0, 129], [32, 4, 9], 2
    recs, st = oracle.decode_cycles_dyn(kc, vc, lens, kl, k_min, sets)
    dkc, dvc = kc.to(DEV), vc.to(DEV)
    dlen = torch.tensor(lens, dtype=torch.int32, device=DEV)
    dblk = torch.tensor(kl, dtype=torch.int32, device=DEV)
    drv = DecodeCycles(dkc, dvc, dlen, _to_dev(sets), blk_len=dblk, k_min=k_min)
    drv.run(len(sets))
    torch.cuda.synchronize()
    for c, rec in enumerate(recs):
        for name in ("accept_len", "correction", "next_anchor", "tokens", "n_tokens"):
            got = getattr(drv, name)[c].cpu().numpy()
            assert np.array_equal(got, rec[name]), f"cycle {c} {name}: {got} vs {rec[name]}"
        k_in = rec["blk_len_in"]
        D = w.head_dim
        for layer in range(w.layers):
            for view, outs in (("diff", drv.diff_out), ("verify", drv.verify_out)):
                got = torch.cat([outs[c][layer][b, :, :k_in[b]].reshape(-1, D) for b in range(w.batch)])
                ref = np.concatenate([rec[f"{view}_out"][layer][b, :, :k_in[b]].reshape(-1, D)
                                      for b in range(w.batch)])
                assert_attn_close(got, ref, f"c{c}/l{layer}/{view}")
    assert dlen.cpu().tolist() == st["cache_len"].tolist()
    assert dblk.cpu().tolist() == st["blk_len"].tolist()
    assert drv.accept_stat.cpu().tolist() == st["accept_stat"].tolist()
    assert torch.equal(dkc.cpu(), bits_to_bf16(st["k_cache"]))
    assert torch.equal(dvc.cpu(), bits_to_bf16(st["v_cache"]))
    print("block lengths per cycle:", [r["blk_len_in"].tolist() for r in recs], "->", st["blk_len"].tolist(),
          flush=True)


def test_adaptive_cycles_graph_replay_matches_eager():
    """A captured round of 3 adaptive cycles replayed twice, with eager work
    and synchronisations between the replays, equals 6 eager cycles bit for
    bit after each replay (lengths, block lengths and cache)."""
    w = Workload("dcyc_g", 2, 2, 8, 2, 128, 600, 32, 2048, 3.0, 25, max_len=600 + 6 * 32)
    sets, kc, vc = _cycle_case(w, 3, 0.7, 13)
    lens, kl = [600, 41], [32, 8]
    dev_sets = _to_dev(sets)

    def state():
        return (kc.to(DEV), vc.to(DEV), torch.tensor(lens, dtype=torch.int32, device=DEV),
                torch.tensor(kl, dtype=torch.int32, device=DEV))

    ek, ev, el, eb = state()
    eager = DecodeCycles(ek, ev, el, dev_sets, blk_len=eb, k_min=2)
    gk, gv, gl, gb = state()
    graphed = DecodeCycles(gk, gv, gl, dev_sets, blk_len=gb, k_min=2)
    graphed.run(1)  # warm the calls once, then restore the state before capture
    torch.cuda.synchronize()
    for t, s in zip((gk, gv, gl, gb), state()):
        t.copy_(s)
    graphed.accept_stat.zero_()
    graphed.capture()
    for rnd in range(2):
        eager.run(3, first_cycle=3 * rnd)
        torch.cuda.synchronize()
        graphed.replay()
        torch.cuda.synchronize()
        assert gl.cpu().tolist() == el.cpu().tolist(), rnd
        assert gb.cpu().tolist() == eb.cpu().tolist(), rnd
        assert graphed.accept_stat.cpu().tolist() == eager.accept_stat.cpu().tolist(), rnd
        assert torch.equal(gk, ek) and torch.equal(gv, ev), rnd
    print(f"graph replay: lengths {el.cpu().tolist()}, block lengths {eb.cpu().tolist()}", flush=True)


def _random_case(seed):
    rng = np.random.default_rng(1000 + seed)
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 4, 8]))
    D = int(rng.choice([64, 128]))
    K = int(rng.choice([1, 3, 8, 16, 24, 32, 40, 64, 100, 128]))
    B = int(rng.integers(1, 7))
    lens = [int(v) for v in rng.integers(0, 3000, size=B)]
    kl = [int(v) for v in rng.integers(1, K + 1, size=B)]
    cap = int(max(max(lens), 64) + rng.integers(0, 200))
    return B, Hkv * G, Hkv, D, K, lens, cap, kl


@pytest.mark.parametrize("seed", range(24))
def test_random_shapes(seed):
    """Seeded random shapes: batch 1..6, KV heads 1..8, GQA group 1..8,
    head_dim 64/128, K up to 128, cached lengths 0..3000 and block lengths
    1..K; the view alternates with the seed."""
    B, Hq, Hkv, D, K, lens, cap, kl = _random_case(seed)
    x = _inputs(B, Hq, Hkv, D, K, lens, cap, seed=2000 + seed)
    _check_attn(x, kl, "diff" if seed % 2 == 0 else "verify",
                f"random B{B} Hq{Hq} Hkv{Hkv} D{D} K{K} L{lens} cap{cap}")


@pytest.mark.parametrize("mode", ["diff", "verify"])
@pytest.mark.parametrize("B,Hq,Hkv,D,K,lens,cap", [
    (1, 32, 8, 128, 32, [32768], 32768),      # the benchmark shape
    (3, 16, 8, 64, 20, [0, 900, 2500], 2560),  # balanced placement, a dead query block
    (2, 32, 8, 128, 128, [700, 33], 1024),     # row groups
])
def test_full_block_lengths_give_the_fixed_length_bits(mode, B, Hq, Hkv, D, K, lens, cap):
    """Every k_b = K: the per-sequence-length call is the fixed-K call, bit
    for bit (out and lse)."""
    x = _inputs(B, Hq, Hkv, D, K, lens, cap, seed=K + B)
    blk = torch.full((B,), K, dtype=torch.int32, device=DEV)
    args = (x["q"], x["k_blk"], x["v_blk"], x["k_cache"], x["v_cache"], x["cache_len"])
    o1, l1 = dvb.orthrus_block_attn(*args, MODES[mode])
    o2, l2 = dvb.orthrus_block_attn_dyn(*args, blk, MODES[mode])
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
    print(f"full-length bits B{B} K{K} {mode}: identical", flush=True)


@pytest.mark.parametrize("mode", ["diff", "verify"])
def test_unsplit_batch_with_short_blocks(mode):
    """40 sequences with K = 128 capacity and 8 KV heads: 1280 groups, one
    work-group each, no split.  Short blocks deal each head's 4 work-groups to
    its live row groups, so the call takes the merge instead of writing the
    rows directly."""
    rng = np.random.default_rng(77)
    lens = [int(v) for v in rng.integers(0, 1500, size=40)]
    kl = [int(v) for v in rng.integers(1, 129, size=40)]
    x = _inputs(40, 32, 8, 128, 128, lens, 1536, seed=77)
    assert dvb.orthrus_attn_num_splits(dvb.attn_desc(x["q"], x["k_cache"])) == 1
    _check_attn(x, kl, mode, "unsplit K=128")


def test_adaptive_cycles_follow_a_change_of_match_rate():
    """24 cycles of three sequences whose draft matches well for 12 cycles
    (rate 0.95) and poorly after (rate 0.4): the block lengths grow to the
    capacity, then shrink, on the device, and after every cycle the
    integers, lengths, statistics and block lengths equal the oracle's, and
    so does the final cache.  The attention outputs are checked by the
    six-cycle test above, not here."""
    w = Workload("dcyc_switch", 1, 3, 8, 2, 64, 300, 32, 512, 3.0, 26, max_len=300 + 24 * 32)
    hi = cycle_inputs(w, 12, accept_rate=0.95, seed_offset=41)
    lo = cycle_inputs(w, 12, accept_rate=0.4, seed_offset=43)
    sets = hi + lo
    shape = (w.layers, w.batch, w.n_kv_heads, w.capacity, w.head_dim)
    kc = torch.randn(shape, generator=torch.Generator().manual_seed(45)).to(torch.bfloat16)
    vc = torch.randn(shape, generator=torch.Generator().manual_seed(46)).to(torch.bfloat16)
    lens, kl, k_min = [300, 17, 0], [4, 32, 8], 2
    recs, st = oracle.decode_cycles_dyn(kc, vc, lens, kl, k_min, sets, keep_attention=False)
    dkc, dvc = kc.to(DEV), vc.to(DEV)
    dlen = torch.tensor(lens, dtype=torch.int32, device=DEV)
    dblk = torch.tensor(kl, dtype=torch.int32, device=DEV)
    drv = DecodeCycles(dkc, dvc, dlen, _to_dev(sets), blk_len=dblk, k_min=k_min)
    ks = []
    for c in range(len(sets)):
        drv.issue(c)
        torch.cuda.synchronize()
        ks.append(dblk.cpu().tolist())
        rec = recs[c]
        assert ks[-1] == rec["blk_len"].tolist(), f"cycle {c}"
        assert drv.accept_stat.cpu().tolist() == rec["accept_stat"].tolist(), f"cycle {c}"
        assert dlen.cpu().tolist() == rec["cache_len"].tolist(), f"cycle {c}"
        for name in ("accept_len", "correction", "next_anchor", "tokens", "n_tokens"):
            got = getattr(drv, name)[c].cpu().numpy()
            assert np.array_equal(got, rec[name]), f"cycle {c} {name}: {got} vs {rec[name]}"
    assert torch.equal(dkc.cpu(), bits_to_bf16(st["k_cache"]))
    assert torch.equal(dvc.cpu(), bits_to_bf16(st["v_cache"]))
    # the lengths reached the capacity while the draft matched and came down
    # after (the statistics forget by 7/8 per cycle)
    assert ks[11] == [32, 32, 32] and all(ks[-1][b] < ks[11][b] for b in range(3))
    print("block lengths:", ks, flush=True)


@pytest.mark.parametrize("mode", ["diff", "verify"])
def test_block_lengths_out_of_range_are_clamped(mode):
    """blk_len 0, -5 and 200 with K = 32 read as 1, 1 and 32 (attention)."""
    x = _inputs(3, 32, 8, 128, 32, [900, 0, 2048], 2048, seed=91)
    B, Hq, K, D = x["q"].shape
    raw = [0, -5, 200]
    blk = torch.tensor(raw, dtype=torch.int32, device=DEV)
    out = torch.full_like(x["q"], MARK_OUT)
    lse = torch.full(x["q"].shape[:3], MARK_LSE, dtype=torch.float32, device=DEV)
    dvb.orthrus_block_attn_dyn(x["q"], x["k_blk"], x["v_blk"], x["k_cache"], x["v_cache"], x["cache_len"], blk,
                               MODES[mode], out=out, lse=lse)
    torch.cuda.synchronize()
    kl = [1, 1, 32]
    ref, ref_lse = oracle.block_attention_dyn(x["q"], x["k_blk"], x["v_blk"], x["k_cache"], x["v_cache"],
                                              x["cache_len"], raw, MODES[mode])
    assert_attn_close(torch.cat([out[b, :, :k].reshape(-1, D) for b, k in enumerate(kl)]),
                      np.concatenate([ref[b, :, :k].reshape(-1, D) for b, k in enumerate(kl)]), "clamped")
    for b, k in enumerate(kl):
        assert bool((out[b, :, k:] == MARK_OUT).all()) and bool((lse[b, :, k:] == MARK_LSE).all())


def test_consensus_block_lengths_out_of_range_are_clamped():
    w = Workload("gc", 1, 3, 32, 8, 128, 1, 32, 4096, 3.0, 53)
    logits, cand, _ = greedy_inputs(w, first_mismatch=torch.tensor([32, 32, 32]))
    raw = [0, -5, 200]
    ref_a, ref_am, ref_c = oracle.greedy_consensus_dyn(logits, cand, raw)
    a, am, c = dvb.orthrus_consensus_greedy_dyn(logits.to(DEV), cand.to(DEV),
                                                torch.tensor(raw, dtype=torch.int32, device=DEV))
    ws = sample_inputs(w.replace(block_k=32), draft_noise=0.3)
    ref_sa, ref_sc = oracle.sample_consensus_dyn(*ws, raw)
    sa, sc = dvb.orthrus_consensus_sample_dyn(*[t.to(DEV) for t in ws], torch.tensor(raw, dtype=torch.int32,
                                                                                      device=DEV))
    torch.cuda.synchronize()
    assert a.cpu().tolist() == ref_a.tolist() == [1, 1, 32]
    assert c.cpu().tolist() == ref_c.tolist() and np.array_equal(am.cpu().numpy(), ref_am)
    assert sa.cpu().tolist() == ref_sa.tolist() and sc.cpu().tolist() == ref_sc.tolist()


def test_sample_decode_cycles_with_adaptive_block_lengths():
    """T > 0 cycles with adaptive block lengths: three sequences starting at
    block lengths 32, 3 and 12; the sampler reads only the live rows and
    uniforms u_0..u_{k-1} and u_K; every cycle's integers, the statistics,
    the block lengths and the final cache match the oracle's cycles."""
    from synth import sample_cycle_inputs
    w = Workload("dscyc", 2, 3, 8, 2, 128, 500, 32, 4096, 3.0, 26, max_len=500 + 6 * 32)
    sets = sample_cycle_inputs(w, 6, draft_noise=0.4, seed_offset=7)
    _, kc, vc = _cycle_case(w, 1, 0.5, 17)
    lens, kl, k_min = [500, 0, 64], [32, 3, 12], 2
    recs, st = oracle.decode_cycles_dyn(kc, vc, lens, kl, k_min, sets)
    dkc, dvc = kc.to(DEV), vc.to(DEV)
    dlen = torch.tensor(lens, dtype=torch.int32, device=DEV)
    dblk = torch.tensor(kl, dtype=torch.int32, device=DEV)
    drv = DecodeCycles(dkc, dvc, dlen, _to_dev(sets), blk_len=dblk, k_min=k_min)
    drv.run(len(sets))
    torch.cuda.synchronize()
    D = w.head_dim
    for c, rec in enumerate(recs):
        for name in ("accept_len", "correction", "next_anchor", "tokens", "n_tokens"):
            got = getattr(drv, name)[c].cpu().numpy()
            assert np.array_equal(got, rec[name]), f"cycle {c} {name}: {got} vs {rec[name]}"
        k_in = rec["blk_len_in"]
        for layer in range(w.layers):
            got = torch.cat([drv.verify_out[c][layer][b, :, :k_in[b]].reshape(-1, D) for b in range(w.batch)])
            ref = np.concatenate([rec["verify_out"][layer][b, :, :k_in[b]].reshape(-1, D) for b in range(w.batch)])
            assert_attn_close(got, ref, f"c{c}/l{layer}/verify")
    assert dlen.cpu().tolist() == st["cache_len"].tolist()
    assert dblk.cpu().tolist() == st["blk_len"].tolist()
    assert drv.accept_stat.cpu().tolist() == st["accept_stat"].tolist()
    assert torch.equal(dkc.cpu(), bits_to_bf16(st["k_cache"]))
    assert torch.equal(dvc.cpu(), bits_to_bf16(st["v_cache"]))
    print("T>0 block lengths per cycle:", [r["blk_len_in"].tolist() for r in recs], flush=True)


def test_adaptive_sample_cycles_graph_replay_matches_eager():
    """T > 0 cycles with adaptive block lengths, captured as a round of 3 and
    replayed twice with eager work and synchronisations between the replays:
    lengths, block lengths, statistics and cache equal 6 eager cycles bit for
    bit after each replay."""
    from synth import sample_cycle_inputs
    w = Workload("dscyc_g", 2, 2, 8, 2, 128, 600, 32, 2048, 3.0, 27, max_len=600 + 6 * 32)
    sets = _to_dev(sample_cycle_inputs(w, 3, draft_noise=0.5, seed_offset=19))
    _, kc, vc = _cycle_case(w, 1, 0.5, 21)
    lens, kl = [600, 41], [32, 8]

    def state():
        return (kc.to(DEV), vc.to(DEV), torch.tensor(lens, dtype=torch.int32, device=DEV),
                torch.tensor(kl, dtype=torch.int32, device=DEV))

    ek, ev, el, eb = state()
    eager = DecodeCycles(ek, ev, el, sets, blk_len=eb, k_min=2)
    gk, gv, gl, gb = state()
    graphed = DecodeCycles(gk, gv, gl, sets, blk_len=gb, k_min=2)
    graphed.run(1)  # warm the calls once, then restore the state before capture
    torch.cuda.synchronize()
    for t, s in zip((gk, gv, gl, gb), state()):
        t.copy_(s)
    graphed.accept_stat.zero_()
    graphed.capture()
    for rnd in range(2):
        eager.run(3, first_cycle=3 * rnd)
        torch.cuda.synchronize()
        graphed.replay()
        torch.cuda.synchronize()
        _ = gk.float().sum()
        torch.cuda.synchronize()
        assert gl.cpu().tolist() == el.cpu().tolist(), rnd
        assert gb.cpu().tolist() == eb.cpu().tolist(), rnd
        assert graphed.accept_stat.cpu().tolist() == eager.accept_stat.cpu().tolist(), rnd
        assert torch.equal(gk, ek) and torch.equal(gv, ev), rnd
    print(f"T>0 graph replay: lengths {el.cpu().tolist()}, block lengths {eb.cpu().tolist()}", flush=True)
