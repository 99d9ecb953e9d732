"""GPU parity of the cycle commit and of whole synthetic decode cycles.

The commit is byte and integer work, so every comparison with the oracle is
bit-exact: cache contents, advanced lengths, emitted tokens, token counts and
next anchors.  Whole cycles (both views' attention per layer, greedy or
T > 0 consensus, commit, repeated with the state carried on the device) are checked
cycle by cycle: integers bit-exact, attention outputs within max-abs 2e-2 and
relative L2 5e-3 of the fp64 oracle.  A captured HIP graph of a round of
cycles must replay bit-identically to the same cycles issued eagerly.
"""
import numpy as np
import pytest
import torch

import dual_view_block_amd as dvb
import oracle
from dual_view_block_amd.cycle import DecodeCycles
from oracle.cycle import bits_to_bf16
from synth import WORKLOADS, Workload, cycle_inputs, sample_cycle_inputs
from tests._parity import assert_attn_close

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _bf16(shape, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=DEV).to(torch.bfloat16)


def _commit_case(n_layers, B, Hkv, D, K, max_len, lens, acc, seed=0):
    kc = _bf16((n_layers, B, Hkv, max_len, D), seed + 1)
    vc = _bf16((n_layers, B, Hkv, max_len, D), seed + 2)
    kb = _bf16((n_layers, B, Hkv, K, D), seed + 3)
    vb = _bf16((n_layers, B, Hkv, K, D), seed + 4)
    g = torch.Generator().manual_seed(seed + 5)
    cand = torch.randint(0, 151936, (B, K), generator=g, dtype=torch.int32)
    corr = torch.randint(0, 151936, (B,), generator=g, dtype=torch.int32)
    acc_t = torch.tensor(acc, dtype=torch.int32)
    corr = torch.where(acc_t < K, corr, torch.full_like(corr, -1))
    return dict(kc=kc, vc=vc, kb=kb, vb=vb, lens=torch.tensor(lens, dtype=torch.int32),
                acc=acc_t, corr=corr, cand=cand)


def _check_commit(x, what):
    ref = oracle.commit_block(x["kc"], x["vc"], x["kb"], x["vb"], x["lens"], x["acc"], x["corr"], x["cand"])
    lens = x["lens"].to(DEV)
    anchor, toks, ntok = dvb.orthrus_cache_commit(x["kc"], x["vc"], x["kb"], x["vb"], lens, x["acc"].to(DEV),
                                                  x["corr"].to(DEV), x["cand"].to(DEV))
    torch.cuda.synchronize()
    assert lens.cpu().tolist() == ref["cache_len"].tolist(), what
    assert ntok.cpu().tolist() == ref["n_tokens"].tolist(), what
    assert anchor.cpu().tolist() == ref["next_anchor"].tolist(), what
    assert toks.cpu().tolist() == ref["tokens"].tolist(), what
    assert torch.equal(x["kc"].cpu(), bits_to_bf16(ref["k_cache"])), what
    assert torch.equal(x["vc"].cpu(), bits_to_bf16(ref["v_cache"])), what
    print(f"{what}: n_tokens={ntok.cpu().tolist()[:8]}", flush=True)


@pytest.mark.parametrize("a", [0, 1, 3, 4])
def test_commit_tiny_every_accept_length(a):
    """1 layer, 1 KV head, D=64, K=4, L=256 (the tiny shape), capacity 264."""
    _check_commit(_commit_case(1, 1, 1, 64, 4, 264, [256], [a]), f"tiny/a{a}")


def test_commit_batched_ragged_with_refusals_and_edges():
    """16 sequences, 3 layers, 8 KV heads, D=128, K=32: every accept length class,
    an empty cache, a commit that exactly fills the cache, and refused commits
    (overflow, a > K, a < 0, negative length)."""
    max_len = 400
    lens = [0, 17, 100, 368, 369, 399, 400, 5, 64, 65, 250, 333, 10, -3, 7, 300]
    acc = [0, 31, 32, 31, 31, 0, 0, 33, -1, 1, 16, 2, 32, 4, 5, 12]
    _check_commit(_commit_case(3, 16, 8, 128, 32, max_len, lens, acc, seed=10), "ragged16")


@pytest.mark.parametrize("shape", [
    # (n_layers, B, Hkv, D, K, max_len)
    (2, 2, 2, 8, 1, 9),       # K = 1: always one row; tiny rows of 16 bytes
    (1, 3, 1, 1024, 5, 40),   # widest rows
    (4, 2, 3, 64, 64, 200),   # K beyond the attention's 32 (the commit allows it)
    (1, 1, 8, 128, 32, 32),   # capacity equals K
])
def test_commit_general_shapes(shape):
    n_layers, B, Hkv, D, K, max_len = shape
    g = torch.Generator().manual_seed(sum(shape))
    lens = torch.randint(0, max_len + 1, (B,), generator=g).tolist()
    acc = torch.randint(0, K + 1, (B,), generator=g).tolist()
    _check_commit(_commit_case(n_layers, B, Hkv, D, K, max_len, lens, acc, seed=sum(shape)), f"shape{shape}")


def test_commit_full_qwen3_8b_32k():
    """All 36 layers of the Qwen3-8B shape at L = 32768, K = 32, in one call:
    only rows [L, L + r) of every plane change, and they hold the block's rows
    0..r-1; checked against the oracle on a window around the committed rows."""
    n_layers, B, Hkv, D, K, L = 36, 1, 8, 128, 32, 32768
    max_len = L + 64
    for a in (5, 32):
        x = _commit_case(n_layers, B, Hkv, D, K, max_len, [L], [a], seed=40 + a)
        before_k, before_v = x["kc"].clone(), x["vc"].clone()
        lens = x["lens"].to(DEV)
        anchor, toks, ntok = dvb.orthrus_cache_commit(x["kc"], x["vc"], x["kb"], x["vb"], lens,
                                                      x["acc"].to(DEV), x["corr"].to(DEV), x["cand"].to(DEV))
        torch.cuda.synchronize()
        r = a + (a < K)
        for after, before in ((x["kc"], before_k), (x["vc"], before_v)):
            changed = (after.view(torch.int16) != before.view(torch.int16)).any(dim=-1)  # [n, B, Hkv, rows]
            rows = changed.nonzero()[:, 3]
            assert rows.numel() > 0 and int(rows.min()) >= L and int(rows.max()) < L + r
        lo = L - 3
        win = lambda t: t[:, :, :, lo:max_len].cpu()
        ref = oracle.commit_block(win(before_k), win(before_v), x["kb"].cpu(), x["vb"].cpu(),
                                  torch.tensor([L - lo]), x["acc"], x["corr"], x["cand"])
        assert torch.equal(win(x["kc"]), bits_to_bf16(ref["k_cache"]))
        assert torch.equal(win(x["vc"]), bits_to_bf16(ref["v_cache"]))
        assert lens.cpu().tolist() == [L + r] and ntok.cpu().tolist() == [r]
        assert toks.cpu().tolist() == ref["tokens"].tolist()
        assert anchor.cpu().tolist() == ref["next_anchor"].tolist()
        print(f"full 36-layer commit a={a}: rows {L}..{L + r - 1} written", flush=True)


def test_commit_rejects_block_inside_cache():
    """Block rows that alias the cache are refused before anything is launched."""
    x = _commit_case(1, 1, 1, 64, 4, 16, [3], [1])
    lens = x["lens"].to(DEV)
    before = x["kc"].clone()
    with pytest.raises(dvb.OrthrusError) as e:
        dvb.orthrus_cache_commit(x["kc"], x["vc"], x["kc"][:, :, :, :4], x["vb"], lens, x["acc"].to(DEV),
                                 x["corr"].to(DEV), x["cand"].to(DEV))
    assert e.value.status == 2
    torch.cuda.synchronize()
    assert torch.equal(x["kc"], before) and lens.cpu().tolist() == [3]


# ------------------------------------------------------- whole cycles ----
def _to_dev(sets):
    out = []
    for s in sets:
        d = {"diff": [tuple(t.to(DEV) for t in v) for v in s["diff"]],
             "verify": [tuple(t.to(DEV) for t in v) for v in s["verify"]]}
        for k in ("logits", "cand", "p", "q", "uniforms"):
            if k in s:
                d[k] = s[k].to(DEV)
        if "j_star" in s:
            d["j_star"] = s["j_star"]
        out.append(d)
    return out


def _cycle_setup(w, n_sets, lens, rate, seed):
    sets = cycle_inputs(w, n_sets, accept_rate=rate, seed_offset=seed)
    shape = (w.layers, w.batch, w.n_kv_heads, w.capacity, w.head_dim)
    kc = torch.randn(shape, generator=torch.Generator().manual_seed(seed + 1)).to(torch.bfloat16)
    vc = torch.randn(shape, generator=torch.Generator().manual_seed(seed + 2)).to(torch.bfloat16)
    return sets, kc, vc, torch.tensor(lens, dtype=torch.int32)


@pytest.mark.parametrize("case", [
    # (workload, initial lengths, accept rate, cycles)
    (Workload("cyc_small", 2, 2, 4, 2, 64, 300, 4, 1000, 4.0, 21, max_len=300 + 6 * 4), [300, 77], 0.6, 6),
    (Workload("cyc_gqa4", 3, 3, 8, 2, 128, 700, 32, 4096, 3.0, 22, max_len=700 + 4 * 32), [700, 0, 129], 0.85, 4),
])
def test_decode_cycles_match_oracle(case):
    w, lens, rate, n_cycles = case
    sets, kc, vc, L = _cycle_setup(w, n_cycles, lens, rate, seed=7)
    recs, state = oracle.decode_cycles(kc, vc, L, sets)
    dkc, dvc, dlen = kc.to(DEV), vc.to(DEV), L.to(DEV)
    drv = DecodeCycles(dkc, dvc, dlen, _to_dev(sets))
    drv.run(n_cycles)
    torch.cuda.synchronize()
    for c, rec in enumerate(recs):
        for name in ("accept_len", "correction", "next_anchor", "tokens", "n_tokens"):
            got = getattr(drv, name)[c].cpu().numpy()
            assert np.array_equal(got, rec[name]), f"cycle {c} {name}: {got} vs {rec[name]}"
        assert rec["accept_len"].tolist() == sets[c]["j_star"].tolist()
        for layer in range(w.layers):
            assert_attn_close(drv.diff_out[c][layer], rec["diff_out"][layer], f"c{c}/l{layer}/diff")
            assert_attn_close(drv.verify_out[c][layer], rec["verify_out"][layer], f"c{c}/l{layer}/verify")
    assert dlen.cpu().tolist() == state["cache_len"].tolist()
    assert torch.equal(dkc.cpu(), bits_to_bf16(state["k_cache"]))
    assert torch.equal(dvc.cpu(), bits_to_bf16(state["v_cache"]))
    print(f"{w.name}: lengths {lens} -> {dlen.cpu().tolist()}", flush=True)


def test_decode_cycles_graph_replay_matches_eager():
    """A captured round of 3 cycles, replayed 3 times with eager work and
    synchronisations between replays, equals 9 eagerly issued cycles bit for bit
    after every replay."""
    w = Workload("cyc_graph", 2, 2, 8, 2, 128, 1000, 32, 2048, 3.0, 23, max_len=1000 + 9 * 32)
    sets, kc, vc, L = _cycle_setup(w, 3, [1000, 333], 0.8, seed=11)
    dev_sets = _to_dev(sets)
    ek, ev, el = kc.to(DEV), vc.to(DEV), L.to(DEV)
    eager = DecodeCycles(ek, ev, el, dev_sets)
    gk, gv, gl = kc.to(DEV), vc.to(DEV), L.to(DEV)
    graphed = DecodeCycles(gk, gv, gl, dev_sets)
    # warm up the graphed driver's calls once on a scratch copy of the state, then restore
    graphed.run(1)
    torch.cuda.synchronize()
    gk.copy_(kc.to(DEV))
    gv.copy_(vc.to(DEV))
    gl.copy_(L.to(DEV))
    graphed.capture()
    for rnd in range(3):
        eager.run(3, first_cycle=3 * rnd)
        torch.cuda.synchronize()
        snap = [t.clone() for t in eager.tokens] + [t.clone() for t in eager.n_tokens]
        graphed.replay()
        torch.cuda.synchronize()
        _ = (gk.float().sum())  # some eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(gl, el), f"round {rnd}"
        got = [t for t in graphed.tokens] + [t for t in graphed.n_tokens]
        for a, b in zip(got, snap):
            assert torch.equal(a, b), f"round {rnd}"
        for s in range(3):
            for layer in range(w.layers):
                assert torch.equal(graphed.verify_out[s][layer], eager.verify_out[s][layer])
                assert torch.equal(graphed.diff_out[s][layer], eager.diff_out[s][layer])
        assert torch.equal(gk, ek) and torch.equal(gv, ev), f"round {rnd}"
    print(f"graph replay: lengths {el.cpu().tolist()}", flush=True)


def _check_cycles(w, drv, recs, state, dkc, dvc, dlen):
    for c, rec in enumerate(recs):
        for name in ("accept_len", "correction", "next_anchor", "tokens", "n_tokens"):
            got = getattr(drv, name)[c].cpu().numpy()
            assert np.array_equal(got, rec[name]), f"cycle {c} {name}: {got} vs {rec[name]}"
        for layer in range(w.layers):
            assert_attn_close(drv.diff_out[c][layer], rec["diff_out"][layer], f"c{c}/l{layer}/diff")
            assert_attn_close(drv.verify_out[c][layer], rec["verify_out"][layer], f"c{c}/l{layer}/verify")
    assert dlen.cpu().tolist() == state["cache_len"].tolist()
    assert torch.equal(dkc.cpu(), bits_to_bf16(state["k_cache"]))
    assert torch.equal(dvc.cpu(), bits_to_bf16(state["v_cache"]))


@pytest.mark.parametrize("case", [
    # (workload, initial lengths, draft noise, cycles)
    (Workload("scyc_small", 2, 2, 4, 2, 64, 300, 4, 1000, 4.0, 31, max_len=300 + 6 * 4), [300, 77], 0.5, 6),
    (Workload("scyc_gqa4", 2, 3, 8, 2, 128, 700, 32, 4096, 3.0, 32, max_len=700 + 4 * 32), [700, 0, 129], 0.3, 4),
    # K 64 and 128: two and four row groups of 128 query rows per KV head
    (Workload("scyc_k64", 2, 2, 8, 2, 128, 900, 64, 2048, 3.0, 35, max_len=900 + 3 * 64), [900, 333], 0.2, 3),
    (Workload("scyc_k128", 1, 2, 8, 2, 64, 600, 128, 1024, 3.0, 36, max_len=600 + 3 * 128), [600, 5], 0.1, 3),
])
def test_sample_decode_cycles_match_oracle(case):
    """T > 0 cycles (rejection-sampling consensus over a near draft): every
    cycle's accepted prefix, sampled correction, emitted tokens and anchors
    bit-exact, attention rows within tolerance, final cache bit-exact."""
    w, lens, noise, n_cycles = case
    sets = sample_cycle_inputs(w, n_cycles, draft_noise=noise, seed_offset=3)
    kc, vc = _cycle_setup(w, 1, lens, 0.5, seed=9)[1:3]
    L = torch.tensor(lens, dtype=torch.int32)
    recs, state = oracle.decode_cycles(kc, vc, L, sets)
    dkc, dvc, dlen = kc.to(DEV), vc.to(DEV), L.to(DEV)
    drv = DecodeCycles(dkc, dvc, dlen, _to_dev(sets))
    drv.run(n_cycles)
    torch.cuda.synchronize()
    _check_cycles(w, drv, recs, state, dkc, dvc, dlen)
    print(f"{w.name}: accept lengths {[r['accept_len'].tolist() for r in recs]}", flush=True)


def test_sample_decode_cycles_graph_replay_matches_eager():
    """A captured round of 2 T > 0 cycles replayed twice, with eager work and
    synchronisations between the replays, equals 4 eager cycles bit for bit."""
    w = Workload("scyc_graph", 2, 2, 8, 2, 128, 900, 32, 2048, 3.0, 33, max_len=900 + 4 * 32)
    sets = _to_dev(sample_cycle_inputs(w, 2, draft_noise=0.3, seed_offset=5))
    kc, vc = _cycle_setup(w, 1, [900, 50], 0.5, seed=13)[1:3]
    L = torch.tensor([900, 50], dtype=torch.int32)
    ek, ev, el = kc.to(DEV), vc.to(DEV), L.to(DEV)
    eager = DecodeCycles(ek, ev, el, sets)
    gk, gv, gl = kc.to(DEV), vc.to(DEV), L.to(DEV)
    graphed = DecodeCycles(gk, gv, gl, sets)
    graphed.run(1)
    torch.cuda.synchronize()
    gk.copy_(kc.to(DEV))
    gv.copy_(vc.to(DEV))
    gl.copy_(L.to(DEV))
    graphed.capture()
    for rnd in range(2):
        eager.run(2, first_cycle=2 * rnd)
        torch.cuda.synchronize()
        graphed.replay()
        torch.cuda.synchronize()
        _ = gk.float().sum()
        torch.cuda.synchronize()
        assert torch.equal(gl, el), f"round {rnd}"
        for a, b in zip(graphed.tokens + graphed.accept_len, eager.tokens + eager.accept_len):
            assert torch.equal(a, b), f"round {rnd}"
        assert torch.equal(gk, ek) and torch.equal(gv, ev), f"round {rnd}"
    print(f"sample graph replay: lengths {el.cpu().tolist()}", flush=True)


def test_prepared_calls_reject_wrong_outputs():
    """The prepared calls check their output and workspace tensors (dtype,
    shape, device) before any launch: a short output would be written past
    its end."""
    B, K, V = 2, 4, 100
    i32 = dict(dtype=torch.int32, device=DEV)
    logits = torch.zeros((B, K, V), device=DEV)
    cand = torch.zeros((B, K), **i32)
    ws = torch.empty(max(dvb.orthrus_consensus_workspace_size(B, K, V), 16), dtype=torch.uint8, device=DEV)
    good = dict(accept_len=torch.empty(B, **i32), correction=torch.empty(B, **i32))
    dvb.PreparedGreedy(logits, cand, good["accept_len"], None, good["correction"], ws)
    with pytest.raises(ValueError):
        dvb.PreparedGreedy(logits, cand, torch.empty(B - 1, **i32), None, good["correction"], ws)
    with pytest.raises(TypeError):
        dvb.PreparedGreedy(logits, cand, good["accept_len"], None, torch.empty(B, dtype=torch.int64, device=DEV), ws)
    u = torch.zeros((B, K + 1), device=DEV)
    with pytest.raises(ValueError):
        dvb.PreparedSample(logits, logits, cand, u, good["accept_len"], torch.empty(B + 1, **i32), ws)
    w = Workload("chk", 1, B, 4, 2, 64, 100, K, V, 1.0, 3)
    from synth import attention_inputs
    x = attention_inputs(w, device=DEV)
    desc = dvb.attn_desc(x["q"], x["k_cache"])
    aws = torch.empty(max(dvb.orthrus_attn_workspace_size(desc), 16), dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError):
        dvb.PreparedAttention(dvb.ORTHRUS_MASK_VERIFY_CAUSAL, x["q"], x["k_blk"], x["v_blk"], x["k_cache"],
                              x["v_cache"], x["cache_len"], torch.empty_like(x["q"])[:, :, :-1].contiguous(),
                              None, aws)


def test_sample_decode_cycles_ragged_batch_of_16():
    """T > 0 cycles over 16 sequences of ragged length (0 to 3000 keys, the
    balanced placement of the streaming kernel), a far draft (noise 1.0, so
    that accept lengths spread over the whole range): every cycle's integers
    and the final cache bit-exact against the oracle's cycles."""
    lens = [int(v) for v in np.random.default_rng(41).integers(0, 3000, size=16)]
    lens[3], lens[7] = 0, 1
    w = Workload("scyc_b16", 2, 16, 8, 2, 64, 3000, 16, 512, 3.0, 34, max_len=3000 + 5 * 16)
    sets = sample_cycle_inputs(w, 5, draft_noise=1.0, seed_offset=11)
    kc, vc = _cycle_setup(w, 1, lens, 0.5, seed=17)[1:3]
    L = torch.tensor(lens, dtype=torch.int32)
    recs, state = oracle.decode_cycles(kc, vc, L, sets, keep_attention=False)
    dkc, dvc, dlen = kc.to(DEV), vc.to(DEV), L.to(DEV)
    drv = DecodeCycles(dkc, dvc, dlen, _to_dev(sets))
    drv.run(len(sets))
    torch.cuda.synchronize()
    seen = set()
    for c, rec in enumerate(recs):
        for name in ("accept_len", "correction", "next_anchor", "tokens", "n_tokens"):
            got = getattr(drv, name)[c].cpu().numpy()
            assert np.array_equal(got, rec[name]), f"cycle {c} {name}: {got} vs {rec[name]}"
        seen.update(rec["accept_len"].tolist())
    assert len(seen) >= 4, seen
    assert dlen.cpu().tolist() == state["cache_len"].tolist()
    assert torch.equal(dkc.cpu(), bits_to_bf16(state["k_cache"]))
    assert torch.equal(dvc.cpu(), bits_to_bf16(state["v_cache"]))
    print(f"ragged T>0 cycles: accept lengths seen {sorted(seen)}", flush=True)
