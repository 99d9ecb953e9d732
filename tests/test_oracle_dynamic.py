"""Pins for the dynamic-block oracle (CPU only).

Each test ties ``oracle.dynamic`` to something other than itself:

* attention: torch's float64 scaled_dot_product_attention over the keys a
  k_b-position block sees, with the mask built here from the definition
  (cache positions all visible; block keys j < k_b, all of them or j <= i);
* greedy consensus: a pure-Python scan written out here;
* T > 0 consensus: properties the definition fixes (rows past k_b are never
  read, a <= k_b, a = k_b exactly when every live test passes, the residual
  draw uses u_K), and identity with the static sampler when k_b = K;
* commit: a hand-worked cycle (rows, length, tokens, anchor) with marked
  block rows past k_b that must never reach the cache;
* the block-length rule: statistics and decisions worked out by hand, and the
  float rule (smallest power of two k with p^k <= 1/8) on a grid of rates.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle.attention import MASK_DIFF_BIDIR as DIFF, MASK_VERIFY_CAUSAL as VERIFY
from synth import Workload, attention_inputs


def _case(B, Hq, Hkv, K, D, lens, seed):
    w = Workload("dyn", 1, B, Hq, Hkv, D, max(max(lens), 1), K, 10, 1.0, seed)
    x = attention_inputs(w, seed_offset=seed)
    x["cache_len"] = torch.tensor(lens, dtype=torch.int32)
    return x


@pytest.mark.parametrize("mode", [DIFF, VERIFY])
def test_attention_matches_sdpa_on_the_live_block(mode):
    B, Hq, Hkv, K, D = 3, 4, 2, 6, 16
    lens = [9, 0, 14]
    kl = [1, 6, 4]
    x = _case(B, Hq, Hkv, K, D, lens, 3)
    out, lse = oracle.block_attention_dyn(x["q"], x["k_blk"], x["v_blk"], x["k_cache"], x["v_cache"],
                                          x["cache_len"], torch.tensor(kl, dtype=torch.int32), mode)
    G = Hq // Hkv
    for b in range(B):
        L, k = lens[b], kl[b]
        for h in range(Hq):
            g = h // G
            keys = torch.cat([x["k_cache"][b, g, :L], x["k_blk"][b, g, :k]]).double()
            vals = torch.cat([x["v_cache"][b, g, :L], x["v_blk"][b, g, :k]]).double()
            mask = torch.zeros((k, L + k), dtype=torch.bool)
            mask[:, :L] = True
            for i in range(k):
                for j in range(k):
                    mask[i, L + j] = mode == DIFF or j <= i
            qr = x["q"][b, h, :k].double()
            ref = F.scaled_dot_product_attention(qr[None], keys[None], vals[None], attn_mask=mask[None],
                                                 scale=1.0 / np.sqrt(D))[0]
            s = (qr @ keys.T) / np.sqrt(D)
            ref_lse = torch.logsumexp(s.masked_fill(~mask, float("-inf")), dim=1)
            np.testing.assert_allclose(out[b, h, :k], ref.numpy(), rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[b, h, :k], ref_lse.numpy(), rtol=0, atol=1e-12)
            assert np.isnan(out[b, h, k:]).all() and np.isnan(lse[b, h, k:]).all()


def test_attention_ignores_dead_block_rows_and_keys():
    """Rows and keys past k_b may hold anything: the live rows do not change."""
    B, Hq, Hkv, K, D = 2, 2, 1, 8, 8
    x = _case(B, Hq, Hkv, K, D, [5, 3], 7)
    kl = torch.tensor([3, 5], dtype=torch.int32)
    out, lse = oracle.block_attention_dyn(x["q"], x["k_blk"], x["v_blk"], x["k_cache"], x["v_cache"],
                                          x["cache_len"], kl, VERIFY)
    y = {n: t.clone() for n, t in x.items()}
    for b, k in enumerate(kl.tolist()):
        y["q"][b, :, k:] = 100.0
        y["k_blk"][b, :, k:] = -50.0
        y["v_blk"][b, :, k:] = 1e4
    out2, lse2 = oracle.block_attention_dyn(y["q"], y["k_blk"], y["v_blk"], y["k_cache"], y["v_cache"],
                                            y["cache_len"], kl, VERIFY)
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(lse, lse2)


def test_lengths_are_clamped():
    np.testing.assert_array_equal(oracle.live_lengths([-3, 0, 1, 7, 9, 40], 9), [1, 1, 1, 7, 9, 9])


def _greedy_scan(logits, cand, k):
    """Greedy rule written out: first-index argmax per row, first mismatch."""
    am = []
    for i in range(k):
        row = logits[i]
        best = 0
        for v in range(1, len(row)):
            if row[v] > row[best]:
                best = v
        am.append(best)
    a = 0
    while a < k and cand[a] == am[a]:
        a += 1
    return a, am, (am[a] if a < k else -1)


def test_greedy_consensus_matches_a_written_out_scan():
    rng = np.random.default_rng(5)
    B, K, V = 5, 7, 11
    logits = rng.normal(size=(B, K, V))
    am_true = logits.argmax(axis=2)
    cand = am_true.copy()
    cand[0, 2] = (cand[0, 2] + 1) % V     # mismatch inside the live block
    cand[1, 5] = (cand[1, 5] + 1) % V     # mismatch past k_b = 3: must not count
    cand[3, 0] = (cand[3, 0] + 1) % V     # mismatch at row 0
    kl = [4, 3, 7, 1, 2]
    acc, am, corr = oracle.greedy_consensus_dyn(logits, cand, kl)
    for b in range(B):
        a, m, c = _greedy_scan(logits[b], cand[b], kl[b])
        assert acc[b] == a and corr[b] == c
        assert list(am[b, :kl[b]]) == m and (am[b, kl[b]:] == -1).all()
    assert list(acc) == [2, 3, 7, 0, 2]
    assert list(corr[[1, 2, 4]]) == [-1, -1, -1]


def _probs(rng, B, K, V):
    z = rng.normal(size=(B, K, V)) * 2.0
    p = np.exp(z - z.max(axis=2, keepdims=True))
    return (p / p.sum(axis=2, keepdims=True)).astype(np.float32)


def test_sampler_reads_no_dead_row_and_uses_the_last_uniform():
    rng = np.random.default_rng(11)
    B, K, V = 6, 5, 13
    P, Q = _probs(rng, B, K, V), _probs(rng, B, K, V)
    cand = rng.integers(0, V, size=(B, K))
    U = (rng.integers(0, 2 ** 24, size=(B, K + 1)) / 2 ** 24).astype(np.float32)
    kl = [1, 2, 3, 5, 4, 2]
    acc, corr = oracle.sample_consensus_dyn(P, Q, cand, U, kl)
    # dead rows, their candidates and their accept uniforms changed: same result
    P2, Q2, c2, U2 = P.copy(), Q.copy(), cand.copy(), U.copy()
    for b, k in enumerate(kl):
        P2[b, k:] = 1.0 / V
        Q2[b, k:] = 0.5
        c2[b, k:] = 0
        U2[b, k:K] = 0.0
    acc2, corr2 = oracle.sample_consensus_dyn(P2, Q2, c2, U2, kl)
    np.testing.assert_array_equal(acc, acc2)
    np.testing.assert_array_equal(corr, corr2)
    assert (acc <= np.array(kl)).all()
    # the residual draw moves with u_K, not with u_{k_b}
    U3 = U.copy()
    U3[:, K] = 1.0 - U3[:, K]
    _, corr3 = oracle.sample_consensus_dyn(P, Q, cand, U3, kl)
    rejected = acc < np.array(kl)
    assert rejected.any()
    assert (corr3[rejected] != corr[rejected]).any()


def test_sampler_accepts_the_whole_live_block_when_every_test_passes():
    rng = np.random.default_rng(2)
    B, K, V = 4, 6, 9
    P = _probs(rng, B, K, V)
    cand = P.argmax(axis=2)
    U = np.zeros((B, K + 1), dtype=np.float32)   # u = 0 < p/q: every live test passes
    kl = [1, 3, 6, 2]
    acc, corr = oracle.sample_consensus_dyn(P, P, cand, U, kl)
    assert list(acc) == kl and (corr == -1).all()
    # one failing test at row k_b - 1 (q = 2p there, u just below 1)
    P2 = P.copy()
    Qm = P.copy()
    U2 = U.copy()
    for b, k in enumerate(kl):
        U2[b, k - 1] = np.float32(1.0 - 2.0 ** -24)
        Qm[b, k - 1, cand[b, k - 1]] = min(1.0, 2.0 * P2[b, k - 1, cand[b, k - 1]])
    acc2, corr2 = oracle.sample_consensus_dyn(P2, Qm, cand, U2, kl)
    assert list(acc2) == [k - 1 for k in kl]
    assert (corr2 >= 0).all()


def test_sampler_with_the_full_block_is_the_static_sampler():
    rng = np.random.default_rng(4)
    B, K, V = 3, 4, 7
    P, Q = _probs(rng, B, K, V), _probs(rng, B, K, V)
    cand = rng.integers(0, V, size=(B, K))
    U = (rng.integers(0, 2 ** 24, size=(B, K + 1)) / 2 ** 24).astype(np.float32)
    a1, c1 = oracle.sample_consensus_dyn(P, Q, cand, U, [K] * B)
    a2, c2 = oracle.sample_consensus(P, Q, cand, U)
    np.testing.assert_array_equal(a1, a2)
    np.testing.assert_array_equal(c1, c2)


def test_acceptance_statistic_update_by_hand():
    """A and N (high and low 16 bits, units of 1/16 candidate) decay by 7/8
    and add the cycle's accepted and tested candidates (R30)."""
    s1 = oracle.update_accept_stat(0, 3, 32)          # 3 accepted, then a rejection: 4 tested
    assert s1 == (48 << 16) | 64
    s2 = oracle.update_accept_stat(s1, 8, 8)          # whole block of 8: 8 tested, no rejection
    assert s2 == ((48 - 6 + 128) << 16) | (64 - 8 + 128)
    s3 = oracle.update_accept_stat(0, 0, 4)           # rejected at once: 1 tested
    assert s3 == 16


# (packed statistic, K, k_min) -> next block length, worked out by hand:
#   (48, 64): P = 49152 -> 36864 (k 2) -> 20736 (k 4) -> 6561 (k 8) <= 8192
#   (170, 184): P = 60549 -> 55941 -> 47750 -> 34790 -> 18468 (k 16) -> 5204 (k 32)
#   (0, 16): P = 0 <= 8192 at k = 1
#   (16, 32): P = 32768 -> 16384 (k 2) -> 4096 (k 4)
HAND = [
    (0, 32, 4, 32),                          # no evidence: K
    ((48 << 16) | 64, 32, 2, 8),
    ((48 << 16) | 64, 32, 16, 16),           # floor
    ((170 << 16) | 184, 32, 1, 32),
    ((170 << 16) | 184, 24, 1, 24),          # capped at a K that is no power of two
    (16, 32, 1, 1),
    (16, 32, 4, 4),
    ((16 << 16) | 32, 32, 1, 4),
    ((100 << 16) | 50, 32, 1, 32),           # A above N counts as N: p = 1
]


@pytest.mark.parametrize("stat,K,k_min,k", HAND)
def test_block_length_from_statistic_by_hand(stat, K, k_min, k):
    assert oracle.block_len_from_stat(stat, K, k_min) == k


@pytest.mark.parametrize("p,K,k", [(0.3, 32, 2), (0.5, 32, 4), (0.6, 32, 8), (0.7, 32, 8), (0.75, 32, 8),
                                   (0.85, 32, 16), (0.9, 32, 32), (0.95, 32, 32), (0.95, 128, 64),
                                   (0.99, 128, 128), (0.1, 32, 1)])
def test_block_length_is_the_smallest_power_of_two_with_rare_overrun(p, K, k):
    """Away from the boundaries (1/8)^(1/k) the integer rule picks what the
    float rule does: the smallest power of two k with p^k <= 1/8."""
    want = 1
    while want < K and p ** want > 0.125:
        want *= 2
    assert want == k
    N = 16000
    stat = (int(round(p * N)) << 16) | N
    assert oracle.block_len_from_stat(stat, K, 1) == k


def test_block_length_grows_with_the_match_rate():
    ks = [oracle.block_len_from_stat((a << 16) | 4096, 128, 1) for a in range(0, 4097, 64)]
    assert ks == sorted(ks) and ks[0] == 1 and ks[-1] == 128


def test_commit_hand_worked():
    """One layer, one KV head, D = 8 (one 16-byte vector per row), K = 6,
    max_len 16.  Block row i holds the value 100 + 10 b + i in every lane;
    rows past k_b hold 0x7777, which must never reach the cache."""
    n_layers, B, Hkv, K, D, max_len = 1, 4, 1, 6, 8, 16
    kc = np.zeros((n_layers, B, Hkv, max_len, D), dtype=np.uint16)
    vc = np.zeros_like(kc)
    kb = np.zeros((n_layers, B, Hkv, K, D), dtype=np.uint16)
    kl = [3, 3, 6, 2]
    for b in range(B):
        for i in range(K):
            kb[:, b, :, i] = 100 + 10 * b + i if i < kl[b] else 0x7777
    vb = kb + np.uint16(1000)
    lens = [5, 5, 0, 15]
    acc = [3, 1, 6, 2]        # b0: whole block; b1: one accepted; b2: whole block; b3: no room
    corr = [-1, 77, -1, 55]
    cand = np.arange(B * K).reshape(B, K) + 10
    r = oracle.commit_block_dyn(kc, vc, kb, vb, lens, acc, corr, cand, kl, [0, 0, 0, 0], k_min=2)
    # b0: k_b = 3, a = 3: rows 0..2 at 5..7, tokens cand[0..2], anchor cand[2]
    assert r["cache_len"][0] == 8 and r["n_tokens"][0] == 3
    assert list(r["tokens"][0]) == [10, 11, 12, -1, -1, -1] and r["next_anchor"][0] == 12
    assert (r["k_cache"][0, 0, 0, 5:8, 0] == [100, 101, 102]).all()
    assert (r["k_cache"][0, 0, 0, 8:, 0] == 0).all()
    # 3 of 3: A = N = 48, p = 1: the whole capacity
    assert r["accept_stat"][0] == (48 << 16) | 48 and r["blk_len"][0] == 6
    # b1: a = 1 < k_b: rows 0..1 at 5..6, tokens cand[0], 77; anchor 77
    assert r["cache_len"][1] == 7 and list(r["tokens"][1][:2]) == [16, 77] and r["next_anchor"][1] == 77
    assert (r["v_cache"][0, 1, 0, 5:7, 0] == [1110, 1111]).all() and (r["v_cache"][0, 1, 0, 7:, 0] == 0).all()
    # 1 of 3, then a rejection: A = 16, N = 32, p = 1/2: p^4 = 1/16 <= 1/8
    assert r["accept_stat"][1] == (16 << 16) | 32 and r["blk_len"][1] == 4
    # b2: k_b = K = 6, a = 6: the static commit of the whole block
    assert r["cache_len"][2] == 6 and r["next_anchor"][2] == cand[2, 5] and r["blk_len"][2] == 6
    # b3: 15 + 2 > 16: refused, nothing written, length and block length kept
    assert r["cache_len"][3] == 15 and r["n_tokens"][3] == 0 and r["blk_len"][3] == 2
    assert r["accept_stat"][3] == 0
    assert (r["k_cache"][0, 3] == 0).all()
    assert not (r["k_cache"] == 0x7777).any() and not (r["v_cache"] == 0x7777 + 1000).any()


def _cycles(w, n, rate, seed):
    from synth import cycle_inputs
    sets = cycle_inputs(w, n, accept_rate=rate, seed_offset=seed)
    shape = (w.layers, w.batch, w.n_kv_heads, w.capacity, w.head_dim)
    kc = torch.randn(shape, generator=torch.Generator().manual_seed(seed + 1)).to(torch.bfloat16)
    vc = torch.randn(shape, generator=torch.Generator().manual_seed(seed + 2)).to(torch.bfloat16)
    return sets, kc, vc


def test_cycles_with_every_block_at_capacity_are_the_static_cycles():
    """k_b = K and k_min = K: the rule can never move k, so every cycle is the
    static (pinned) cycle."""
    w = Workload("dyncyc", 2, 2, 4, 2, 16, 40, 4, 50, 4.0, 5, max_len=40 + 4 * 4)
    sets, kc, vc = _cycles(w, 4, 0.6, 3)
    L = torch.tensor([40, 9], dtype=torch.int32)
    r1, s1 = oracle.decode_cycles(kc, vc, L, sets)
    r2, s2 = oracle.decode_cycles_dyn(kc, vc, L, [4, 4], 4, sets)  # k_min = K: the rule can only give K
    for a, b in zip(r1, r2):
        for n in ("accept_len", "correction", "cache_len", "next_anchor", "tokens", "n_tokens"):
            np.testing.assert_array_equal(a[n], b[n])
        for x, y in zip(a["diff_out"] + a["verify_out"], b["diff_out"] + b["verify_out"]):
            np.testing.assert_array_equal(x, y)
        assert b["blk_len"].tolist() == [4, 4]
    np.testing.assert_array_equal(s1["k_cache"], s2["k_cache"])
    np.testing.assert_array_equal(s1["cache_len"], s2["cache_len"])


def test_cycle_block_lengths_follow_the_rule_and_the_lengths_add_up():
    w = Workload("dyncyc2", 1, 3, 2, 1, 16, 30, 8, 40, 4.0, 6, max_len=30 + 8 * 6)
    sets, kc, vc = _cycles(w, 6, 0.7, 9)
    recs, st = oracle.decode_cycles_dyn(kc, vc, [30, 0, 12], [8, 2, 5], 2, sets)
    lens = np.array([30, 0, 12])
    k = np.array([8, 2, 5])
    stat = [0, 0, 0]
    for c, rec in enumerate(recs):
        assert rec["blk_len_in"].tolist() == k.tolist()
        a = rec["accept_len"]
        # the planted first mismatch j*, cut at the block length
        assert (a == np.minimum(sets[c]["j_star"].numpy(), k)).all()
        n = a + (a < k)
        assert rec["n_tokens"].tolist() == n.tolist()
        lens = lens + n
        assert rec["cache_len"].tolist() == lens.tolist()
        stat = [oracle.update_accept_stat(stat[b], int(a[b]), int(k[b])) for b in range(3)]
        assert rec["accept_stat"].tolist() == stat
        k = np.array([oracle.block_len_from_stat(stat[b], 8, 2) for b in range(3)])
        assert rec["blk_len"].tolist() == k.tolist()
        for out in rec["verify_out"]:
            for b in range(3):
                assert np.isnan(out[b, :, rec["blk_len_in"][b]:]).all()
                assert np.isfinite(out[b, :, :rec["blk_len_in"][b]]).all()
    assert st["blk_len"].tolist() == k.tolist()


def test_sample_cycles_with_a_one_hot_target_are_the_greedy_cycles():
    """With block lengths adapting, T > 0 cycles whose target is a point mass
    at the argmax retrace the greedy cycles: same accepted prefixes (the
    planted mismatch cut at k_b), corrections, statistics and block lengths."""
    w = Workload("dyns", 1, 3, 4, 2, 16, 30, 8, 40, 4.0, 7, max_len=30 + 6 * 8)
    sets, kc, vc = _cycles(w, 6, 0.7, 4)
    g = torch.Generator().manual_seed(8)
    tsets = []
    for s in sets:
        B, K, V = s["logits"].shape
        p = torch.zeros(B, K, V)
        p.scatter_(2, s["logits"].argmax(-1, keepdim=True), 1.0)
        q = torch.softmax(torch.randn(B, K, V, generator=g, dtype=torch.float64), -1).float()
        u = (torch.randint(0, 1 << 24, (B, K + 1), generator=g).double() / (1 << 24)).float()
        tsets.append({"diff": s["diff"], "verify": s["verify"], "cand": s["cand"], "p": p, "q": q, "uniforms": u})
    r1, s1 = oracle.decode_cycles_dyn(kc, vc, [30, 0, 12], [8, 2, 5], 2, sets, keep_attention=False)
    r2, s2 = oracle.decode_cycles_dyn(kc, vc, [30, 0, 12], [8, 2, 5], 2, tsets, keep_attention=False)
    for c, (a, b) in enumerate(zip(r1, r2)):
        for n in ("accept_len", "correction", "cache_len", "tokens", "n_tokens", "accept_stat", "blk_len"):
            np.testing.assert_array_equal(a[n], b[n], err_msg=f"cycle {c} {n}")
    np.testing.assert_array_equal(s1["k_cache"], s2["k_cache"])


def test_sample_cycles_with_the_draft_equal_to_the_target_grow_the_block():
    """q = p keeps every live candidate, so a = k_b each cycle; the estimate
    of the match rate stays at 1 and the block length climbs to K."""
    from synth import sample_cycle_inputs
    w = Workload("dyns2", 1, 2, 4, 2, 16, 20, 16, 30, 3.0, 9, max_len=20 + 8 * 16)
    sets = sample_cycle_inputs(w, 8, draft_noise=0.3)
    for s in sets:
        s["q"] = s["p"].clone()
    kc = torch.randn((1, 2, 2, w.capacity, 16), generator=torch.Generator().manual_seed(1)).to(torch.bfloat16)
    vc = torch.randn((1, 2, 2, w.capacity, 16), generator=torch.Generator().manual_seed(2)).to(torch.bfloat16)
    recs, st = oracle.decode_cycles_dyn(kc, vc, [20, 4], [1, 3], 1, sets, keep_attention=False)
    for rec in recs:
        np.testing.assert_array_equal(rec["accept_len"], rec["blk_len_in"])
        assert (rec["correction"] == -1).all()
    assert st["blk_len"].tolist() == [16, 16]
