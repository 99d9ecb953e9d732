"""Pins for the cycle-commit oracle (CPU only).

* Hand-worked cases: the rows, length, emitted tokens and next anchor of a
  commit with a mismatch at the first candidate, in the middle, and with all
  K candidates accepted, written out from the paper notes' §4.1 description.
* Capacity and bad-input cases: refused commits leave everything untouched;
  a commit that exactly fills the cache is accepted.
* Sequential decoding: after the commit, the AR verify output of every
  committed block row equals one plain single-token decode step (K = 1) over
  the committed cache at that row's position -- the "verify over K tokens is
  K sequential causal decode steps" invariant carried across the commit.  A
  row written to the wrong position, in the wrong order, or a K/V mix-up
  breaks it.
* Losslessness at T = 0 (paper notes §4.2): a toy deterministic AR model
  driven through many cycles of greedy consensus and commit emits exactly the
  AR model's own greedy sequence, and the cache ends up holding that sequence
  position by position; every cycle emits between 1 and K tokens.
"""
import random

import numpy as np
import pytest
import torch

import oracle
from oracle.cycle import bits_to_bf16, commit_block, decode_cycles
from synth import Workload, cycle_inputs, first_mismatch_geometric


def _planes(n_layers, B, Hkv, rows, D, base):
    """uint16 planes whose rows carry recognisable values: base + 100*layer + 10*g + row
    in element 0, the sequence index in element 1."""
    x = np.zeros((n_layers, B, Hkv, rows, D), dtype=np.uint16)
    for layer in range(n_layers):
        for b in range(B):
            for g in range(Hkv):
                for r in range(rows):
                    x[layer, b, g, r, 0] = base + 100 * layer + 10 * g + r
                    x[layer, b, g, r, 1] = b
    return x


# ----------------------------------------------------------- hand cases ----
@pytest.mark.parametrize("a,rows_written,new_len,tokens,anchor", [
    # first candidate rejected: the anchor's row is committed, the correction emitted
    (0, [0], 4, [90, -1, -1, -1], 90),
    # two accepted: anchor + 2 candidates committed; tokens c0, c1, correction
    (2, [0, 1, 2], 6, [70, 71, 90, -1], 90),
    # all K accepted, no bonus: rows 0..K-1 committed, next anchor = last candidate
    (4, [0, 1, 2, 3], 7, [70, 71, 72, 73], 73),
])
def test_commit_hand_cases(a, rows_written, new_len, tokens, anchor):
    L, K, max_len, D = 3, 4, 10, 8
    kc = _planes(1, 1, 1, max_len, D, 1000)
    vc = _planes(1, 1, 1, max_len, D, 3000)
    kb = _planes(1, 1, 1, K, D, 2000)
    vb = _planes(1, 1, 1, K, D, 4000)
    cand = np.array([[70, 71, 72, 73]])
    corr = np.array([90 if a < K else -1])
    r = commit_block(kc, vc, kb, vb, np.array([L]), np.array([a]), corr, cand)
    assert r["cache_len"].tolist() == [new_len]
    assert r["n_tokens"].tolist() == [new_len - L]
    assert r["tokens"].tolist() == [tokens]
    assert r["next_anchor"].tolist() == [anchor]
    col_k = r["k_cache"][0, 0, 0, :, 0].tolist()
    col_v = r["v_cache"][0, 0, 0, :, 0].tolist()
    want_k = [1000 + p for p in range(max_len)]
    want_v = [3000 + p for p in range(max_len)]
    for i in rows_written:
        want_k[L + i] = 2000 + i
        want_v[L + i] = 4000 + i
    assert col_k == want_k and col_v == want_v
    # inputs are not modified
    assert kc[0, 0, 0, L, 0] == 1000 + L


def test_commit_layers_heads_and_batch():
    """Every layer and KV head gets its own block rows; sequences are independent."""
    n_layers, B, Hkv, max_len, K, D = 3, 3, 2, 12, 3, 8
    kc, vc = _planes(n_layers, B, Hkv, max_len, D, 1000), _planes(n_layers, B, Hkv, max_len, D, 5000)
    kb, vb = _planes(n_layers, B, Hkv, K, D, 3000), _planes(n_layers, B, Hkv, K, D, 7000)
    lens, acc = np.array([0, 5, 9]), np.array([1, 3, 0])
    corr, cand = np.array([11, -1, 12]), np.array([[1, 2, 3], [4, 5, 6], [7, 8, 9]])
    r = commit_block(kc, vc, kb, vb, lens, acc, corr, cand)
    assert r["cache_len"].tolist() == [2, 8, 10]
    assert r["next_anchor"].tolist() == [11, 6, 12]
    assert r["tokens"].tolist() == [[1, 11, -1], [4, 5, 6], [12, -1, -1]]
    for b in range(B):
        solo = commit_block(kc[:, b:b + 1], vc[:, b:b + 1], kb[:, b:b + 1], vb[:, b:b + 1],
                            lens[b:b + 1], acc[b:b + 1], corr[b:b + 1], cand[b:b + 1])
        assert np.array_equal(solo["k_cache"][:, 0], r["k_cache"][:, b])
        assert np.array_equal(solo["v_cache"][:, 0], r["v_cache"][:, b])
    # layer 2, head 1 of sequence 1: rows 5..7 hold block rows 0..2 of that layer/head
    assert r["k_cache"][2, 1, 1, 5:8, 0].tolist() == [3000 + 200 + 10 + i for i in range(3)]
    assert r["v_cache"][2, 1, 1, 5:8, 0].tolist() == [7000 + 200 + 10 + i for i in range(3)]
    assert r["k_cache"][2, 1, 1, 8, 0] == 1000 + 200 + 10 + 8


@pytest.mark.parametrize("L,a,ok", [
    (7, 2, True),     # 7 + 3 = 10 = max_len: fills the cache exactly
    (7, 3, False),    # 7 + 4 > 10
    (6, 4, True),     # all accepted: 6 + 4 = 10
    (7, 4, False),
    (3, 5, False),    # a > K
    (3, -1, False),   # a < 0
    (-1, 1, False),   # negative length
    (11, 0, False),   # length beyond capacity
])
def test_commit_refused_leaves_state(L, a, ok):
    K, max_len, D = 4, 10, 8
    kc, vc = _planes(1, 1, 1, max_len, D, 1000), _planes(1, 1, 1, max_len, D, 3000)
    kb, vb = _planes(1, 1, 1, K, D, 2000), _planes(1, 1, 1, K, D, 4000)
    r = commit_block(kc, vc, kb, vb, np.array([L]), np.array([a]), np.array([50]),
                     np.array([[1, 2, 3, 4]]))
    if ok:
        assert r["n_tokens"][0] == a + (a < K)
        assert r["cache_len"][0] == L + a + (a < K)
    else:
        assert r["n_tokens"].tolist() == [0]
        assert r["cache_len"].tolist() == [L]
        assert r["next_anchor"].tolist() == [-1]
        assert r["tokens"].tolist() == [[-1] * K]
        assert np.array_equal(r["k_cache"], kc) and np.array_equal(r["v_cache"], vc)


def test_commit_accepts_torch_bf16():
    g = torch.Generator().manual_seed(5)
    kc = torch.randn((1, 1, 2, 9, 16), generator=g).to(torch.bfloat16)
    vc = torch.randn((1, 1, 2, 9, 16), generator=g).to(torch.bfloat16)
    kb = torch.randn((1, 1, 2, 3, 16), generator=g).to(torch.bfloat16)
    vb = torch.randn((1, 1, 2, 3, 16), generator=g).to(torch.bfloat16)
    r = commit_block(kc, vc, kb, vb, torch.tensor([4]), torch.tensor([1]), torch.tensor([7]),
                     torch.tensor([[3, 4, 5]]))
    got_k, got_v = bits_to_bf16(r["k_cache"]), bits_to_bf16(r["v_cache"])
    assert torch.equal(got_k[0, 0, :, 4:6], kb[0, 0, :, 0:2])
    assert torch.equal(got_v[0, 0, :, 4:6], vb[0, 0, :, 0:2])
    assert torch.equal(got_k[0, 0, :, :4], kc[0, 0, :, :4])
    assert torch.equal(got_k[0, 0, :, 6:], kc[0, 0, :, 6:])


# ---------------------------------------------- sequential decode link ----
@pytest.mark.parametrize("lens,acc,K", [([7, 0], [2, 5], 5), ([3, 12], [0, 1], 4), ([5], [1], 1)])
def test_commit_then_single_token_decode_reproduces_verify_rows(lens, acc, K):
    B, Hq, Hkv, D, max_len = len(lens), 4, 2, 64, 24
    g = torch.Generator().manual_seed(11 + K)
    bf = lambda *s: torch.randn(s, generator=g).to(torch.bfloat16)
    q = bf(B, Hq, K, D)
    kb, vb = bf(B, Hkv, K, D), bf(B, Hkv, K, D)
    kc, vc = bf(B, Hkv, max_len, D), bf(B, Hkv, max_len, D)
    L = torch.tensor(lens, dtype=torch.int32)
    verify, _ = oracle.block_attention(q, kb, vb, kc, vc, L, oracle.MASK_VERIFY_CAUSAL)
    cand = torch.arange(B * K).reshape(B, K)
    corr = torch.tensor([100 + b if acc[b] < K else -1 for b in range(B)])
    r = commit_block(kc[None], vc[None], kb[None], vb[None], L, torch.tensor(acc), corr, cand)
    kc2, vc2 = bits_to_bf16(r["k_cache"])[0], bits_to_bf16(r["v_cache"])[0]
    for b in range(B):
        committed = int(r["n_tokens"][b])
        assert committed == acc[b] + (acc[b] < K)
        for i in range(committed):
            # one decode step of the token at position lens[b] + i: its own K/V is the
            # single block key, everything before it comes from the committed cache
            one, _ = oracle.block_attention(q[b:b + 1, :, i:i + 1], kb[b:b + 1, :, i:i + 1],
                                            vb[b:b + 1, :, i:i + 1], kc2[b:b + 1], vc2[b:b + 1],
                                            torch.tensor([lens[b] + i]), oracle.MASK_DIFF_BIDIR)
            np.testing.assert_allclose(one[0, :, 0], verify[b, :, i], rtol=0, atol=1e-12)


# ------------------------------------------------- lossless toy AR loop ----
class ToyAR:
    """A deterministic stand-in for a frozen AR model over a small vocabulary:
    the greedy next token is a hash of the last few tokens."""

    def __init__(self, vocab, seed):
        self.V = vocab
        self.salt = seed * 2654435761 % (1 << 31)

    def next_token(self, seq):
        h = self.salt
        for p, tok in enumerate(seq[-5:]):
            h = (h * 1000003 + (tok + 1) * 7919 + p) % (1 << 31)
        return h % self.V


def _enc(token, pos, layer, g, D, kind):
    row = np.zeros(D, dtype=np.uint16)
    row[0], row[1], row[2], row[3], row[4] = token, pos & 0xFF, pos >> 8, layer, g
    row[5] = kind
    return row


def _run_toy(B, K, accept_rate, n_cycles, seed, n_layers=2, Hkv=2, D=8, V=37, prompt_len=5):
    rng = random.Random(seed)
    model = ToyAR(V, seed)
    max_len = prompt_len + n_cycles * K + 1
    streams = [[rng.randrange(V) for _ in range(prompt_len)] for _ in range(B)]
    kc = np.zeros((n_layers, B, Hkv, max_len, D), dtype=np.uint16)
    vc = np.zeros_like(kc)
    for b in range(B):                       # the prompt except its last token is cached
        for p in range(prompt_len - 1):
            for layer in range(n_layers):
                for g in range(Hkv):
                    kc[layer, b, g, p] = _enc(streams[b][p], p, layer, g, D, 1)
                    vc[layer, b, g, p] = _enc(streams[b][p], p, layer, g, D, 2)
    lens = np.full(B, prompt_len - 1)
    for _ in range(n_cycles):
        cand = np.zeros((B, K), dtype=np.int64)
        logits = np.zeros((B, K, V))
        kb = np.zeros((n_layers, B, Hkv, K, D), dtype=np.uint16)
        vb = np.zeros_like(kb)
        for b in range(B):
            seq = list(streams[b])           # ends with the anchor
            t = int(lens[b])
            assert t == len(seq) - 1
            # diffusion candidates: right with probability accept_rate, else surely wrong
            draft = []
            for k in range(K):
                right = model.next_token(seq + draft)
                draft.append(right if rng.random() < accept_rate
                             else (right + 1 + rng.randrange(V - 1)) % V)
            cand[b] = draft
            block = [seq[-1]] + draft[:K - 1]  # verify rows: anchor, y1 .. y(K-1)
            for i in range(K):
                top = model.next_token(seq + draft[:i])
                row = np.array([rng.gauss(0.0, 3.0) for _ in range(V)])
                row[top] = row.max() + 1.0
                logits[b, i] = row
                for layer in range(n_layers):
                    for g in range(Hkv):
                        kb[layer, b, g, i] = _enc(block[i], t + i, layer, g, D, 1)
                        vb[layer, b, g, i] = _enc(block[i], t + i, layer, g, D, 2)
        acc, _, corr = oracle.greedy_consensus(logits, cand)
        r = commit_block(kc, vc, kb, vb, lens, acc, corr, cand)
        for b in range(B):
            n = int(r["n_tokens"][b])
            assert 1 <= n <= K                # at least one token per two forwards, at most K
            emitted = r["tokens"][b, :n].tolist()
            assert r["tokens"][b, n:].tolist() == [-1] * (K - n)
            assert r["next_anchor"][b] == emitted[-1]
            streams[b].extend(emitted)
        kc, vc, lens = r["k_cache"], r["v_cache"], r["cache_len"]
    return model, streams, kc, vc, lens, prompt_len


@pytest.mark.parametrize("B,K,rate,cycles", [(3, 4, 0.7, 12), (2, 8, 0.9, 8), (2, 1, 0.5, 10),
                                            (1, 6, 1.0, 4), (1, 5, 0.0, 6)])
def test_toy_decode_is_lossless_and_cache_holds_the_sequence(B, K, rate, cycles):
    model, streams, kc, vc, lens, P = _run_toy(B, K, rate, cycles, seed=K * 100 + B)
    n_layers, _, Hkv, _, D = kc.shape
    for b in range(B):
        s = streams[b]
        ar = list(s[:P])
        while len(ar) < len(s):
            ar.append(model.next_token(ar))
        assert s == ar, "the emitted sequence must be the AR model's own greedy sequence"
        assert lens[b] == len(s) - 1, "every position except the new anchor is cached"
        for p in range(len(s) - 1):
            for layer in range(n_layers):
                for g in range(Hkv):
                    assert np.array_equal(kc[layer, b, g, p], _enc(s[p], p, layer, g, D, 1))
                    assert np.array_equal(vc[layer, b, g, p], _enc(s[p], p, layer, g, D, 2))
        assert not kc[:, b, :, len(s) - 1:].any(), "no row past the committed prefix is written"
    if rate == 1.0:
        assert all(len(s) == P + cycles * K for s in streams)
    if rate == 0.0:
        assert all(len(s) == P + cycles for s in streams)


# ---------------------------------------------------- whole cycles ----
def test_decode_cycles_follow_the_planted_acceptance():
    w = Workload("t", 2, 2, 4, 2, 64, 40, 4, 50, 4.0, 9, max_len=40 + 3 * 4)
    cyc = cycle_inputs(w, 3, accept_rate=0.6)
    kc = torch.randn((2, 2, 2, w.capacity, 64), generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    vc = torch.randn((2, 2, 2, w.capacity, 64), generator=torch.Generator().manual_seed(4)).to(torch.bfloat16)
    lens = torch.tensor([40, 33], dtype=torch.int32)
    recs, state = decode_cycles(kc, vc, lens, cyc)
    cur = lens.numpy().astype(np.int64)
    for rec, c in zip(recs, cyc):
        assert np.array_equal(rec["cache_len_in"], cur)
        assert rec["accept_len"].tolist() == c["j_star"].tolist()
        n = rec["n_tokens"]
        assert np.array_equal(n, c["j_star"].numpy() + (c["j_star"].numpy() < 4))
        cur = cur + n
        assert np.array_equal(rec["cache_len"], cur)
        assert len(rec["diff_out"]) == 2 and rec["verify_out"][1].shape == (2, 4, 4, 64)
    assert np.array_equal(state["cache_len"], cur)


@pytest.mark.parametrize("rate", [0.815, 0.912])
def test_geometric_first_mismatch_mean(rate):
    j = first_mismatch_geometric(100000, 32, rate, 1)
    assert j.min() >= 0 and j.max() <= 32
    n = (j + (j < 32).long()).double().mean().item()
    # E[j*] = sum_{i=1..K} P(j* >= i) = sum rate^i; plus P(j* < K) = 1 - rate^K
    expected = sum(rate ** i for i in range(1, 33)) + 1 - rate ** 32
    assert abs(n - expected) < 0.05 * expected
    if rate == 0.912:
        assert abs(expected - 2 * 5.39) < 0.1


def test_quantile_first_mismatch_follow_the_law():
    from synth import first_mismatch_quantiles
    j = first_mismatch_quantiles(16, 32, 0.815, 3)
    # P(j* <= j) = 1 - 0.815^(j+1): the (s+1/2)/16 quantiles, worked out by hand
    assert sorted(j.tolist()) == [0, 0, 0, 1, 1, 2, 2, 3, 3, 4, 5, 6, 7, 9, 11, 16]
    n = j + (j < 32).long()
    assert abs(n.double().mean().item() - 5.4) < 0.1
    j = first_mismatch_quantiles(32, 32, 0.912, 3)
    n = j + (j < 32).long()
    assert abs(n.double().mean().item() - 10.8) < 0.1
    assert first_mismatch_quantiles(4, 8, 1.0, 0).tolist() == [8, 8, 8, 8]
    assert first_mismatch_quantiles(4, 8, 0.0, 0).tolist() == [0, 0, 0, 0]


# ------------------------------------------------- T > 0 whole cycles ----
def _one_hot_target_sets(sets, seed):
    """The greedy cycle sets turned into T > 0 sets: the target puts all its
    mass on each row's argmax of the logits, the draft is a full-support
    softmax, and the uniforms lie on the 2**-24 grid in [0, 1)."""
    g = torch.Generator().manual_seed(seed)
    out = []
    for s in sets:
        B, K, V = s["logits"].shape
        p = torch.zeros(B, K, V)
        p.scatter_(2, s["logits"].argmax(-1, keepdim=True), 1.0)
        q = torch.softmax(torch.randn(B, K, V, generator=g, dtype=torch.float64), -1).float()
        u = (torch.randint(0, 1 << 24, (B, K + 1), generator=g).double() / (1 << 24)).float()
        t = {k: v for k, v in s.items() if k != "logits"}
        t.update(p=p, q=q, uniforms=u)
        out.append(t)
    return out


def _cycle_state(w, seed):
    shape = (w.layers, w.batch, w.n_kv_heads, w.capacity, w.head_dim)
    kc = torch.randn(shape, generator=torch.Generator().manual_seed(seed + 1)).to(torch.bfloat16)
    vc = torch.randn(shape, generator=torch.Generator().manual_seed(seed + 2)).to(torch.bfloat16)
    return kc, vc


def test_sample_cycles_with_a_one_hot_target_are_the_greedy_cycles():
    """A target with all its mass on the argmax turns rejection sampling into
    greedy consensus (notes §4.2-4.3): a candidate at the argmax has ratio
    1/q > u and is kept, any other has p = 0 and is refused, and the residual
    max(p - q, 0) is a point mass at the argmax.  The T > 0 cycles must then
    retrace the greedy cycles, and the planted first mismatch."""
    w = Workload("t0", 2, 3, 4, 2, 32, 60, 6, 40, 4.0, 11, max_len=60 + 5 * 6)
    greedy = cycle_inputs(w, 5, accept_rate=0.7)
    kc, vc = _cycle_state(w, 5)
    lens = torch.tensor([60, 0, 17], dtype=torch.int32)
    r1, s1 = decode_cycles(kc, vc, lens, greedy, keep_attention=False)
    r2, s2 = decode_cycles(kc, vc, lens, _one_hot_target_sets(greedy, 3), keep_attention=False)
    for c, (a, b) in enumerate(zip(r1, r2)):
        assert b["accept_len"].tolist() == greedy[c]["j_star"].tolist()
        for n in ("accept_len", "correction", "cache_len", "next_anchor", "tokens", "n_tokens"):
            np.testing.assert_array_equal(a[n], b[n], err_msg=f"cycle {c} {n}")
    np.testing.assert_array_equal(s1["k_cache"], s2["k_cache"])
    np.testing.assert_array_equal(s1["v_cache"], s2["v_cache"])


def test_sample_cycles_with_the_draft_equal_to_the_target_keep_every_candidate():
    """q = p makes every ratio exactly 1 > u: each cycle keeps all K
    candidates, emits no correction, and the cache grows by K per cycle with
    the candidates as the emitted tokens."""
    from synth import sample_cycle_inputs
    w = Workload("t1", 1, 2, 4, 2, 32, 50, 5, 30, 3.0, 12, max_len=50 + 4 * 5)
    sets = sample_cycle_inputs(w, 4, draft_noise=0.3)
    for s in sets:
        s["q"] = s["p"].clone()
    kc, vc = _cycle_state(w, 6)
    recs, st = decode_cycles(kc, vc, torch.tensor([50, 3], dtype=torch.int32), sets, keep_attention=False)
    for c, rec in enumerate(recs):
        assert rec["accept_len"].tolist() == [5, 5] and rec["correction"].tolist() == [-1, -1]
        assert rec["cache_len"].tolist() == [50 + 5 * (c + 1), 3 + 5 * (c + 1)]
        assert rec["tokens"][:, :5].tolist() == sets[c]["cand"].tolist()
    assert st["cache_len"].tolist() == [70, 23]


def test_sample_cycles_commit_what_the_sampler_decides():
    """Cycles over a near draft: each cycle commits the accepted prefix plus
    the sampled correction, and the lengths add up from cycle to cycle."""
    from synth import sample_cycle_inputs
    w = Workload("t2", 2, 3, 4, 2, 32, 40, 8, 60, 3.0, 13, max_len=40 + 6 * 8)
    sets = sample_cycle_inputs(w, 6, draft_noise=0.5)
    kc, vc = _cycle_state(w, 7)
    recs, st = decode_cycles(kc, vc, torch.tensor([40, 1, 25], dtype=torch.int32), sets, keep_attention=False)
    cur = np.array([40, 1, 25])
    seen = set()
    for c, rec in enumerate(recs):
        acc, corr = oracle.sample_consensus(sets[c]["p"], sets[c]["q"], sets[c]["cand"], sets[c]["uniforms"])
        np.testing.assert_array_equal(rec["accept_len"], acc)
        np.testing.assert_array_equal(rec["correction"], corr)
        n = acc + (acc < 8)
        cur = cur + n
        np.testing.assert_array_equal(rec["cache_len"], cur)
        for b in range(3):
            assert rec["tokens"][b, :acc[b]].tolist() == sets[c]["cand"][b, :acc[b]].tolist()
            if acc[b] < 8:
                assert rec["tokens"][b, acc[b]] == corr[b]
        seen.update(acc.tolist())
    assert len(seen) > 2, "the near draft should give a spread of accept lengths"
    np.testing.assert_array_equal(st["cache_len"], cur)
