"""Pins for the tree-verification oracle (CPU only).

* Masks: a chain gives the causal (verify) mask, a star gives {root, self},
  unused nodes see only themselves; a hand-drawn tree.
* Masked attention: the explicit causal / all-ones masks reproduce the verify
  / diffusion modes; an empty row gives 0 and lse -inf; every tree row equals
  one plain decode step over the cache plus its root path (sequential decode
  along the path).
* Tree consensus: on a chain it emits exactly the tokens of the linear greedy
  rule (R2/R3) on the same rows; a brute-force walk over all root paths; a
  hand-worked tree.
* Path commit: on a chain it equals the linear commit; a toy AR model driven
  through many cycles of random draft trees emits exactly its own greedy
  sequence and the cache holds it (lossless at T = 0).
* Top-M: against torch.topk over torch.log_softmax, with planted ties.
* Tree building: the node set equals the n-1 best prefixes found by brute
  enumeration; M = 1 gives the chain of top-1 tokens; scores never increase
  in creation order.
"""
import itertools
import math
import random

import numpy as np
import pytest
import torch

import oracle
from oracle.consensus import greedy_consensus
from oracle.cycle import bits_to_bf16, commit_block
from oracle.tree import (ancestor_masks, build_tree, commit_path, masks_to_bits, topk_logprobs,
                         tree_greedy_consensus)


def test_masks_chain_star_unused_and_hand_tree():
    K = 6
    chain = np.array([[-1, 0, 1, 2, 3, 4]])
    assert np.array_equal(ancestor_masks(chain)[0], np.tril(np.ones((K, K), dtype=bool)))
    star = np.array([[-1, 0, 0, 0, 0, 0]])
    m = ancestor_masks(star)[0]
    assert np.array_equal(m, np.eye(K, dtype=bool) | (np.arange(K)[None, :] == 0))
    unused = np.array([[-1, 0, -1, 1, -1, 3]])
    m = ancestor_masks(unused)[0]
    assert m[2].tolist() == [False, False, True, False, False, False]
    assert m[5].tolist() == [True, True, False, True, False, True]
    # hand tree: 0 -> {1, 2}, 1 -> {3, 4}, 2 -> {5}
    hand = np.array([[-1, 0, 0, 1, 1, 2]])
    m = ancestor_masks(hand)[0]
    want = {0: {0}, 1: {0, 1}, 2: {0, 2}, 3: {0, 1, 3}, 4: {0, 1, 4}, 5: {0, 2, 5}}
    for i in range(K):
        assert set(np.nonzero(m[i])[0].tolist()) == want[i]
    bits = masks_to_bits(ancestor_masks(hand))[0]
    assert [int(x) for x in bits] == [1, 3, 5, 11, 19, 37]


def _attn_inputs(B, Hq, Hkv, K, D, L, seed):
    g = torch.Generator().manual_seed(seed)
    bf = lambda *s: torch.randn(s, generator=g).to(torch.bfloat16)
    return bf(B, Hq, K, D), bf(B, Hkv, K, D), bf(B, Hkv, K, D), bf(B, Hkv, L + 4, D), bf(B, Hkv, L + 4, D)


def test_explicit_masks_reproduce_the_two_views_and_empty_rows():
    B, Hq, Hkv, K, D, L = 2, 4, 2, 5, 16, 9
    q, kb, vb, kc, vc = _attn_inputs(B, Hq, Hkv, K, D, L, 1)
    lens = torch.tensor([L, 3])
    causal = np.broadcast_to(np.tril(np.ones((K, K), dtype=bool)), (B, K, K))
    ones = np.ones((B, K, K), dtype=bool)
    for mode, m in ((oracle.MASK_VERIFY_CAUSAL, causal), (oracle.MASK_DIFF_BIDIR, ones)):
        ref, ref_l = oracle.block_attention(q, kb, vb, kc, vc, lens, mode)
        got, got_l = oracle.block_attention(q, kb, vb, kc, vc, lens, oracle.MASK_EXPLICIT, block_masks=m)
        np.testing.assert_array_equal(got, ref)
        np.testing.assert_array_equal(got_l, ref_l)
    empty = np.zeros((B, K, K), dtype=bool)
    out, lse = oracle.block_attention(q, kb, vb, kc, vc, torch.tensor([0, 0]), oracle.MASK_EXPLICIT,
                                      block_masks=empty)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_tree_rows_are_decode_steps_along_their_path():
    B, Hq, Hkv, K, D, L = 1, 4, 2, 6, 16, 7
    q, kb, vb, kc, vc = _attn_inputs(B, Hq, Hkv, K, D, L, 2)
    parent = np.array([[-1, 0, 0, 1, 1, 2]])
    m = ancestor_masks(parent)
    out, _ = oracle.block_attention(q, kb, vb, kc, vc, torch.tensor([L]), oracle.MASK_EXPLICIT, block_masks=m)
    for i in range(K):
        path = []
        j = i
        while j >= 0:
            path.append(j)
            j = int(parent[0, j]) if j > 0 else -1
        path = path[::-1]  # root .. i
        # cache extended by the ancestors' rows, then node i as the single block key
        ext_k = torch.cat([kc[:, :, :L], kb[:, :, path[:-1]]], dim=2)
        ext_v = torch.cat([vc[:, :, :L], vb[:, :, path[:-1]]], dim=2)
        one, _ = oracle.block_attention(q[:, :, i:i + 1], kb[:, :, i:i + 1], vb[:, :, i:i + 1], ext_k, ext_v,
                                        torch.tensor([L + len(path) - 1]), oracle.MASK_DIFF_BIDIR)
        np.testing.assert_allclose(out[0, :, i], one[0, :, 0], rtol=0, atol=1e-12)


def _planted_logits(B, K, V, tops, seed):
    rng = np.random.default_rng(seed)
    lg = rng.normal(0.0, 3.0, (B, K, V))
    for b in range(B):
        for i in range(K):
            lg[b, i, tops[b][i]] = 30.0
    return lg


def test_tree_consensus_on_a_chain_emits_the_linear_tokens():
    rng = random.Random(3)
    K, V = 8, 50
    for trial in range(40):
        tops = [[rng.randrange(V) for _ in range(K)]]
        a_plant = rng.randrange(K + 1)
        cand = [tops[0][i] if i < a_plant else (tops[0][i] + 1) % V for i in range(K)]
        lg = _planted_logits(1, K, V, tops, trial)
        acc, am, corr = greedy_consensus(lg, np.array([cand]))
        linear = cand[:acc[0]] + ([int(corr[0])] if acc[0] < K else [])
        # chain tree: node i+1 carries cand[i] (i < K-1), row i checks node i+1
        tok = np.array([[999] + cand[:K - 1]])
        par = np.array([[-1] + list(range(K - 1))])
        t_acc, path, t_corr, _ = tree_greedy_consensus(lg, tok, par)
        tree = [int(tok[0, n]) for n in path[0, 1:t_acc[0] + 1]] + [int(t_corr[0])]
        assert tree == linear, (trial, tree, linear)


def test_tree_consensus_brute_force_and_hand_tree():
    rng = random.Random(4)
    K, V = 7, 6
    for trial in range(60):
        par = [-1] + [rng.randrange(i) for i in range(1, K)]
        tok = [0] + [rng.randrange(V) for _ in range(1, K)]
        lg = np.random.default_rng(trial).normal(0.0, 1.0, (1, K, V))
        am = [int(np.argmax(lg[0, i])) for i in range(K)]
        # brute force: follow, from the root, the lowest-index child that matches
        paths = [[0]]
        best = [0]
        for _ in range(K):
            nxt = []
            for p in paths:
                kids = [c for c in range(1, K) if par[c] == p[-1] and tok[c] == am[p[-1]]]
                if kids:
                    nxt.append(p + [min(kids)])
            if not nxt:
                break
            paths = nxt
            best = nxt[0]
        acc, path, corr, _ = tree_greedy_consensus(lg, np.array([tok]), np.array([par]))
        assert path[0, :acc[0] + 1].tolist() == best
        assert corr[0] == am[best[-1]]
    # hand tree: root argmax 7 -> node 2 (token 7; node 1 has token 3), node 2's argmax 9 -> node 4
    par = np.array([[-1, 0, 0, 1, 2, 2]])
    tok = np.array([[0, 3, 7, 9, 9, 5]])
    lg = _planted_logits(1, 6, 20, [[7, 1, 9, 1, 12, 1]], 9)
    acc, path, corr, _ = tree_greedy_consensus(lg, tok, par)
    assert acc.tolist() == [2] and path[0, :3].tolist() == [0, 2, 4] and corr.tolist() == [12]


def test_path_commit_on_a_chain_equals_the_linear_commit():
    n_layers, B, Hkv, max_len, K, D = 2, 3, 2, 20, 5, 8
    g = torch.Generator().manual_seed(8)
    bf = lambda *s: torch.randn(s, generator=g).to(torch.bfloat16)
    kc, vc = bf(n_layers, B, Hkv, max_len, D), bf(n_layers, B, Hkv, max_len, D)
    kb, vb = bf(n_layers, B, Hkv, K, D), bf(n_layers, B, Hkv, K, D)
    lens = np.array([3, 0, 14])
    acc = np.array([2, 0, 4])          # a <= K-1 on the tree
    corr = np.array([40, 41, 42])
    cand = np.array([[10, 11, 12, 13, 14]] * B)
    path = np.array([[i if i <= a else -1 for i in range(K)] for a in acc])
    tok = np.concatenate([np.full((B, 1), 99), cand[:, :K - 1]], axis=1)
    lin = commit_block(kc, vc, kb, vb, lens, acc, corr, cand)
    tr = commit_path(kc, vc, kb, vb, lens, acc, path, tok, corr)
    for key in ("k_cache", "v_cache", "cache_len", "next_anchor", "tokens", "n_tokens"):
        assert np.array_equal(lin[key], tr[key]), key


class ToyAR:
    def __init__(self, vocab, seed):
        self.V, self.salt = vocab, seed * 2654435761 % (1 << 31)

    def next_token(self, seq):
        h = self.salt
        for p, t in enumerate(seq[-4:]):
            h = (h * 1000003 + (t + 1) * 7919 + p) % (1 << 31)
        return h % self.V


@pytest.mark.parametrize("K,seed", [(6, 1), (10, 2), (16, 3)])
def test_tree_decoding_is_lossless_and_cache_holds_the_sequence(K, seed):
    rng = random.Random(seed)
    V, P, D, cycles = 11, 4, 4, 15
    model = ToyAR(V, seed)
    seq = [rng.randrange(V) for _ in range(P)]
    max_len = P + cycles * K
    enc = lambda tok, pos: np.array([tok, pos, 7, 0][:D], dtype=np.uint16)
    kc = np.zeros((1, 1, 1, max_len, D), dtype=np.uint16)
    for p in range(P - 1):
        kc[0, 0, 0, p] = enc(seq[p], p)
    vc = kc.copy()
    L = np.array([P - 1])
    for _ in range(cycles):
        # a random draft tree whose tokens are sometimes the AR model's choice
        par = [-1] + [rng.randrange(i) for i in range(1, K)]
        paths = {0: []}
        tok = [seq[-1]]
        for i in range(1, K):
            ctx = seq + paths[par[i]]
            right = model.next_token(ctx)
            t = right if rng.random() < 0.6 else rng.randrange(V)
            tok.append(t)
            paths[i] = paths[par[i]] + [t]
        logits = np.zeros((1, K, V))
        kb = np.zeros((1, 1, 1, K, D), dtype=np.uint16)
        for i in range(K):
            logits[0, i, model.next_token(seq + paths[i])] = 1.0
            kb[0, 0, 0, i] = enc(tok[i], int(L[0]) + len(paths[i]))
        acc, path, corr, _ = tree_greedy_consensus(logits, np.array([tok]), np.array([par]))
        r = commit_path(kc, vc, kb, kb.copy(), L, acc, path, np.array([tok]), corr)
        n = int(r["n_tokens"][0])
        assert n == acc[0] + 1 >= 1
        seq += r["tokens"][0, :n].tolist()
        kc, vc, L = r["k_cache"], r["v_cache"], r["cache_len"]
    ar = seq[:P]
    while len(ar) < len(seq):
        ar.append(model.next_token(ar))
    assert seq == ar
    assert int(L[0]) == len(seq) - 1
    for p in range(len(seq) - 1):
        assert kc[0, 0, 0, p].tolist() == enc(seq[p], p).tolist()


def test_topk_logprobs_against_torch_with_ties():
    g = torch.Generator().manual_seed(5)
    lg = torch.randn((6, 300), generator=g, dtype=torch.float64) * 3
    lg[0, 10] = lg[0, 200] = lg[0, 5] = 20.0      # a three-way tie at the top
    lg[1, 7] = lg[1, 8] = 15.0
    logp, idx = topk_logprobs(lg, 5)
    ls = torch.log_softmax(lg, dim=1)
    for r in range(6):
        vals, _ = torch.topk(lg[r], 5)
        np.testing.assert_allclose(lg[r, idx[r]].numpy(), vals.numpy(), rtol=0, atol=0)
        np.testing.assert_allclose(logp[r], ls[r, idx[r]].numpy(), rtol=0, atol=1e-12)
    assert idx[0, :3].tolist() == [5, 10, 200] and idx[1, :2].tolist() == [7, 8]


def _brute_prefixes(lp, Dd, M, n_best):
    """All prefixes (rank tuples) with float32 path-sum scores, best n."""
    scored = []
    for d in range(1, Dd + 1):
        for ranks in itertools.product(range(M), repeat=d):
            s = np.float32(0.0)
            for depth, r in enumerate(ranks):
                s = np.float32(s + lp[depth, r])
            scored.append((float(s), ranks))
    scored.sort(key=lambda x: -x[0])
    return {r for _, r in scored[:n_best]}


@pytest.mark.parametrize("Dd,M,n", [(3, 3, 10), (4, 2, 12), (2, 4, 9), (5, 1, 6)])
def test_tree_building_picks_the_best_prefixes(Dd, M, n):
    rng = np.random.default_rng(Dd * 10 + M)
    lp = -np.sort(rng.exponential(1.0, (1, Dd, M)).astype(np.float32), axis=2)  # descending, <= 0
    tok = np.arange(Dd * M).reshape(1, Dd, M) + 100
    parent, tokens, depth, score = build_tree(lp, tok, [7], n)
    assert tokens[0, 0] == 7 and parent[0, 0] == -1
    # every node is its parent's prefix plus one token; scores never increase
    prefixes = {0: ()}
    for i in range(1, n):
        p = int(parent[0, i])
        assert 0 <= p < i and depth[0, i] == depth[0, p] + 1
        d = int(depth[0, i]) - 1
        r = int(np.nonzero(tok[0, d] == tokens[0, i])[0][0])
        prefixes[i] = prefixes[p] + (r,)
        if i > 1:
            assert score[0, i] <= score[0, i - 1]
    want = _brute_prefixes(lp[0], Dd, M, min(n - 1, sum(M ** d for d in range(1, Dd + 1))))
    assert set(prefixes[i] for i in range(1, n)) == want
    if M == 1:
        assert parent[0].tolist() == [-1] + list(range(n - 1))
