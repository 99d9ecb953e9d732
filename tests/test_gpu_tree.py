"""GPU parity of the variants: K = 64 / 128 blocks, explicit (tree) block
masks, and the tree-verification pieces (top-m marginals, best-first draft
trees, ancestor masks, greedy tree consensus, path commit).

Attention against the fp64 oracle at the attention bar (max-abs 2e-2,
rel-L2 5e-3, lse 1e-3).  Integer work bit-exact: consensus results, masks,
trees built from the same fp32 marginals, committed caches and state.  Top-m
indices exact (the order of fp32 logits is exact); log-probabilities within
1e-4 (fp32 log-sum-exp over up to 151936 terms).
"""
import numpy as np
import pytest
import torch

import dual_view_block_amd as dvb
import oracle
from oracle.cycle import bits_to_bf16
from synth import (WORKLOADS, Workload, attention_inputs, draft_marginals, greedy_inputs, random_trees,
                   tree_verify_logits)
from tests._parity import assert_attn_close, assert_lse_close

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _attn_check(x, mode, what, masks=None):
    if masks is None:
        fn = dvb.orthrus_block_attn_diff if mode == oracle.MASK_DIFF_BIDIR else dvb.orthrus_block_attn_verify
        out, lse = fn(x["q"], x["k_blk"], x["v_blk"], x["k_cache"], x["v_cache"], x["cache_len"])
    else:
        bits = torch.from_numpy(oracle.masks_to_bits(masks).view(np.int64)).to(DEV)
        out, lse = dvb.orthrus_block_attn_masked(x["q"], x["k_blk"], x["v_blk"], x["k_cache"], x["v_cache"],
                                                 x["cache_len"], bits)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.block_attention(x["q"], x["k_blk"], x["v_blk"], x["k_cache"], x["v_cache"],
                                          x["cache_len"], mode, block_masks=masks)
    e = assert_attn_close(out, ref, what)
    finite = np.isfinite(ref_lse)
    got_lse = lse.cpu().double().numpy()
    assert np.array_equal(np.isfinite(got_lse), finite), what
    assert_lse_close(torch.from_numpy(np.where(finite, got_lse, 0.0)), np.where(finite, ref_lse, 0.0), what)
    print(f"{what}: max_abs={e[0]:.2e} rel_l2={e[1]:.2e}", flush=True)
    return out, lse


@pytest.mark.parametrize("K", [64, 128])
@pytest.mark.parametrize("mode", [oracle.MASK_DIFF_BIDIR, oracle.MASK_VERIFY_CAUSAL])
def test_large_blocks(mode, K):
    """K = 64 (one block tile, 256 rows per KV head) and K = 128 (two block
    tiles, 512 rows), Qwen3-8B heads, L 2048 and a ragged batch."""
    w = WORKLOADS["qwen3_1p7b_layer"].replace(n_q_heads=32, block_k=K, seed=K)
    _attn_check(attention_inputs(w, device=DEV), mode, f"K{K}/mode{mode}")
    wr = Workload("ragged", 1, 3, 8, 2, 128, 700, K, 100, 3.0, K + 1, max_len=700, ragged_min=0)
    x = attention_inputs(wr, device=DEV)
    x["cache_len"] = torch.tensor([0, 65, 700], dtype=torch.int32, device=DEV)
    _attn_check(x, mode, f"K{K}/ragged/mode{mode}")


@pytest.mark.parametrize("K", [8, 32, 64])
def test_tree_masked_attention(K):
    """Ancestor masks of random trees (with unused nodes) at K 8 / 32 / 64."""
    w = Workload("tree", 1, 3, 8, 2, 128, 300, K, 100, 3.0, 40 + K, max_len=300)
    x = attention_inputs(w, device=DEV)
    x["cache_len"] = torch.tensor([300, 17, 0], dtype=torch.int32, device=DEV)
    par = random_trees(3, K, seed=K, unused_frac=0.2)
    _attn_check(x, oracle.MASK_EXPLICIT, f"tree{K}", masks=oracle.ancestor_masks(par))


def test_explicit_masks_match_the_views_and_empty_rows():
    w = Workload("m", 1, 2, 4, 1, 64, 200, 16, 100, 3.0, 7, max_len=200)
    x = attention_inputs(w, device=DEV)
    K = 16
    causal = np.broadcast_to(np.tril(np.ones((K, K), dtype=bool)), (2, K, K)).copy()
    ones = np.ones((2, K, K), dtype=bool)
    out_c, _ = _attn_check(x, oracle.MASK_EXPLICIT, "explicit-causal", masks=causal)
    out_v, _ = _attn_check(x, oracle.MASK_VERIFY_CAUSAL, "verify")
    _attn_check(x, oracle.MASK_EXPLICIT, "explicit-ones", masks=ones)
    # rows with nothing visible: no cache and an empty mask row
    x["cache_len"] = torch.tensor([0, 0], dtype=torch.int32, device=DEV)
    empty = causal.copy()
    empty[:, 3] = False
    out, lse = _attn_check(x, oracle.MASK_EXPLICIT, "explicit-empty-rows", masks=empty)
    assert torch.all(out[:, :, 3] == 0) and torch.all(torch.isneginf(lse[:, :, 3]))


@pytest.mark.parametrize("K", [64, 128])
def test_greedy_consensus_large_blocks(K):
    w = WORKLOADS["ragged_b16"].replace(block_k=K, vocab=32768)
    for j in (0, K // 2 - 1, K // 2 + 5, K - 1, K):
        logits, cand, _ = greedy_inputs(w, device=DEV, first_mismatch=j, seed_offset=j)
        acc, am, corr = dvb.orthrus_consensus_greedy(logits, cand)
        torch.cuda.synchronize()
        r_acc, r_am, r_corr = oracle.greedy_consensus(logits.cpu(), cand.cpu())
        assert acc.cpu().tolist() == r_acc.tolist() and corr.cpu().tolist() == r_corr.tolist()
        assert np.array_equal(am.cpu().numpy(), r_am)


@pytest.mark.parametrize("K", [64, 128])
def test_sample_consensus_large_blocks(K):
    from synth import sample_inputs
    w = Workload("s", 1, 3, 4, 1, 64, 8, K, 2000, 3.0, K)
    p, q, cand, u = sample_inputs(w, device=DEV, draft_noise=0.3)
    acc, corr = dvb.orthrus_consensus_sample(p, q, cand, u)
    torch.cuda.synchronize()
    r_acc, r_corr = oracle.sample_consensus(p.cpu(), q.cpu(), cand.cpu(), u.cpu())
    assert acc.cpu().tolist() == r_acc.tolist() and corr.cpu().tolist() == r_corr.tolist()
    print(f"sample K{K}: accept {acc.cpu().tolist()}", flush=True)


@pytest.mark.parametrize("K,unused", [(8, 0.0), (32, 0.3), (64, 0.1)])
def test_tree_masks(K, unused):
    par = random_trees(16, K, seed=K, unused_frac=unused)
    got = dvb.orthrus_tree_masks(par.to(DEV))
    torch.cuda.synchronize()
    want = oracle.masks_to_bits(oracle.ancestor_masks(par)).view(np.int64)
    assert np.array_equal(got.cpu().numpy(), want)


@pytest.mark.parametrize("K,V,rate", [(8, 1000, 0.7), (32, 151936, 0.8), (64, 4099, 0.9), (128, 2048, 0.85)])
def test_tree_consensus(K, V, rate):
    B = 6
    par = random_trees(B, K, seed=K + 1, unused_frac=0.1)
    g = torch.Generator().manual_seed(K)
    tok = torch.randint(0, V, (B, K), generator=g, dtype=torch.int32)
    logits = tree_verify_logits(par, tok, V, accept_rate=rate, seed=K)
    acc, path, corr, am = dvb.orthrus_consensus_tree_greedy(logits.to(DEV), tok.to(DEV), par.to(DEV),
                                                            want_row_argmax=True)
    torch.cuda.synchronize()
    r_acc, r_path, r_corr, r_am = oracle.tree_greedy_consensus(logits, tok, par)
    assert acc.cpu().tolist() == r_acc.tolist()
    assert np.array_equal(path.cpu().numpy(), r_path)
    assert corr.cpu().tolist() == r_corr.tolist()
    assert np.array_equal(am.cpu().numpy(), r_am)
    print(f"tree consensus K{K}: accepted {acc.cpu().tolist()}", flush=True)


def test_tree_consensus_on_chains_matches_the_linear_rule():
    B, K, V = 8, 32, 5000
    w = Workload("c", 1, B, 4, 1, 64, 8, K, V, 3.0, 77)
    logits, cand, _ = greedy_inputs(w, device=DEV)
    acc, _, corr = dvb.orthrus_consensus_greedy(logits, cand)
    par = torch.tensor([[-1] + list(range(K - 1))] * B, dtype=torch.int32, device=DEV)
    tok = torch.cat([torch.full((B, 1), 999, dtype=torch.int32, device=DEV), cand[:, :K - 1]], dim=1)
    t_acc, t_path, t_corr, _ = dvb.orthrus_consensus_tree_greedy(logits, tok, par)
    torch.cuda.synchronize()
    for b in range(B):
        a = int(acc[b])
        linear = cand[b, :a].cpu().tolist() + ([int(corr[b])] if a < K else [])
        ta = int(t_acc[b])
        tree = [int(tok[b, n]) for n in t_path[b, 1:ta + 1].cpu().tolist()] + [int(t_corr[b])]
        assert tree == linear


def test_path_commit():
    n_layers, B, Hkv, D, K, max_len = 3, 8, 4, 128, 16, 64
    g = torch.Generator(device=DEV)
    g.manual_seed(3)
    bf = lambda *s: torch.randn(s, generator=g, device=DEV).to(torch.bfloat16)
    kc, vc = bf(n_layers, B, Hkv, max_len, D), bf(n_layers, B, Hkv, max_len, D)
    kb, vb = bf(n_layers, B, Hkv, K, D), bf(n_layers, B, Hkv, K, D)
    par = random_trees(B, K, seed=9)
    tok = torch.randint(0, 1000, (B, K), generator=torch.Generator().manual_seed(4), dtype=torch.int32)
    logits = tree_verify_logits(par, tok, 1000, accept_rate=0.9, seed=9)
    acc, path, corr, _ = oracle.tree_greedy_consensus(logits, tok, par)
    lens = torch.tensor([0, 10, 48, 63, 60, 5, -1, 20], dtype=torch.int32)
    acc = torch.tensor(acc, dtype=torch.int32)
    acc[5] = K          # out of range: refused
    path = torch.tensor(path, dtype=torch.int32)
    corr = torch.tensor(corr, dtype=torch.int32)
    ref = oracle.commit_path(kc.cpu(), vc.cpu(), kb.cpu(), vb.cpu(), lens, acc, path, tok, corr)
    dl = lens.to(DEV)
    anchor, toks, ntok = dvb.orthrus_cache_commit_path(kc, vc, kb, vb, dl, acc.to(DEV), path.to(DEV), tok.to(DEV),
                                                       corr.to(DEV))
    torch.cuda.synchronize()
    assert dl.cpu().tolist() == ref["cache_len"].tolist()
    assert ntok.cpu().tolist() == ref["n_tokens"].tolist()
    assert anchor.cpu().tolist() == ref["next_anchor"].tolist()
    assert np.array_equal(toks.cpu().numpy(), ref["tokens"])
    assert torch.equal(kc.cpu(), bits_to_bf16(ref["k_cache"])) and torch.equal(vc.cpu(), bits_to_bf16(ref["v_cache"]))
    print(f"path commit: n_tokens {ntok.cpu().tolist()}", flush=True)


@pytest.mark.parametrize("R,V,m", [(32, 151936, 8), (5, 1001, 1), (7, 4096, 32), (3, 40, 16)])
def test_topk_logprobs(R, V, m):
    g = torch.Generator().manual_seed(V)
    logits = torch.randn((R, V), generator=g) * 3
    logits[0, 17] = logits[0, 900 % V] = logits[0, 5] = 25.0   # ties at the top: lower index first
    logp, idx = dvb.orthrus_topk_logprobs(logits.to(DEV), m)
    torch.cuda.synchronize()
    r_logp, r_idx = oracle.topk_logprobs(logits, m)
    assert np.array_equal(idx.cpu().numpy(), r_idx)
    err = float(np.abs(logp.cpu().double().numpy() - r_logp).max())
    assert err <= 1e-4, err
    print(f"topk R{R} V{V} m{m}: logp max err {err:.2e}", flush=True)


@pytest.mark.parametrize("Dd,m,n,ties", [(31, 4, 32, False), (8, 8, 64, True), (3, 2, 20, False),
                                         (1, 1, 4, False), (63, 1, 64, False), (5, 3, 1, False)])
def test_tree_build(Dd, m, n, ties):
    B = 12
    logp, tok = draft_marginals(B, Dd, m, 50000, seed=Dd * m + n, ties=ties)
    anchor = torch.arange(B, dtype=torch.int32) + 7
    par, tks, dep = dvb.orthrus_tree_build(logp.to(DEV), tok.to(DEV), anchor.to(DEV), n)
    torch.cuda.synchronize()
    r_par, r_tok, r_dep, _ = oracle.build_tree(logp.numpy(), tok, anchor, n)
    assert np.array_equal(par.cpu().numpy(), r_par)
    assert np.array_equal(tks.cpu().numpy(), r_tok)
    assert np.array_equal(dep.cpu().numpy(), r_dep)


def test_tree_pipeline_on_device():
    """topk -> build -> masks -> masked verify attention -> tree consensus ->
    path commit, chained on the device for a batch of 4 at K = 32.  The first
    stage is compared with the oracle on the synthetic logits; the later
    stages run on device results, so they are checked through properties that
    must hold for any input: a well-formed tree whose depth-d tokens come from
    position d's top-m, masks that are the ancestor sets of that tree, an
    accepted path that descends the tree, emitted tokens = path tokens + the
    correction, and lengths grown by a + 1 with the path rows in the cache."""
    B, K, V, m = 4, 32, 8192, 4
    g = torch.Generator().manual_seed(21)
    diff_logits = torch.randn((B * (K - 1), V), generator=g) * 3
    logp, idx = dvb.orthrus_topk_logprobs(diff_logits.to(DEV), m)
    torch.cuda.synchronize()
    r_logp, r_idx = oracle.topk_logprobs(diff_logits, m)
    assert np.array_equal(idx.cpu().numpy(), r_idx)
    assert float(np.abs(logp.cpu().double().numpy() - r_logp).max()) <= 1e-4
    logp3, idx3 = logp.view(B, K - 1, m), idx.view(B, K - 1, m)
    anchor = torch.tensor([11, 12, 13, 14], dtype=torch.int32, device=DEV)
    par, tok, dep = dvb.orthrus_tree_build(logp3, idx3, anchor, K)
    masks = dvb.orthrus_tree_masks(par)
    torch.cuda.synchronize()
    P, T, Dp, M = par.cpu().tolist(), tok.cpu().tolist(), dep.cpu().tolist(), masks.cpu().tolist()
    top = idx3.cpu().tolist()
    for b in range(B):
        assert P[b][0] == -1 and T[b][0] == int(anchor[b]) and Dp[b][0] == 0
        for i in range(1, K):
            p = P[b][i]
            assert 0 <= p < i and Dp[b][i] == Dp[b][p] + 1 and T[b][i] in top[b][Dp[b][i] - 1]
        for i in range(K):
            anc, j = 0, i
            while True:
                anc |= 1 << j
                if j == 0:
                    break
                j = P[b][j]
            assert (M[b][i] & ((1 << 64) - 1)) == anc
    w = Workload("pipe", 1, B, 8, 2, 128, 512, K, V, 3.0, 5, max_len=512 + 2 * K)
    x = attention_inputs(w, device=DEV)
    out, _ = dvb.orthrus_block_attn_masked(x["q"], x["k_blk"], x["v_blk"], x["k_cache"], x["v_cache"],
                                           x["cache_len"], masks)
    ver_logits = (torch.randn((B, K, V), generator=g) * 3).to(DEV)
    acc, path, corr, am = dvb.orthrus_consensus_tree_greedy(ver_logits, tok, par, want_row_argmax=True)
    kc, vc = x["k_cache"][None].clone(), x["v_cache"][None].clone()
    lens = x["cache_len"].clone()
    anchor2, toks, ntok = dvb.orthrus_cache_commit_path(kc, vc, x["k_blk"][None], x["v_blk"][None], lens, acc, path,
                                                        tok, corr)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    A, PT, C, AM = acc.cpu().tolist(), path.cpu().tolist(), corr.cpu().tolist(), am.cpu().tolist()
    for b in range(B):
        nodes = PT[b][:A[b] + 1]
        assert nodes[0] == 0 and all(P[b][nodes[i + 1]] == nodes[i] for i in range(A[b]))
        assert all(T[b][nodes[i + 1]] == AM[b][nodes[i]] for i in range(A[b]))
        assert C[b] == AM[b][nodes[-1]] and int(anchor2[b]) == C[b]
        assert toks[b, :A[b] + 1].cpu().tolist() == [T[b][n] for n in nodes[1:]] + [C[b]]
        assert int(ntok[b]) == A[b] + 1 and int(lens[b]) == 512 + A[b] + 1
        for i, n in enumerate(nodes):
            assert torch.equal(kc[0, b, :, 512 + i], x["k_blk"][b, :, n])
    print(f"pipeline: accepted {A}, tokens {ntok.cpu().tolist()}", flush=True)
