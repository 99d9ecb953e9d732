"""Oracle for tree verification: draft trees from the diffusion marginals,
tree-masked verify attention, greedy consensus along the tree, and the commit
of the accepted path.

TEST INFRASTRUCTURE ONLY -- never imported by the product path.

Sources (the Orthrus pages): paper notes on Orthrus (zhangshuibai.github.io
paper-notes), §7.4-7.5 and §9.6, name tree verification over the K diffusion
marginals (DDTree-style: best-first prefixes under a tree attention mask) and
a dynamic block size as open directions, beside the linear cycle of §4.1-4.2
(left-to-right match, correction from the AR argmax, lossless at T = 0).

Readings (the pages only name the idea; the plainest construction is taken):

* R22 -- explicit block masks.  A block row may see any given subset of the
  block keys (plus the whole cache); a row that sees no key at all returns 0
  with lse = -inf.
* R23 -- the tree.  Node 0 is the anchor; every other node i has a parent
  p(i) < i and a token; parent -1 marks an unused node (a ragged block).
  Verify row i is the AR distribution after the path root..i, so row i sees
  exactly the block keys of its ancestors and itself.
* R24 -- greedy tree consensus.  Starting at the root, move to the child
  (lowest node index first) whose token equals the AR argmax of the current
  node's row; stop when none does.  The accepted path is root, n_1, .., n_a;
  the correction is the argmax of the last node's row, always emitted (every
  node has a verify row), so a cycle emits a + 1 tokens.  On a chain (node i
  the child of i-1) this emits exactly the tokens of the linear rule of R2/R3
  on the same K rows.
* R25 -- commit of a path: verify rows root, n_1, .., n_a are appended to the
  cache in that order, the length grows by a + 1, the correction becomes the
  next anchor (refusal as in R17).
* R26 -- the draft tree.  Per block position d = 1..Dd the diffusion marginal
  is given by its top M tokens and log-probabilities (sorted, descending).  A
  node at depth d has candidate children at depth d+1, one per rank r, with
  score(child) = score(node) + logp[d][r] in float32 (score(root) = 0).
  Best-first: repeatedly add the candidate with the highest score (ties: lower
  parent index, then lower rank) until the tree has n nodes.  Log-probs are
  <= 0, so this is the set of the n-1 highest-scoring prefixes.
* R27 -- top-M log-probabilities of a logit row: the M largest logits (ties:
  lower index first), each minus the row's natural log-sum-exp.

Integer and ordering decisions are exact; scores are summed in float32 in a
fixed order on both sides.
"""
from __future__ import annotations

import numpy as np

from .attention import _as_f64, _as_int
from .consensus import row_argmax
from .cycle import _bits


def ancestor_masks(parent) -> np.ndarray:
    """bool [B, K, K]: row i sees block key j iff j is i or an ancestor of i."""
    par = _as_int(parent)
    B, K = par.shape
    m = np.zeros((B, K, K), dtype=bool)
    for b in range(B):
        for i in range(K):
            j = i
            while True:
                m[b, i, j] = True
                p = int(par[b, j]) if j > 0 else -1
                if p < 0 or p >= j:  # the root, an unused node, or a malformed link: stop
                    break
                j = p
    return m


def masks_to_bits(masks) -> np.ndarray:
    """bool [B, K, K] (K <= 64) -> uint64 [B, K], bit j = key j visible."""
    m = np.asarray(masks, dtype=bool)
    B, K, _ = m.shape
    out = np.zeros((B, K), dtype=np.uint64)
    for j in range(K):
        out |= (m[:, :, j].astype(np.uint64) << np.uint64(j))
    return out


def tree_greedy_consensus(logits, tokens, parent):
    """Greedy consensus along a draft tree (R24).

    logits [B, K, V] (row i: AR distribution after the path to node i),
    tokens [B, K] (token of node i; node 0 unchecked), parent [B, K].
    Returns (accept_len [B], path [B, K] (-1 padded; path[0] = 0),
    correction [B], row_argmax [B, K]) as int64.
    """
    lg = _as_f64(logits)
    tok = _as_int(tokens)
    par = _as_int(parent)
    B, K, _ = lg.shape
    am = np.array([[row_argmax(lg[b, i]) for i in range(K)] for b in range(B)], dtype=np.int64)
    acc = np.zeros(B, dtype=np.int64)
    path = np.full((B, K), -1, dtype=np.int64)
    corr = np.zeros(B, dtype=np.int64)
    for b in range(B):
        cur, a = 0, 0
        path[b, 0] = 0
        while True:
            nxt = -1
            for c in range(cur + 1, K):  # children come after their parent
                if par[b, c] == cur and tok[b, c] == am[b, cur]:
                    nxt = c
                    break
            if nxt < 0:
                break
            a += 1
            path[b, a] = nxt
            cur = nxt
        acc[b] = a
        corr[b] = am[b, cur]
    return acc, path, corr, am


def commit_path(k_cache, v_cache, k_blk, v_blk, cache_len, accept_len, path, tokens, correction):
    """Commit an accepted tree path (R25), all layers.  Shapes as
    ``oracle.cycle.commit_block``; path [B, K], tokens [B, K] (node tokens).
    Returns the same dict (k_cache, v_cache bits, cache_len, next_anchor,
    tokens [B, K] emitted, n_tokens)."""
    kc, vc = _bits(k_cache), _bits(v_cache)
    kb, vb = _bits(k_blk), _bits(v_blk)
    lens, acc = _as_int(cache_len), _as_int(accept_len)
    pth, tok, corr = _as_int(path), _as_int(tokens), _as_int(correction)
    n_layers, B, Hkv, max_len, D = kc.shape
    K = kb.shape[3]
    new_len = lens.copy()
    anchor = np.full(B, -1, dtype=np.int64)
    emitted = np.full((B, K), -1, dtype=np.int64)
    n_tok = np.zeros(B, dtype=np.int64)
    for b in range(B):
        t, a = int(lens[b]), int(acc[b])
        if t < 0 or a < 0 or a > K - 1 or t + a + 1 > max_len:
            continue
        nodes = [int(pth[b, i]) for i in range(a + 1)]
        if any(nd < 0 or nd >= K for nd in nodes):
            continue
        for layer in range(n_layers):
            for g in range(Hkv):
                for i, nd in enumerate(nodes):
                    kc[layer, b, g, t + i] = kb[layer, b, g, nd]
                    vc[layer, b, g, t + i] = vb[layer, b, g, nd]
        out = [int(tok[b, nd]) for nd in nodes[1:]] + [int(corr[b])]
        emitted[b, :len(out)] = out
        n_tok[b] = len(out)
        anchor[b] = int(corr[b])
        new_len[b] = t + a + 1
    return {"k_cache": kc, "v_cache": vc, "cache_len": new_len, "next_anchor": anchor,
            "tokens": emitted, "n_tokens": n_tok}


def topk_logprobs(logits, m: int):
    """R27: per row the m largest logits (ties: lower index first) and their
    log-probabilities logit - logsumexp(row) (float64).
    Returns (logp [R, m], idx [R, m])."""
    lg = _as_f64(logits)
    R, V = lg.shape
    logp = np.zeros((R, m))
    idx = np.zeros((R, m), dtype=np.int64)
    for r in range(R):
        row = lg[r]
        mx = row.max()
        lse = mx + np.log(np.sum(np.exp(row - mx)))
        order = sorted(range(V), key=lambda v: (-row[v], v))[:m]
        idx[r] = order
        logp[r] = row[order] - lse
    return logp, idx


def build_tree(logp, tok, anchor, n_nodes: int):
    """R26: best-first draft tree of n_nodes nodes from per-depth top-M
    marginals.  logp float32 [B, Dd, M] (descending per depth), tok [B, Dd, M],
    anchor [B].  Returns (parent, tokens, depth) int64 [B, n_nodes] and score
    float32 [B, n_nodes]."""
    lp = np.asarray(logp, dtype=np.float32)
    tk = _as_int(tok)
    anc = _as_int(anchor)
    B, Dd, M = lp.shape
    parent = np.full((B, n_nodes), -1, dtype=np.int64)
    tokens = np.full((B, n_nodes), -1, dtype=np.int64)
    depth = np.zeros((B, n_nodes), dtype=np.int64)
    score = np.zeros((B, n_nodes), dtype=np.float32)
    for b in range(B):
        tokens[b, 0] = anc[b]
        cands = [(np.float32(0.0) + lp[b, 0, 0], 0, 0)] if Dd > 0 and M > 0 else []
        made = 1
        while made < n_nodes and cands:
            best = min(range(len(cands)), key=lambda k: (-float(cands[k][0]), cands[k][1], cands[k][2]))
            sc, p, r = cands.pop(best)
            d = int(depth[b, p])
            node = made
            made += 1
            parent[b, node] = p
            depth[b, node] = d + 1
            tokens[b, node] = tk[b, d, r]
            score[b, node] = sc
            if d + 1 < Dd:  # its first child
                cands.append((np.float32(sc + lp[b, d + 1, 0]), node, 0))
            if r + 1 < M:   # the parent's next-ranked child
                cands.append((np.float32(score[b, p] + lp[b, d, r + 1]), p, r + 1))
    return parent, tokens, depth, score
