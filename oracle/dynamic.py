"""Oracle for dynamic block sizes: a block length per sequence, chosen from acceptance.

TEST INFRASTRUCTURE ONLY -- never imported by the product path.

Sources (the Orthrus pages):

* Paper notes on Orthrus (zhangshuibai.github.io paper-notes), §7.4 (the
  comparison with speculative verification: deciding the verify length
  dynamically is orthogonal to Orthrus, which runs a fixed K = 32, and K could
  be made adaptive on top of it) and §9.6 (dynamic K as an unexplored
  direction: a large K where acceptance is high, a small K where it is low).
* The same notes, §4.1 (one cycle: diffusion forward over the block, causal
  AR forward over the candidates, left-to-right consensus, commit) -- the
  cycle below is that cycle with the block cut to its first k_b positions.

Readings of points the pages leave open:

* R29 -- a dynamic block.  Buffers keep the capacity K ([.., K, ..] block
  layouts); sequence b's block in this cycle is its first
  k_b = clamp(blk_len[b], 1, K) positions: the anchor and k_b - 1 mask
  positions in the diffusion view, the anchor and k_b - 1 candidates in the
  verify view.  Block rows i >= k_b are not part of the cycle (their outputs
  are not written: NaN here) and block keys j >= k_b are invisible.  The
  consensus runs over rows [0, k_b): a <= k_b, and the correction is drawn at
  row a when a < k_b (the T > 0 sampler keeps its uniform layout [B, K+1]:
  u_0 .. u_{k_b-1} for the accept tests, u_K for the residual draw).  The
  commit treats the block as k_b positions long: a = k_b means no correction
  and cand[k_b - 1] becomes the next anchor (R3 with K = k_b).
* R30 -- the block-length rule.  After a committed cycle with accepted length
  a under block length k (capacity K, floor k_min):
      k' = min(2k, K)            if a = k        (the whole block was accepted)
      k' = max(ceil(k/2), k_min) if 2(a + 1) <= k (at most half of it was used)
      k' = k                     otherwise,
  then clamped to [k_min, K].  A refused commit (R17) keeps k.  The pages name
  only the direction (large K where acceptance is high); doubling and halving
  is the plainest rule with that direction whose state is one integer per
  sequence.

Each function applies the static definitions (``oracle.attention``,
``oracle.consensus``, ``oracle.cycle``) to each sequence's sliced block.
"""
from __future__ import annotations

import math

import numpy as np

from .attention import MASK_DIFF_BIDIR, MASK_VERIFY_CAUSAL, _as_f64, _as_int, block_attention
from .consensus import _np, greedy_consensus, sample_consensus
from .cycle import _bits, _ints, bits_to_bf16, commit_block


def live_lengths(blk_len, block_k: int) -> np.ndarray:
    """k_b = clamp(blk_len[b], 1, K) for every sequence (R29)."""
    return np.clip(_as_int(blk_len).astype(np.int64), 1, int(block_k))


def block_attention_dyn(q, k_blk, v_blk, k_cache, v_cache, cache_len, blk_len, mode: int,
                        scale: float | None = None):
    """Block attention of sequence b over its first k_b block positions (R29).

    Shapes as ``block_attention``; blk_len [B].  Rows i >= k_b of out and lse
    are NaN (not part of the block).
    """
    qd, kb, vb = _as_f64(q), _as_f64(k_blk), _as_f64(v_blk)
    kc, vc = _as_f64(k_cache), _as_f64(v_cache)
    lens = _as_int(cache_len)
    B, Hq, K, D = qd.shape
    kl = live_lengths(blk_len, K)
    out = np.full((B, Hq, K, D), np.nan)
    lse = np.full((B, Hq, K), np.nan)
    for b in range(B):
        k = int(kl[b])
        o, l = block_attention(qd[b:b + 1, :, :k], kb[b:b + 1, :, :k], vb[b:b + 1, :, :k],
                               kc[b:b + 1], vc[b:b + 1], lens[b:b + 1], mode, scale)
        out[b, :, :k] = o[0]
        lse[b, :, :k] = l[0]
    return out, lse


def greedy_consensus_dyn(logits, cand, blk_len):
    """Greedy consensus over the first k_b rows of every sequence (R29).

    Returns (accept_len [B], row_argmax [B, K] with -1 for rows >= k_b,
    correction [B]: argmax of row a if a < k_b, else -1).
    """
    lg = _np(logits, np.float64)
    cd = _np(cand, np.int64)
    B, K, _ = lg.shape
    kl = live_lengths(blk_len, K)
    acc = np.zeros(B, dtype=np.int64)
    am = np.full((B, K), -1, dtype=np.int64)
    corr = np.zeros(B, dtype=np.int64)
    for b in range(B):
        k = int(kl[b])
        a, m, c = greedy_consensus(lg[b:b + 1, :k], cd[b:b + 1, :k])
        acc[b], corr[b] = a[0], c[0]
        am[b, :k] = m[0]
    return acc, am, corr


def sample_consensus_dyn(p_target, q_draft, cand, uniforms, blk_len):
    """T > 0 consensus over the first k_b rows of every sequence (R29): the
    accept tests use u_0 .. u_{k_b-1}, the residual draw u_K."""
    P = _np(p_target, np.float32)
    Q = _np(q_draft, np.float32)
    cd = _np(cand, np.int64)
    U = _np(uniforms, np.float32)
    B, K, _ = P.shape
    kl = live_lengths(blk_len, K)
    acc = np.zeros(B, dtype=np.int64)
    corr = np.zeros(B, dtype=np.int64)
    for b in range(B):
        k = int(kl[b])
        u = np.concatenate([U[b, :k], U[b, K:K + 1]])[None, :]
        a, c = sample_consensus(P[b:b + 1, :k], Q[b:b + 1, :k], cd[b:b + 1, :k], u)
        acc[b], corr[b] = a[0], c[0]
    return acc, corr


def next_block_len(a: int, k: int, block_k: int, k_min: int) -> int:
    """The block length after a committed cycle (R30)."""
    if a == k:
        nk = min(2 * k, block_k)
    elif 2 * (a + 1) <= k:
        nk = max(math.ceil(k / 2), k_min)
    else:
        nk = k
    return int(min(max(nk, k_min), block_k))


def commit_block_dyn(k_cache, v_cache, k_blk, v_blk, cache_len, accept_len, correction, cand,
                     blk_len, k_min: int):
    """The commit of ``oracle.cycle.commit_block`` with sequence b's block cut
    to its first k_b positions (R29), then the block-length rule (R30).

    Returns the dict of ``commit_block`` (tokens padded to [B, K] with -1) plus
    ``blk_len`` int64 [B], the next cycle's block lengths.
    """
    kc, vc = _bits(k_cache), _bits(v_cache)
    kb, vb = _bits(k_blk), _bits(v_blk)
    lens, acc = _ints(cache_len), _ints(accept_len)
    corr, cd = _ints(correction), _ints(cand)
    n_layers, B, Hkv, max_len, D = kc.shape
    K = kb.shape[3]
    if not 1 <= int(k_min) <= K:
        raise ValueError("k_min must lie in [1, K]")
    kl = live_lengths(blk_len, K)
    new_len = lens.copy()
    next_anchor = np.full(B, -1, dtype=np.int64)
    tokens = np.full((B, K), -1, dtype=np.int64)
    n_tokens = np.zeros(B, dtype=np.int64)
    new_k = kl.copy()
    for b in range(B):
        k = int(kl[b])
        r = commit_block(kc[:, b:b + 1], vc[:, b:b + 1], kb[:, b:b + 1, :, :k], vb[:, b:b + 1, :, :k],
                         lens[b:b + 1], acc[b:b + 1], corr[b:b + 1], cd[b:b + 1, :k])
        kc[:, b:b + 1], vc[:, b:b + 1] = r["k_cache"], r["v_cache"]
        new_len[b] = r["cache_len"][0]
        next_anchor[b] = r["next_anchor"][0]
        tokens[b, :k] = r["tokens"][0]
        n_tokens[b] = r["n_tokens"][0]
        if n_tokens[b] > 0:  # committed (a refused commit emits nothing and keeps k)
            new_k[b] = next_block_len(int(acc[b]), k, K, int(k_min))
    return {"k_cache": kc, "v_cache": vc, "cache_len": new_len, "next_anchor": next_anchor,
            "tokens": tokens, "n_tokens": n_tokens, "blk_len": new_k}


def decode_cycles_dyn(k_cache, v_cache, cache_len, blk_len, k_min: int, cycles, scale=None,
                      keep_attention=True):
    """``oracle.cycle.decode_cycles`` with a block length per sequence: each
    cycle runs both views' attention, the greedy consensus and the commit over
    each sequence's first k_b positions, and the commit's block-length rule
    sets the next cycle's k_b (R29, R30).

    Returns (records, state) as ``decode_cycles``; every record also holds
    ``blk_len_in`` (the lengths the cycle ran with) and ``blk_len`` (the next
    ones), attention outputs NaN past k_b, and ``state`` the final ``blk_len``.
    """
    kc, vc = _bits(k_cache), _bits(v_cache)
    lens = _ints(cache_len).copy()
    K = _as_f64(cycles[0]["diff"][0][0]).shape[2]
    kl = live_lengths(blk_len, K)
    records = []
    for cyc in cycles:
        rec = {"cache_len_in": lens.copy(), "blk_len_in": kl.copy()}
        kc_t, vc_t = bits_to_bf16(kc), bits_to_bf16(vc)
        if keep_attention:
            rec["diff_out"], rec["verify_out"] = [], []
            for layer, (dv, vv) in enumerate(zip(cyc["diff"], cyc["verify"])):
                od, _ = block_attention_dyn(dv[0], dv[1], dv[2], kc_t[layer], vc_t[layer], lens, kl,
                                            MASK_DIFF_BIDIR, scale)
                ov, _ = block_attention_dyn(vv[0], vv[1], vv[2], kc_t[layer], vc_t[layer], lens, kl,
                                            MASK_VERIFY_CAUSAL, scale)
                rec["diff_out"].append(od)
                rec["verify_out"].append(ov)
        acc, _, corr = greedy_consensus_dyn(cyc["logits"], cyc["cand"], kl)
        kb = np.stack([_bits(vv[1]) for vv in cyc["verify"]])
        vb = np.stack([_bits(vv[2]) for vv in cyc["verify"]])
        res = commit_block_dyn(kc, vc, kb, vb, lens, acc, corr, cyc["cand"], kl, k_min)
        kc, vc, lens, kl = res["k_cache"], res["v_cache"], res["cache_len"], res["blk_len"]
        rec.update(accept_len=acc, correction=corr, cache_len=lens.copy(), blk_len=kl.copy(),
                   next_anchor=res["next_anchor"], tokens=res["tokens"], n_tokens=res["n_tokens"])
        records.append(rec)
    return records, {"k_cache": kc, "v_cache": vc, "cache_len": lens, "blk_len": kl}
