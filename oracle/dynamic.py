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
* R30 -- the block-length rule.  The pages tie the block size to a task's
  acceptance rate (large K where it is high, small where it is low) and name
  no rule.  Reading: the acceptance rate is the probability p that a draft
  candidate matches, given the ones before it matched (the run of accepted
  candidates is then geometric, as the pages' accept-length figures suggest).
  Each sequence keeps an exponentially forgetting estimate of it -- accepted
  candidates A over tested candidates N, both decayed by 7/8 per cycle (the
  maximum-likelihood estimate of p from runs cut at the block end) -- and the
  next block is the smallest power of two k with p^k <= 1/8 (the whole block
  is accepted, and tokens possibly left on the table, in at most one cycle in
  eight), clamped to [k_min, K]; with no evidence yet (N = 0) it is K.  All in
  integers so that every implementation takes the same decision: A and N are
  16-bit fields of one int32 (A high, N low) in units of 1/16 candidate; a
  committed cycle with a accepted of k (t = a + [a < k] tested) sets
  A <- A - floor(A/8) + 16 a and N <- N - floor(N/8) + 16 t (N saturating
  at 65535, A at N); p is
  P = floor(65536 A / N) (A above N counts as N), P^k is formed by squaring
  with floor(x^2 / 65536), and 1/8 is 8192.  A refused commit (R17) changes
  neither the statistics nor k.

Each function applies the static definitions (``oracle.attention``,
``oracle.consensus``, ``oracle.cycle``) to each sequence's sliced block.
"""
from __future__ import annotations

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


STAT_UNIT = 16        # one candidate in the acceptance statistics (R30)
OVERRUN_Q16 = 8192    # 1/8: the largest whole-block acceptance probability wanted


def stat_fields(stat: int):
    """(A, N) of a packed acceptance statistic (R30); A is at most N."""
    s = int(stat) & 0xFFFFFFFF
    a_, n_ = s >> 16, s & 0xFFFF
    return min(a_, n_), n_


def update_accept_stat(stat: int, a: int, k: int) -> int:
    """The statistic after a committed cycle that accepted a of k (R30)."""
    A, N = stat_fields(stat)
    t = a + (1 if a < k else 0)
    N = min(N - N // 8 + STAT_UNIT * t, 0xFFFF)   # both fields saturate (blocks past 511)
    A = min(A - A // 8 + STAT_UNIT * a, N)
    return (A << 16) | N


def block_len_from_stat(stat: int, block_k: int, k_min: int) -> int:
    """The smallest power of two k with p^k <= 1/8 under the estimate (R30),
    clamped to [k_min, K]; K with no evidence."""
    A, N = stat_fields(stat)
    if N == 0:
        k = block_k
    else:
        x = (A * 65536) // N      # p in Q16
        k = 1
        while k < block_k and x > OVERRUN_Q16:
            x = (x * x) >> 16     # p^(2k)
            k *= 2
    return int(min(max(k, k_min), block_k))


def commit_block_dyn(k_cache, v_cache, k_blk, v_blk, cache_len, accept_len, correction, cand,
                     blk_len, accept_stat, k_min: int):
    """The commit of ``oracle.cycle.commit_block`` with sequence b's block cut
    to its first k_b positions (R29), then the block-length rule (R30) from the
    packed acceptance statistics ``accept_stat`` [B].

    Returns the dict of ``commit_block`` (tokens padded to [B, K] with -1) plus
    ``blk_len`` and ``accept_stat`` int64 [B], the next cycle's lengths and
    statistics.
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
    stats = [int(x) & 0xFFFFFFFF for x in _ints(accept_stat)]
    new_stat = np.array(stats, dtype=np.int64)
    for b in range(B):
        k = int(kl[b])
        r = commit_block(kc[:, b:b + 1], vc[:, b:b + 1], kb[:, b:b + 1, :, :k], vb[:, b:b + 1, :, :k],
                         lens[b:b + 1], acc[b:b + 1], corr[b:b + 1], cd[b:b + 1, :k])
        kc[:, b:b + 1], vc[:, b:b + 1] = r["k_cache"], r["v_cache"]
        new_len[b] = r["cache_len"][0]
        next_anchor[b] = r["next_anchor"][0]
        tokens[b, :k] = r["tokens"][0]
        n_tokens[b] = r["n_tokens"][0]
        if n_tokens[b] > 0:  # committed (a refused commit emits nothing and keeps k and the statistics)
            new_stat[b] = update_accept_stat(stats[b], int(acc[b]), k)
            new_k[b] = block_len_from_stat(int(new_stat[b]), K, int(k_min))
    return {"k_cache": kc, "v_cache": vc, "cache_len": new_len, "next_anchor": next_anchor,
            "tokens": tokens, "n_tokens": n_tokens, "blk_len": new_k, "accept_stat": new_stat}


def decode_cycles_dyn(k_cache, v_cache, cache_len, blk_len, k_min: int, cycles, scale=None,
                      keep_attention=True, accept_stat=None):
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
    stat = np.zeros(len(lens), dtype=np.int64) if accept_stat is None else _ints(accept_stat).copy()
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
        if "p" in cyc:  # T>0 consensus
            acc, corr = sample_consensus_dyn(cyc["p"], cyc["q"], cyc["cand"], cyc["uniforms"], kl)
        else:
            acc, _, corr = greedy_consensus_dyn(cyc["logits"], cyc["cand"], kl)
        kb = np.stack([_bits(vv[1]) for vv in cyc["verify"]])
        vb = np.stack([_bits(vv[2]) for vv in cyc["verify"]])
        res = commit_block_dyn(kc, vc, kb, vb, lens, acc, corr, cyc["cand"], kl, stat, k_min)
        kc, vc, lens, kl, stat = res["k_cache"], res["v_cache"], res["cache_len"], res["blk_len"], res["accept_stat"]
        rec.update(accept_len=acc, correction=corr, cache_len=lens.copy(), blk_len=kl.copy(),
                   accept_stat=stat.copy(),
                   next_anchor=res["next_anchor"], tokens=res["tokens"], n_tokens=res["n_tokens"])
        records.append(rec)
    return records, {"k_cache": kc, "v_cache": vc, "cache_len": lens, "blk_len": kl, "accept_stat": stat}
