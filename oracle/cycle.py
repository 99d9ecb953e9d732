"""Oracle for closing one Orthrus decode cycle: the commit into the shared cache.

TEST INFRASTRUCTURE ONLY -- never imported by the product path.

Sources (the Orthrus pages):

* Paper notes on Orthrus (zhangshuibai.github.io paper-notes), §4.1: a cycle
  is one diffusion forward over [anchor, mask x (K-1)], one causal AR forward
  over the K candidates, and a left-to-right consensus.  At the first mismatch
  (1-based position j) the j-1 matching candidates are kept, one correction
  token is drawn from the AR distribution at j, the cache is cut back to
  position t+j, and the next cycle starts from there.  Every cycle runs exactly
  two forwards and commits at least one token.  §4.2: at T=0 the emitted
  sequence equals the AR model's own greedy sequence token for token.
* Paper notes §2.2 and the hotdry.top blog post (dual-view attention
  section): only the AR path writes the shared cache; the diffusion view's
  block K/V are transient.

Readings of points the pages leave open:

* R1 -- the cache handed to a cycle holds every position strictly before the
  anchor (``cache_len[b]`` = t positions); the anchor is verify row 0.
* R2 -- verify block row i is the token at position t+i: the anchor for i = 0,
  candidate i (``cand[i-1]``) for i >= 1; its AR keys/values are the verify
  call's k_blk/v_blk row i.
* R3 -- no bonus token: with all K candidates accepted the cycle emits
  ŷ1..ŷK, and ŷK (``cand[K-1]``, whose AR K/V the verify pass did not
  compute) becomes the next anchor.
* R16 -- "cut the cache back to t+j" is realised by never writing the
  unverified rows: rows 0..min(a, K-1) of the verify block (the anchor and the
  a accepted candidates) are appended at position t, the length becomes
  t + a + [a < K], and nothing else of the cache changes.
* R17 -- a sequence whose commit would not fit (t < 0, a outside [0, K], or
  t + a + [a < K] > max_len) is left untouched: no row is written, its length
  stays, it emits no token (n_tokens = 0, tokens and next anchor -1).

All work here is on integers and raw bf16 bit patterns (uint16), so the
result is exact; the loops run one sequence, layer and head at a time.
"""
from __future__ import annotations

import numpy as np

from .attention import MASK_DIFF_BIDIR, MASK_VERIFY_CAUSAL, block_attention
from .consensus import greedy_consensus, sample_consensus


def _bits(x) -> np.ndarray:
    """bf16 data as its uint16 bit patterns (a copy; torch bf16 or numpy uint16)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            t = x.detach().to("cpu").contiguous()
            if t.dtype == torch.bfloat16:
                t = t.view(torch.int16)
            return t.numpy().view(np.uint16).copy()
    except ImportError:  # pragma: no cover
        pass
    a = np.asarray(x)
    if a.dtype != np.uint16:
        raise TypeError("expected bf16 bit patterns (uint16) or a torch bfloat16 tensor")
    return a.copy()


def _ints(x) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.int64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.int64)


def bits_to_bf16(bits: np.ndarray):
    """uint16 bit patterns back to a torch bfloat16 tensor (CPU)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


def commit_block(k_cache, v_cache, k_blk, v_blk, cache_len, accept_len, correction, cand):
    """Commit one cycle's verified rows for every layer and sequence.

    k_cache, v_cache  bf16 [n_layers, B, Hkv, max_len, D]
    k_blk, v_blk      bf16 [n_layers, B, Hkv, K, D]   (the AR verify block K/V)
    cache_len, accept_len, correction  int [B];  cand int [B, K]

    Returns a dict of new arrays (inputs are not modified):
      k_cache, v_cache  uint16 bit patterns, same shapes
      cache_len   int64 [B]   t + a + [a < K]  (unchanged for a refused commit)
      next_anchor int64 [B]   correction if a < K, else cand[K-1]; -1 if refused
      tokens      int64 [B, K]  tokens emitted by the cycle (cand[0..a-1], then
                                the correction if a < K), -1 beyond
      n_tokens    int64 [B]   a + [a < K], or 0 if refused
    """
    kc, vc = _bits(k_cache), _bits(v_cache)
    kb, vb = _bits(k_blk), _bits(v_blk)
    lens, acc = _ints(cache_len), _ints(accept_len)
    corr, cd = _ints(correction), _ints(cand)
    n_layers, B, Hkv, max_len, D = kc.shape
    K = kb.shape[3]
    if kb.shape != (n_layers, B, Hkv, K, D) or vb.shape != kb.shape or vc.shape != kc.shape:
        raise ValueError("inconsistent cache / block shapes")
    new_len = lens.copy()
    next_anchor = np.full(B, -1, dtype=np.int64)
    tokens = np.full((B, K), -1, dtype=np.int64)
    n_tokens = np.zeros(B, dtype=np.int64)
    for b in range(B):
        t, a = int(lens[b]), int(acc[b])
        if t < 0 or a < 0 or a > K:
            continue
        mismatch = a < K
        rows = a + 1 if mismatch else K        # anchor + accepted candidates (R2, R3)
        if t + rows > max_len:
            continue
        for layer in range(n_layers):
            for g in range(Hkv):
                for i in range(rows):          # verify row i is the token at position t+i
                    kc[layer, b, g, t + i] = kb[layer, b, g, i]
                    vc[layer, b, g, t + i] = vb[layer, b, g, i]
        emitted = [int(cd[b, k]) for k in range(a)]
        if mismatch:
            emitted.append(int(corr[b]))
            next_anchor[b] = int(corr[b])
        else:
            next_anchor[b] = int(cd[b, K - 1])
        tokens[b, :len(emitted)] = emitted
        n_tokens[b] = len(emitted)
        new_len[b] = t + rows
    return {"k_cache": kc, "v_cache": vc, "cache_len": new_len, "next_anchor": next_anchor,
            "tokens": tokens, "n_tokens": n_tokens}


def decode_cycles(k_cache, v_cache, cache_len, cycles, scale=None, keep_attention=True):
    """Run whole synthetic decode cycles: per layer the diffusion and the verify
    block attention over the current cache, one greedy consensus, one commit.

    k_cache, v_cache  bf16 [n_layers, B, Hkv, max_len, D];  cache_len int [B]
    cycles  list of dicts, one per cycle, with
        "diff", "verify": per-layer lists of (q, k_blk, v_blk) bf16
                          ([B,Hq,K,D], [B,Hkv,K,D], [B,Hkv,K,D])
        "logits" fp32 [B,K,V], "cand" int [B,K]  (greedy consensus), or
        "p", "q" fp32 [B,K,V], "cand" int [B,K], "uniforms" fp32 [B,K+1]
        (T>0 consensus by exact rejection sampling, notes §4.3)
    There is no model between the calls: the block inputs and the verify logits
    of each cycle are given, and the cycle's state (cache rows, lengths) flows
    from one cycle to the next exactly as in decoding.

    Returns (records, state): one record per cycle with the attention outputs
    of every layer (float64, if ``keep_attention``), the consensus results and
    the commit results; ``state`` holds the final cache bits and lengths.
    """
    kc, vc = _bits(k_cache), _bits(v_cache)
    lens = _ints(cache_len).copy()
    records = []
    for cyc in cycles:
        rec = {"cache_len_in": lens.copy()}
        kc_t, vc_t = bits_to_bf16(kc), bits_to_bf16(vc)
        if keep_attention:
            rec["diff_out"], rec["verify_out"] = [], []
        for layer, (dv, vv) in enumerate(zip(cyc["diff"], cyc["verify"])):
            if keep_attention:
                od, _ = block_attention(dv[0], dv[1], dv[2], kc_t[layer], vc_t[layer], lens,
                                        MASK_DIFF_BIDIR, scale)
                ov, _ = block_attention(vv[0], vv[1], vv[2], kc_t[layer], vc_t[layer], lens,
                                        MASK_VERIFY_CAUSAL, scale)
                rec["diff_out"].append(od)
                rec["verify_out"].append(ov)
        if "p" in cyc:
            acc, corr = sample_consensus(cyc["p"], cyc["q"], cyc["cand"], cyc["uniforms"])
        else:
            acc, _, corr = greedy_consensus(cyc["logits"], cyc["cand"])
        kb = np.stack([_bits(vv[1]) for vv in cyc["verify"]])
        vb = np.stack([_bits(vv[2]) for vv in cyc["verify"]])
        res = commit_block(kc, vc, kb, vb, lens, acc, corr, cyc["cand"])
        kc, vc, lens = res["k_cache"], res["v_cache"], res["cache_len"]
        rec.update(accept_len=acc, correction=corr, cache_len=lens.copy(),
                   next_anchor=res["next_anchor"], tokens=res["tokens"], n_tokens=res["n_tokens"])
        records.append(rec)
    return records, {"k_cache": kc, "v_cache": vc, "cache_len": lens}
