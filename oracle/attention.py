"""Oracle for the dual-view block attention (diffusion view and AR verify).

TEST INFRASTRUCTURE ONLY -- never imported by the product path.

Sources (the Orthrus pages):

* Paper notes on Orthrus (zhangshuibai.github.io paper-notes, "Orthrus:
  Memory-Efficient Parallel Token Generation via Dual-View Diffusion"),
  §2.1 (the diffusion view has its own Q/K/V projections; its K/V for the K
  future positions are transient and never become history), §2.2 (only the AR
  path writes the shared cache), §3.2 (the diffusion positions of a block see
  the clean context before their anchor and each other, bidirectionally, under
  one block mask), §4.1 step 1 (block = anchor + K-1 mask positions, one
  diffusion forward) and step 2 (the K candidates go through one causal AR
  forward, giving K next-token distributions).
* hotdry.top blog post on Orthrus dual-view diffusion decoding, sections on
  the dual-view attention architecture and on the training mask (same facts).

Readings of points the pages leave open:

* R1 -- the cache given holds every position strictly before the anchor
  (``cache_len[b]`` positions); the anchor itself is block row 0.
* R4 -- cache keys and block keys share one softmax (one mask over the
  concatenated key sequence, as in the training mask).
* R5 -- scale 1/sqrt(D) unless given; q head h reads KV head h // (Hq/Hkv);
  q and k arrive already projected (RoPE/norms are upstream).
* R15 -- ``cache_len`` = 0 and K = 1 are valid.

Everything is float64, one (sequence, q head) at a time, with an explicit
boolean mask; ``numpy.matmul`` and ``numpy.exp`` are the only library steps.
"""
from __future__ import annotations

import math

import numpy as np

MASK_DIFF_BIDIR = 0      # diffusion view: every block row sees every block key
MASK_VERIFY_CAUSAL = 1   # AR verify: block row i sees block keys j <= i
MASK_EXPLICIT = 2        # a given per-row set of visible block keys (tree / ragged blocks)


def _as_f64(x) -> np.ndarray:
    """Widen to float64 (bf16/fp32 -> fp64 is exact)."""
    try:  # torch tensors, including bfloat16 ones
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def _as_int(x) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.int64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.int64)


def block_mask(L: int, K: int, mode: int, explicit=None) -> np.ndarray:
    """Boolean mask [K, L+K]: row i (block position i) may attend key column c.

    Columns 0..L-1 are the cached positions (all before the anchor: visible to
    every block row in both views).  Column L+j is block key j: always visible
    in the diffusion view (bidirectional block), visible iff j <= i in the
    verify view (causal AR forward over the block).
    """
    m = np.zeros((K, L + K), dtype=bool)
    m[:, :L] = True
    if mode == MASK_DIFF_BIDIR:
        m[:, L:] = True
    elif mode == MASK_VERIFY_CAUSAL:
        for i in range(K):
            m[i, L:L + i + 1] = True
    elif mode == MASK_EXPLICIT:
        # explicit[i][j]: block key j visible to block row i (R22)
        for i in range(K):
            for j in range(K):
                m[i, L + j] = bool(explicit[i][j])
    else:
        raise ValueError(f"unknown mask mode {mode}")
    return m


def _attend(qrows: np.ndarray, keys: np.ndarray, vals: np.ndarray,
            mask: np.ndarray, scale: float):
    """Masked softmax attention of qrows [n, D] over keys/vals [m, D].

    s = scale * q k^T, -inf where the mask is False; p = softmax(s);
    out = p v; lse = log sum exp(s) (natural log).
    """
    s = scale * (qrows @ keys.T)
    s = np.where(mask, s, -np.inf)
    seen = mask.any(axis=1)  # a row with no visible key: output 0, lse -inf (R22)
    smax = np.where(seen, s.max(axis=1), 0.0)[:, None]
    e = np.where(mask, np.exp(s - smax), 0.0)
    denom = e.sum(axis=1, keepdims=True)
    p = np.where(seen[:, None], e / np.where(denom > 0, denom, 1.0), 0.0)
    out = p @ vals
    with np.errstate(divide="ignore"):
        lse = np.where(seen, smax[:, 0] + np.log(np.where(seen, denom[:, 0], 1.0)), -np.inf)
    return out, lse


def block_attention(q, k_blk, v_blk, k_cache, v_cache, cache_len, mode: int,
                    scale: float | None = None, block_masks=None):
    """Dual-view block attention for every (sequence, q head, block row).

    Shapes: q [B,Hq,K,D]; k_blk, v_blk [B,Hkv,K,D]; k_cache, v_cache
    [B,Hkv,max_len,D]; cache_len [B] (clamped to [0, max_len]).  With mode
    MASK_EXPLICIT, block_masks [B,K,K] (bool) gives the visible block keys of
    every row.
    Returns (out [B,Hq,K,D] float64, lse [B,Hq,K] float64).
    """
    qd, kb, vb = _as_f64(q), _as_f64(k_blk), _as_f64(v_blk)
    kc, vc = _as_f64(k_cache), _as_f64(v_cache)
    lens = _as_int(cache_len)
    B, Hq, K, D = qd.shape
    Hkv = kb.shape[1]
    max_len = kc.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    sc = 1.0 / math.sqrt(D) if not scale else float(scale)
    out = np.zeros((B, Hq, K, D))
    lse = np.zeros((B, Hq, K))
    for b in range(B):
        L = int(min(max(int(lens[b]), 0), max_len))
        mask = block_mask(L, K, mode, None if block_masks is None else block_masks[b])
        for h in range(Hq):
            g = h // G
            keys = np.concatenate([kc[b, g, :L], kb[b, g]], axis=0)
            vals = np.concatenate([vc[b, g, :L], vb[b, g]], axis=0)
            out[b, h], lse[b, h] = _attend(qd[b, h], keys, vals, mask, sc)
    return out, lse


def block_attention_rows(q, k_blk, v_blk, k_cache, v_cache, cache_len,
                         mode: int, rows, scale: float | None = None):
    """The same definition evaluated only at selected outputs.

    ``rows`` is an iterable of (b, h, i).  Used to check full-size launches on
    sampled outputs.  Inputs may be torch tensors (any device); only the
    slices a row needs are widened to float64.
    Returns (out [n, D] float64, lse [n] float64) in the order of ``rows``.
    """
    rows = list(rows)
    Hq = q.shape[1]
    Hkv = k_blk.shape[1]
    K = q.shape[2]
    D = q.shape[3]
    max_len = k_cache.shape[2]
    G = Hq // Hkv
    sc = 1.0 / math.sqrt(D) if not scale else float(scale)
    lens = _as_int(cache_len)
    outs, lses = [], []
    cache_kv = {}
    for (b, h, i) in rows:
        g = h // G
        L = int(min(max(int(lens[b]), 0), max_len))
        key = (b, g)
        if key not in cache_kv:
            keys = np.concatenate([_as_f64(k_cache[b, g, :L]), _as_f64(k_blk[b, g])], axis=0)
            vals = np.concatenate([_as_f64(v_cache[b, g, :L]), _as_f64(v_blk[b, g])], axis=0)
            cache_kv[key] = (keys, vals)
        keys, vals = cache_kv[key]
        mask = block_mask(L, K, mode)[i:i + 1]
        qrow = _as_f64(q[b, h, i]).reshape(1, D)
        o, l = _attend(qrow, keys, vals, mask, sc)
        outs.append(o[0])
        lses.append(l[0])
    return np.stack(outs), np.array(lses)


def transient_kv_bytes(n_layers: int, n_kv_heads: int, head_dim: int,
                       block_k: int, bytes_per_elem: int = 2) -> int:
    """Bytes of the transient diffusion-view K/V for one block, all layers.

    The diffusion view's K_diff/V_diff exist only for the K block positions of
    the current cycle (paper notes §2.1 and §2.3; the notes' §9.5 check of the
    constant ~4.5 MiB overhead).  Per layer: K and V, each [Hkv, K, D].
    Cache length does not appear: the size is independent of L.
    """
    return n_layers * n_kv_heads * block_k * head_dim * 2 * bytes_per_elem
