"""Seeded synthetic inputs for the dual-view decode step.

This module only draws and lays out inputs; it holds none of the method's
arithmetic (no attention, no argmax, no accept test).  Both the HIP path and
the CPU oracle are fed from the tensors it returns, so the two sides always see
bit-identical inputs.

Workloads (shapes and value laws) stand in for the pages' settings: Qwen3
1.7B / 8B attention shapes, block size K = 32 (the pages' default), a frozen
model's KV cache modelled as N(0, 1) values rounded to bf16, and vocab-sized
logits.  The public evaluation suites the pages measure on are not needed:
only context length and acceptance pattern reach this path, and both are
swept synthetically (L from 256 to 131072, first-mismatch index over 0..K).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

VOCAB_QWEN3 = 151936


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    layers: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    cache_len: int            # L (for ragged: the largest allowed L)
    block_k: int
    vocab: int
    logit_sigma: float
    seed: int
    max_len: Optional[int] = None     # cache capacity; defaults to cache_len
    ragged_min: Optional[int] = None  # ragged: L_b ~ U{ragged_min..cache_len}

    @property
    def capacity(self) -> int:
        return self.max_len if self.max_len is not None else self.cache_len

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    # 1 layer, 2 q heads, 1 KV head, D=64, L=256, K=4; vocab 1000, logits sigma 4
    "tiny": Workload("tiny", 1, 1, 2, 1, 64, 256, 4, 1000, 4.0, 1),
    # Qwen3-1.7B-shaped single layer: 16 q heads / 8 KV heads, D=128, L=2048
    "qwen3_1p7b_layer": Workload("qwen3_1p7b_layer", 1, 1, 16, 8, 128, 2048, 32,
                                 VOCAB_QWEN3, 3.0, 2),
    # Qwen3-8B-shaped: 36 layers, 32 q heads / 8 KV heads, D=128, L=8192
    "qwen3_8b_8k": Workload("qwen3_8b_8k", 36, 1, 32, 8, 128, 8192, 32,
                            VOCAB_QWEN3, 3.0, 3),
    # Qwen3-8B-shaped long context, L=32768, K=32 (K and L are swept around it)
    "qwen3_8b_32k": Workload("qwen3_8b_32k", 36, 1, 32, 8, 128, 32768, 32,
                             VOCAB_QWEN3, 3.0, 4),
    "qwen3_8b_128k": Workload("qwen3_8b_128k", 36, 1, 32, 8, 128, 131072, 32,
                              VOCAB_QWEN3, 3.0, 4),
    # batched ragged: 16 sequences, L_b ~ U{1024..16384}, capacity 16384
    "ragged_b16": Workload("ragged_b16", 36, 16, 32, 8, 128, 16384, 32,
                           VOCAB_QWEN3, 3.0, 5, max_len=16384, ragged_min=1024),
}

K_SWEEP = (1, 4, 8, 16, 32)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randn_bf16(shape, g, device) -> torch.Tensor:
    """N(0, 1) float32 draws rounded once to bf16 (round-to-nearest-even)."""
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


def cache_lengths(w: Workload, device="cpu") -> torch.Tensor:
    """int32 [B]: L for every sequence, or seeded U{ragged_min..cache_len}."""
    if w.ragged_min is None:
        return torch.full((w.batch,), w.cache_len, dtype=torch.int32, device=device)
    g = _gen(w.seed * 1000 + 7, "cpu")
    lens = torch.randint(w.ragged_min, w.cache_len + 1, (w.batch,), generator=g, dtype=torch.int64)
    return lens.to(torch.int32).to(device)


def attention_inputs(w: Workload, layer: int = 0, device="cpu", seed_offset: int = 0):
    """One layer's attention inputs (identical tensors go to both views).

    Returns a dict: q [B,Hq,K,D], k_blk / v_blk [B,Hkv,K,D] (the block's
    keys/values: K_diff/V_diff for the diffusion view, the AR K/V of the block
    tokens for the verify view), k_cache / v_cache [B,Hkv,max_len,D], all
    bf16, and cache_len int32 [B].  Cache rows at and beyond L_b hold ordinary
    N(0,1) draws (tests that need poison there write it themselves).
    """
    g = _gen(w.seed * 7919 + 104729 * layer + seed_offset, device)
    B, Hq, Hkv, D, K, S = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.block_k, w.capacity
    return {
        "q": _randn_bf16((B, Hq, K, D), g, device),
        "k_blk": _randn_bf16((B, Hkv, K, D), g, device),
        "v_blk": _randn_bf16((B, Hkv, K, D), g, device),
        "k_cache": _randn_bf16((B, Hkv, S, D), g, device),
        "v_cache": _randn_bf16((B, Hkv, S, D), g, device),
        "cache_len": cache_lengths(w, device),
    }


def layer_cache(w: Workload, layer: int, device="cpu"):
    """One layer's shared KV cache (k_cache, v_cache) bf16 [B,Hkv,max_len,D]."""
    g = _gen(w.seed * 7919 + 104729 * layer + 1, device)
    shape = (w.batch, w.n_kv_heads, w.capacity, w.head_dim)
    return _randn_bf16(shape, g, device), _randn_bf16(shape, g, device)


def model_cache(w: Workload, device="cpu"):
    """The shared KV cache of every layer as two layer-major tensors
    (k_cache, v_cache) bf16 [layers, B, Hkv, max_len, D]; layer l holds the
    same draws as ``layer_cache(w, l)``."""
    shape = (w.layers, w.batch, w.n_kv_heads, w.capacity, w.head_dim)
    k = torch.empty(shape, dtype=torch.bfloat16, device=device)
    v = torch.empty(shape, dtype=torch.bfloat16, device=device)
    for layer in range(w.layers):
        g = _gen(w.seed * 7919 + 104729 * layer + 1, device)
        k[layer] = _randn_bf16(shape[1:], g, device)
        v[layer] = _randn_bf16(shape[1:], g, device)
    return k, v


def view_inputs(w: Workload, layer: int, view: str, device="cpu"):
    """The block inputs of one view at one layer: (q, k_blk, v_blk) bf16.

    The diffusion view and the verify view get independent draws (different
    projections of different block tokens in the real model)."""
    g = _gen(w.seed * 7919 + 104729 * layer + (2 if view == "diff" else 3) + 17 * w.block_k, device)
    B, Hq, Hkv, D, K = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.block_k
    return (_randn_bf16((B, Hq, K, D), g, device), _randn_bf16((B, Hkv, K, D), g, device),
            _randn_bf16((B, Hkv, K, D), g, device))


def greedy_inputs(w: Workload, device="cpu", first_mismatch=None, ties: bool = False,
                  seed_offset: int = 0):
    """Verify logits [B,K,V] float32 and candidates [B,K] int32.

    Logits are N(0, sigma) clamped to +-6 sigma; in each row one seeded token t
    is set to 6 sigma + 1, so the row's top token is known by construction.
    With ``ties`` a second seeded token t2 gets the same top value (the lower
    of t, t2 is then the lowest-index top).  Candidates copy the top token up
    to the seeded first-mismatch index j* (0..K; K = all match), differ from it
    at j*, and are random after j*.
    Returns (logits, cand, j_star [B] int64).
    """
    g = _gen(w.seed * 31 + 17 + seed_offset, "cpu")
    B, K, V, s = w.batch, w.block_k, w.vocab, float(w.logit_sigma)
    logits = torch.randn((B, K, V), generator=g, dtype=torch.float32) * s
    logits.clamp_(-6.0 * s, 6.0 * s)
    top = torch.randint(0, V, (B, K), generator=g)
    top_val = 6.0 * s + 1.0
    b_idx = torch.arange(B).unsqueeze(1).expand(B, K)
    k_idx = torch.arange(K).unsqueeze(0).expand(B, K)
    logits[b_idx, k_idx, top] = top_val
    first_top = top.clone()
    if ties:
        t2 = torch.randint(0, V, (B, K), generator=g)
        logits[b_idx, k_idx, t2] = top_val
        first_top = torch.minimum(top, t2)
    if first_mismatch is None:
        j_star = torch.randint(0, K + 1, (B,), generator=g)
    else:
        j_star = torch.as_tensor(first_mismatch, dtype=torch.int64).expand(B).clone()
    rand_tok = torch.randint(0, V, (B, K), generator=g)
    shift = torch.randint(1, V, (B, K), generator=g)
    cand = torch.where(k_idx < j_star.unsqueeze(1), first_top, rand_tok)
    at_j = k_idx == j_star.unsqueeze(1)
    cand = torch.where(at_j, (first_top + shift) % V, cand)
    return logits.to(device), cand.to(torch.int32).to(device), j_star


# Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as
# easy as 1, 2, 3", SC 2011): a counter-based generator.  Each 128-bit counter
# (four 32-bit words) and 64-bit key give four independent 32-bit outputs;
# ten rounds, each two 32x32->64 multiplications whose halves are mixed with
# the other words and the key, the key bumped by the Weyl constants between
# rounds.
_PHILOX_M = (0xD2511F53, 0xCD9E8D57)
_PHILOX_W = (0x9E3779B9, 0xBB67AE85)
_U32 = 0xFFFFFFFF


def philox4x32(counters, key):
    """Philox4x32-10 of uint64 arrays holding 32-bit words.

    counters: int array [..., 4]; key: (k0, k1).  Returns uint64 [..., 4]."""
    import numpy as np

    c = np.asarray(counters, dtype=np.uint64) & np.uint64(_U32)
    c0, c1, c2, c3 = (c[..., i].copy() for i in range(4))
    k0, k1 = np.uint64(key[0] & _U32), np.uint64(key[1] & _U32)
    m0, m1 = np.uint64(_PHILOX_M[0]), np.uint64(_PHILOX_M[1])
    lo = np.uint64(_U32)
    for r in range(10):
        p0, p1 = m0 * c0, m1 * c2            # exact: both factors < 2^32
        c0, c1, c2, c3 = ((p1 >> np.uint64(32)) ^ c1 ^ k0, p1 & lo,
                          (p0 >> np.uint64(32)) ^ c3 ^ k1, p0 & lo)
        if r < 9:
            k0 = (k0 + np.uint64(_PHILOX_W[0])) & lo
            k1 = (k1 + np.uint64(_PHILOX_W[1])) & lo
    return np.stack([c0, c1, c2, c3], axis=-1)


def philox_uniforms(n: int, seed: int) -> torch.Tensor:
    """float64 [n] uniforms on the 2**-24 grid in [0, 1): output word j of
    the Philox4x32-10 block with counter (j // 4, 0, 0, 0) and key (seed mod
    2^32, seed >> 32), top 24 bits."""
    import numpy as np

    blocks = (n + 3) // 4
    ctr = np.zeros((blocks, 4), dtype=np.uint64)
    ctr[:, 0] = np.arange(blocks, dtype=np.uint64)
    words = philox4x32(ctr, (int(seed) & _U32, (int(seed) >> 32) & _U32)).reshape(-1)[:n]
    return torch.from_numpy((words >> np.uint64(8)).astype(np.float64) / 16777216.0)


def quantise_uniforms(u: torch.Tensor) -> torch.Tensor:
    """Put float uniforms on the 2**-24 grid in [0, 1) (exact in float32)."""
    return (torch.floor(u.double() * 16777216.0).clamp(0, 16777215) / 16777216.0).float()


def sample_inputs(w: Workload, device="cpu", draft_noise: Optional[float] = None,
                  seed_offset: int = 0):
    """Target/draft probabilities, candidates and uniforms for T>0 consensus.

    z_p ~ N(0, sigma); z_q ~ N(0, sigma) independent, or z_q = z_p + N(0,
    draft_noise) when ``draft_noise`` is set (a draft close to the target, so
    acceptance runs long).  p, q = softmax in float64 rounded to float32.
    cand[b, i] ~ q[b, i] by inverse CDF of a Philox4x32-10 uniform; uniforms
    [B, K+1] on the 2**-24 grid from a second Philox stream.  Returns (p, q,
    cand int32, uniforms float32).
    """
    g = _gen(w.seed * 131 + 5 + seed_offset, "cpu")
    B, K, V, s = w.batch, w.block_k, w.vocab, float(w.logit_sigma)
    zp = torch.randn((B, K, V), generator=g, dtype=torch.float64) * s
    if draft_noise is None:
        zq = torch.randn((B, K, V), generator=g, dtype=torch.float64) * s
    else:
        zq = zp + torch.randn((B, K, V), generator=g, dtype=torch.float64) * float(draft_noise)
    p64 = torch.softmax(zp, dim=-1)
    q64 = torch.softmax(zq, dim=-1)
    del zp, zq
    # cand ~ q by inverse CDF of one Philox uniform per row; the accept and
    # residual uniforms from a second Philox stream
    uc = philox_uniforms(B * K, w.seed * 131 + 6 + seed_offset).reshape(B * K, 1)
    cdf = torch.cumsum(q64.reshape(B * K, V), dim=-1)
    cand = torch.searchsorted(cdf, uc * cdf[:, -1:], right=True).clamp_(max=V - 1).reshape(B, K)
    u = quantise_uniforms(philox_uniforms(B * (K + 1), w.seed * 131 + 7 + seed_offset).reshape(B, K + 1))
    return (p64.float().to(device), q64.float().to(device),
            cand.to(torch.int32).to(device), u.to(device))


def first_mismatch_geometric(n: int, block_k: int, accept_rate: float, seed: int) -> torch.Tensor:
    """int64 [n] first-mismatch indices j* in 0..K: the number of leading
    successes of independent trials with success probability ``accept_rate``,
    capped at K.  With accept_rate 0.912 and K = 32 the mean of
    j* + [j* < K] is about 10.8 tokens per cycle: two forwards per cycle at
    the average 5.39 tokens per forward the pages report for the 8B model."""
    g = _gen(seed, "cpu")
    u = torch.rand((n, block_k), generator=g, dtype=torch.float64)
    fail = u >= float(accept_rate)
    first = torch.where(fail.any(dim=1), fail.to(torch.int64).argmax(dim=1),
                        torch.full((n,), block_k, dtype=torch.int64))
    return first


def first_mismatch_quantiles(n: int, block_k: int, accept_rate: float, seed: int) -> torch.Tensor:
    """int64 [n] first-mismatch indices that follow the law of
    ``first_mismatch_geometric`` as closely as n values can: the (s + 1/2)/n
    quantiles, s = 0..n-1, in a seeded random order.  For a benchmark that
    cycles through a few input sets, this keeps the mean tokens per cycle at
    the law's mean instead of a small random sample's."""
    vals = []
    for s in range(n):
        u = (s + 0.5) / n
        j = 0
        while j < block_k and 1.0 - float(accept_rate) ** (j + 1) < u:
            j += 1
        vals.append(j)
    perm = torch.randperm(n, generator=_gen(seed, "cpu"))
    return torch.tensor(vals, dtype=torch.int64)[perm]


def cycle_inputs(w: Workload, n_cycles: int, accept_rate: float = 0.912, device="cpu",
                 seed_offset: int = 0, layers: Optional[int] = None, stratified: bool = False):
    """Inputs of ``n_cycles`` synthetic decode cycles (no model between calls).

    Each cycle gets fresh block inputs for every layer and both views (q,
    k_blk, v_blk drawn as in ``view_inputs``) and fresh verify logits and
    candidates (``greedy_inputs``) whose first-mismatch index per sequence is
    drawn by ``first_mismatch_geometric`` (or, with ``stratified``, taken from
    ``first_mismatch_quantiles`` over all cycles and sequences).  Returns a list of dicts with keys
    "diff", "verify" (per-layer (q, k_blk, v_blk) tuples), "logits", "cand"
    and "j_star".
    """
    n_layers = w.layers if layers is None else layers
    strata = None
    if stratified:
        strata = first_mismatch_quantiles(n_cycles * w.batch, w.block_k, accept_rate,
                                          w.seed * 1009 + seed_offset + 5).reshape(n_cycles, w.batch)
    out = []
    for c in range(n_cycles):
        wc = w.replace(seed=w.seed * 1009 + 31 * c + seed_offset)
        if strata is not None:
            js = strata[c].clone()
        else:
            js = first_mismatch_geometric(w.batch, w.block_k, accept_rate, wc.seed * 13 + 3)
        diff = [view_inputs(wc, layer, "diff", device) for layer in range(n_layers)]
        verify = [view_inputs(wc, layer, "verify", device) for layer in range(n_layers)]
        logits, cand, j_star = greedy_inputs(wc, device, first_mismatch=js)
        out.append({"diff": diff, "verify": verify, "logits": logits, "cand": cand, "j_star": j_star})
    return out


def sample_cycle_inputs(w: Workload, n_cycles: int, draft_noise: Optional[float] = 0.3, device="cpu",
                        seed_offset: int = 0, layers: Optional[int] = None):
    """Inputs of ``n_cycles`` synthetic T>0 decode cycles: per cycle fresh
    block inputs for every layer and both views (as ``cycle_inputs``) and the
    target/draft probabilities, candidates and uniforms of ``sample_inputs``
    (a draft close to the target with ``draft_noise``).  Returns dicts with
    "diff", "verify", "p", "q", "cand" and "uniforms"."""
    n_layers = w.layers if layers is None else layers
    out = []
    for c in range(n_cycles):
        wc = w.replace(seed=w.seed * 1009 + 31 * c + seed_offset)
        diff = [view_inputs(wc, layer, "diff", device) for layer in range(n_layers)]
        verify = [view_inputs(wc, layer, "verify", device) for layer in range(n_layers)]
        p, q, cand, u = sample_inputs(wc, device, draft_noise=draft_noise)
        out.append({"diff": diff, "verify": verify, "p": p, "q": q, "cand": cand, "uniforms": u})
    return out


def kl_inputs(rows: int, vocab: int, sigma: float = 3.0, dtype=torch.float32, seed: int = 0,
              draft_noise: Optional[float] = None, device="cpu"):
    """Target (AR) and draft (diffusion) logits [rows, vocab] for the forward-KL
    loss: target ~ N(0, sigma); draft independent N(0, sigma), or target +
    N(0, draft_noise) for a draft close to its teacher (late in training).
    Drawn in float32 and rounded once to ``dtype``."""
    g = _gen(seed * 7 + 101, device)
    a = torch.randn((rows, vocab), generator=g, device=device, dtype=torch.float32) * float(sigma)
    if draft_noise is None:
        b = torch.randn((rows, vocab), generator=g, device=device, dtype=torch.float32) * float(sigma)
    else:
        b = a + torch.randn((rows, vocab), generator=g, device=device, dtype=torch.float32) * float(draft_noise)
    return a.to(dtype), b.to(dtype)


def train_attn_inputs(n_q_heads: int, n_kv_heads: int, seq_len: int, n_blocks: int, block_k: int,
                      head_dim: int, seed: int = 0, device="cpu", anchors=None):
    """One packed training sequence for the dual-pass attention: head-major
    bf16 N(0, 1) q/k/v of the clean path ([H, L, D]) and of the diffusion
    blocks ([H, N*K, D]), and N anchor positions drawn uniformly from
    [0, L - K] (the pages sample 256 random anchors per 2048-token sequence)."""
    g = _gen(seed * 613 + 29, device)
    Hq, Hkv, L, N, K, D = n_q_heads, n_kv_heads, seq_len, n_blocks, block_k, head_dim
    out = {
        "q_ar": _randn_bf16((Hq, L, D), g, device),
        "k_ar": _randn_bf16((Hkv, L, D), g, device),
        "v_ar": _randn_bf16((Hkv, L, D), g, device),
        "q_diff": _randn_bf16((Hq, N * K, D), g, device),
        "k_diff": _randn_bf16((Hkv, N * K, D), g, device),
        "v_diff": _randn_bf16((Hkv, N * K, D), g, device),
    }
    if anchors is None:
        ga = _gen(seed * 613 + 30, "cpu")
        anchors = torch.randint(0, max(L - K, 0) + 1, (N,), generator=ga)
    out["anchors"] = torch.as_tensor(anchors, dtype=torch.int32).to(device)
    out["block_k"] = K
    return out


def random_trees(batch: int, n_nodes: int, seed: int = 0, unused_frac: float = 0.0) -> torch.Tensor:
    """int32 [B, n] draft-tree parents: node 0 is the root (-1); node i > 0
    picks a uniform parent among the used nodes before it, or is unused (-1)
    with probability ``unused_frac``."""
    g = _gen(seed * 17 + 3, "cpu")
    par = torch.full((batch, n_nodes), -1, dtype=torch.int32)
    u = torch.rand((batch, n_nodes), generator=g)
    pick = torch.rand((batch, n_nodes), generator=g)
    for b in range(batch):
        used = [0]
        for i in range(1, n_nodes):
            if float(u[b, i]) < unused_frac:
                continue
            par[b, i] = used[int(float(pick[b, i]) * len(used))]
            used.append(i)
    return par


def tree_verify_logits(parent: torch.Tensor, tokens: torch.Tensor, vocab: int, accept_rate: float = 0.7,
                       sigma: float = 3.0, seed: int = 0) -> torch.Tensor:
    """fp32 [B, n, V] verify logits for draft trees with a planted top token
    per node row: with probability ``accept_rate`` the token of one of the
    node's children (uniform among them), else a uniform token.  Rows are
    N(0, sigma) clamped to +-6 sigma with the planted token at 6 sigma + 1, so
    each row's argmax is known by construction."""
    g = _gen(seed * 29 + 11, "cpu")
    B, n = parent.shape
    s = float(sigma)
    logits = (torch.randn((B, n, vocab), generator=g) * s).clamp_(-6 * s, 6 * s)
    coin = torch.rand((B, n), generator=g)
    pick = torch.rand((B, n), generator=g)
    rand_tok = torch.randint(0, vocab, (B, n), generator=g)
    for b in range(B):
        kids = {i: [] for i in range(n)}
        for i in range(1, n):
            p = int(parent[b, i])
            if 0 <= p < i:
                kids[p].append(i)
        for i in range(n):
            if kids[i] and float(coin[b, i]) < accept_rate:
                top = int(tokens[b, kids[i][int(float(pick[b, i]) * len(kids[i]))]])
            else:
                top = int(rand_tok[b, i])
            logits[b, i, top] = 6 * s + 1
    return logits


def draft_marginals(batch: int, depth: int, m: int, vocab: int, seed: int = 0, ties: bool = False):
    """Per-depth top-m marginals for tree building: logp fp32 [B, depth, m]
    descending and <= 0 (the top entries of a uniformly drawn probability
    vector over m + 4 outcomes, logged),
    tok int32 [B, depth, m] distinct tokens per depth.  With ``ties`` some
    log-probs repeat, exercising the tie rule."""
    g = _gen(seed * 37 + 5, "cpu")
    # a uniform random probability vector over m + 4 outcomes (normalised exponentials)
    e = -torch.log(torch.rand((batch, depth, m + 4), generator=g, dtype=torch.float64).clamp_min(1e-300))
    p = e / e.sum(dim=-1, keepdim=True)
    top = torch.sort(p, dim=-1, descending=True).values[..., :m]
    logp = torch.log(top).to(torch.float32)
    if ties:
        logp[:, :, 1::3] = logp[:, :, 0::3][:, :, :logp[:, :, 1::3].shape[2]]
        logp = torch.sort(logp, dim=-1, descending=True).values
    tok = torch.stack([torch.randperm(vocab, generator=g)[:m] for _ in range(batch * depth)]).reshape(batch, depth, m)
    return logp, tok.to(torch.int32)
