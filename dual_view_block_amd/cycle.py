"""Synthetic multi-cycle decode driver over the C ABI.

One Orthrus decode cycle (paper notes §4.1) is the diffusion-view block
attention of every layer, then the AR verify block attention of every layer
(both over the shared cache), then one consensus over the verify
distributions, then the commit that writes the verified rows into the cache
and advances the lengths.  This driver issues
exactly those calls, cycle after cycle, on one HIP stream: lengths live on the
device and every call reads them there, so the host never waits for a cycle to
finish before issuing the next one.  There is no model between the calls: each
cycle's block inputs and verify logits come from a given input set, and sets
are reused round-robin.

The driver computes nothing itself; it only resolves pointers once and
launches.  A whole round of cycles (one per input set) can be captured into a
HIP graph and replayed.
"""
from __future__ import annotations

import torch

from . import (ORTHRUS_MASK_DIFF_BIDIR, ORTHRUS_MASK_EXPLICIT, ORTHRUS_MASK_VERIFY_CAUSAL, PreparedAttention,
               PreparedCommit, PreparedGreedy, PreparedSample, _need, attn_desc, orthrus_attn_workspace_size,
               orthrus_consensus_workspace_size)


class DecodeCycles:
    """Synthetic decode cycles over caches of ``n_layers`` layers.

    k_cache, v_cache  bf16 [n_layers, B, Hkv, max_len, D] (updated in place)
    cache_len         int32 [B] (advanced in place by every commit)
    sets              list of input sets, each a dict with
        "diff", "verify": per-layer lists of (q [B,Hq,K,D], k_blk [B,Hkv,K,D],
                          v_blk [B,Hkv,K,D]) bf16 device tensors
        "logits" fp32 [B,K,V] and "cand" int32 [B,K] device tensors (greedy
        consensus), or "p", "q" fp32 [B,K,V], "cand" int32 [B,K] and
        "uniforms" fp32 [B,K+1] (T>0 consensus by rejection sampling)
    Cycle c uses set c % len(sets) and writes that set's outputs:
    ``diff_out[s][layer]``, ``verify_out[s][layer]`` (bf16 [B,Hq,K,D]),
    ``accept_len[s]``, ``correction[s]``, ``next_anchor[s]``, ``tokens[s]``,
    ``n_tokens[s]``.

    Dynamic block sizes (paper notes §7.4, §9.6): with ``blk_len`` (int32 [B]
    on the device) every call of a cycle runs over each sequence's first
    blk_len[b] block positions (the K of the inputs is the capacity), and the
    commit rewrites blk_len with the next cycle's lengths (floor ``k_min``)
    from each sequence's acceptance statistics ``accept_stat`` (int32 [B] on
    the device; zeros, no history, when not given), so the block size follows
    acceptance without the host.
    """

    def __init__(self, k_cache, v_cache, cache_len, sets, softmax_scale: float = 0.0, blk_len=None,
                 k_min: int = 1, accept_stat=None):
        if k_cache.dim() != 5:
            raise ValueError("k_cache must be [n_layers, B, Hkv, max_len, D]")
        self.n_layers = k_cache.shape[0]
        dev = k_cache.device
        self.k_cache, self.v_cache, self.cache_len = k_cache, v_cache, cache_len
        self.blk_len = blk_len
        if blk_len is not None and accept_stat is None:
            accept_stat = torch.zeros(k_cache.shape[1], dtype=torch.int32, device=dev)
        self.accept_stat = accept_stat
        B = k_cache.shape[1]
        first_q = sets[0]["diff"][0][0]
        K = first_q.shape[2]
        V = (sets[0]["p"] if "p" in sets[0] else sets[0]["logits"]).shape[2]
        desc = attn_desc(first_q, k_cache[0], softmax_scale)
        self.attn_ws = torch.empty(max(orthrus_attn_workspace_size(desc), 16), dtype=torch.uint8, device=dev)
        self.cons_ws = torch.empty(max(orthrus_consensus_workspace_size(B, K, V), 16), dtype=torch.uint8,
                                   device=dev)
        i32 = dict(dtype=torch.int32, device=dev)
        self.diff_out, self.verify_out = [], []
        self.accept_len, self.correction, self.next_anchor, self.tokens, self.n_tokens = [], [], [], [], []
        self._calls = []          # per set: the ordered list of prepared calls of one cycle
        self._blocks = []         # per set: stacked verify k/v blocks (the commit reads them)
        for s in sets:
            if len(s["diff"]) != self.n_layers or len(s["verify"]) != self.n_layers:
                raise ValueError("every input set needs one (q, k_blk, v_blk) per layer and view")
            kb = torch.stack([v[1] for v in s["verify"]])   # [n_layers, B, Hkv, K, D]
            vb = torch.stack([v[2] for v in s["verify"]])
            d_out = [torch.empty_like(s["diff"][l][0]) for l in range(self.n_layers)]
            v_out = [torch.empty_like(s["verify"][l][0]) for l in range(self.n_layers)]
            acc, corr = torch.empty(B, **i32), torch.empty(B, **i32)
            anchor, toks, ntok = torch.empty(B, **i32), torch.empty((B, K), **i32), torch.empty(B, **i32)
            _need(s["cand"], "cand", torch.int32, (B, K), dev)
            # the whole diffusion forward (every layer), then the whole verify
            # forward: the verify pass needs the candidates the diffusion pass
            # produces, so a real cycle cannot interleave the two per layer
            calls = []
            for l in range(self.n_layers):
                q, k_blk, v_blk = s["diff"][l]
                calls.append(PreparedAttention(ORTHRUS_MASK_DIFF_BIDIR, q, k_blk, v_blk, k_cache[l], v_cache[l],
                                               cache_len, d_out[l], None, self.attn_ws, softmax_scale,
                                               blk_len=blk_len))
            for l in range(self.n_layers):
                calls.append(PreparedAttention(ORTHRUS_MASK_VERIFY_CAUSAL, s["verify"][l][0], kb[l], vb[l],
                                               k_cache[l], v_cache[l], cache_len, v_out[l], None, self.attn_ws,
                                               softmax_scale, blk_len=blk_len))
            if "p" in s:
                calls.append(PreparedSample(s["p"], s["q"], s["cand"], s["uniforms"], acc, corr, self.cons_ws,
                                            blk_len=blk_len))
            else:
                calls.append(PreparedGreedy(s["logits"], s["cand"], acc, None, corr, self.cons_ws, blk_len=blk_len))
            calls.append(PreparedCommit(k_cache, v_cache, kb, vb, cache_len, acc, corr, s["cand"], anchor,
                                        toks, ntok, blk_len=blk_len, accept_stat=accept_stat, k_min=k_min))
            self._calls.append(calls)
            self._blocks.append((kb, vb))
            self.diff_out.append(d_out)
            self.verify_out.append(v_out)
            self.accept_len.append(acc)
            self.correction.append(corr)
            self.next_anchor.append(anchor)
            self.tokens.append(toks)
            self.n_tokens.append(ntok)
        self.sets = sets
        self.graph = None

    @property
    def n_sets(self) -> int:
        return len(self._calls)

    def issue(self, cycle: int, stream=None) -> None:
        """Issue one cycle (input set cycle % n_sets) on ``stream`` (default:
        torch's current stream).  Returns at once; nothing is waited for."""
        sp = (stream or torch.cuda.current_stream()).cuda_stream
        for call in self._calls[cycle % self.n_sets]:
            call(sp)

    def run(self, n_cycles: int, first_cycle: int = 0, stream=None) -> None:
        for c in range(first_cycle, first_cycle + n_cycles):
            self.issue(c, stream)

    def capture(self) -> None:
        """Capture one round (one cycle per input set, in order) into a HIP graph."""
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                self.run(self.n_sets)
        torch.cuda.current_stream().wait_stream(side)
        self.graph = g

    def replay(self, rounds: int = 1) -> None:
        """Replay the captured round ``rounds`` times on torch's current stream."""
        if self.graph is None:
            raise RuntimeError("capture() first")
        for _ in range(rounds):
            self.graph.replay()


class TreeDecodeCycles:
    """Synthetic decode cycles with tree verification (one draft tree of
    ``n_nodes`` nodes per sequence and cycle).

    Per cycle, on one stream: the diffusion-view attention of every layer;
    the top-``m`` marginals of the diffusion logits of block positions
    1..n_nodes-1; the best-first draft tree (rooted at the current anchor,
    which the previous commit wrote on the device); its ancestor masks; the
    tree-masked verify attention of every layer; greedy consensus along the
    tree; the commit of the accepted path.

    sets: dicts with "diff", "verify" (per-layer (q, k_blk, v_blk) with K =
    n_nodes block rows), "diff_logits" fp32 [B*(n_nodes-1), V] and
    "verify_logits" fp32 [B, n_nodes, V].
    """

    def __init__(self, k_cache, v_cache, cache_len, anchor, sets, m: int = 4, softmax_scale: float = 0.0):
        self.n_layers = k_cache.shape[0]
        dev = k_cache.device
        B = k_cache.shape[1]
        first_q = sets[0]["diff"][0][0]
        K = first_q.shape[2]
        V = sets[0]["verify_logits"].shape[2]
        self.B, self.K, self.V, self.m = B, K, V, m
        self.k_cache, self.v_cache, self.cache_len, self.anchor = k_cache, v_cache, cache_len, anchor
        desc = attn_desc(first_q, k_cache[0], softmax_scale)
        self.attn_ws = torch.empty(max(orthrus_attn_workspace_size(desc), 16), dtype=torch.uint8, device=dev)
        self.cons_ws = torch.empty(max(orthrus_consensus_workspace_size(B, K, V), 16), dtype=torch.uint8,
                                   device=dev)
        from . import _lib
        self.topk_ws = torch.empty(max(int(_lib.load().orthrus_topk_workspace_size(B * (K - 1), V, m)), 16),
                                   dtype=torch.uint8, device=dev)
        i32 = dict(dtype=torch.int32, device=dev)
        self.logp = torch.empty((B * (K - 1), m), dtype=torch.float32, device=dev)
        self.idx = torch.empty((B * (K - 1), m), **i32)
        self.parent, self.tokens, self.depth = (torch.empty((B, K), **i32) for _ in range(3))
        self.mask = torch.empty((B, K), dtype=torch.int64, device=dev)
        self.accept_len, self.correction = torch.empty(B, **i32), torch.empty(B, **i32)
        self.path = torch.empty((B, K), **i32)
        self.out_tokens, self.n_tokens = torch.empty((B, K), **i32), torch.empty(B, **i32)
        self._sets = []
        for s in sets:
            kb = torch.stack([v[1] for v in s["verify"]])
            vb = torch.stack([v[2] for v in s["verify"]])
            d_out = [torch.empty_like(s["diff"][l][0]) for l in range(self.n_layers)]
            v_out = [torch.empty_like(s["verify"][l][0]) for l in range(self.n_layers)]
            diff_calls, ver_calls = [], []
            for l in range(self.n_layers):
                q, k_blk, v_blk = s["diff"][l]
                diff_calls.append(PreparedAttention(ORTHRUS_MASK_DIFF_BIDIR, q, k_blk, v_blk, k_cache[l], v_cache[l],
                                                    cache_len, d_out[l], None, self.attn_ws, softmax_scale))
                ver_calls.append(PreparedAttention(ORTHRUS_MASK_EXPLICIT, s["verify"][l][0], kb[l], vb[l],
                                                   k_cache[l], v_cache[l], cache_len, v_out[l], None, self.attn_ws,
                                                   softmax_scale, block_mask=self.mask))
            self._sets.append(dict(diff=diff_calls, verify=ver_calls, kb=kb, vb=vb, d_out=d_out, v_out=v_out,
                                   diff_logits=s["diff_logits"], verify_logits=s["verify_logits"]))
        self.graph = None

    def issue(self, cycle: int, stream=None) -> None:
        from . import (orthrus_cache_commit_path, orthrus_consensus_tree_greedy, orthrus_topk_logprobs,
                       orthrus_tree_build, orthrus_tree_masks)
        st = stream or torch.cuda.current_stream()
        sp = st.cuda_stream
        s = self._sets[cycle % len(self._sets)]
        for c in s["diff"]:
            c(sp)
        orthrus_topk_logprobs(s["diff_logits"], self.m, logp=self.logp, idx=self.idx, workspace=self.topk_ws,
                              stream=sp)
        orthrus_tree_build(self.logp.view(self.B, self.K - 1, self.m), self.idx.view(self.B, self.K - 1, self.m),
                           self.anchor, self.K, parent=self.parent, tokens=self.tokens, depth=self.depth, stream=sp)
        orthrus_tree_masks(self.parent, mask=self.mask, stream=sp)
        for c in s["verify"]:
            c(sp)
        orthrus_consensus_tree_greedy(s["verify_logits"], self.tokens, self.parent, accept_len=self.accept_len,
                                      path=self.path, correction=self.correction, workspace=self.cons_ws, stream=sp)
        orthrus_cache_commit_path(self.k_cache, self.v_cache, s["kb"], s["vb"], self.cache_len, self.accept_len,
                                  self.path, self.tokens, self.correction, next_anchor=self.anchor,
                                  tokens=self.out_tokens, n_tokens=self.n_tokens, stream=sp)

    def run(self, n_cycles: int, first_cycle: int = 0, stream=None) -> None:
        for c in range(first_cycle, first_cycle + n_cycles):
            self.issue(c, stream)

    def capture(self) -> None:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                self.run(len(self._sets))
        torch.cuda.current_stream().wait_stream(side)
        self.graph = g

    def replay(self, rounds: int = 1) -> None:
        for _ in range(rounds):
            self.graph.replay()
