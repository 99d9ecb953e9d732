"""Synthetic multi-cycle decode driver over the C ABI.

One Orthrus decode cycle (paper notes §4.1) is, per layer, the diffusion-view
block attention and the AR verify block attention over the shared cache, then
one consensus over the verify distributions, then the commit that writes the
verified rows into the cache and advances the lengths.  This driver issues
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

from . import (ORTHRUS_MASK_DIFF_BIDIR, ORTHRUS_MASK_VERIFY_CAUSAL, PreparedAttention, PreparedCommit,
               PreparedGreedy, _need, attn_desc, orthrus_attn_workspace_size,
               orthrus_consensus_workspace_size)


class DecodeCycles:
    """Synthetic decode cycles over caches of ``n_layers`` layers.

    k_cache, v_cache  bf16 [n_layers, B, Hkv, max_len, D] (updated in place)
    cache_len         int32 [B] (advanced in place by every commit)
    sets              list of input sets, each a dict with
        "diff", "verify": per-layer lists of (q [B,Hq,K,D], k_blk [B,Hkv,K,D],
                          v_blk [B,Hkv,K,D]) bf16 device tensors
        "logits" fp32 [B,K,V] and "cand" int32 [B,K] device tensors
    Cycle c uses set c % len(sets) and writes that set's outputs:
    ``diff_out[s][layer]``, ``verify_out[s][layer]`` (bf16 [B,Hq,K,D]),
    ``accept_len[s]``, ``correction[s]``, ``next_anchor[s]``, ``tokens[s]``,
    ``n_tokens[s]``.
    """

    def __init__(self, k_cache, v_cache, cache_len, sets, softmax_scale: float = 0.0):
        if k_cache.dim() != 5:
            raise ValueError("k_cache must be [n_layers, B, Hkv, max_len, D]")
        self.n_layers = k_cache.shape[0]
        dev = k_cache.device
        self.k_cache, self.v_cache, self.cache_len = k_cache, v_cache, cache_len
        B = k_cache.shape[1]
        first_q = sets[0]["diff"][0][0]
        K = first_q.shape[2]
        V = sets[0]["logits"].shape[2]
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
            calls = []
            for l in range(self.n_layers):
                q, k_blk, v_blk = s["diff"][l]
                calls.append(PreparedAttention(ORTHRUS_MASK_DIFF_BIDIR, q, k_blk, v_blk, k_cache[l], v_cache[l],
                                               cache_len, d_out[l], None, self.attn_ws, softmax_scale))
                calls.append(PreparedAttention(ORTHRUS_MASK_VERIFY_CAUSAL, s["verify"][l][0], kb[l], vb[l],
                                               k_cache[l], v_cache[l], cache_len, v_out[l], None, self.attn_ws,
                                               softmax_scale))
            calls.append(PreparedGreedy(s["logits"], s["cand"], acc, None, corr, self.cons_ws))
            calls.append(PreparedCommit(k_cache, v_cache, kb, vb, cache_len, acc, corr, s["cand"], anchor,
                                        toks, ntok))
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
