"""MI355X-native Orthrus dual-view decode step (C ABI + thin torch binding).

The functions carry the C ABI's names (include/orthrus.h) and only marshal
arguments: they check dtypes, shapes, devices and contiguity, allocate missing
outputs / workspace with torch on the tensors' device, and call the library on
torch's current HIP stream.  All computation happens in the gfx950 kernels.

Sources for what each call computes: Orthrus paper notes (zhangshuibai.github.io
paper-notes), §2.1, §3.2 and §4.1 (block attention of both views over the
shared KV cache), §4.2 (greedy consensus), §4.3 and §7.2 (rejection-sampling
consensus), §4.1 step 3 (closing the cycle: the verified rows go into the cache,
the correction becomes the next anchor), §3.3 (the forward-KL distillation loss
of training), §3.1-3.2 (the training-time dual-pass block-mask attention).
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import (ORTHRUS_MASK_DIFF_BIDIR, ORTHRUS_MASK_EXPLICIT, ORTHRUS_MASK_VERIFY_CAUSAL, AttnDesc, CommitDesc,
                   OrthrusError, TrainAttnDesc, status_string)

__all__ = [
    "AttnDesc", "OrthrusError", "ORTHRUS_MASK_DIFF_BIDIR", "ORTHRUS_MASK_VERIFY_CAUSAL",
    "attn_desc", "orthrus_attn_workspace_size", "orthrus_attn_num_splits", "orthrus_block_attn",
    "orthrus_block_attn_diff", "orthrus_block_attn_verify", "orthrus_consensus_workspace_size",
    "orthrus_consensus_greedy", "orthrus_consensus_sample", "orthrus_status_string",
    "PreparedAttention", "PreparedGreedy", "PreparedSample", "library_path", "CommitDesc", "orthrus_cache_commit",
    "PreparedCommit", "orthrus_kl_workspace_size", "orthrus_forward_kl", "PreparedForwardKL",
    "TrainAttnDesc", "orthrus_train_attn_fwd", "orthrus_train_attn_bwd", "orthrus_block_attn_masked",
    "orthrus_topk_logprobs", "orthrus_tree_build", "orthrus_tree_masks", "orthrus_consensus_tree_greedy",
    "orthrus_cache_commit_path", "orthrus_block_attn_noalloc", "orthrus_block_attn_dyn",
    "orthrus_consensus_greedy_dyn", "orthrus_consensus_sample_dyn", "orthrus_cache_commit_dyn",
]


def library_path() -> str:
    return _lib.LIB_PATH


def orthrus_status_string(status: int) -> str:
    return status_string(status)


def _stream_ptr(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _need(t: torch.Tensor, name: str, dtype, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device (the library has no CPU path)")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def attn_desc(q: torch.Tensor, k_cache: torch.Tensor, softmax_scale: float = 0.0) -> AttnDesc:
    B, Hq, K, D = q.shape
    _, Hkv, max_len, _ = k_cache.shape
    return AttnDesc(B, Hq, Hkv, D, K, max_len, float(softmax_scale))


def orthrus_attn_workspace_size(desc: AttnDesc) -> int:
    return int(_lib.load().orthrus_attn_workspace_size(ctypes.byref(desc)))


def orthrus_attn_num_splits(desc: AttnDesc) -> int:
    return int(_lib.load().orthrus_attn_num_splits(ctypes.byref(desc)))


def orthrus_consensus_workspace_size(batch: int, block_k: int, vocab: int) -> int:
    return int(_lib.load().orthrus_consensus_workspace_size(batch, block_k, vocab))


def _workspace(nbytes: int, device, workspace):
    if workspace is None:  # scratch only: no initialisation needed
        return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)
    _need(workspace, "workspace", torch.uint8, device=device)
    return workspace


def _check_attn(q, k_blk, v_blk, k_cache, v_cache, cache_len):
    if q.dim() != 4 or k_cache.dim() != 4:
        raise ValueError("q and k_cache must be 4-D")
    B, Hq, K, D = q.shape
    _, Hkv, max_len, _ = k_cache.shape
    dev = q.device
    _need(q, "q", torch.bfloat16, (B, Hq, K, D))
    _need(k_blk, "k_blk", torch.bfloat16, (B, Hkv, K, D), dev)
    _need(v_blk, "v_blk", torch.bfloat16, (B, Hkv, K, D), dev)
    _need(k_cache, "k_cache", torch.bfloat16, (B, Hkv, max_len, D), dev)
    _need(v_cache, "v_cache", torch.bfloat16, (B, Hkv, max_len, D), dev)
    _need(cache_len, "cache_len", torch.int32, (B,), dev)


def orthrus_block_attn(q, k_blk, v_blk, k_cache, v_cache, cache_len, mode: int, out=None, lse=None,
                       workspace=None, softmax_scale: float = 0.0, want_lse: bool = True,
                       stream=None):
    """Block attention of one layer; returns (out bf16 [B,Hq,K,D], lse fp32 [B,Hq,K] or None)."""
    _check_attn(q, k_blk, v_blk, k_cache, v_cache, cache_len)
    desc = attn_desc(q, k_cache, softmax_scale)
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16, tuple(q.shape), dev)
    if lse is None and want_lse:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, tuple(q.shape[:3]), dev)
    nbytes = orthrus_attn_workspace_size(desc)
    ws = _workspace(nbytes, dev, workspace)
    st = _lib.load().orthrus_block_attn(
        ctypes.byref(desc), int(mode), q.data_ptr(), k_blk.data_ptr(), v_blk.data_ptr(),
        k_cache.data_ptr(), v_cache.data_ptr(), cache_len.data_ptr(), out.data_ptr(),
        lse.data_ptr() if lse is not None else None, ws.data_ptr(), ws.numel(), _stream_ptr(stream))
    _lib.check("orthrus_block_attn", st)
    return out, lse


def orthrus_block_attn_noalloc(q, k_blk, v_blk, k_cache, v_cache, cache_len, mode: int, out, lse=None,
                               softmax_scale: float = 0.0, stream=None):
    """orthrus_block_attn on the library's own device scratch: the C call
    allocates nothing (the caller passes `out`, and `lse` or None)."""
    _check_attn(q, k_blk, v_blk, k_cache, v_cache, cache_len)
    desc = attn_desc(q, k_cache, softmax_scale)
    _need(out, "out", torch.bfloat16, tuple(q.shape), q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32, tuple(q.shape[:3]), q.device)
    st = _lib.load().orthrus_block_attn_noalloc(
        ctypes.byref(desc), int(mode), q.data_ptr(), k_blk.data_ptr(), v_blk.data_ptr(), k_cache.data_ptr(),
        v_cache.data_ptr(), cache_len.data_ptr(), out.data_ptr(), lse.data_ptr() if lse is not None else None,
        _stream_ptr(stream))
    _lib.check("orthrus_block_attn_noalloc", st)
    return out, lse


def orthrus_block_attn_diff(q, k_blk, v_blk, k_cache, v_cache, cache_len, **kw):
    """Diffusion-view block attention (bidirectional within the block)."""
    return orthrus_block_attn(q, k_blk, v_blk, k_cache, v_cache, cache_len, ORTHRUS_MASK_DIFF_BIDIR, **kw)


def orthrus_block_attn_verify(q, k_blk, v_blk, k_cache, v_cache, cache_len, **kw):
    """AR verify block attention (causal within the block)."""
    return orthrus_block_attn(q, k_blk, v_blk, k_cache, v_cache, cache_len, ORTHRUS_MASK_VERIFY_CAUSAL,
                              **kw)


class PreparedAttention:
    """A block-attention call with every pointer resolved once.

    For launch loops (one call per layer per view): calling the object issues
    exactly one C call on the given stream.  The tensors are held so that
    their memory stays alive as long as the object.
    """

    def __init__(self, mode, q, k_blk, v_blk, k_cache, v_cache, cache_len, out, lse, workspace,
                 softmax_scale: float = 0.0, block_mask=None, blk_len=None):
        _check_attn(q, k_blk, v_blk, k_cache, v_cache, cache_len)
        _need(out, "out", torch.bfloat16, tuple(q.shape), q.device)
        if lse is not None:
            _need(lse, "lse", torch.float32, tuple(q.shape[:3]), q.device)
        _need(workspace, "workspace", torch.uint8, None, q.device)
        self.desc = attn_desc(q, k_cache, softmax_scale)
        self._keep = (q, k_blk, v_blk, k_cache, v_cache, cache_len, out, lse, workspace, block_mask, blk_len)
        nbytes = orthrus_attn_workspace_size(self.desc)
        if workspace.numel() < nbytes:
            raise ValueError(f"workspace has {workspace.numel()} bytes, needs {nbytes}")
        lib = _lib.load()
        if (mode == ORTHRUS_MASK_EXPLICIT) != (block_mask is not None):
            raise ValueError("an explicit block mask goes with mode ORTHRUS_MASK_EXPLICIT, and only with it")
        self._fn = lib.orthrus_block_attn
        self._args = (ctypes.byref(self.desc), int(mode), q.data_ptr(), k_blk.data_ptr(), v_blk.data_ptr(),
                      k_cache.data_ptr(), v_cache.data_ptr(), cache_len.data_ptr(), out.data_ptr(),
                      lse.data_ptr() if lse is not None else None, workspace.data_ptr(),
                      workspace.numel())

        self._partial = lib.orthrus_block_attn_partial
        self._partial_args = self._args[:8] + self._args[10:]
        self._merge = lib.orthrus_block_attn_merge
        self._merge_args = (self._args[0],) + self._args[8:]
        if block_mask is not None:  # the whole call only (the halves take mode masks)
            _need(block_mask, "block_mask", torch.int64, (q.shape[0], q.shape[2]), q.device)
            self._fn = lib.orthrus_block_attn_masked
            a = self._args
            self._args = (a[0],) + a[2:8] + (block_mask.data_ptr(),) + a[8:]
            self._partial = self._merge = None
        if blk_len is not None:  # dynamic block sizes: the whole call only
            if block_mask is not None:
                raise ValueError("a block length per sequence goes with the mode masks only")
            _need(blk_len, "blk_len", torch.int32, (q.shape[0],), q.device)
            self._fn = lib.orthrus_block_attn_dyn
            a = self._args
            self._args = a[:8] + (blk_len.data_ptr(),) + a[8:]
            self._partial = self._merge = None

    def __call__(self, stream_ptr: int) -> None:
        st = self._fn(*self._args, stream_ptr)
        if st:
            _lib.check("orthrus_block_attn", st)

    def partial(self, stream_ptr: int) -> None:
        """First half only: stream the cache into the split partials."""
        st = self._partial(*self._partial_args, stream_ptr)
        if st:
            _lib.check("orthrus_block_attn_partial", st)

    def merge(self, stream_ptr: int) -> None:
        """Second half only: merge the split partials into out / lse."""
        st = self._merge(*self._merge_args, stream_ptr)
        if st:
            _lib.check("orthrus_block_attn_merge", st)


class PreparedGreedy:
    """A greedy-consensus call with every pointer resolved once."""

    def __init__(self, logits, cand, accept_len, row_argmax, correction, workspace, blk_len=None):
        B, K, V = logits.shape
        dev = logits.device
        _need(logits, "logits", torch.float32, (B, K, V))
        _need(cand, "cand", torch.int32, (B, K), dev)
        _need(accept_len, "accept_len", torch.int32, (B,), dev)
        _need(correction, "correction", torch.int32, (B,), dev)
        if row_argmax is not None:
            _need(row_argmax, "row_argmax", torch.int32, (B, K), dev)
        _need(workspace, "workspace", torch.uint8, None, dev)
        nbytes = orthrus_consensus_workspace_size(B, K, V)
        if workspace.numel() < nbytes:
            raise ValueError(f"workspace has {workspace.numel()} bytes, needs {nbytes}")
        self._keep = (logits, cand, accept_len, row_argmax, correction, workspace, blk_len)
        lib = _lib.load()
        self._fn = lib.orthrus_consensus_greedy
        self._args = (B, K, V, logits.data_ptr(), cand.data_ptr(), accept_len.data_ptr(),
                      row_argmax.data_ptr() if row_argmax is not None else None, correction.data_ptr(),
                      workspace.data_ptr(), workspace.numel())
        if blk_len is not None:  # dynamic block sizes
            _need(blk_len, "blk_len", torch.int32, (B,), dev)
            self._fn = lib.orthrus_consensus_greedy_dyn
            self._args = self._args[:5] + (blk_len.data_ptr(),) + self._args[5:]

    def __call__(self, stream_ptr: int) -> None:
        st = self._fn(*self._args, stream_ptr)
        if st:
            _lib.check("orthrus_consensus_greedy", st)


class PreparedSample:
    """A T>0 consensus call with every pointer resolved once."""

    def __init__(self, p_target, q_draft, cand, uniforms, accept_len, correction, workspace, blk_len=None):
        B, K, V = p_target.shape
        dev = p_target.device
        _need(p_target, "p_target", torch.float32, (B, K, V))
        _need(q_draft, "q_draft", torch.float32, (B, K, V), dev)
        _need(cand, "cand", torch.int32, (B, K), dev)
        _need(uniforms, "uniforms", torch.float32, (B, K + 1), dev)
        _need(accept_len, "accept_len", torch.int32, (B,), dev)
        _need(correction, "correction", torch.int32, (B,), dev)
        _need(workspace, "workspace", torch.uint8, None, dev)
        nbytes = orthrus_consensus_workspace_size(B, K, V)
        if workspace.numel() < nbytes:
            raise ValueError(f"workspace has {workspace.numel()} bytes, needs {nbytes}")
        self._keep = (p_target, q_draft, cand, uniforms, accept_len, correction, workspace, blk_len)
        lib = _lib.load()
        self._fn = lib.orthrus_consensus_sample
        self._args = (B, K, V, p_target.data_ptr(), q_draft.data_ptr(), cand.data_ptr(), uniforms.data_ptr(),
                      accept_len.data_ptr(), correction.data_ptr(), workspace.data_ptr(), workspace.numel())
        if blk_len is not None:  # dynamic block sizes
            _need(blk_len, "blk_len", torch.int32, (B,), dev)
            self._fn = lib.orthrus_consensus_sample_dyn
            self._args = self._args[:7] + (blk_len.data_ptr(),) + self._args[7:]

    def __call__(self, stream_ptr: int) -> None:
        st = self._fn(*self._args, stream_ptr)
        if st:
            _lib.check("orthrus_consensus_sample", st)


def orthrus_consensus_greedy(logits, cand, accept_len=None, row_argmax=None, correction=None,
                             workspace=None, want_row_argmax: bool = True, stream=None):
    """Greedy consensus; returns (accept_len [B], row_argmax [B,K] or None, correction [B])."""
    if logits.dim() != 3:
        raise ValueError("logits must be [B, K, V]")
    B, K, V = logits.shape
    dev = logits.device
    _need(logits, "logits", torch.float32, (B, K, V))
    _need(cand, "cand", torch.int32, (B, K), dev)
    if accept_len is None:
        accept_len = torch.empty(B, dtype=torch.int32, device=dev)
    if correction is None:
        correction = torch.empty(B, dtype=torch.int32, device=dev)
    if row_argmax is None and want_row_argmax:
        row_argmax = torch.empty((B, K), dtype=torch.int32, device=dev)
    _need(accept_len, "accept_len", torch.int32, (B,), dev)
    _need(correction, "correction", torch.int32, (B,), dev)
    if row_argmax is not None:
        _need(row_argmax, "row_argmax", torch.int32, (B, K), dev)
    ws = _workspace(orthrus_consensus_workspace_size(B, K, V), dev, workspace)
    st = _lib.load().orthrus_consensus_greedy(
        B, K, V, logits.data_ptr(), cand.data_ptr(), accept_len.data_ptr(),
        row_argmax.data_ptr() if row_argmax is not None else None, correction.data_ptr(),
        ws.data_ptr(), ws.numel(), _stream_ptr(stream))
    _lib.check("orthrus_consensus_greedy", st)
    return accept_len, row_argmax, correction


def orthrus_consensus_sample(p_target, q_draft, cand, uniforms, accept_len=None, correction=None,
                             workspace=None, stream=None):
    """T>0 rejection-sampling consensus; returns (accept_len [B], correction [B])."""
    if p_target.dim() != 3:
        raise ValueError("p_target must be [B, K, V]")
    B, K, V = p_target.shape
    dev = p_target.device
    _need(p_target, "p_target", torch.float32, (B, K, V))
    _need(q_draft, "q_draft", torch.float32, (B, K, V), dev)
    _need(cand, "cand", torch.int32, (B, K), dev)
    _need(uniforms, "uniforms", torch.float32, (B, K + 1), dev)
    if accept_len is None:
        accept_len = torch.empty(B, dtype=torch.int32, device=dev)
    if correction is None:
        correction = torch.empty(B, dtype=torch.int32, device=dev)
    _need(accept_len, "accept_len", torch.int32, (B,), dev)
    _need(correction, "correction", torch.int32, (B,), dev)
    ws = _workspace(orthrus_consensus_workspace_size(B, K, V), dev, workspace)
    st = _lib.load().orthrus_consensus_sample(
        B, K, V, p_target.data_ptr(), q_draft.data_ptr(), cand.data_ptr(), uniforms.data_ptr(),
        accept_len.data_ptr(), correction.data_ptr(), ws.data_ptr(), ws.numel(), _stream_ptr(stream))
    _lib.check("orthrus_consensus_sample", st)
    return accept_len, correction


def _check_commit(k_cache, v_cache, k_blk, v_blk, cache_len, accept_len, correction, cand):
    """Shapes of a commit; 4-D caches/blocks are one layer.  Returns the descriptor."""
    if k_cache.dim() == 4:
        k_cache, v_cache = k_cache.unsqueeze(0), v_cache.unsqueeze(0)
    if k_blk.dim() == 4:
        k_blk, v_blk = k_blk.unsqueeze(0), v_blk.unsqueeze(0)
    if k_cache.dim() != 5 or k_blk.dim() != 5:
        raise ValueError("caches must be [n_layers, B, Hkv, max_len, D] and blocks [n_layers, B, Hkv, K, D]")
    n_layers, B, Hkv, max_len, D = k_cache.shape
    K = k_blk.shape[3]
    dev = k_cache.device
    _need(k_cache, "k_cache", torch.bfloat16, (n_layers, B, Hkv, max_len, D))
    _need(v_cache, "v_cache", torch.bfloat16, (n_layers, B, Hkv, max_len, D), dev)
    _need(k_blk, "k_blk", torch.bfloat16, (n_layers, B, Hkv, K, D), dev)
    _need(v_blk, "v_blk", torch.bfloat16, (n_layers, B, Hkv, K, D), dev)
    _need(cache_len, "cache_len", torch.int32, (B,), dev)
    _need(accept_len, "accept_len", torch.int32, (B,), dev)
    _need(correction, "correction", torch.int32, (B,), dev)
    _need(cand, "cand", torch.int32, (B, K), dev)
    return CommitDesc(n_layers, B, Hkv, D, K, max_len)


class PreparedCommit:
    """A cache-commit call with every pointer resolved once (see
    ``orthrus_cache_commit``); calling it issues one C call on the stream."""

    def __init__(self, k_cache, v_cache, k_blk, v_blk, cache_len, accept_len, correction, cand,
                 next_anchor, tokens, n_tokens, blk_len=None, accept_stat=None, k_min: int = 1):
        self.desc = _check_commit(k_cache, v_cache, k_blk, v_blk, cache_len, accept_len, correction, cand)
        B, K, dev = self.desc.batch, self.desc.block_k, k_cache.device
        _need(next_anchor, "next_anchor", torch.int32, (B,), dev)
        _need(tokens, "tokens", torch.int32, (B, K), dev)
        _need(n_tokens, "n_tokens", torch.int32, (B,), dev)
        self._keep = (k_cache, v_cache, k_blk, v_blk, cache_len, accept_len, correction, cand,
                      next_anchor, tokens, n_tokens)
        lib = _lib.load()
        self._fn = lib.orthrus_cache_commit
        self._args = (ctypes.byref(self.desc),) + tuple(t.data_ptr() for t in self._keep)
        if blk_len is not None:  # dynamic block sizes: the commit also advances blk_len
            _need(blk_len, "blk_len", torch.int32, (B,), dev)
            _need(accept_stat, "accept_stat", torch.int32, (B,), dev)
            self._keep = self._keep + (blk_len, accept_stat)
            self._fn = lib.orthrus_cache_commit_dyn
            self._args = self._args + (blk_len.data_ptr(), accept_stat.data_ptr(), int(k_min))

    def __call__(self, stream_ptr: int) -> None:
        st = self._fn(*self._args, stream_ptr)
        if st:
            _lib.check("orthrus_cache_commit", st)


def orthrus_cache_commit(k_cache, v_cache, k_blk, v_blk, cache_len, accept_len, correction, cand,
                         next_anchor=None, tokens=None, n_tokens=None, stream=None):
    """Close one decode cycle on the device: the verified block rows go into the
    caches and ``cache_len`` advances, both in place.

    Caches bf16 [n_layers, B, Hkv, max_len, D] (or [B, Hkv, max_len, D] for one
    layer), blocks bf16 [n_layers, B, Hkv, K, D] (or 4-D).  Returns
    (next_anchor [B], tokens [B, K], n_tokens [B]), all int32."""
    desc = _check_commit(k_cache, v_cache, k_blk, v_blk, cache_len, accept_len, correction, cand)
    B, K, dev = desc.batch, desc.block_k, k_cache.device
    if next_anchor is None:
        next_anchor = torch.empty(B, dtype=torch.int32, device=dev)
    if tokens is None:
        tokens = torch.empty((B, K), dtype=torch.int32, device=dev)
    if n_tokens is None:
        n_tokens = torch.empty(B, dtype=torch.int32, device=dev)
    _need(next_anchor, "next_anchor", torch.int32, (B,), dev)
    _need(tokens, "tokens", torch.int32, (B, K), dev)
    _need(n_tokens, "n_tokens", torch.int32, (B,), dev)
    st = _lib.load().orthrus_cache_commit(
        ctypes.byref(desc), k_cache.data_ptr(), v_cache.data_ptr(), k_blk.data_ptr(), v_blk.data_ptr(),
        cache_len.data_ptr(), accept_len.data_ptr(), correction.data_ptr(), cand.data_ptr(),
        next_anchor.data_ptr(), tokens.data_ptr(), n_tokens.data_ptr(), _stream_ptr(stream))
    _lib.check("orthrus_cache_commit", st)
    return next_anchor, tokens, n_tokens


def orthrus_block_attn_dyn(q, k_blk, v_blk, k_cache, v_cache, cache_len, blk_len, mode: int, out=None, lse=None,
                           workspace=None, softmax_scale: float = 0.0, want_lse: bool = True, stream=None):
    """Block attention with a block length per sequence (int32 [B] on the
    device): rows past a sequence's length are not written.  Returns
    (out, lse or None) as ``orthrus_block_attn``."""
    _check_attn(q, k_blk, v_blk, k_cache, v_cache, cache_len)
    desc = attn_desc(q, k_cache, softmax_scale)
    dev = q.device
    _need(blk_len, "blk_len", torch.int32, (q.shape[0],), dev)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", torch.bfloat16, tuple(q.shape), dev)
    if lse is None and want_lse:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, tuple(q.shape[:3]), dev)
    ws = _workspace(orthrus_attn_workspace_size(desc), dev, workspace)
    st = _lib.load().orthrus_block_attn_dyn(
        ctypes.byref(desc), int(mode), q.data_ptr(), k_blk.data_ptr(), v_blk.data_ptr(), k_cache.data_ptr(),
        v_cache.data_ptr(), cache_len.data_ptr(), blk_len.data_ptr(), out.data_ptr(),
        lse.data_ptr() if lse is not None else None, ws.data_ptr(), ws.numel(), _stream_ptr(stream))
    _lib.check("orthrus_block_attn_dyn", st)
    return out, lse


def orthrus_consensus_greedy_dyn(logits, cand, blk_len, accept_len=None, row_argmax=None, correction=None,
                                 workspace=None, want_row_argmax: bool = True, stream=None):
    """Greedy consensus over each sequence's first blk_len[b] rows; returns
    (accept_len [B], row_argmax [B,K] (-1 past the block) or None, correction [B])."""
    B, K, V = logits.shape
    dev = logits.device
    _need(logits, "logits", torch.float32, (B, K, V))
    _need(cand, "cand", torch.int32, (B, K), dev)
    _need(blk_len, "blk_len", torch.int32, (B,), dev)
    if accept_len is None:
        accept_len = torch.empty(B, dtype=torch.int32, device=dev)
    if correction is None:
        correction = torch.empty(B, dtype=torch.int32, device=dev)
    if row_argmax is None and want_row_argmax:
        row_argmax = torch.empty((B, K), dtype=torch.int32, device=dev)
    ws = _workspace(orthrus_consensus_workspace_size(B, K, V), dev, workspace)
    st = _lib.load().orthrus_consensus_greedy_dyn(
        B, K, V, logits.data_ptr(), cand.data_ptr(), blk_len.data_ptr(), accept_len.data_ptr(),
        row_argmax.data_ptr() if row_argmax is not None else None, correction.data_ptr(),
        ws.data_ptr(), ws.numel(), _stream_ptr(stream))
    _lib.check("orthrus_consensus_greedy_dyn", st)
    return accept_len, row_argmax, correction


def orthrus_consensus_sample_dyn(p_target, q_draft, cand, uniforms, blk_len, accept_len=None, correction=None,
                                 workspace=None, stream=None):
    """T>0 consensus over each sequence's first blk_len[b] rows; returns
    (accept_len [B], correction [B])."""
    B, K, V = p_target.shape
    dev = p_target.device
    _need(p_target, "p_target", torch.float32, (B, K, V))
    _need(q_draft, "q_draft", torch.float32, (B, K, V), dev)
    _need(cand, "cand", torch.int32, (B, K), dev)
    _need(uniforms, "uniforms", torch.float32, (B, K + 1), dev)
    _need(blk_len, "blk_len", torch.int32, (B,), dev)
    if accept_len is None:
        accept_len = torch.empty(B, dtype=torch.int32, device=dev)
    if correction is None:
        correction = torch.empty(B, dtype=torch.int32, device=dev)
    ws = _workspace(orthrus_consensus_workspace_size(B, K, V), dev, workspace)
    st = _lib.load().orthrus_consensus_sample_dyn(
        B, K, V, p_target.data_ptr(), q_draft.data_ptr(), cand.data_ptr(), uniforms.data_ptr(),
        blk_len.data_ptr(), accept_len.data_ptr(), correction.data_ptr(), ws.data_ptr(), ws.numel(),
        _stream_ptr(stream))
    _lib.check("orthrus_consensus_sample_dyn", st)
    return accept_len, correction


def orthrus_cache_commit_dyn(k_cache, v_cache, k_blk, v_blk, cache_len, accept_len, correction, cand, blk_len,
                             accept_stat, k_min: int = 1, next_anchor=None, tokens=None, n_tokens=None,
                             stream=None):
    """``orthrus_cache_commit`` over each sequence's first blk_len[b] block
    positions; the acceptance statistics (int32 [B], 0 for a new sequence) and
    blk_len are then advanced in place to the next cycle's.
    Returns (next_anchor [B], tokens [B, K], n_tokens [B])."""
    desc = _check_commit(k_cache, v_cache, k_blk, v_blk, cache_len, accept_len, correction, cand)
    B, K, dev = desc.batch, desc.block_k, k_cache.device
    _need(blk_len, "blk_len", torch.int32, (B,), dev)
    _need(accept_stat, "accept_stat", torch.int32, (B,), dev)
    if next_anchor is None:
        next_anchor = torch.empty(B, dtype=torch.int32, device=dev)
    if tokens is None:
        tokens = torch.empty((B, K), dtype=torch.int32, device=dev)
    if n_tokens is None:
        n_tokens = torch.empty(B, dtype=torch.int32, device=dev)
    st = _lib.load().orthrus_cache_commit_dyn(
        ctypes.byref(desc), k_cache.data_ptr(), v_cache.data_ptr(), k_blk.data_ptr(), v_blk.data_ptr(),
        cache_len.data_ptr(), accept_len.data_ptr(), correction.data_ptr(), cand.data_ptr(),
        next_anchor.data_ptr(), tokens.data_ptr(), n_tokens.data_ptr(), blk_len.data_ptr(), accept_stat.data_ptr(),
        int(k_min), _stream_ptr(stream))
    _lib.check("orthrus_cache_commit_dyn", st)
    return next_anchor, tokens, n_tokens


_KL_DTYPES = {torch.float32: _lib.ORTHRUS_DTYPE_F32, torch.bfloat16: _lib.ORTHRUS_DTYPE_BF16}


def orthrus_kl_workspace_size(rows: int, vocab: int, dtype) -> int:
    return int(_lib.load().orthrus_kl_workspace_size(rows, vocab, _KL_DTYPES[dtype]))


def _check_kl(target, draft):
    if target.dim() != 2:
        raise ValueError("logits must be [rows, V]")
    if target.dtype not in _KL_DTYPES:
        raise TypeError("logits must be float32 or bfloat16")
    rows, V = target.shape
    _need(target, "target_logits", target.dtype, (rows, V))
    _need(draft, "draft_logits", target.dtype, (rows, V), target.device)
    return rows, V


class PreparedForwardKL:
    """A forward-KL call with every pointer resolved once (see ``orthrus_forward_kl``)."""

    def __init__(self, target, draft, kl, grad, workspace, grad_scale: float = 1.0):
        rows, V = _check_kl(target, draft)
        dev = target.device
        _need(kl, "kl", torch.float32, (rows,), dev)
        if grad is not None:
            _need(grad, "grad", target.dtype, (rows, V), dev)
        nbytes = orthrus_kl_workspace_size(rows, V, target.dtype)
        if workspace.numel() < nbytes:
            raise ValueError(f"workspace has {workspace.numel()} bytes, needs {nbytes}")
        self._keep = (target, draft, kl, grad, workspace)
        self._fn = _lib.load().orthrus_forward_kl
        self._args = (rows, V, _KL_DTYPES[target.dtype], target.data_ptr(), draft.data_ptr(), kl.data_ptr(),
                      grad.data_ptr() if grad is not None else None, float(grad_scale), workspace.data_ptr(),
                      workspace.numel())

    def __call__(self, stream_ptr: int) -> None:
        st = self._fn(*self._args, stream_ptr)
        if st:
            _lib.check("orthrus_forward_kl", st)


def orthrus_forward_kl(target_logits, draft_logits, kl=None, grad=None, want_grad: bool = False,
                       grad_scale: float = 1.0, workspace=None, stream=None):
    """Forward KL(softmax(target) || softmax(draft)) per row, and optionally its
    gradient with respect to the draft logits (times ``grad_scale``).

    Logits [rows, V], float32 or bfloat16.  Returns (kl fp32 [rows], grad
    [rows, V] in the logits' dtype, or None)."""
    rows, V = _check_kl(target_logits, draft_logits)
    dev = target_logits.device
    if kl is None:
        kl = torch.empty(rows, dtype=torch.float32, device=dev)
    _need(kl, "kl", torch.float32, (rows,), dev)
    if grad is None and want_grad:
        grad = torch.empty_like(target_logits)
    if grad is not None:
        _need(grad, "grad", target_logits.dtype, (rows, V), dev)
    ws = _workspace(orthrus_kl_workspace_size(rows, V, target_logits.dtype), dev, workspace)
    st = _lib.load().orthrus_forward_kl(
        rows, V, _KL_DTYPES[target_logits.dtype], target_logits.data_ptr(), draft_logits.data_ptr(),
        kl.data_ptr(), grad.data_ptr() if grad is not None else None, float(grad_scale), ws.data_ptr(),
        ws.numel(), _stream_ptr(stream))
    _lib.check("orthrus_forward_kl", st)
    return kl, grad


def _check_train(q_ar, k_ar, v_ar, q_diff, k_diff, v_diff, anchors, block_k):
    if k_ar.dim() != 3:
        raise ValueError("k_ar must be [Hkv, L, D]")
    Hkv, L, D = k_ar.shape
    dev = k_ar.device
    _need(k_ar, "k_ar", torch.bfloat16, (Hkv, L, D))
    _need(v_ar, "v_ar", torch.bfloat16, (Hkv, L, D), dev)
    Hq = None
    if q_ar is not None:
        Hq = q_ar.shape[0]
        _need(q_ar, "q_ar", torch.bfloat16, (Hq, L, D), dev)
    N = 0
    if q_diff is not None:
        Hq = q_diff.shape[0] if Hq is None else Hq
        N = anchors.shape[0]
        _need(q_diff, "q_diff", torch.bfloat16, (Hq, N * block_k, D), dev)
        _need(k_diff, "k_diff", torch.bfloat16, (Hkv, N * block_k, D), dev)
        _need(v_diff, "v_diff", torch.bfloat16, (Hkv, N * block_k, D), dev)
        _need(anchors, "anchors", torch.int32, (N,), dev)
    if Hq is None:
        raise ValueError("need q_ar or q_diff")
    return Hq, Hkv, L, D, N


def orthrus_train_attn_fwd(q_ar, k_ar, v_ar, q_diff=None, k_diff=None, v_diff=None, anchors=None, block_k=32,
                           out_ar=None, lse_ar=None, out_diff=None, lse_diff=None, want_lse: bool = True,
                           softmax_scale: float = 0.0, stream=None):
    """Training dual-pass attention forward of one packed sequence (head-major
    bf16 layouts).  q_ar may be None to skip the AR rows, q_diff None for no
    blocks.  Returns (out_ar, lse_ar, out_diff, lse_diff); absent parts are None."""
    Hq, Hkv, L, D, N = _check_train(q_ar, k_ar, v_ar, q_diff, k_diff, v_diff, anchors, block_k)
    dev = k_ar.device
    if q_ar is not None:
        out_ar = torch.empty_like(q_ar) if out_ar is None else out_ar
        _need(out_ar, "out_ar", torch.bfloat16, tuple(q_ar.shape), dev)
        if lse_ar is None and want_lse:
            lse_ar = torch.empty((Hq, L), dtype=torch.float32, device=dev)
    else:
        out_ar = lse_ar = None
    if q_diff is not None:
        out_diff = torch.empty_like(q_diff) if out_diff is None else out_diff
        _need(out_diff, "out_diff", torch.bfloat16, tuple(q_diff.shape), dev)
        if lse_diff is None and want_lse:
            lse_diff = torch.empty((Hq, N * block_k), dtype=torch.float32, device=dev)
    else:
        out_diff = lse_diff = None
    desc = TrainAttnDesc(L, N, block_k, Hq, Hkv, D, float(softmax_scale))
    ptr = lambda t: t.data_ptr() if t is not None else None
    st = _lib.load().orthrus_train_attn_fwd(
        ctypes.byref(desc), ptr(q_ar), k_ar.data_ptr(), v_ar.data_ptr(), ptr(q_diff), ptr(k_diff), ptr(v_diff),
        ptr(anchors), ptr(out_ar), ptr(lse_ar), ptr(out_diff), ptr(lse_diff), _stream_ptr(stream))
    _lib.check("orthrus_train_attn_fwd", st)
    return out_ar, lse_ar, out_diff, lse_diff


def orthrus_train_attn_bwd(k_ar, v_ar, q_diff, k_diff, v_diff, anchors, block_k, out_diff, lse_diff, d_out_diff,
                           dq=None, dk=None, dv=None, softmax_scale: float = 0.0, stream=None):
    """Backward of the diffusion rows of the training dual-pass attention.
    Returns (dq_diff [Hq,N*K,D], dk_diff [Hkv,N*K,D], dv_diff [Hkv,N*K,D]) bf16."""
    Hq, Hkv, L, D, N = _check_train(None, k_ar, v_ar, q_diff, k_diff, v_diff, anchors, block_k)
    dev = k_ar.device
    _need(out_diff, "out_diff", torch.bfloat16, tuple(q_diff.shape), dev)
    _need(lse_diff, "lse_diff", torch.float32, (Hq, N * block_k), dev)
    _need(d_out_diff, "d_out_diff", torch.bfloat16, tuple(q_diff.shape), dev)
    dq = torch.empty_like(q_diff) if dq is None else dq
    dk = torch.empty_like(k_diff) if dk is None else dk
    dv = torch.empty_like(v_diff) if dv is None else dv
    _need(dq, "dq", torch.bfloat16, tuple(q_diff.shape), dev)
    _need(dk, "dk", torch.bfloat16, tuple(k_diff.shape), dev)
    _need(dv, "dv", torch.bfloat16, tuple(v_diff.shape), dev)
    desc = TrainAttnDesc(L, N, block_k, Hq, Hkv, D, float(softmax_scale))
    st = _lib.load().orthrus_train_attn_bwd(
        ctypes.byref(desc), k_ar.data_ptr(), v_ar.data_ptr(), q_diff.data_ptr(), k_diff.data_ptr(),
        v_diff.data_ptr(), anchors.data_ptr(), out_diff.data_ptr(), lse_diff.data_ptr(), d_out_diff.data_ptr(),
        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), _stream_ptr(stream))
    _lib.check("orthrus_train_attn_bwd", st)
    return dq, dk, dv


# ------------------------------------------------------------ tree verification
def orthrus_block_attn_masked(q, k_blk, v_blk, k_cache, v_cache, cache_len, block_mask, out=None, lse=None,
                              workspace=None, softmax_scale: float = 0.0, want_lse: bool = True, stream=None):
    """Block attention with explicit per-row block masks (int64 [B, K], bit j
    = block key j visible).  Returns (out, lse)."""
    _check_attn(q, k_blk, v_blk, k_cache, v_cache, cache_len)
    desc = attn_desc(q, k_cache, softmax_scale)
    dev = q.device
    B, Hq, K, D = q.shape
    _need(block_mask, "block_mask", torch.int64, (B, K), dev)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    ws = _workspace(orthrus_attn_workspace_size(desc), dev, workspace)
    st = _lib.load().orthrus_block_attn_masked(
        ctypes.byref(desc), q.data_ptr(), k_blk.data_ptr(), v_blk.data_ptr(), k_cache.data_ptr(),
        v_cache.data_ptr(), cache_len.data_ptr(), block_mask.data_ptr(), out.data_ptr(),
        lse.data_ptr() if lse is not None else None, ws.data_ptr(), ws.numel(), _stream_ptr(stream))
    _lib.check("orthrus_block_attn_masked", st)
    return out, lse


def orthrus_topk_logprobs(logits, m: int, logp=None, idx=None, workspace=None, stream=None):
    """Top-m logits per row and their log-probabilities.  logits fp32 [R, V].
    Returns (logp fp32 [R, m], idx int32 [R, m])."""
    R, V = logits.shape
    dev = logits.device
    _need(logits, "logits", torch.float32, (R, V))
    logp = torch.empty((R, m), dtype=torch.float32, device=dev) if logp is None else logp
    idx = torch.empty((R, m), dtype=torch.int32, device=dev) if idx is None else idx
    _need(logp, "logp", torch.float32, (R, m), dev)
    _need(idx, "idx", torch.int32, (R, m), dev)
    ws = _workspace(int(_lib.load().orthrus_topk_workspace_size(R, V, m)), dev, workspace)
    st = _lib.load().orthrus_topk_logprobs(R, V, m, logits.data_ptr(), logp.data_ptr(), idx.data_ptr(),
                                           ws.data_ptr(), ws.numel(), _stream_ptr(stream))
    _lib.check("orthrus_topk_logprobs", st)
    return logp, idx


def orthrus_tree_build(logp, tok, anchor, n_nodes: int, parent=None, tokens=None, depth=None, stream=None):
    """Best-first draft trees.  logp fp32 [B, Dd, m], tok int32 [B, Dd, m],
    anchor int32 [B].  Returns (parent, tokens, depth) int32 [B, n_nodes]."""
    B, Dd, m = logp.shape
    dev = logp.device
    _need(logp, "logp", torch.float32, (B, Dd, m))
    _need(tok, "tok", torch.int32, (B, Dd, m), dev)
    _need(anchor, "anchor", torch.int32, (B,), dev)
    mk = lambda t: torch.empty((B, n_nodes), dtype=torch.int32, device=dev) if t is None else t
    parent, tokens, depth = mk(parent), mk(tokens), mk(depth)
    for t, nm in ((parent, "parent"), (tokens, "tokens"), (depth, "depth")):
        _need(t, nm, torch.int32, (B, n_nodes), dev)
    st = _lib.load().orthrus_tree_build(B, Dd, m, n_nodes, logp.data_ptr(), tok.data_ptr(), anchor.data_ptr(),
                                        parent.data_ptr(), tokens.data_ptr(), depth.data_ptr(), _stream_ptr(stream))
    _lib.check("orthrus_tree_build", st)
    return parent, tokens, depth


def orthrus_tree_masks(parent, mask=None, stream=None):
    """Ancestor-or-self bitmasks (int64 [B, K]) of draft trees (parent int32 [B, K])."""
    B, K = parent.shape
    dev = parent.device
    _need(parent, "parent", torch.int32, (B, K))
    mask = torch.empty((B, K), dtype=torch.int64, device=dev) if mask is None else mask
    _need(mask, "mask", torch.int64, (B, K), dev)
    st = _lib.load().orthrus_tree_masks(B, K, parent.data_ptr(), mask.data_ptr(), _stream_ptr(stream))
    _lib.check("orthrus_tree_masks", st)
    return mask


def orthrus_consensus_tree_greedy(logits, tokens, parent, accept_len=None, path=None, correction=None,
                                  row_argmax=None, workspace=None, want_row_argmax: bool = False, stream=None):
    """Greedy consensus along draft trees.  Returns (accept_len [B], path [B, K],
    correction [B], row_argmax [B, K] or None), int32."""
    B, K, V = logits.shape
    dev = logits.device
    _need(logits, "logits", torch.float32, (B, K, V))
    _need(tokens, "tokens", torch.int32, (B, K), dev)
    _need(parent, "parent", torch.int32, (B, K), dev)
    i32 = dict(dtype=torch.int32, device=dev)
    accept_len = torch.empty(B, **i32) if accept_len is None else accept_len
    path = torch.empty((B, K), **i32) if path is None else path
    correction = torch.empty(B, **i32) if correction is None else correction
    if row_argmax is None and want_row_argmax:
        row_argmax = torch.empty((B, K), **i32)
    ws = _workspace(orthrus_consensus_workspace_size(B, K, V), dev, workspace)
    st = _lib.load().orthrus_consensus_tree_greedy(
        B, K, V, logits.data_ptr(), tokens.data_ptr(), parent.data_ptr(), accept_len.data_ptr(), path.data_ptr(),
        correction.data_ptr(), row_argmax.data_ptr() if row_argmax is not None else None, ws.data_ptr(),
        ws.numel(), _stream_ptr(stream))
    _lib.check("orthrus_consensus_tree_greedy", st)
    return accept_len, path, correction, row_argmax


def orthrus_cache_commit_path(k_cache, v_cache, k_blk, v_blk, cache_len, accept_len, path, node_tokens,
                              correction, next_anchor=None, tokens=None, n_tokens=None, stream=None):
    """Commit accepted tree paths (caches and cache_len updated in place).
    Returns (next_anchor [B], tokens [B, K], n_tokens [B])."""
    desc = _check_commit(k_cache, v_cache, k_blk, v_blk, cache_len, accept_len, correction, node_tokens)
    B, K, dev = desc.batch, desc.block_k, k_cache.device
    _need(path, "path", torch.int32, (B, K), dev)
    i32 = dict(dtype=torch.int32, device=dev)
    next_anchor = torch.empty(B, **i32) if next_anchor is None else next_anchor
    tokens = torch.empty((B, K), **i32) if tokens is None else tokens
    n_tokens = torch.empty(B, **i32) if n_tokens is None else n_tokens
    st = _lib.load().orthrus_cache_commit_path(
        ctypes.byref(desc), k_cache.data_ptr(), v_cache.data_ptr(), k_blk.data_ptr(), v_blk.data_ptr(),
        cache_len.data_ptr(), accept_len.data_ptr(), path.data_ptr(), node_tokens.data_ptr(), correction.data_ptr(),
        next_anchor.data_ptr(), tokens.data_ptr(), n_tokens.data_ptr(), _stream_ptr(stream))
    _lib.check("orthrus_cache_commit_path", st)
    return next_anchor, tokens, n_tokens
