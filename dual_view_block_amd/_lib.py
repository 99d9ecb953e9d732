"""ctypes binding of liborthrus.so (the C ABI in include/orthrus.h).

Argument marshalling only: every step of the decode path runs in the HIP
kernels behind the C ABI.  torch supplies device memory (``data_ptr``) and the
current HIP stream; nothing here computes on tensor values, and there is no
CPU fallback -- if the library is missing, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# ORTHRUS_LIBRARY names another build of the same library (for instance the
# host-sanitised one that dual_view_block_amd.build makes for the CPU tests)
LIB_PATH = os.environ.get("ORTHRUS_LIBRARY") or os.path.join(HERE, "liborthrus.so")

ORTHRUS_OK = 0
ORTHRUS_ERR_NULL_PTR = 1
ORTHRUS_ERR_BAD_SHAPE = 2
ORTHRUS_ERR_UNSUPPORTED = 3
ORTHRUS_ERR_MISALIGNED = 4
ORTHRUS_ERR_WORKSPACE_TOO_SMALL = 5
ORTHRUS_ERR_HIP = 6
ORTHRUS_MASK_DIFF_BIDIR = 0
ORTHRUS_MASK_VERIFY_CAUSAL = 1
ORTHRUS_MASK_EXPLICIT = 2
ORTHRUS_DTYPE_F32 = 0
ORTHRUS_DTYPE_BF16 = 1

# every symbol include/orthrus.h declares
EXPORTS = (
    "orthrus_attn_workspace_size", "orthrus_attn_num_splits", "orthrus_block_attn",
    "orthrus_block_attn_diff", "orthrus_block_attn_verify", "orthrus_block_attn_partial",
    "orthrus_block_attn_merge", "orthrus_consensus_workspace_size",
    "orthrus_consensus_greedy", "orthrus_consensus_sample", "orthrus_cache_commit",
    "orthrus_kl_workspace_size", "orthrus_forward_kl", "orthrus_train_attn_fwd", "orthrus_train_attn_bwd",
    "orthrus_block_attn_masked", "orthrus_topk_workspace_size", "orthrus_topk_logprobs", "orthrus_tree_build",
    "orthrus_tree_masks", "orthrus_consensus_tree_greedy", "orthrus_cache_commit_path", "orthrus_status_string",
    "orthrus_block_attn_noalloc", "orthrus_block_attn_dyn", "orthrus_consensus_greedy_dyn",
    "orthrus_consensus_sample_dyn", "orthrus_cache_commit_dyn",
)
# bytes of the device scratch behind orthrus_block_attn_noalloc
ORTHRUS_NOALLOC_SCRATCH_BYTES = 32 << 20


class AttnDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_k", ctypes.c_int32),
        ("max_len", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
    ]


class CommitDesc(ctypes.Structure):
    _fields_ = [
        ("n_layers", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_k", ctypes.c_int32),
        ("max_len", ctypes.c_int32),
    ]


class TrainAttnDesc(ctypes.Structure):
    _fields_ = [
        ("seq_len", ctypes.c_int32),
        ("n_blocks", ctypes.c_int32),
        ("block_k", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
    ]


class OrthrusError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn} failed: {message}")
        self.status = status


_P = ctypes.c_void_p
_SZ = ctypes.c_size_t
_I32 = ctypes.c_int32
_DESC = ctypes.POINTER(AttnDesc)

_SIGS = {
    "orthrus_attn_workspace_size": (_SZ, [_DESC]),
    "orthrus_attn_num_splits": (_I32, [_DESC]),
    "orthrus_block_attn": (_I32, [_DESC, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "orthrus_block_attn_diff": (_I32, [_DESC, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "orthrus_block_attn_verify": (_I32, [_DESC, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "orthrus_block_attn_partial": (_I32, [_DESC, _I32, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "orthrus_block_attn_merge": (_I32, [_DESC, _P, _P, _P, _SZ, _P]),
    "orthrus_consensus_workspace_size": (_SZ, [_I32, _I32, _I32]),
    "orthrus_consensus_greedy": (_I32, [_I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "orthrus_consensus_sample": (_I32, [_I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "orthrus_cache_commit": (_I32, [ctypes.POINTER(CommitDesc), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                    _P, _P]),
    "orthrus_kl_workspace_size": (_SZ, [_I32, _I32, _I32]),
    "orthrus_forward_kl": (_I32, [_I32, _I32, _I32, _P, _P, _P, _P, ctypes.c_float, _P, _SZ, _P]),
    "orthrus_train_attn_fwd": (_I32, [ctypes.POINTER(TrainAttnDesc)] + [_P] * 12),
    "orthrus_train_attn_bwd": (_I32, [ctypes.POINTER(TrainAttnDesc)] + [_P] * 13),
    "orthrus_block_attn_masked": (_I32, [_DESC, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "orthrus_topk_workspace_size": (_SZ, [_I32, _I32, _I32]),
    "orthrus_topk_logprobs": (_I32, [_I32, _I32, _I32, _P, _P, _P, _P, _SZ, _P]),
    "orthrus_tree_build": (_I32, [_I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P]),
    "orthrus_tree_masks": (_I32, [_I32, _I32, _P, _P, _P]),
    "orthrus_consensus_tree_greedy": (_I32, [_I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "orthrus_cache_commit_path": (_I32, [ctypes.POINTER(CommitDesc)] + [_P] * 13),
    "orthrus_status_string": (ctypes.c_char_p, [_I32]),
    "orthrus_block_attn_noalloc": (_I32, [_DESC, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "orthrus_block_attn_dyn": (_I32, [_DESC, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "orthrus_consensus_greedy_dyn": (_I32, [_I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "orthrus_consensus_sample_dyn": (_I32, [_I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "orthrus_cache_commit_dyn": (_I32, [ctypes.POINTER(CommitDesc)] + [_P] * 13 + [_I32, _P]),
}

_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load liborthrus.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m dual_view_block_amd.build` "
                          "(there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().orthrus_status_string(int(status)).decode()


def check(fn: str, status: int) -> None:
    if status != ORTHRUS_OK:
        raise OrthrusError(fn, status, status_string(status))
