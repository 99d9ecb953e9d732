"""CPU tests of the C ABI: the library loads, exports every declared symbol,
and rejects bad arguments with the documented status before touching HIP.
No compute call runs here (no GPU in this process)."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

import dual_view_block_amd as dvb
from dual_view_block_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "orthrus.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"\b(orthrus_[a-z0-9_]+)\s*\(", src)
    return sorted(set(names))


def test_header_declares_the_four_named_entry_points():
    names = _declared_functions()
    for n in ("orthrus_block_attn_diff", "orthrus_block_attn_verify", "orthrus_consensus_greedy",
              "orthrus_consensus_sample"):
        assert n in names
    assert sorted(_lib.EXPORTS) == names


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    for n in _declared_functions():
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True)
    if out.returncode == 0:
        exported = set(re.findall(r"\bT (orthrus_\w+)", out.stdout))
        assert exported == set(_declared_functions())


def test_status_strings():
    for code in range(7):
        s = dvb.orthrus_status_string(code)
        assert s.startswith("ORTHRUS_")
    assert "UNKNOWN" in dvb.orthrus_status_string(99)


def _desc(**kw):
    base = dict(batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128, block_k=32, max_len=32768,
                softmax_scale=0.0)
    base.update(kw)
    return _lib.AttnDesc(**base)


def test_workspace_query_depends_on_shapes_only():
    lib = _lib.load()
    ws = lib.orthrus_attn_workspace_size(ctypes.byref(_desc()))
    assert ws > 0
    # the same descriptor always gives the same size: there is no length input at all
    assert ws == lib.orthrus_attn_workspace_size(ctypes.byref(_desc()))
    assert lib.orthrus_attn_num_splits(ctypes.byref(_desc())) >= 1
    assert lib.orthrus_attn_workspace_size(ctypes.byref(_desc(head_dim=96))) == 0
    assert lib.orthrus_attn_num_splits(ctypes.byref(_desc(n_q_heads=30))) == -1
    assert lib.orthrus_consensus_workspace_size(1, 32, 151936) > 0
    assert lib.orthrus_consensus_workspace_size(1, 128, 151936) > 0
    assert lib.orthrus_consensus_workspace_size(1, 129, 151936) == 0


def _attn_call(desc, mode=0, ptrs=None, ws_bytes=1 << 30):
    lib = _lib.load()
    p = dict(q=4096, kb=4096, vb=4096, kc=4096, vc=4096, lens=4096, out=4096, lse=4096, ws=4096)
    p.update(ptrs or {})
    return lib.orthrus_block_attn(ctypes.byref(desc) if desc is not None else None, mode, p["q"], p["kb"],
                                  p["vb"], p["kc"], p["vc"], p["lens"], p["out"], p["lse"], p["ws"],
                                  ws_bytes, None)


@pytest.mark.parametrize("case,expected", [
    (dict(desc=None), _lib.ORTHRUS_ERR_NULL_PTR),
    (dict(desc=_desc(batch=0)), _lib.ORTHRUS_ERR_BAD_SHAPE),
    (dict(desc=_desc(n_q_heads=30)), _lib.ORTHRUS_ERR_BAD_SHAPE),
    (dict(desc=_desc(block_k=0)), _lib.ORTHRUS_ERR_BAD_SHAPE),
    (dict(desc=_desc(max_len=-1)), _lib.ORTHRUS_ERR_BAD_SHAPE),
    (dict(desc=_desc(softmax_scale=float("nan"))), _lib.ORTHRUS_ERR_BAD_SHAPE),
    (dict(desc=_desc(softmax_scale=-1.0)), _lib.ORTHRUS_ERR_BAD_SHAPE),
    (dict(desc=_desc(head_dim=96)), _lib.ORTHRUS_ERR_UNSUPPORTED),
    (dict(desc=_desc(block_k=129)), _lib.ORTHRUS_ERR_UNSUPPORTED),
    (dict(desc=_desc(), mode=3), _lib.ORTHRUS_ERR_BAD_SHAPE),
    (dict(desc=_desc(), mode=2), _lib.ORTHRUS_ERR_NULL_PTR),   # explicit masks need orthrus_block_attn_masked
    (dict(desc=_desc(), ptrs=dict(kc=None)), _lib.ORTHRUS_ERR_NULL_PTR),
    (dict(desc=_desc(), ptrs=dict(lens=None)), _lib.ORTHRUS_ERR_NULL_PTR),
    (dict(desc=_desc(), ptrs=dict(q=4104)), _lib.ORTHRUS_ERR_MISALIGNED),
    (dict(desc=_desc(), ptrs=dict(ws=4100)), _lib.ORTHRUS_ERR_MISALIGNED),
    (dict(desc=_desc(), ws_bytes=16), _lib.ORTHRUS_ERR_WORKSPACE_TOO_SMALL),
])
def test_attention_argument_checks(case, expected):
    assert _attn_call(case.get("desc"), case.get("mode", 0), case.get("ptrs"),
                      case.get("ws_bytes", 1 << 30)) == expected


def test_consensus_argument_checks():
    lib = _lib.load()
    P = 4096
    assert lib.orthrus_consensus_greedy(0, 4, 10, P, P, P, P, P, P, 1 << 20, None) == _lib.ORTHRUS_ERR_BAD_SHAPE
    assert lib.orthrus_consensus_greedy(1, 129, 10, P, P, P, P, P, P, 1 << 20, None) == _lib.ORTHRUS_ERR_UNSUPPORTED
    assert lib.orthrus_consensus_greedy(1, 4, 10, None, P, P, P, P, P, 1 << 20, None) == _lib.ORTHRUS_ERR_NULL_PTR
    assert lib.orthrus_consensus_greedy(1, 4, 10, P + 4, P, P, P, P, P, 1 << 20, None) == _lib.ORTHRUS_ERR_MISALIGNED
    assert lib.orthrus_consensus_greedy(1, 4, 10, P, P, P, P, P, P, 1, None) == _lib.ORTHRUS_ERR_WORKSPACE_TOO_SMALL
    assert lib.orthrus_consensus_sample(1, 4, 10, P, P, P, None, P, P, P, 1 << 20, None) == _lib.ORTHRUS_ERR_NULL_PTR
    assert lib.orthrus_consensus_sample(1, 4, 0, P, P, P, P, P, P, P, 1 << 20, None) == _lib.ORTHRUS_ERR_BAD_SHAPE


def _commit(desc, **ptrs):
    lib = _lib.load()
    p = dict(kc=1 << 40, vc=2 << 40, kb=3 << 40, vb=4 << 40, lens=4096, acc=8192, corr=12288, cand=16384,
             anchor=20480, toks=24576, ntok=28672)
    p.update(ptrs)
    return lib.orthrus_cache_commit(ctypes.byref(desc) if desc is not None else None, p["kc"], p["vc"],
                                    p["kb"], p["vb"], p["lens"], p["acc"], p["corr"], p["cand"],
                                    p["anchor"], p["toks"], p["ntok"], None)


def _cdesc(**kw):
    base = dict(n_layers=36, batch=1, n_kv_heads=8, head_dim=128, block_k=32, max_len=32768 + 64)
    base.update(kw)
    return _lib.CommitDesc(**base)


@pytest.mark.parametrize("desc,ptrs,expected", [
    (None, {}, _lib.ORTHRUS_ERR_NULL_PTR),
    (_cdesc(n_layers=0), {}, _lib.ORTHRUS_ERR_BAD_SHAPE),
    (_cdesc(batch=0), {}, _lib.ORTHRUS_ERR_BAD_SHAPE),
    (_cdesc(block_k=0), {}, _lib.ORTHRUS_ERR_BAD_SHAPE),
    (_cdesc(max_len=-1), {}, _lib.ORTHRUS_ERR_BAD_SHAPE),
    (_cdesc(head_dim=12), {}, _lib.ORTHRUS_ERR_UNSUPPORTED),
    (_cdesc(head_dim=2048), {}, _lib.ORTHRUS_ERR_UNSUPPORTED),
    (_cdesc(block_k=2000), {}, _lib.ORTHRUS_ERR_UNSUPPORTED),
    (_cdesc(n_layers=1 << 16, batch=1 << 16), {}, _lib.ORTHRUS_ERR_BAD_SHAPE),
    (_cdesc(), dict(kb=None), _lib.ORTHRUS_ERR_NULL_PTR),
    (_cdesc(), dict(ntok=None), _lib.ORTHRUS_ERR_NULL_PTR),
    (_cdesc(), dict(kc=(1 << 40) + 8), _lib.ORTHRUS_ERR_MISALIGNED),
    (_cdesc(), dict(lens=4098), _lib.ORTHRUS_ERR_MISALIGNED),
    # block rows inside the K cache, and K and V caches that overlap
    (_cdesc(), dict(kb=(1 << 40) + 4096), _lib.ORTHRUS_ERR_BAD_SHAPE),
    (_cdesc(), dict(vc=(1 << 40) + (1 << 20)), _lib.ORTHRUS_ERR_BAD_SHAPE),
])
def test_commit_argument_checks(desc, ptrs, expected):
    assert _commit(desc, **ptrs) == expected


def test_forward_kl_argument_checks():
    lib = _lib.load()
    P, Q, K, G, W = 1 << 40, 2 << 40, 4096, 3 << 40, 8192
    ok = lib.orthrus_kl_workspace_size(8192, 151936, _lib.ORTHRUS_DTYPE_BF16)
    assert ok > 0 and lib.orthrus_kl_workspace_size(8192, 151936, 7) == 0
    assert lib.orthrus_kl_workspace_size(70000, 10, _lib.ORTHRUS_DTYPE_F32) == 0
    f = lib.orthrus_forward_kl
    BF = _lib.ORTHRUS_DTYPE_BF16
    assert f(0, 10, BF, P, Q, K, G, 1.0, W, ok, None) == _lib.ORTHRUS_ERR_BAD_SHAPE
    assert f(4, 0, BF, P, Q, K, G, 1.0, W, ok, None) == _lib.ORTHRUS_ERR_BAD_SHAPE
    assert f(4, 10, 5, P, Q, K, G, 1.0, W, ok, None) == _lib.ORTHRUS_ERR_BAD_SHAPE
    assert f(70000, 10, BF, P, Q, K, G, 1.0, W, ok, None) == _lib.ORTHRUS_ERR_UNSUPPORTED
    assert f(4, 10, BF, None, Q, K, G, 1.0, W, ok, None) == _lib.ORTHRUS_ERR_NULL_PTR
    assert f(4, 10, BF, P, Q, None, G, 1.0, W, ok, None) == _lib.ORTHRUS_ERR_NULL_PTR
    assert f(4, 10, BF, P, Q, K, G, float("inf"), W, ok, None) == _lib.ORTHRUS_ERR_BAD_SHAPE
    assert f(4, 10, BF, P + 2, Q, K, G, 1.0, W, ok, None) == _lib.ORTHRUS_ERR_MISALIGNED
    assert f(4, 10, BF, P, Q, K, G + 8, 1.0, W, ok, None) == _lib.ORTHRUS_ERR_MISALIGNED
    assert f(8192, 151936, BF, P, Q, K, G, 1.0, W, ok - 1, None) == _lib.ORTHRUS_ERR_WORKSPACE_TOO_SMALL


def test_tree_argument_checks():
    lib = _lib.load()
    P, W = 4096, 8192
    desc = _lib.AttnDesc(1, 32, 8, 128, 65, 4096, 0.0)
    assert lib.orthrus_block_attn_masked(ctypes.byref(desc), P, P, P, P, P, P, P, P, P, W, 1 << 30, None) == \
        _lib.ORTHRUS_ERR_UNSUPPORTED                       # explicit masks: K <= 64
    desc = _lib.AttnDesc(1, 32, 8, 128, 32, 4096, 0.0)
    assert lib.orthrus_block_attn_masked(ctypes.byref(desc), P, P, P, P, P, P, None, P, P, W, 1 << 30, None) == \
        _lib.ORTHRUS_ERR_NULL_PTR
    assert lib.orthrus_tree_masks(1, 65, P, P, None) == _lib.ORTHRUS_ERR_UNSUPPORTED
    assert lib.orthrus_tree_masks(1, 8, P, P + 4, None) == _lib.ORTHRUS_ERR_MISALIGNED
    assert lib.orthrus_tree_masks(0, 8, P, P, None) == _lib.ORTHRUS_ERR_BAD_SHAPE
    assert lib.orthrus_topk_workspace_size(4, 100, 33) == 0 and lib.orthrus_topk_workspace_size(4, 10, 11) == 0
    assert lib.orthrus_topk_workspace_size(32, 151936, 8) > 0
    assert lib.orthrus_topk_logprobs(4, 10, 11, P, P, P, W, 1 << 20, None) == _lib.ORTHRUS_ERR_BAD_SHAPE
    assert lib.orthrus_topk_logprobs(4, 100, 33, P, P, P, W, 1 << 20, None) == _lib.ORTHRUS_ERR_UNSUPPORTED
    assert lib.orthrus_topk_logprobs(4, 100, 8, P, P, P, W, 1, None) == _lib.ORTHRUS_ERR_WORKSPACE_TOO_SMALL
    assert lib.orthrus_tree_build(1, 4, 2, 65, P, P, P, P, P, P, None) == _lib.ORTHRUS_ERR_UNSUPPORTED
    assert lib.orthrus_tree_build(1, 4, 2, 0, P, P, P, P, P, P, None) == _lib.ORTHRUS_ERR_BAD_SHAPE
    assert lib.orthrus_tree_build(1, 4, 2, 8, None, P, P, P, P, P, None) == _lib.ORTHRUS_ERR_NULL_PTR
    assert lib.orthrus_consensus_tree_greedy(1, 129, 10, P, P, P, P, P, P, P, W, 1 << 20, None) == \
        _lib.ORTHRUS_ERR_UNSUPPORTED
    assert lib.orthrus_consensus_tree_greedy(1, 8, 10, P, P, None, P, P, P, P, W, 1 << 20, None) == \
        _lib.ORTHRUS_ERR_NULL_PTR
    c = _lib.CommitDesc(1, 1, 1, 64, 4, 256)
    assert lib.orthrus_cache_commit_path(ctypes.byref(c), 1 << 40, 2 << 40, 3 << 40, 4 << 40, P, P, None, P, P, P,
                                         P, P, None) == _lib.ORTHRUS_ERR_NULL_PTR
    assert lib.orthrus_cache_commit_path(ctypes.byref(c), 1 << 40, 1 << 40, 3 << 40, 4 << 40, P, P, P, P, P, P,
                                         P, P, None) == _lib.ORTHRUS_ERR_BAD_SHAPE


def test_valid_call_without_gpu_reports_hip_error():
    """Run in a child process: a well-formed call on a host with no GPU must
    come back as ORTHRUS_ERR_HIP (validation passed, the launch was refused)."""
    code = (
        "import ctypes, sys; sys.path.insert(0, %r)\n"
        "from dual_view_block_amd import _lib\n"
        "lib = _lib.load()\n"
        "d = _lib.AttnDesc(1, 2, 1, 64, 4, 256, 0.0)\n"
        "P = 4096\n"
        "print(lib.orthrus_block_attn(ctypes.byref(d), 0, P, P, P, P, P, P, P, P, P, 1 << 30, None))\n"
        "c = _lib.CommitDesc(1, 1, 1, 64, 4, 256)\n"
        "print(lib.orthrus_cache_commit(ctypes.byref(c), 1 << 40, 2 << 40, 3 << 40, 4 << 40, P, P, P, P, P, P, "
        "P, None))\n"
        "print(lib.orthrus_block_attn_dyn(ctypes.byref(d), 1, P, P, P, P, P, P, P, P, P, P, 1 << 30, None))\n"
        "print(lib.orthrus_cache_commit_dyn(ctypes.byref(c), 1 << 40, 2 << 40, 3 << 40, 4 << 40, P, P, P, P, P, "
        "P, P, P, P, 2, None))\n"
    ) % ROOT
    env = dict(os.environ, HIP_VISIBLE_DEVICES="")
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120, env=env)
    assert res.returncode == 0, res.stderr
    assert [int(x) for x in res.stdout.strip().splitlines()[-4:]] == [_lib.ORTHRUS_ERR_HIP] * 4


def test_product_path_never_touches_the_oracle():
    pkg = os.path.join(ROOT, "dual_view_block_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in src.lower(), f


def test_noalloc_entry_point_rejects_before_any_hip_call():
    """orthrus_block_attn_noalloc: a descriptor whose workspace exceeds the
    16 MiB scratch is refused with ORTHRUS_ERR_UNSUPPORTED, and bad pointers,
    alignment and modes are refused as in orthrus_block_attn -- all on the host."""
    lib = _lib.load()

    def call(desc, mode=0, **ptrs):
        p = dict(q=4096, kb=4096, vb=4096, kc=4096, vc=4096, lens=4096, out=4096, lse=4096)
        p.update(ptrs)
        return lib.orthrus_block_attn_noalloc(ctypes.byref(desc), mode, p["q"], p["kb"], p["vb"], p["kc"],
                                              p["vc"], p["lens"], p["out"], p["lse"], None)

    big = _desc(batch=256)  # 2048 groups of 128 rows: ~69 MB of split partials
    assert lib.orthrus_attn_workspace_size(ctypes.byref(big)) > _lib.ORTHRUS_NOALLOC_SCRATCH_BYTES
    assert call(big) == _lib.ORTHRUS_ERR_UNSUPPORTED
    assert lib.orthrus_attn_workspace_size(ctypes.byref(_desc())) <= _lib.ORTHRUS_NOALLOC_SCRATCH_BYTES
    assert call(_desc(), mode=_lib.ORTHRUS_MASK_EXPLICIT) == _lib.ORTHRUS_ERR_BAD_SHAPE
    assert call(_desc(), q=None) == _lib.ORTHRUS_ERR_NULL_PTR
    assert call(_desc(), out=None) == _lib.ORTHRUS_ERR_NULL_PTR
    assert call(_desc(), kc=4104) == _lib.ORTHRUS_ERR_MISALIGNED
    assert call(_desc(head_dim=96)) == _lib.ORTHRUS_ERR_UNSUPPORTED


def test_dynamic_block_entry_points_check_arguments_on_the_host():
    """The per-sequence block-length variants need their length array and the
    mode masks; the commit's floor must lie in [1, K]; the rest is checked as
    in the fixed-length calls."""
    lib = _lib.load()
    P = 4096
    d = _desc()

    def attn(mode=0, blk=P, **ptrs):
        p = dict(q=P, kb=P, vb=P, kc=P, vc=P, lens=P, out=P, lse=P, ws=P)
        p.update(ptrs)
        return lib.orthrus_block_attn_dyn(ctypes.byref(d), mode, p["q"], p["kb"], p["vb"], p["kc"], p["vc"],
                                          p["lens"], blk, p["out"], p["lse"], p["ws"], 1 << 30, None)

    assert attn(blk=None) == _lib.ORTHRUS_ERR_NULL_PTR
    assert attn(mode=_lib.ORTHRUS_MASK_EXPLICIT) == _lib.ORTHRUS_ERR_BAD_SHAPE
    assert attn(blk=P + 2) == _lib.ORTHRUS_ERR_MISALIGNED
    assert attn(q=None) == _lib.ORTHRUS_ERR_NULL_PTR
    assert lib.orthrus_consensus_greedy_dyn(1, 4, 10, P, P, None, P, P, P, P, 1 << 20, None) == \
        _lib.ORTHRUS_ERR_NULL_PTR
    assert lib.orthrus_consensus_greedy_dyn(1, 4, 10, P, P, P + 2, P, P, P, P, 1 << 20, None) == \
        _lib.ORTHRUS_ERR_MISALIGNED
    assert lib.orthrus_consensus_greedy_dyn(1, 129, 10, P, P, P, P, P, P, P, 1 << 20, None) == \
        _lib.ORTHRUS_ERR_UNSUPPORTED
    assert lib.orthrus_consensus_sample_dyn(1, 4, 10, P, P, P, P, None, P, P, P, 1 << 20, None) == \
        _lib.ORTHRUS_ERR_NULL_PTR
    assert lib.orthrus_consensus_sample_dyn(1, 4, 10, P, P, P, P, P, P, P, P, 1, None) == \
        _lib.ORTHRUS_ERR_WORKSPACE_TOO_SMALL
    c = _cdesc()

    def commit(blk=P, stat=P, k_min=1):
        return lib.orthrus_cache_commit_dyn(ctypes.byref(c), 1 << 40, 2 << 40, 3 << 40, 4 << 40, P, P, P, P, P,
                                            P, P, blk, stat, k_min, None)

    assert commit(blk=None) == _lib.ORTHRUS_ERR_NULL_PTR
    assert commit(stat=None) == _lib.ORTHRUS_ERR_NULL_PTR
    assert commit(stat=P + 1) == _lib.ORTHRUS_ERR_MISALIGNED
    assert commit(k_min=0) == _lib.ORTHRUS_ERR_BAD_SHAPE
    assert commit(k_min=33) == _lib.ORTHRUS_ERR_BAD_SHAPE
    assert commit(blk=P + 2) == _lib.ORTHRUS_ERR_MISALIGNED
