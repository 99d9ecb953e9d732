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

# calls that pass the host checks carry made-up device pointers: never where a GPU could run them
pytestmark = pytest.mark.nogpu

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
    32 MiB scratch is refused with ORTHRUS_ERR_UNSUPPORTED, and bad pointers,
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


# ---------------------------------------------------- randomized host checks ----
from hypothesis import given, settings, strategies as st  # noqa: E402

_I32 = st.one_of(st.integers(-3, 300), st.sampled_from([0, 1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 4096,
                                                         65535, 65536, 1 << 20, (1 << 31) - 1, -(1 << 31)]))


@settings(max_examples=300, deadline=None)
@given(batch=_I32, hq=_I32, hkv=_I32, d=st.sampled_from([0, 32, 64, 96, 128, 256, -64]), k=_I32,
       max_len=_I32, scale=st.sampled_from([0.0, 0.088, 1.0, -1.0, float("nan"), float("inf")]),
       mode=st.integers(-1, 3))
def test_attention_descriptors_at_random_never_launch_without_a_gpu(batch, hq, hkv, d, k, max_len, scale, mode):
    """Any descriptor: the size queries agree on which ones are accepted, an
    accepted one gets a split count in [1, 64] and a workspace that holds its
    split partials, and a call with valid-looking pointers and that workspace
    ends in a documented status -- ORTHRUS_ERR_HIP for an accepted one, as
    there is no GPU in this process -- without reaching a launch.  Under the
    host sanitizers (tests/test_abi_hostsan.py) this also checks the planning
    arithmetic for overflow and out-of-range reads."""
    lib = _lib.load()
    desc = _desc(batch=batch, n_q_heads=hq, n_kv_heads=hkv, head_dim=d, block_k=k, max_len=max_len,
                 softmax_scale=scale)
    ws = lib.orthrus_attn_workspace_size(ctypes.byref(desc))
    splits = lib.orthrus_attn_num_splits(ctypes.byref(desc))
    assert (ws == 0) == (splits == -1), (ws, splits)
    if ws:
        assert 1 <= splits <= 64
        rows = (hq // hkv) * k
        per_wg = 32 if rows <= 32 else (64 if rows <= 64 else 128)
        groups = batch * hkv * -(-rows // per_wg)
        assert ws >= groups * splits * per_wg * (8 + 2 * d)
    st_ = _attn_call(desc, mode, ws_bytes=max(ws, 16))
    documented = {_lib.ORTHRUS_ERR_NULL_PTR, _lib.ORTHRUS_ERR_BAD_SHAPE, _lib.ORTHRUS_ERR_UNSUPPORTED,
                  _lib.ORTHRUS_ERR_HIP, _lib.ORTHRUS_ERR_WORKSPACE_TOO_SMALL, _lib.ORTHRUS_ERR_MISALIGNED}
    assert st_ in documented, st_
    if ws and mode in (0, 1):
        assert st_ == _lib.ORTHRUS_ERR_HIP


@settings(max_examples=200, deadline=None)
@given(batch=_I32, k=_I32, vocab=_I32)
def test_consensus_sizes_at_random(batch, k, vocab):
    """Consensus workspace sizes for any (B, K, V): zero exactly for the
    shapes the header rules out (B < 1, K outside [1, 128], B K > 65535,
    V outside [1, 2^30]), and a valid call without a GPU ends in
    ORTHRUS_ERR_HIP before any launch.  Under the host sanitizers this found
    an int overflow in the sampler's plan at V = 2^31 - 1."""
    lib = _lib.load()
    ws = lib.orthrus_consensus_workspace_size(batch, k, vocab)
    ok = batch >= 1 and 1 <= k <= 128 and batch * k <= 65535 and 1 <= vocab <= 1 << 30
    assert (ws > 0) == ok, (batch, k, vocab, ws)
    if ok:
        st_ = lib.orthrus_consensus_greedy(batch, k, vocab, 4096, 4096, 4096, None, 4096, 4096, ws, None)
        assert st_ == _lib.ORTHRUS_ERR_HIP, st_


@settings(max_examples=200, deadline=None)
@given(rows=_I32, vocab=_I32, dtype=st.integers(-1, 3), m=_I32)
def test_kl_and_topk_sizes_at_random(rows, vocab, dtype, m):
    """Workspace queries of the forward KL and of the top-m marginals for any
    sizes: zero exactly outside the documented ranges (rows in [1, 65535], V in
    [1, 2^30], a known dtype; 1 <= m <= min(32, V))."""
    lib = _lib.load()
    kl_ok = 1 <= rows <= 65535 and 1 <= vocab <= 1 << 30 and dtype in (0, 1)
    assert (lib.orthrus_kl_workspace_size(rows, vocab, dtype) > 0) == kl_ok
    tk_ok = 1 <= rows <= 65535 and 1 <= vocab <= 1 << 30 and 1 <= m <= min(32, vocab)
    assert (lib.orthrus_topk_workspace_size(rows, vocab, m) > 0) == tk_ok


def test_extreme_sizes_are_refused_without_overflow():
    """Sizes at the ends of int32 (regressions: the host planning summed a
    length or a vocabulary with a tile or chunk size in int, and multiplied
    three commit dimensions in 64 bits, both past their range; under the host
    sanitizers (tests/test_abi_hostsan.py) an overflow fails this test)."""
    lib = _lib.load()
    big = (1 << 31) - 1
    for max_len in (big, (1 << 30) + 1):
        d = _desc(max_len=max_len)
        assert lib.orthrus_attn_workspace_size(ctypes.byref(d)) == 0
        assert lib.orthrus_attn_num_splits(ctypes.byref(d)) == -1
        assert _attn_call(d) == _lib.ORTHRUS_ERR_UNSUPPORTED
    assert lib.orthrus_attn_workspace_size(ctypes.byref(_desc(max_len=1 << 30))) > 0
    for v in (big, (1 << 30) + 1):
        assert lib.orthrus_consensus_workspace_size(1, 32, v) == 0
        assert lib.orthrus_kl_workspace_size(8, v, 1) == 0
        assert lib.orthrus_topk_workspace_size(8, v, 4) == 0
        assert lib.orthrus_consensus_greedy(1, 32, v, 4096, 4096, 4096, None, 4096, 4096, 1 << 40, None) == \
            _lib.ORTHRUS_ERR_UNSUPPORTED
    assert lib.orthrus_consensus_workspace_size(1, 32, 1 << 30) > 0
    p = [1 << 20] * 12
    for fields, expected in ((dict(n_layers=big, batch=big, n_kv_heads=big), _lib.ORTHRUS_ERR_BAD_SHAPE),
                             (dict(n_layers=65536, batch=65536, n_kv_heads=1), _lib.ORTHRUS_ERR_BAD_SHAPE),
                             (dict(max_len=big), _lib.ORTHRUS_ERR_UNSUPPORTED)):
        base = dict(n_layers=36, batch=1, n_kv_heads=8, head_dim=128, block_k=32, max_len=36864)
        base.update(fields)
        cd = _lib.CommitDesc(**base)
        assert lib.orthrus_cache_commit(ctypes.byref(cd), *p) == expected, fields
