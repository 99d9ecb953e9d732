"""The C ABI driven from a C++ program with no Python in the call path.

`tests/c/decode_step` (built from `tests/c/decode_step.cpp` by
`tests/c/build_example.py`, which `__graft_entry__.build()` runs) loads
liborthrus.so through the linker, runs the diffusion-view and the verify
block attention over one shared cache and the greedy consensus, and writes
the results to files.  Without a GPU it prints the host-side workspace sizes
and exits with status 2; the CPU test checks those sizes against the
library's own answer through the Python binding.  The GPU test compares every
result with the fp64 oracle: attention within max-abs 2e-2, relative L2
5e-3 and lse 1e-3, consensus bit-exact.
"""
import os
import subprocess

import numpy as np
import pytest
import torch

import dual_view_block_amd as dvb
from synth import Workload, attention_inputs, greedy_inputs, view_inputs

HERE = os.path.dirname(os.path.abspath(__file__))
BIN = os.path.join(HERE, "c", "decode_step")
W = Workload("c_abi", 1, 3, 8, 2, 128, 700, 16, 3000, 3.0, 91, max_len=800)
LENS = [700, 0, 129]


def _binary() -> str:
    if not os.path.exists(BIN):
        import importlib.util
        spec = importlib.util.spec_from_file_location("build_example", os.path.join(HERE, "c", "build_example.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    return BIN


def _meta(d):
    with open(os.path.join(d, "meta.txt"), "w") as f:
        f.write(f"{W.batch} {W.n_q_heads} {W.n_kv_heads} {W.head_dim} {W.block_k} {W.capacity} {W.vocab}\n")
        f.write(" ".join(str(v) for v in LENS) + "\n")


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="checks the no-GPU path")
def test_c_program_links_and_reports_sizes_without_a_gpu(tmp_path):
    _meta(tmp_path)
    r = subprocess.run([_binary(), str(tmp_path)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 2, (r.returncode, r.stdout, r.stderr)
    sizes = dict(line.split() for line in r.stdout.splitlines() if line.endswith(tuple("0123456789")))
    q = torch.empty((W.batch, W.n_q_heads, W.block_k, W.head_dim), dtype=torch.bfloat16)
    kc = torch.empty((W.batch, W.n_kv_heads, W.capacity, W.head_dim), dtype=torch.bfloat16)
    assert int(sizes["attn_workspace_bytes"]) == dvb.orthrus_attn_workspace_size(dvb.attn_desc(q, kc))
    assert int(sizes["consensus_workspace_bytes"]) == dvb.orthrus_consensus_workspace_size(
        W.batch, W.block_k, W.vocab)
    assert "no GPU" in r.stdout


def _bits(t: torch.Tensor) -> bytes:
    return t.contiguous().view(torch.int16).numpy().tobytes()


@pytest.mark.gpu
def test_c_program_decode_step_matches_oracle(tmp_path):
    import oracle

    _meta(tmp_path)
    x = attention_inputs(W)
    x["cache_len"] = torch.tensor(LENS, dtype=torch.int32)
    views = {v: view_inputs(W, 0, v) for v in ("diff", "verify")}
    logits, cand, j_star = greedy_inputs(W, first_mismatch=torch.tensor([5, 0, 16]))
    files = {"q_diff.bin": _bits(views["diff"][0]), "q_verify.bin": _bits(views["verify"][0]),
             "k_blk_diff.bin": _bits(views["diff"][1]), "v_blk_diff.bin": _bits(views["diff"][2]),
             "k_blk_verify.bin": _bits(views["verify"][1]), "v_blk_verify.bin": _bits(views["verify"][2]),
             "k_cache.bin": _bits(x["k_cache"]), "v_cache.bin": _bits(x["v_cache"]),
             "logits.bin": logits.float().contiguous().numpy().tobytes(),
             "cand.bin": cand.to(torch.int32).contiguous().numpy().tobytes()}
    for name, data in files.items():
        (tmp_path / name).write_bytes(data)
    print(f"c_abi: B {W.batch} Hq {W.n_q_heads} Hkv {W.n_kv_heads} D {W.head_dim} K {W.block_k} lens {LENS}",
          flush=True)
    r = subprocess.run([_binary(), str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)

    def arr(name, dtype, shape):
        return np.frombuffer((tmp_path / name).read_bytes(), dtype=dtype).reshape(shape)

    qshape = (W.batch, W.n_q_heads, W.block_k, W.head_dim)
    for view, mode in (("diff", oracle.MASK_DIFF_BIDIR), ("verify", oracle.MASK_VERIFY_CAUSAL)):
        q, kb, vb = views[view]
        ref, ref_lse = oracle.block_attention(q, kb, vb, x["k_cache"], x["v_cache"], x["cache_len"], mode)
        out = torch.from_numpy(arr(f"out_{view}.bin", np.int16, qshape).copy()).view(torch.bfloat16).double()
        got = out.numpy()
        max_abs = float(np.abs(got - ref).max())
        rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
        lse_err = float(np.abs(arr(f"lse_{view}.bin", np.float32, qshape[:3]).astype(np.float64) - ref_lse).max())
        print(f"c_abi {view}: max_abs={max_abs:.2e} rel_l2={rel:.2e} lse={lse_err:.2e}", flush=True)
        assert max_abs <= 2e-2 and rel <= 5e-3 and lse_err <= 1e-3, view
    acc, am, corr = oracle.greedy_consensus(logits, cand)
    assert np.array_equal(arr("accept_len.bin", np.int32, (W.batch,)), acc)
    assert np.array_equal(arr("correction.bin", np.int32, (W.batch,)), corr)
    assert np.array_equal(arr("row_argmax.bin", np.int32, (W.batch, W.block_k)), am)
    assert acc.tolist() == j_star.tolist()
