"""Host logic of bench.py (no GPU): the algorithmic byte and flop counts it
divides by, the HBM-traffic record built from counter CSVs, the code
fingerprint that voids a stale record, and the refusal of more than one GPU.

Expected values are closed forms written out here from the shapes, not
re-calls of bench.py's own helpers."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from synth import WORKLOADS  # noqa: E402

W = WORKLOADS["qwen3_8b_32k"]  # 36 layers, Hq 32, Hkv 8, D 128, L 32768, K 32, V 151936


def test_layer_view_bytes_at_the_benchmark_shape():
    # cache K+V rows [0, L) of 8 KV heads, q, k/v block, out (bf16)
    cache = 2 * 8 * 32768 * 128 * 2
    q = 32 * 32 * 128 * 2
    blk = 2 * 8 * 32 * 128 * 2
    assert bench.stream_bytes(W) == cache + q + blk == 134_610_944
    assert bench.attn_bytes(W) == cache + 2 * q + blk == 134_873_088


def test_step_bytes():
    logits = 32 * (151936 * 4 + 4)  # fp32 logits + candidates
    outs = 4 + 4 + 32 * 4           # accept_len, correction, row_argmax
    assert bench.greedy_bytes(W) == logits + outs
    assert 72 * 134_873_088 + logits + outs == 9_730_310_408
    # the ragged-batch form reduces to the uniform one when every length is L
    assert bench.step_bytes_lens(W, W.batch * W.cache_len) == 9_730_310_408
    w16 = W.replace(batch=16)
    assert (bench.step_bytes_lens(w16, 16 * 32768)
            == 72 * 16 * 134_873_088 + bench.greedy_bytes(w16))


@pytest.mark.parametrize("causal", [False, True])
def test_layer_view_flops(causal):
    # 2 products (QK^T, PV) x 2 flops per multiply-add over the visible keys:
    # every row sees L cache keys plus all K block keys (diffusion) or, on
    # average, (K + 1) / 2 of them (verify)
    L, K = 32768, 32
    visible = 32 * K * (L + ((K + 1) / 2 if causal else K))
    assert bench.attn_flops(W, causal) == int(4 * 128 * visible)
    if not causal:
        assert round(bench.attn_flops(W, False) / 1e9, 2) == 17.20


def _counter_csv(path, rows):
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for r in rows:
            wr.writerow(r)


def test_traffic_record_scales_by_the_copy_kernel(tmp_path):
    k = "orthrus::(anonymous namespace)::attn_stream_kernel<128, 4, false>(...)"
    c = "__amd_rocclr_copyBuffer"
    _counter_csv(tmp_path / "f.csv", [{"Kernel_Name": k, "Counter_Name": "FETCH_SIZE", "Counter_Value": v}
                                      for v in (1000.0, 1200.0)])
    _counter_csv(tmp_path / "w.csv", [{"Kernel_Name": k, "Counter_Name": "WRITE_SIZE", "Counter_Value": 300.0}])
    _counter_csv(tmp_path / "cf.csv", [{"Kernel_Name": c, "Counter_Name": "FETCH_SIZE", "Counter_Value": 512.0}])
    _counter_csv(tmp_path / "cw.csv", [{"Kernel_Name": c, "Counter_Name": "WRITE_SIZE", "Counter_Value": 1024.0}])
    out = tmp_path / "traffic.json"
    bench.make_traffic([str(tmp_path / n) for n in ("f.csv", "w.csv", "cf.csv", "cw.csv")], str(out), copy_mib=1)
    rec = json.load(open(out))
    # a 1 MiB copy read as 512 KiB: 2048 true bytes per counted KiB; written as 1024 KiB: 1024
    assert rec["fetch_bytes_per_kib"] == 2048.0 and rec["write_bytes_per_kib"] == 1024.0
    assert rec["read_bytes_per_launch"] == 1100 * 2048        # mean of the two dispatches
    assert rec["write_bytes_per_launch"] == 300 * 1024
    assert rec["bytes_per_launch"] == 1100 * 2048 + 300 * 1024
    assert rec["code_sha256"] == bench._code_sha256(bench.ATTN_SOURCE)
    assert bench.load_traffic(str(out)) == rec["bytes_per_launch"]
    # a record taken with other code is reported as null
    rec["code_sha256"] = "0" * 64
    json.dump(rec, open(out, "w"))
    assert bench.load_traffic(str(out)) is None
    assert bench.load_traffic(str(tmp_path / "missing.json")) is None


def test_code_fingerprint_ignores_comments_and_whitespace(tmp_path):
    a, b, c = tmp_path / "a.hip", tmp_path / "b.hip", tmp_path / "c.hip"
    a.write_text("int f(int x) {\n  return x + 1;  // one\n}\n")
    b.write_text("/* header */ int f(int x) { return x + 1; }\n")
    c.write_text("int f(int x) { return x + 2; }\n")
    assert bench._code_sha256(str(a)) == bench._code_sha256(str(b))
    assert bench._code_sha256(str(a)) != bench._code_sha256(str(c))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_trace_summary_phases(tmp_path, capsys):
    """--summarize-trace with --trace-phases: the streaming kernel's dispatches
    a..b-1 of its most frequent launch shape, in launch order, summarised per
    phase (values written out here: durations 10, 20, ... µs)."""
    import sqlite3

    db = tmp_path / "t.db"
    con = sqlite3.connect(db)
    con.execute("create table kernels (name text, start integer, end integer, grid_x integer, grid_y integer, "
                "grid_z integer, workgroup_x integer)")
    k = "void orthrus::(anonymous namespace)::attn_stream_kernel<128, 4, false, false>(orthrus::AttnArgs)"
    m = "void orthrus::(anonymous namespace)::attn_merge_kernel<128, 32>(orthrus::AttnArgs)"
    t = 0
    for i in range(6):  # stream dispatch i lasts 10 (i + 1) us, each followed by a merge of 1 us
        con.execute("insert into kernels values (?, ?, ?, 16384, 1, 8, 512)", (k, t, t + 10_000 * (i + 1)))
        t += 10_000 * (i + 1)
        con.execute("insert into kernels values (?, ?, ?, 65536, 1, 1, 256)", (m, t, t + 1_000))
        t += 1_000
    # one dispatch of another launch shape, which must not count
    con.execute("insert into kernels values (?, ?, ?, 1024, 1, 128, 512)", (k, t, t + 999_000))
    con.commit()
    con.close()
    bench.summarize_trace(str(db), "first=0:2,rest=2:6")
    out = capsys.readouterr().out
    assert "| first | 2 | 15.00 | 15.00 | 10.00 |" in out
    assert "| rest | 4 | 45.00 | 45.00 | 30.00 |" in out
    assert "(16384 × 1 × 8)" in out
