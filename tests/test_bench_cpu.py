"""Host logic of bench.py, without a GPU: the one-GPU guard, the rocprofv3 traffic
arithmetic (counter KiB scaled by a copy of known size), the source hash that ties
a profile to its kernel, and the traffic lookup that refuses a stale profile."""

import csv
import json
import os
import shutil
import subprocess
import sys

import numpy as np
import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _csv(path, rows):
    with open(path, "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(HDR)
        wr.writerows(rows)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=300)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_traffic_summary_scales_counters_by_the_copy(tmp_path):
    chunk = "void kvq::(anonymous namespace)::decode_chunk_kernel<1, 1, 128, 2, false>(kvq::Params)"
    red = "void kvq::(anonymous namespace)::decode_reduce_rows_kernel<128>(kvq::Params)"
    copy = "__amd_rocclr_copyBuffer"
    # FETCH_SIZE reads half the bytes moved, WRITE_SIZE all of them (in KiB), on the copy of 1 MiB
    _csv(tmp_path / "cf.csv", [[1, copy, "FETCH_SIZE", 512.0], [2, copy, "FETCH_SIZE", 512.0]])
    _csv(tmp_path / "cw.csv", [[1, copy, "WRITE_SIZE", 1024.0]])
    # two chunk dispatches of 100 and 300 KiB fetched, one reduce of 10; writes 4 and 2
    _csv(tmp_path / "f.csv", [[5, chunk, "FETCH_SIZE", 100.0], [6, chunk, "FETCH_SIZE", 300.0],
                              [7, red, "FETCH_SIZE", 10.0]])
    _csv(tmp_path / "w.csv", [[5, chunk, "WRITE_SIZE", 4.0], [7, red, "WRITE_SIZE", 2.0]])
    out = tmp_path / "traffic.txt"
    bench.traffic_summary("tiny_int8", str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(tmp_path / "cf.csv"),
                          str(tmp_path / "cw.csv"), str(1 << 20), str(out), "cmd")
    vals = dict(l.split(": ", 1) for l in out.read_text().splitlines() if ": " in l)
    assert float(vals["fetch_scale (copy bytes / copy FETCH_SIZE bytes)"]) == pytest.approx(2.0)
    assert float(vals["write_scale (copy bytes / copy WRITE_SIZE bytes)"]) == pytest.approx(1.0)
    # per call: (mean chunk 200 + reduce 10) KiB x 2 fetched, (4 + 2) KiB written
    assert float(vals["hbm_bytes_per_launch"]) == pytest.approx((210 * 2 + 6) * 1024)
    assert vals["kernel_source_hash"] == bench.decode_source_hash()
    # tiny_int8: sequences of 17 and 33 tokens, 4 KV heads, 2 x 64 bytes per token-head
    assert int(vals["algorithmic_kv_bytes"]) == (17 + 33) * 4 * 128
    assert float(vals["traffic_over_algorithmic"]) == pytest.approx((210 * 2 + 6) * 1024 / ((17 + 33) * 4 * 128),
                                                                     rel=1e-4)


def test_source_hash_ignores_comments_only(tmp_path, monkeypatch):
    src = os.path.join(ROOT, "quantized_paged_kv_absmax_amd", "csrc")
    dst = tmp_path / "quantized_paged_kv_absmax_amd" / "csrc"
    dst.mkdir(parents=True)
    for f in ("decode_kernel.h", "decode.hip", "kvq_device.h", "kvq_rows.h"):
        shutil.copy(os.path.join(src, f), dst / f)
    h_repo = bench.decode_source_hash()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.decode_source_hash()
    assert h0 == h_repo                      # the same sources
    k = dst / "decode_kernel.h"
    k.write_text(k.read_text() + "\n// a new comment\n/* and a block\n comment */\n")
    assert bench.decode_source_hash() == h0
    k.write_text(k.read_text() + "\nnamespace kvq { constexpr int kAnotherConstant = 1; }\n")
    assert bench.decode_source_hash() != h0


def test_stale_traffic_profile_is_not_reported(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "decode_llama8b_int8_traffic.txt").write_text("kernel_source_hash: abc\nhbm_bytes_per_launch: 123\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.read_traffic("llama8b_int8", "abc") == 123.0
    assert bench.read_traffic("llama8b_int8", "def") is None
    assert bench.read_traffic("fp8_e4m3", "abc") is None


def test_oracle_write_rates_cover_the_three_write_side_steps():
    from workloads import WORKLOADS, make_decode_inputs
    w = WORKLOADS["llama8b_int8"]
    inp = make_decode_inputs(w)
    r = bench.oracle_write_rates(w, inp, n_tok=512)
    assert r["tokens"] == 512
    for k in ("calibrate_gbs", "write_int8_gbs", "convert_int4_gbs"):
        assert r[k] > 0


def test_page_list_is_the_decode_order():
    # every page of every non-empty sequence, sequence by sequence
    class Inp:
        seq_lens = np.array([17, 0, 16, 1], np.int32)
        block_tables = np.array([[5, 6, 9], [1, 2, 3], [7, 8, 0], [4, 0, 0]], np.int32)
    assert bench.page_list(Inp).tolist() == [5, 6, 7, 4]


def test_read_probe_library_loads_and_checks_arguments():
    # the probe's host-side checks return hipErrorInvalidValue (1) before any launch
    f = bench._probe_fn()
    P = 1 << 20
    assert f(None, P, None, None, P, 10, 8, 2048, 256, 100, P, None) == 1       # no K pages
    assert f(P, P, None, None, P, 0, 8, 2048, 256, 100, P, None) == 1           # no pages to read
    assert f(P, P, None, None, P, 10, 8, 8192, 256, 100, P, None) == 1          # pages over 4 KB
    assert f(P, P, None, None, P, 10, 8, 2050, 256, 100, P, None) == 1          # not a multiple of 16 bytes
