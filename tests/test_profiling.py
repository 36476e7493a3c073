"""CPU checks of the profile post-processing that bench.py's `traffic` field
and the committed summaries come from: counter scaling by a copy of known
size, the source-hash guard that turns a stale record into null, and the
parity table."""
import csv
import json
import os
import types

import pytest

from mixture_experts_ffn_gemv_amd import profiling as P


def _write_counters(d, rows):
    """rows: (kernel name, counter name, value) -> one rocprofv3 counter CSV."""
    os.makedirs(os.path.join(d, "host"), exist_ok=True)
    with open(os.path.join(d, "host", "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Kernel_Name", "Counter_Name", "Counter_Value"])
        for r in rows:
            w.writerow(r)


def test_traffic_is_scaled_by_the_copy_and_keyed_to_the_sources(tmp_path, monkeypatch):
    fetch, write = str(tmp_path / "f"), str(tmp_path / "w")
    # a 1 MiB copy reads as 2048 KiB fetched and 1024 KiB written
    _write_counters(fetch, [("__amd_rocclr_copyBuffer", "FETCH_SIZE", 2048.0),
                            ("void moe::k_gemm_dma<0, 0, 64, 3>(moe::GemmParams)", "FETCH_SIZE", 300.0),
                            ("void moe::k_gemm_dma<0, 0, 64, 3>(moe::GemmParams)", "FETCH_SIZE", 500.0)])
    _write_counters(write, [("__amd_rocclr_copyBuffer", "WRITE_SIZE", 1024.0),
                            ("void moe::k_gemm_dma<0, 0, 64, 3>(moe::GemmParams)", "WRITE_SIZE", 64.0)])
    out = str(tmp_path / "traffic.json")
    a = types.SimpleNamespace(fetch=fetch, write=write, workload="w", copy_mib=1,
                              kernel=["gemm_gateup=k_gemm_dma<0"], out=out)
    P.cmd_traffic(a)
    rec = json.load(open(out))
    k = rec["kernels"]["w"]["gemm_gateup"]
    assert k["fetch_kib"] == 400.0 and k["write_kib"] == 64.0
    assert k["fetch_bytes"] == pytest.approx(400.0 * 1024 * 0.5)  # 1024 KiB known / 2048 read
    assert k["write_bytes"] == pytest.approx(64.0 * 1024 * 1.0)
    assert k["source_sha256"] == P.kernel_source_sha("gemm_gateup")
    monkeypatch.setattr(P, "TRAFFIC_JSON", out)
    assert P.recorded_traffic("w", "gemm_gateup") == pytest.approx(400.0 * 512 + 64.0 * 1024)
    assert P.recorded_traffic("w", "gemm_down") is None
    assert P.recorded_traffic("other", "gemm_gateup") is None
    # a record taken on other sources is stale: null, not a number
    rec["kernels"]["w"]["gemm_gateup"]["source_sha256"] = "0" * 64
    json.dump(rec, open(out, "w"))
    assert P.recorded_traffic("w", "gemm_gateup") is None


def test_source_hash_follows_the_named_files_only():
    h = P.kernel_source_sha("wsum_backward")
    assert h == P.kernel_source_sha("wsum_backward")
    assert h != P.kernel_source_sha("gemm_gateup")  # different file lists
    assert len(h) == 64


def test_parity_table_orders_by_error_over_tolerance(tmp_path, capsys):
    log = tmp_path / "p.jsonl"
    rows = [{"case": "a", "T": 4, "tokens": 4, "out_err": 1e-5, "w_err": 0.0, "tol": 1e-4},
            {"case": "b", "T": 1, "tokens": 1, "out_err": 4e-3, "w_err": 1e-7, "tol": 2e-2},
            {"case": "c", "T": 32, "tokens": 32, "out_err": 6e-7, "w_err": None, "tol": 3e-2}]
    log.write_text("\n".join(json.dumps(r) for r in rows) + "\n")
    P.cmd_parity(types.SimpleNamespace(log=str(log)))
    out = capsys.readouterr().out.splitlines()
    assert out[0].startswith("3 comparisons, 3 cases; largest error / tolerance 0.2")
    body = [l for l in out if l.startswith("| ") and not l.startswith("| case")]
    assert [l.split("|")[1].strip() for l in body] == ["b", "a", "c"]
