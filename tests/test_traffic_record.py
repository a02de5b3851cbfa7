"""The HBM-traffic record that bench.py reports as roofline.traffic: its sums
are consistent with the per-dispatch counter readings it holds, its
algorithmic bytes are those of the workload it names, and bench.py drops it
(reports null) once the decode sources differ from the ones it was taken on."""
import json

import bench
import workloads as W


def _record():
    with open(bench.TRAFFIC_FILE) as f:
        return json.load(f)


def test_record_sums_follow_its_counter_readings():
    rec = _record()
    copy_bytes = rec["scale"]["copy_kernel_bytes_each_way"]
    fk, wk = rec["fetch_size_kib_per_dispatch"], rec["write_size_kib_per_dispatch"]
    f_scale = copy_bytes / 1024 / fk["stream_copy_kernel"]
    w_scale = copy_bytes / 1024 / wk["stream_copy_kernel"]
    assert abs(f_scale - rec["scale"]["fetch"]) < 1e-4 and abs(w_scale - rec["scale"]["write"]) < 1e-4
    fetch = sum(v for k, v in fk.items() if k != "stream_copy_kernel") * 1024 * f_scale
    write = sum(v for k, v in wk.items() if k != "stream_copy_kernel") * 1024 * w_scale
    assert abs(fetch - rec["fetch_bytes_per_call"]) < 1e-6 * fetch
    assert abs(write - rec["write_bytes_per_call"]) < 1e-6 * write + 1
    assert rec["hbm_bytes_per_call"] == rec["fetch_bytes_per_call"] + rec["write_bytes_per_call"]
    # every KV byte is read at least once; more than a few percent over would be re-reads
    assert 1.0 <= rec["hbm_bytes_per_call"] / rec["algorithmic_bytes_per_call"] < 1.05


def test_record_names_the_default_workload():
    rec = _record()
    w = W.llama8b_decode()
    assert rec["workload"] == w.name
    assert rec["algorithmic_bytes_per_call"] == w.kv_bytes()
    assert rec["call"] == "pa_decode_append"


def test_bench_drops_a_record_taken_on_other_sources(monkeypatch):
    rec = _record()
    monkeypatch.setattr(bench, "decode_sources_sha256", lambda: rec["source_sha256"])
    assert bench.recorded_traffic(rec["workload"], rec["call"]) == rec["hbm_bytes_per_call"]
    assert bench.recorded_traffic(rec["workload"], "pa_decode") is None
    assert bench.recorded_traffic("cb_mix_b256_gqa8", rec["call"]) is None
    monkeypatch.setattr(bench, "decode_sources_sha256", lambda: "0" * 64)
    assert bench.recorded_traffic(rec["workload"], rec["call"]) is None
