"""The HBM-traffic records that bench.py reports as roofline.traffic: their
sums are consistent with the per-dispatch counter readings they hold, their
algorithmic bytes are those of the workload they name, and bench.py drops a
record (reports null) once the decode sources differ from the ones it was
taken on, or when it names another workload or entry point."""
import pytest

import bench
import workloads as W

_BY_NAME = {W.CONFIGS[k]().name: k for k in W.CONFIGS if k not in ("tiny", "chunked_prefill_mix")}


def _records():
    recs = bench.traffic_records()
    assert recs, "no traffic record under profiles/"
    return recs


@pytest.mark.parametrize("i", range(8))
def test_record_sums_follow_its_counter_readings(i):
    recs = _records()
    if i >= len(recs):
        pytest.skip("fewer records")
    _, rec = recs[i]
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
    # the record names a workload of this repository and its algorithmic bytes
    assert rec["workload"] in _BY_NAME, rec["workload"]
    assert rec["algorithmic_bytes_per_call"] == W.CONFIGS[_BY_NAME[rec["workload"]]]().kv_bytes()
    assert rec["call"] in ("pa_decode_append", "pa_decode")


def test_bench_drops_a_record_taken_on_other_sources(monkeypatch):
    _, rec = _records()[0]
    monkeypatch.setattr(bench, "decode_sources_sha256", lambda: rec["source_sha256"])
    assert bench.recorded_traffic(rec["workload"], rec["call"]) == rec["hbm_bytes_per_call"]
    other_call = "pa_decode" if rec["call"] == "pa_decode_append" else "pa_decode_append"
    assert bench.recorded_traffic(rec["workload"], other_call) is None
    assert bench.recorded_traffic("no_such_workload", rec["call"]) is None
    monkeypatch.setattr(bench, "decode_sources_sha256", lambda: "0" * 64)
    assert bench.recorded_traffic(rec["workload"], rec["call"]) is None


def test_headline_workload_has_a_current_record():
    """The bench's headline workload (batch 64, every context 8192) has a
    traffic record of its one-call step taken on the current decode sources,
    so its line carries roofline.traffic."""
    w = W.llama8b_decode_8k()
    assert bench.recorded_traffic(w.name, "pa_decode_append") is not None
