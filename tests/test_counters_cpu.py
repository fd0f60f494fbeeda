"""CPU checks of the profile-summary host logic (gated_linear_recurrent_amd.counters):
kernel-name shortening, the copy-kernel calibration of FETCH_SIZE and
WRITE_SIZE, the MFMA-busy fraction and the kernel-trace table, on synthetic
rocprofv3 outputs written here (no profiler or GPU involved).
"""
import csv
import os
import sqlite3

import pytest

from gated_linear_recurrent_amd import counters

COPY = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda(at::TensorIteratorBase&)>(int)"
OUT = "void liger::prefill_output_kernel<unsigned short, 128, 0, false>(liger::PrefillParams)"
OTHER = "void liger::prefill_output_kernel<unsigned short, 128, 0, true>(liger::PrefillParams)"


def _write_csv(d, rows):
    os.makedirs(os.path.join(d, "host", "1234"), exist_ok=True)
    with open(os.path.join(d, "host", "1234", "p_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (k, c, v) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def test_short_names():
    assert counters._short(OUT) == "liger::prefill_output_kernel<unsigned short, 128, 0, false>"
    anon = "void liger::(anonymous namespace)::bwd_chunk_kernel<128, 0>(liger::(anonymous namespace)::BwdParams)"
    assert counters._short(anon) == "liger::bwd_chunk_kernel<128, 0>"


def test_traffic_calibration_and_busy(tmp_path):
    fetch, write, busy = (str(tmp_path / n) for n in ("fetch", "write", "busy"))
    # two dispatches each: the per-dispatch mean is used
    _write_csv(fetch, [(COPY, "FETCH_SIZE", 131000), (COPY, "FETCH_SIZE", 131144),
                       (OUT, "FETCH_SIZE", 61000), (OUT, "FETCH_SIZE", 61604),
                       (OTHER, "FETCH_SIZE", 99999)])
    _write_csv(write, [(COPY, "WRITE_SIZE", 262144), (OUT, "WRITE_SIZE", 66048), (OTHER, "WRITE_SIZE", 1)])
    _write_csv(busy, [(OUT, "SQ_VALU_MFMA_BUSY_CYCLES", 2.0e7), (OUT, "GRBM_GUI_ACTIVE", 1.2e6)])
    rec = counters.traffic(fetch, write, busy, 256, "cmd")
    cal = rec["_calibration"]
    assert cal["fetch_kib_read"] == pytest.approx(131072.0)
    assert cal["fetch_scale"] == pytest.approx(2.0) and cal["write_scale"] == pytest.approx(1.0)
    out = rec["prefill_output_kernel"]
    assert out["fetch_kib_per_launch"] == pytest.approx(61302.0)      # the SINK variant is not mixed in
    assert out["hbm_bytes_per_launch"] == pytest.approx((61302.0 * 2.0 + 66048.0) * 1024.0)
    # busy cycles over all 1024 SIMDs; GRBM_GUI_ACTIVE is summed over the 8 XCDs
    assert out["mfma_busy_frac"] == pytest.approx(2.0e7 / (1024 * 1.2e6 / 8))
    assert out["source_sha256"] == counters.source_sha(counters.KERNELS["prefill_output_kernel"][2])
    assert "decode_step_kernel" not in rec   # kernels absent from the run are left out


def test_source_sha_follows_the_sources(tmp_path, monkeypatch):
    (tmp_path / "a.hip").write_text("x")
    monkeypatch.setattr(counters, "ROOT", str(tmp_path))
    h1 = counters.source_sha(["a.hip"])
    (tmp_path / "a.hip").write_text("y")
    assert counters.source_sha(["a.hip"]) != h1


def test_trace_table(tmp_path):
    db = str(tmp_path / "run_results.db")
    con = sqlite3.connect(db)
    con.execute("create table top_kernels (name text, total_calls int, total_duration real, average real, "
                "percentage real)")
    con.execute("insert into top_kernels values (?, ?, ?, ?, ?)", (OUT, 12, 916.2, 76.35, 2.0))
    con.commit()
    con.close()
    text = counters.trace(db, "Kernel trace: test", "rocprofv3 --kernel-trace --stats -- python3 bench.py")
    assert text.startswith("# Kernel trace: test\n")
    assert "| `liger::prefill_output_kernel<unsigned short, 128, 0, false>` | 12 | 916.2 | 76.35 | 2.0 |" in text


DEC = "void liger::decode_step_kernel<unsigned short, 128, 1, 4, false>(liger::DecodeParams)"
RED = "void at::native::reduce_kernel<512, 1, at::native::ReduceOp<float, at::native::func_wrapper<float> > >(int)"
FILL = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<float>, std::array<char*, 1ul> >(int)"


def _write_dispatches(d, dispatches):
    """dispatches: [(kernel, {counter: value})], one dispatch id each, several rows per dispatch."""
    os.makedirs(os.path.join(d, "host", "1"), exist_ok=True)
    with open(os.path.join(d, "host", "1", "p_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (k, cs) in enumerate(dispatches):
            for c, v in cs.items():
                w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def test_busy_fractions_follow_the_profiler_formulas():
    # 8 XCDs at 1000 cycles each; 256 CUs, 1024 SIMDs
    b = {"GRBM_GUI_ACTIVE": 8000.0, "SQ_VALU_MFMA_BUSY_CYCLES": 1024 * 250.0, "SQ_ACTIVE_INST_VALU": 256 * 400.0,
         "SQ_LDS_BANK_CONFLICT": 256 * 50.0, "SQ_LDS_IDX_ACTIVE": 256 * 150.0}
    f = counters.busy_fracs(b)
    assert f["mfma_busy_frac"] == pytest.approx(0.25)
    assert f["valu_busy_frac"] == pytest.approx(0.40)
    assert f["lds_bank_conflict_frac"] == pytest.approx(0.05)
    assert f["lds_conflicts_per_access"] == pytest.approx(0.5)
    lat = counters.read_latency({"TCC_EA0_RDREQ_sum": 200.0, "TCC_EA0_RDREQ_LEVEL_sum": 200.0 * 700,
                                 "TCC_EA0_RDREQ_DRAM_sum": 150.0})
    assert lat == {"read_requests": 200.0, "read_latency_cycles": 700.0, "dram_read_requests": 150.0}


def test_decode_dispatches_split_by_the_preceding_kernel(tmp_path):
    d = str(tmp_path / "tcc")
    seq = [(DEC, {"TCC_EA0_RDREQ_sum": 10.0, "TCC_EA0_RDREQ_LEVEL_sum": 1000.0}),   # first: no predecessor
           (DEC, {"TCC_EA0_RDREQ_sum": 10.0, "TCC_EA0_RDREQ_LEVEL_sum": 2000.0}),   # back to back
           (RED, {"TCC_EA0_RDREQ_sum": 5.0, "TCC_EA0_RDREQ_LEVEL_sum": 5.0}),
           (DEC, {"TCC_EA0_RDREQ_sum": 10.0, "TCC_EA0_RDREQ_LEVEL_sum": 9000.0}),   # after the read eviction
           (FILL, {"TCC_EA0_RDREQ_sum": 0.0, "TCC_EA0_RDREQ_LEVEL_sum": 0.0}),
           (DEC, {"TCC_EA0_RDREQ_sum": 10.0, "TCC_EA0_RDREQ_LEVEL_sum": 12000.0})]  # after the write eviction
    _write_dispatches(d, seq)
    allm = counters._counter_means(d)[DEC]
    assert allm["TCC_EA0_RDREQ_LEVEL_sum"] == pytest.approx((1000 + 2000 + 9000 + 12000) / 4)
    for after, level in (("reduce_kernel", 9000.0), ("FillFunctor", 12000.0), ("decode_step_kernel", 2000.0)):
        m = counters._counter_means(d, after)[DEC]
        assert m["TCC_EA0_RDREQ_LEVEL_sum"] == level
    assert counters.DECODE_REGIMES["after_read_eviction"] in RED
    assert counters.DECODE_REGIMES["after_write_eviction"] in FILL
