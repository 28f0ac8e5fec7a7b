"""Host logic of profiling.py: per-kernel counter means, the calibration
factor taken from the 1 GiB bitwise_not kernel, and stale-record detection."""
import csv
import json
import os

import pytest

from mxfp4_routed_expert_top_amd import profiling


def _write_pass(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "x_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_record_and_staleness(tmp_path):
    cal = "void at::native::vectorized_elementwise_kernel<4, at::native::bitwise_not_kernel_cuda(x)>(int)"
    k = "void (anonymous namespace)::gate_up_kernel<2, false>(void const*, int)"
    # calibration reads 1 GiB but FETCH_SIZE shows half of it; writes show all
    _write_pass(tmp_path / "f", "FETCH_SIZE", [(cal, 524288.0), (k, 1000.0), (k, 3000.0)])
    _write_pass(tmp_path / "w", "WRITE_SIZE", [(cal, 1048576.0), (k, 10.0), (k, 30.0)])
    rec = profiling.traffic_record(str(tmp_path / "f"), str(tmp_path / "w"), "decode")
    assert rec["fetch_factor"] == pytest.approx(2.0) and rec["write_factor"] == pytest.approx(1.0)
    g = rec["kernels"]["gate_up_kernel<2, false>"]
    assert g["dispatches"] == 2
    assert g["fetch_bytes"] == 2000 * 1024 * 2 and g["write_bytes"] == 20 * 1024
    assert g["bytes"] == g["fetch_bytes"] + g["write_bytes"]
    assert not any("bitwise_not" in name for name in rec["kernels"])
    p = tmp_path / "rec.json"
    p.write_text(json.dumps(rec))
    assert profiling.load_traffic(str(p), "gate_up_kernel<2, false>") == g["bytes"]
    assert profiling.load_traffic(str(p), "down_kernel<2, false>") is None
    rec["source_sha256"] = "0" * 64                     # kernel sources changed since
    p.write_text(json.dumps(rec))
    assert profiling.load_traffic(str(p), "gate_up_kernel<2, false>") is None
    assert profiling.load_traffic(str(tmp_path / "missing.json"), "x") is None


def test_calibration_kernel_required(tmp_path):
    _write_pass(tmp_path / "f", "FETCH_SIZE", [("void k(int)", 1.0)])
    _write_pass(tmp_path / "w", "WRITE_SIZE", [("void k(int)", 1.0)])
    with pytest.raises(ValueError):
        profiling.traffic_record(str(tmp_path / "f"), str(tmp_path / "w"), "decode")


def test_committed_records_match_kernel_names():
    # every committed traffic record carries the gate/up kernel bench.py looks up
    import bench
    import synth
    from mxfp4_routed_expert_top_amd import ops
    for name in ("decode", "prefill", "prefill_skewed", "w4a4", "decode_mxfp8", "prefill_mxfp8"):
        cfg = synth.CONFIGS[name]
        path = bench.traffic_path(cfg)
        if not os.path.exists(path):
            continue
        rec = json.load(open(path))
        tile_m = (ops.mxfp8_gemm_tile_m(cfg.T, cfg.Kp, cfg.Ep, cfg.H, cfg.I)
                  if cfg.wfmt == synth.W_MXFP8 else
                  ops.gemm_tile_m(cfg.T, cfg.Kp, cfg.Ep, cfg.H, cfg.I, cfg.act_fmt))
        assert bench.gate_up_kernel_name(cfg, tile_m) in rec["kernels"], name
