"""bench.py end to end on the tiny workload: one JSON line with the fields
the benchmark promises (throughput, the GEMM roofline, per-step latency,
device memory and the plain-torch logits baselines), consistent with one
another; and the default multi-workload line's nesting."""
import json

import pytest

pytestmark = pytest.mark.gpu


def _line(capsys):
    lines = [ln for ln in capsys.readouterr().out.splitlines() if ln.startswith("{")]
    assert len(lines) == 1
    return json.loads(lines[0])


def _check_record(rec, steps):
    assert rec["unit"] == "masked tokens/s" and rec["value"] > 0
    cfg = rec["config"]
    assert cfg["L"] == 512 and cfg["masked_rows_timed"] > 0
    mem = rec["memory"]
    assert mem["mask_only_logits_fp32_bytes"] <= mem["full_logits_fp32_bytes"]
    assert mem["peak_bytes"] == mem["resident_before_step_bytes"] + mem["step_transient_bytes"]
    # the streamed readout allocates nothing per step: its transient is zero
    # (the workspace is resident, allocated by the caller before the step)
    assert mem["step_transient_bytes"] == 0
    assert mem["workspace_bytes"] > 0
    roof = rec["roofline"]
    assert 0 < roof["frac"] <= 1 and roof["achieved"] > 0
    lat = rec["latency"]
    assert lat["steps"] == steps and 0 < lat["median_us"] <= lat["p95_us"]


def test_bench_tiny_json(capsys):
    import bench
    print("[case] bench.py --workload tiny --steps 8 --warmup 2", flush=True)
    rc = bench.main(["--workload", "tiny", "--steps", "8", "--warmup", "2", "--no-cpu-baseline"])
    assert rc == 0
    rec = _line(capsys)
    assert rec["n_gpus"] == 1 and rec["steps"] == 8
    _check_record(rec, 8)
    tb = rec["torch_logits_baseline"]
    assert tb["rows"]["full"] == 512 and 0 < tb["rows"]["mask_only"] <= 512
    for name in ("full", "mask_only"):
        assert tb[name]["ms_per_step"] > 0 and tb[name]["transient_bytes"] > 0
    # the full readout materialises at least the fp32 logits of all L rows
    assert tb["full"]["transient_bytes"] >= rec["memory"]["full_logits_fp32_bytes"]
    assert tb["streamed_transient_bytes"] == 0
    assert rec["cpu_baseline"] is None


def test_bench_default_line_nests_workloads(capsys, monkeypatch):
    import bench
    print("[case] bench.py default line, workloads restricted to tiny", flush=True)
    monkeypatch.setattr(bench, "ALL_ORDER", ("tiny",))
    rc = bench.main(["--steps", "4", "--warmup", "1", "--no-cpu-baseline", "--no-torch-baseline"])
    assert rc == 0
    rec = _line(capsys)
    assert rec["config"]["workload"].startswith("tiny")
    assert list(rec["configs"]) == ["tiny"]
    nested = rec["configs"]["tiny"]
    assert "metric" not in nested and nested["value"] > 0
    _check_record(dict(nested, unit="masked tokens/s"), 4)


def test_bench_gemm_ceiling(capsys):
    """The GEMM instruction-mix probe runs and gives plausible rates: both
    below the published dense peak, the full mix no faster than MFMAs alone
    (within run-to-run noise)."""
    import bench
    print("[case] bench.py --ceiling", flush=True)
    assert bench.main(["--ceiling"]) == 0
    rec = _line(capsys)["gemm_ceiling"]
    a, b = rec["mfma_only"], rec["main_loop_mix"]
    assert 0 < b["tflops"] <= a["tflops"] * 1.1
    assert a["frac_of_peak"] < 1.0 and b["frac_of_peak"] < 1.0
    assert rec["grid"] > 0 and rec["stages"] > 0
    # the sustained shader clock under MFMA load, and the pipe busy fraction at it
    for r in (a, b):
        assert 0.5 < r["shader_clock_ghz"] < 3.0
        assert 0 < r["mfma_busy_at_clock"] <= 1.05
