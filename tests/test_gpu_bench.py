"""bench.py end to end on the tiny workload: one JSON line with the fields
the benchmark promises (throughput, the GEMM roofline, per-step latency and
the plain-torch logits baselines), consistent with one another."""
import json

import pytest

pytestmark = pytest.mark.gpu


def test_bench_tiny_json(capsys):
    import bench
    print("[case] bench.py --workload tiny --steps 8 --warmup 2", flush=True)
    rc = bench.main(["--workload", "tiny", "--steps", "8", "--warmup", "2", "--no-cpu-baseline"])
    assert rc == 0
    lines = [ln for ln in capsys.readouterr().out.splitlines() if ln.startswith("{")]
    assert len(lines) == 1
    rec = json.loads(lines[0])
    assert rec["unit"] == "masked tokens/s" and rec["value"] > 0 and rec["n_gpus"] == 1
    cfg = rec["config"]
    assert cfg["L"] == 512 and cfg["masked_rows_timed"] > 0
    assert cfg["mask_only_logits_fp32_bytes"] <= cfg["full_logits_fp32_bytes"]
    roof = rec["roofline"]
    assert 0 < roof["frac"] <= 1 and roof["achieved"] > 0
    lat = rec["latency"]
    assert lat["steps"] == 8 and 0 < lat["median_us"] <= lat["p95_us"]
    tb = rec["torch_logits_baseline"]
    assert tb["rows"]["full"] == 512 and 0 < tb["rows"]["mask_only"] <= 512
    for name in ("full", "mask_only"):
        assert tb[name]["ms_per_step"] > 0 and tb[name]["transient_bytes"] > 0
    # the full readout materialises at least the fp32 logits of all L rows
    assert tb["full"]["transient_bytes"] >= cfg["full_logits_fp32_bytes"]
    assert tb["streamed_transient_bytes"] == cfg["workspace_bytes"]
    assert rec["cpu_baseline"] is None
