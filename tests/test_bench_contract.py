"""The bench's output contract: one JSON line whose fields agree with each other, a refusal of
more than one GPU, and the CPU baseline's fields (the oracle timed on a bounded sample)."""
import json
import os
import subprocess
import sys

import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True,
                       timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_cpu_baseline_fields():
    sys.path.insert(0, ROOT)
    import bench
    inp = synth.make_inputs(synth.get_config("tiny"), 16)
    cb = bench.cpu_baseline(inp, 1.0)
    assert set(cb) == {"value", "unit", "cores", "kind", "sample"}
    assert cb["kind"] == "oracle" and cb["unit"] == "tokens/s"
    assert cb["value"] > 0 and cb["cores"] >= 1
    assert "16 of 16 tokens" in cb["sample"]


@pytest.mark.gpu
@pytest.mark.timeout(300)
def test_bench_json_line():
    """A short run of the default workload: every contract field is present, the throughput is
    the token count over the step time, and the roofline fraction is achieved over peak."""
    print("bench contract: default workload, 5 steps", flush=True)
    r = subprocess.run([sys.executable, "-u", BENCH, "--steps", "5", "--warmup", "2",
                        "--no-cpu-baseline"], capture_output=True, text=True, timeout=280,
                       cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 2
    assert d["higher_is_better"] is True and d["scaling"] == "weak"
    assert d["vs_baseline"] is None and d["data"] == "synthetic" and d["unit"] == "tokens/s"
    cfg = d["config"]
    assert cfg["workload"] == "mt_encoder_int4_T3840" and cfg["tokens"] == 3840
    assert d["ms_per_step"] > 0
    assert d["value"] == pytest.approx(cfg["tokens"] / (d["ms_per_step"] * 1e-3), rel=1e-9)
    roof = d["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in roof, key
    assert (roof["bound"], roof["unit"], roof["peak"]) in (("mfma", "TFLOP/s", 2500.0),
                                                           ("hbm", "GB/s", 8000.0))
    assert 0 < roof["frac"] < 1
    assert roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"], rel=1e-9)
    assert roof["traffic"] is None or roof["traffic"] > 0
    assert "cpu_baseline" not in d
    # the other layer shapes: graph-replayed step and dominant-kernel roofline each
    pc = d["per_config"]
    assert set(pc) == {"qwen15_moe_int4_T17", "qwen15_moe_int4_T544", "dsv2_lite_int4_T9",
                       "dsv2_lite_int4_T288", "phi35_moe_int4_T1", "phi35_moe_int4_T17",
                       "phi35_moe_int4_T8192"}, sorted(pc)
    for name, c in pc.items():
        assert c["timing"] == "hip-graph replay" and c["ms_per_step"] > 0, name
        assert c["bound"] in ("hbm", "mfma") and 0 < c["frac"] < 1, name
        assert c["dominant_us"] < c["ms_per_step"] * 1e3 * 1.5, name
