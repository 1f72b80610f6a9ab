"""The benchmark's contract: the one-JSON-line output, the one-GPU refusal,
and the FLOP accounting its throughput figures rest on."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PEAK_MIX = (2500.0, 5000.0)   # a mix of fp8 and bf16 MFMA FLOP has a peak between the two
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_executed_flops_counts_valid_rows_and_keys():
    """S = 100: q-blocks of 64 and 36 rows, key tiles of 100 keys (one tile).
    QK^T of both blocks always; P.V only of the kept block."""
    mask = np.array([[[[True], [False]]]])   # block 0 skips tile 0, block 1 keeps it
    D = 128
    want = 2 * D * (64 * 100 + 36 * 100) + 2 * D * (36 * 100)
    assert bench.executed_flops(mask, 100, D=D) == want


def test_executed_flops_dense_equals_the_definition():
    """No skipped tile: executed work is 4 B H S^2 D, the dense count."""
    B, H, S, D = 2, 3, 300, 128
    mask = np.zeros((B, H, -(-S // 64), -(-S // 128)), bool)
    assert bench.executed_flops(mask, S, D=D) == 4 * B * H * S * S * D


def test_issued_mfma_flops_pads_tiles():
    mask = np.array([[[[True, False], [False, False]]]])
    assert bench.issued_mfma_flops(mask) == 2 * 128 * 64 * 128 * (4 + 3)


@pytest.mark.gpu
def test_bench_json_line():
    """A short run prints one JSON line with every field the driver reads."""
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--steps", "2", "--warmup", "1",
                        "--cpu-seconds", "1", "--energy-calls", "40"], capture_output=True, text=True, timeout=280, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    d = json.loads(r.stdout.strip().splitlines()[-1])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert "workload" in d["config"]
    roof = d["roofline"]
    assert roof["bound"] in ("hbm", "mfma", "alu") and roof["unit"] in ("GB/s", "TFLOP/s")
    assert roof["peak"] > 0 and abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    oc = d["other_configs"]
    for key in ("wan_like_skip_0.5", "wan_like_skip_0.9", "long_seq_threshold_1e-3", "varlen_calibrated_0.5",
                "varlen_calibrated_0.7", "varlen_calibrated_0.9"):
        assert oc[key]["dense_ms"] > 0 and oc[key]["skip_ms"] > 0, key
        assert 0.0 <= oc[key]["skip_fraction"] <= 1.0, key
    # more skipping, less time (well separated fractions)
    assert oc["wan_like_skip_0.9"]["skip_ms"] < d["skip_step"]["ms_mean"] < oc["wan_like_skip_0.5"]["skip_ms"]
    assert len(oc["varlen_calibrated_0.9"]["skip_fraction_per_sequence"]) == 3
    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1 and cpu["sample"]
    assert cpu["cpu_model"] and {"tiny_factor_4", "mid_threshold_0.001"} <= set(cpu["full_configs"])
    # kernel durations from the rocprofv3 child run: the roofline uses the traced skip kernel,
    # whose duration cannot exceed the HIP-event time of the same call
    tr = d["rocprof"]
    assert tr is not None and roof["timing"] == "rocprofv3 kernel trace"
    assert tr["kernels"][bench.KERNEL_SKIP]["calls"] == 3 and tr["kernels"][bench.KERNEL_DENSE]["calls"] == 3
    assert roof["kernel_ms"] == tr["skip_kernel_mean_ms"] <= 1.05 * d["ms_per_step"]
    # the variants' kernels against their own rooflines, from the same trace
    var = d["variant_rooflines"]
    for key in ("fp8_scores_kernel", "fp8_quantize", "virtual_tile_means", "virtual_tiles_kernel"):
        assert key in var and var[key]["kernel_ms"] > 0, key
    for key in ("fp8_scores_kernel", "fp8_quantize", "virtual_tile_means"):
        assert 0.0 < var[key]["frac"] < 1.0, (key, var[key])
    f8 = var["fp8_scores_kernel"]
    assert PEAK_MIX[0] <= f8["peak"] <= PEAK_MIX[1]
    assert tr["kernels"][bench.KERNEL_FP8]["calls"] == 3
    # energy figures where the board's power sensor can be read
    en = d["energy"]
    if en is not None:
        assert en["idle_w"] > 0 and en["dense"]["power_w"] > en["idle_w"] and en["skip"]["power_w"] > en["idle_w"]
        assert en["work_energy_ratio"] > 1.0 and en["power_above_idle_ratio"] > 0.0
        # the time ratio of the two calls is the product of the two ratios
        t_ratio = en["dense"]["ms_per_call"] / en["skip"]["ms_per_call"]
        assert abs(en["work_energy_ratio"] * en["power_above_idle_ratio"] - t_ratio) < 0.01 * t_ratio


@pytest.mark.gpu
def test_bench_power_mode():
    """--power prints one JSON line with the cap, idle power and, for the dense
    and skip calls, time, power and energy per call (read-only hwmon)."""
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--power", "30"],
                       capture_output=True, text=True, timeout=280, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    d = json.loads(r.stdout.strip().splitlines()[-1])["power_run"]
    if d is None:
        pytest.skip("no readable hwmon power file on this machine")
    for name in ("dense", "skip"):
        e = d[name]
        assert e["ms_per_call"] > 0 and e["power_w"] > 0
        assert abs(e["energy_j_per_call"] - e["power_w"] * e["ms_per_call"] / 1e3) < 0.01
    assert d["skip"]["ms_per_call"] < d["dense"]["ms_per_call"]
