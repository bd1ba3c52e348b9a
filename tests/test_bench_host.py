"""Host-side parts of bench.py (no device): the one-GPU guard, the roofline
record and the rotating-copy count, and the oracle baseline's record shape."""
import subprocess
import sys
import pathlib

import numpy as np
import pytest

ROOT = pathlib.Path(__file__).resolve().parents[1]
sys.path.insert(0, str(ROOT))

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_before_any_device_work():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "--gpus must be 1" in r.stdout + r.stderr


def test_roof_takes_the_closer_roof():
    t = dict(ms=0.040, min_ms=0.039, max_ms=0.041, launches_per_window=50, ramp_launches=1000)
    # 16 x 1024^3 bf16 products in 40 us: 859 TFLOP/s, far from the 8 TB/s HBM roof for 96 MiB
    r = bench.roof(2.0 * 16 * 1024 ** 3, 96 * 2 ** 20, t)
    assert r["bound"] == "mfma"
    assert r["tflops"] == pytest.approx(2.0 * 16 * 1024 ** 3 / 40e-6 / 1e12, rel=1e-3)
    assert r["frac_mfma"] == pytest.approx(r["tflops"] / bench.PEAK_MFMA_16, abs=1e-4)
    assert r["roofline_frac"] == max(r["frac_mfma"], r["frac_hbm"])
    # a memory-bound call: 32 MiB in 10 us against a few GFLOP
    r = bench.roof(2.0 * 16 * 8192 * 8192, 32 * 2 ** 20, dict(t, ms=0.010))
    assert r["bound"] == "hbm"
    assert r["gbps"] == pytest.approx(32 * 2 ** 20 / 10e-6 / 1e9, rel=1e-3)
    assert bench.roof(1.0, 1.0, t, bound="launch")["bound"] == "launch"


def test_rotating_copies_keep_inputs_out_of_the_caches():
    assert bench.copies_for(bench.ROTATE_TARGET) == 1
    assert bench.copies_for(bench.ROTATE_TARGET * 3) == 1
    n = bench.copies_for(96 * 2 ** 20)
    assert n * 96 * 2 ** 20 >= bench.ROTATE_TARGET and (n - 1) * 96 * 2 ** 20 < bench.ROTATE_TARGET


def test_cpu_baseline_record():
    # a tiny bounded sample of the oracle on headline-shaped batches (two 1024^3 products at most)
    import gmi_inputs as gi

    r = np.random.default_rng(0)
    A = [gi.to_bits(r.standard_normal((1024, 1024)).astype(np.float32), "bf16") for _ in range(2)]
    B = [gi.to_bits(r.standard_normal((1024, 1024)).astype(np.float32), "bf16") for _ in range(2)]
    rec = bench.cpu_baseline(gi, A, B, budget_s=0.0)
    assert rec["kind"] == "oracle" and rec["unit"] == "TFLOP/s"
    assert rec["value"] > 0 and rec["cores"] >= 1
    assert "1 batch products" in rec["sample"]
