"""bench.py's stdout line stays small enough to be read whole from the tail of the output,
and bench.py refuses more than one GPU.  CPU only: the line is composed from stand-in numbers
of the real sizes (eight sweep rows, five kernels, the run state with long strings)."""
import json
import os
import subprocess
import sys
import types

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

LINE_LIMIT = 8192


def _fake():
    args = types.SimpleNamespace(steps=50, warmup=20)
    Ms = (1, 2, 4, 8, 16, 32, 64, 128)
    sweep = [{"M": m, "us": 123456.78, "GBps": 12345.6, "hbm_frac": 0.12345, "TFLOPs": 1234.5,
              "mfma_frac": 0.12345, "roofline_frac": 0.12345, "x_fp16_bound": 1.234,
              "x_fp16_gemm": 1.234} for m in Ms]
    kernels = [{"bound": "hbm", "achieved": 12345.6, "peak": 8000.0, "unit": "GB/s",
                "frac": 0.12345, "traffic": 123456789012.5,
                "kernel": name + " " * 40, "M": list(ms), "mean_launch_us": 123456.78}
               for name, ms, _ in bench.KERNELS]
    cpu = {"value": 0.123456, "unit": "GB/s", "cores": 16, "kind": "oracle",
           "sample": "x" * 200, "cpu_model": "y" * 64, "host_cores": 256}
    refs = {"stream_read_GBps": 6850.1, "stream_read_frac_of_spec": 0.8563,
            "mfma_f16_TFLOPs": {"16x16x32": 1600.0, "32x32x16": 1700.0},
            "mfma_f16_frac_of_spec": {"16x16x32": 0.64, "32x32x16": 0.68}}
    state = {"hip": "7.0.51831-a3e329ad8", "torch": "2.10.0+rocm7.0", "gpu": "z" * 64,
             "arch": "gfx950:sramecc+:xnack-", "cus": 256,
             "gpu_sysfs": {"card": "0000:05:00.0", "sclk_levels": ["0: 500Mhz", "1: 1500Mhz",
                                                                  "2: 2400Mhz"],
                           "mclk_levels": ["0: 900Mhz", "1: 1500Mhz", "2: 1900Mhz", "3: 2000Mhz"],
                           "power_cap_w": 1400.0,
                           "ecc": {"ras_features": "feature mask: 0x3fbfffff" + " " * 100,
                                   "hbm_ecc_enabled": True, "umc_err_count": "ue: 0\nce: 0"}},
             "cpu_model": "y" * 64, "host_cores": 256, "cores_allowed": 256, "omp_num_threads": "16"}
    compute = [{"M": m, "us": 123456.78, "TFLOPs": 1234.5, "mfma_frac": 0.12345}
               for m in (256, 512, 1024)]
    config = {"workload": "single_72kx18k_m1_128", "K": 18432, "N": 73728, "M": list(Ms),
              "group": 128, "weights": "int4 codes + fp16 scales (4.125 bits/weight)",
              "weight_copies_rotated": 9}
    return args, config, kernels, sweep, cpu, refs, state, compute


def test_line_fits_and_has_the_contract_keys():
    args, config, kernels, sweep, cpu, refs, state, compute = _fake()
    line = bench.compose_line(args, 4321.0, 1.2345, config, kernels, sweep, cpu, refs, state,
                              compute, "gpurun_out/bench_details.json")
    assert "\n" not in line
    assert len(line.encode()) < LINE_LIMIT, len(line.encode())
    d = json.loads(line)
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in d, k
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in d["roofline"], k
    for k in ("value", "unit", "cores", "kind", "sample"):
        assert k in d["cpu_baseline"], k
    assert len(d["sweep"]) == 8
    assert d["config"]["workload"]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_oracle_threads_follow_the_process_cpu_share():
    host = {"cores_allowed": 64, "omp_num_threads": "16", "host_cores": 256, "cpu_model": None}
    assert bench.oracle_threads(host) == 16
    host["omp_num_threads"] = None
    assert bench.oracle_threads(host) == 64
