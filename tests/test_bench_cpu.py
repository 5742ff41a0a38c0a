"""Host-side checks of the benchmark and of the product path's isolation (no GPU needed).

* The algorithmic byte and FLOP counts bench.py divides by are the ones stated for the
  workload shapes: each operand read once, each output written once (act_quant reads
  2 B and writes 1 B per element plus a 4-byte scale per 128; weight_dequant reads 1 B
  and writes 2 B; the GEMM reads A, B and both scale grids and writes bf16 C).
* bench.py refuses more than one GPU and the cold mode outside the decode workload,
  before touching a device.
* Nothing in the package imports or loads the CPU oracle: the product path has no CPU
  fallback of any kind.
"""
import ast
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


@pytest.fixture(scope="module")
def bench():
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_module", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_algorithmic_bytes(bench):
    # decode projection 64 x 1536 x 7168
    assert bench.gemm_bytes(64, 1536, 7168) == 64 * 7168 + 1536 * 7168 + 2 * 64 * 1536 + 4 * 64 * 56 + 4 * 12 * 56
    assert bench.gemm_bytes(64, 1536, 7168) == 11_682_432
    # dense MLP up projection 8192 x 18432 x 7168 and down 8192 x 7168 x 18432
    assert bench.gemm_bytes(8192, 18432, 7168) == 494_697_984
    assert bench.gemm_bytes(8192, 7168, 18432) == 405_306_880
    # act_quant of x [8192, 7168] and of H [8192, 18432]; dequant of [18432, 7168]
    assert bench.act_quant_bytes(8192, 7168) == 177_995_776
    assert bench.act_quant_bytes(8192, 18432) == 457_703_424
    assert bench.dequant_bytes(18432, 7168) == 396_393_984
    # grouped: G weight matrices and scale grids, the rows once
    assert bench.gemm_bytes(100, 2048, 7168, G=4) == (100 * 7168 + 4 * 2048 * 7168 + 2 * 100 * 2048
                                                      + 4 * 100 * 56 + 4 * 4 * 16 * 56)


def test_peaks_are_the_datasheet_figures(bench):
    assert bench.PEAK_FP8_TFLOPS == 5000.0
    assert bench.PEAK_BF16_TFLOPS == 2500.0
    assert bench.PEAK_HBM_GBS == 8000.0


def _run_bench(*args):
    env = dict(os.environ, HIP_VISIBLE_DEVICES="")
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, timeout=300, env=env)


def test_bench_refuses_more_than_one_gpu():
    r = _run_bench("--gpus", "2", "--no-cpu-baseline")
    assert r.returncode != 0
    assert "one GPU" in r.stderr or "--gpus 1" in r.stderr


def test_bench_cold_only_for_decode():
    r = _run_bench("--workload", "dense-mlp", "--cold", "--no-cpu-baseline")
    assert r.returncode != 0
    assert "--cold" in (r.stderr + r.stdout)


def _imports(path):
    tree = ast.parse(open(path).read())
    names = set()
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            names.update(a.name.split(".")[0] for a in node.names)
        elif isinstance(node, ast.ImportFrom) and node.module:
            names.add(node.module.split(".")[0])
    return names


def test_package_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "block_scaled_fp8_04_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith(".py"):
                assert "oracle" not in _imports(os.path.join(dirpath, f)), f
            if f.endswith((".hip", ".hpp", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "bfp8_oracle" not in text and "oracle/" not in text, f


def test_traffic_is_tied_to_its_workload(bench):
    """Counter-measured HBM bytes are reported only for the workload they were measured on."""
    assert bench.read_traffic("gemm", "decode") is None
    assert bench.read_traffic("gemm", "moe-pair") is None
    assert bench.read_traffic("gemm_grouped", "moe-layer") is None
    assert bench.read_traffic("no_such_kernel", "dense-mlp") is None
