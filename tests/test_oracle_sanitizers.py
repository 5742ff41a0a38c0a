"""The CPU oracle built with AddressSanitizer and UndefinedBehaviorSanitizer runs every pin cleanly.

The oracle is compiled again with ``-fsanitize=address,undefined`` (host code only; no
GPU code is involved) into a temporary folder and the pins of tests/pins.py run
against that build in a child Python process with the ASan runtime preloaded.  A
second build with a planted one-past-the-block read shows the sanitizer is live:
that child must die with an AddressSanitizer report.
"""
import os
import subprocess
import sys

import pytest

from oracle import build as oracle_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_FLAGS = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
             "-fno-omit-frame-pointer", "-w"]

RUN_PINS = """
import sys
sys.path.insert(0, {tests!r}); sys.path.insert(0, {root!r})
import oracle, pins
orc = oracle.Oracle({lib!r})
for p in pins.ALL_PINS:
    p(orc)
print("pins ok:", len(pins.ALL_PINS))
"""


def _asan_runtime():
    out = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = out.stdout.strip()
    return path if path and os.path.isabs(path) and os.path.exists(path) else None


def _run_pins(lib):
    env = dict(os.environ)
    env["LD_PRELOAD"] = _asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    code = RUN_PINS.format(tests=os.path.join(ROOT, "tests"), root=ROOT, lib=lib)
    return subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                          timeout=600)


@pytest.fixture(scope="module")
def san_dir(tmp_path_factory):
    if _asan_runtime() is None:
        pytest.skip("g++ has no AddressSanitizer runtime here")
    return tmp_path_factory.mktemp("oracle_sanitized")


def test_pins_clean_under_asan_ubsan(san_dir):
    lib = str(san_dir / "libbfp8_oracle_san.so")
    subprocess.run(oracle_build.compile_cmd(oracle_build.SOURCE, lib, SAN_FLAGS), check=True)
    res = _run_pins(lib)
    assert res.returncode == 0, res.stderr[-4000:]
    assert "pins ok" in res.stdout
    assert "runtime error" not in res.stderr, res.stderr[-4000:]


def test_sanitizer_catches_planted_overrun(san_dir):
    src = open(oracle_build.SOURCE).read()
    old = "for (int j = 0; j < ORACLE_BLOCK; ++j) {\n                float a = fabsf("
    assert src.count(old) >= 1
    bad = src.replace(old, "for (int j = 0; j <= ORACLE_BLOCK; ++j) {\n                float a = fabsf(")
    cpp = san_dir / "overrun.cpp"
    cpp.write_text(bad)
    lib = str(san_dir / "liboverrun.so")
    subprocess.run(oracle_build.compile_cmd(str(cpp), lib, SAN_FLAGS), check=True)
    res = _run_pins(lib)
    assert res.returncode != 0
    assert "AddressSanitizer" in res.stderr, res.stderr[-2000:]
