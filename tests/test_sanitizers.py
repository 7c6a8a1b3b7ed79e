"""Host code and the oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two small drivers (tests/sanitize/) are compiled together with the code they exercise and run:

* host_driver.cpp with ternary_weight_quantized_bonsai_amd/csrc/host.cpp, the host-only part of
  the C ABI (pack / unpack of the three weight layouts, the conversions between them and the
  affine scale pairs, the status strings);
* oracle_driver.c with oracle/bonsai_oracle.c, every oracle entry point.

Each driver checks results as well (round trips, cross-layout agreement, error statuses), and
holds every buffer at exactly its documented size, so an out-of-bounds access, a signed overflow
or any other undefined operation fails the run (-fno-sanitize-recover=all).  The kernels are not
covered here: device-side sanitizers need hardware support these GPUs do not offer; the GPU tests
cover the kernels with NaN-poisoned outputs, guard-band canaries and bitwise re-runs instead.
"""
from __future__ import annotations

import shutil
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
OUT = ROOT / "_build" / "sanitize"
SAN = ["-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-ffp-contract=off", "-Wall", "-Wextra", "-Werror"]


def _build_and_run(compiler: str, std: str, sources: list[Path], name: str, libs: tuple[str, ...] = ()) -> str:
    if shutil.which(compiler) is None:
        pytest.skip(f"{compiler} not found")
    OUT.mkdir(parents=True, exist_ok=True)
    exe = OUT / name
    cmd = [compiler, std, *SAN, f"-I{ROOT / 'include'}", *map(str, sources), "-o", str(exe), *libs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"build failed:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}"
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300,
                       env={"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0",
                            "UBSAN_OPTIONS": "print_stacktrace=1"})
    assert r.returncode == 0, f"{name} failed (exit {r.returncode}):\n{r.stdout}{r.stderr}"
    return r.stdout


def test_host_abi_under_sanitizers():
    out = _build_and_run("g++", "-std=c++17",
                         [ROOT / "ternary_weight_quantized_bonsai_amd" / "csrc" / "host.cpp",
                          ROOT / "tests" / "sanitize" / "host_driver.cpp"], "host_driver")
    assert "all checks passed" in out


def test_oracle_under_sanitizers():
    out = _build_and_run("gcc", "-std=c11",
                         [ROOT / "oracle" / "bonsai_oracle.c", ROOT / "tests" / "sanitize" / "oracle_driver.c"],
                         "oracle_driver", libs=("-lm",))
    assert "all checks passed" in out


def test_sanitizers_catch_a_planted_overrun():
    """The harness has teeth: a copy of the oracle whose binary dequantisation writes one row
    past the requested range must fail under AddressSanitizer."""
    src = (ROOT / "oracle" / "bonsai_oracle.c").read_text()
    loop = "    for (int64_t n = n0; n < n1; ++n)\n        for (int64_t k = 0; k < K; ++k)\n            W[(n - n0) * K + k] = q1_weight("
    assert src.count(loop) == 1, "the planted mistake no longer applies: update this test"
    OUT.mkdir(parents=True, exist_ok=True)
    mutant = OUT / "oracle_overrun.c"
    mutant.write_text(src.replace(loop, loop.replace("n < n1", "n <= n1")))
    with pytest.raises(AssertionError, match="AddressSanitizer"):
        _build_and_run("gcc", "-std=c11", [mutant, ROOT / "tests" / "sanitize" / "oracle_driver.c"],
                       "oracle_overrun", libs=("-lm",))
