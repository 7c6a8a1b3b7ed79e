"""Host-side logic of bench.py (CPU only): the one-GPU refusal, the HBM-traffic summary built
from rocprofv3 counter CSVs, and the digest gate that keeps counters taken on one build of the
decode kernel from being reported for another."""
from __future__ import annotations

import csv
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
sys.path.insert(0, str(ROOT))
import bench  # noqa: E402

SRC = "ternary_weight_quantized_bonsai_amd/csrc/q1_gemv.hip"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "--gpus 1" in r.stderr and r.stdout == ""


def _counter_csv(path: Path, counter: str, rows: list[tuple[int, str, int, float]]) -> None:
    path.parent.mkdir(parents=True, exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name",
                                           "Counter_Value"])
        w.writeheader()
        for d, name, grid, v in rows:
            w.writerow({"Dispatch_Id": d, "Kernel_Name": name, "Grid_Size": grid, "Counter_Name": counter,
                        "Counter_Value": v})


@pytest.fixture
def fake_root(tmp_path, monkeypatch):
    """A repository root with a kernel source and build recipe of its own."""
    (tmp_path / SRC).parent.mkdir(parents=True)
    (tmp_path / SRC).write_text("// kernel, first build\n")
    (tmp_path / "ternary_weight_quantized_bonsai_amd" / "build.py").write_text("FLAGS = ['-O3']\n")
    monkeypatch.setattr(bench, "ROOT", tmp_path)
    return tmp_path


def test_traffic_summary_scales_by_the_copy_probe_and_gates_on_the_digest(fake_root, capsys):
    kern = "void bonsai::(anonymous namespace)::q1_gemv_lut4_kernel<64, true, false, 4>(unsigned int const*)"
    copy = "__amd_rocclr_copyBuffer"
    # The copy probe reads 1 GiB as 524288 KiB of FETCH_SIZE (scale 2) and writes it as 1048576
    # KiB of WRITE_SIZE (scale 1); a small weight clone (below 90 % of the largest copy) is not
    # one of its dispatches.  The kernel runs on two grids, FETCH_SIZE split over two rows.
    fetch = [(1, copy, 512, 4096.0), (2, copy, 512, 524288.0), (3, copy, 512, 524288.0),
             (4, copy, 512, 524300.0), (5, kern, 102400, 600.0), (5, kern, 102400, 400.0),
             (6, kern, 138240, 3000.0)]
    write = [(1, copy, 512, 4096.0), (2, copy, 512, 1048576.0), (3, copy, 512, 1048576.0),
             (4, copy, 512, 1048576.0), (5, kern, 102400, 10.0), (6, kern, 138240, 30.0)]
    _counter_csv(fake_root / "f" / "run" / "f_counter_collection.csv", "FETCH_SIZE", fetch)
    _counter_csv(fake_root / "w" / "run" / "w_counter_collection.csv", "WRITE_SIZE", write)
    bench.summarize_pmc(str(fake_root / "f"), str(fake_root / "w"), "traffic.txt", ["cmd one", "cmd two"],
                        "q1_gemv_lut4_kernel", SRC)
    capsys.readouterr()
    text = (fake_root / "profiles" / "traffic.txt").read_text()
    assert "#   cmd one" in text and "#   cmd two" in text
    # scales from the median of the three 1 GiB copies
    assert "fetch_scale: 2.0000" in text and "write_scale: 1.0000" in text
    # grid 102400: (1000 * 2 + 10) KiB; grid 138240: (3000 * 2 + 30) KiB; mean over the launches
    expect = ((1000 * 2 + 10) + (3000 * 2 + 30)) * 1024 / 2
    digest = bench.src_digest(fake_root / SRC)
    assert bench.read_pmc("traffic.txt", digest) == pytest.approx(expect, abs=1)

    # another kernel source, or another build recipe, and the figure is no longer reported
    (fake_root / SRC).write_text("// kernel, second build\n")
    assert bench.src_digest(fake_root / SRC) != digest
    assert bench.read_pmc("traffic.txt", bench.src_digest(fake_root / SRC)) is None
    (fake_root / SRC).write_text("// kernel, first build\n")
    assert bench.src_digest(fake_root / SRC) == digest
    (fake_root / "ternary_weight_quantized_bonsai_amd" / "build.py").write_text("FLAGS = ['-O2']\n")
    assert bench.src_digest(fake_root / SRC) != digest
    assert bench.read_pmc("missing.txt", digest) is None
