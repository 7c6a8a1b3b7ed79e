"""Host-side logic of bench.py (CPU only): the one-GPU refusal, the HBM-traffic summary built
from rocprofv3 counter CSVs and calibrated by the stream probes, the digest gate that keeps
counters taken on one build of a kernel from being reported for another, and the small helpers
of the bench line."""
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


def test_traffic_summary_scales_by_the_stream_probes_and_gates_on_the_digest(fake_root, capsys):
    kern = "void bonsai::(anonymous namespace)::q1_gemv_lut4_kernel<64, true, false, 4>(unsigned int const*)"
    other = "void bonsai::(anonymous namespace)::q1_gemv_lutp_kernel<true, false>(unsigned int const*)"
    rd, lds, wr = "probe_read_kernel", "probe_lds_kernel", "probe_write_kernel"
    pk = bench.PROBE_BYTES / 1024
    # The read probe's PROBE_BYTES show as half as many KiB of FETCH_SIZE (scale 2), the write
    # probe's as exactly as many KiB of WRITE_SIZE (scale 1).  The kernel runs on two grids,
    # FETCH_SIZE of one dispatch split over two rows; another kernel is not counted.
    fetch = [(1, rd, 131072, pk / 2), (2, rd, 131072, pk / 2 + 5), (3, rd, 131072, pk / 2 - 5),
             (4, lds, 131072, pk / 2), (5, kern, 102400, 600.0), (5, kern, 102400, 400.0),
             (6, kern, 138240, 3000.0), (7, other, 131072, 9e6)]
    write = [(8, wr, 131072, pk), (9, wr, 131072, pk), (5, kern, 102400, 10.0), (6, kern, 138240, 30.0),
             (7, other, 131072, 1e4)]
    _counter_csv(fake_root / "f" / "run" / "f_counter_collection.csv", "FETCH_SIZE", fetch)
    _counter_csv(fake_root / "w" / "run" / "w_counter_collection.csv", "WRITE_SIZE", write)
    bench.summarize_pmc(str(fake_root / "f"), str(fake_root / "w"), "traffic.txt", ["cmd one", "cmd two"],
                        "q1_gemv_lut4_kernel", SRC)
    capsys.readouterr()
    text = (fake_root / "profiles" / "traffic.txt").read_text()
    assert "#   cmd one" in text and "#   cmd two" in text
    # scales from the median of the read probe's dispatches and from the write probe
    assert "fetch_scale: 2.0000" in text and "write_scale: 1.0000" in text
    # grid 102400: (1000 * 2 + 10) KiB; grid 138240: (3000 * 2 + 30) KiB; mean over the launches
    expect = ((1000 * 2 + 10) + (3000 * 2 + 30)) * 1024 / 2
    digest = bench.src_digest(fake_root / SRC)
    assert bench.read_pmc("traffic.txt", digest) == pytest.approx(expect, abs=1)
    # one grid only
    bench.summarize_pmc(str(fake_root / "f"), str(fake_root / "w"), "traffic1.txt", [], "q1_gemv_lut4_kernel",
                        SRC, grid=138240)
    capsys.readouterr()
    assert bench.read_pmc("traffic1.txt", digest) == pytest.approx((3000 * 2 + 30) * 1024, abs=1)

    # another kernel source, or another build recipe, and the figure is no longer reported
    (fake_root / SRC).write_text("// kernel, second build\n")
    assert bench.src_digest(fake_root / SRC) != digest
    assert bench.read_pmc("traffic.txt", bench.src_digest(fake_root / SRC)) is None
    (fake_root / SRC).write_text("// kernel, first build\n")
    assert bench.src_digest(fake_root / SRC) == digest
    (fake_root / "ternary_weight_quantized_bonsai_amd" / "build.py").write_text("FLAGS = ['-O2']\n")
    assert bench.src_digest(fake_root / SRC) != digest
    assert bench.read_pmc("missing.txt", digest) is None


def test_launch_distribution_and_kernel_names():
    d = bench.dist_us([0.001 * v for v in range(1, 11)])      # 1 .. 10 us
    assert d["mean_us"] == pytest.approx(5.5) and d["median_us"] == pytest.approx(5.5)
    assert d["p10_us"] == pytest.approx(1.9) and d["p90_us"] == pytest.approx(9.1) and d["launches"] == 10
    assert bench.kernel_of("launch_lutp[AFF = false] grid=256,1 block=512 lds=163840") == "q1_gemv_lutp_kernel"
    assert bench.kernel_of("launch_lut8_t[W = 16, PD = 4, UMAX = 8] grid=256,1 block=1024 lds=141312") == \
        "q1_gemv_lut8_kernel"
    assert bench.kernel_of("q1_gemm_kernel<false, 16> grid=216,1 block=256 lds=0") == "q1_gemm_kernel"
    assert bench.KERNEL_SRC[bench.HEADLINE_KERNEL].endswith(".hip")


def test_sysfs_clocks_without_a_device_are_null():
    assert bench.sysfs_clocks(None) == {"sclk_dpm_mhz": None, "mclk_dpm_mhz": None}
    assert bench.sysfs_clocks("ffff:ff:ff.0") == {"sclk_dpm_mhz": None, "mclk_dpm_mhz": None}
