"""The rocprofv3 summary tool's per-shape grouping (autoregressive_tts_decode_amd/prof_summary.py
--shapes), on a hand-written kernel trace: launches and kernel time per frame by kernel and launch
shape, excluded kernels left out."""
import csv
import subprocess
import sys
from pathlib import Path

ROOT = Path(__file__).resolve().parents[1]
FIELDS = ["Kernel_Name", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z", "Start_Timestamp", "End_Timestamp"]


def _trace(tmp_path: Path, rows) -> str:
    prefix = tmp_path / "bench"
    with open(str(prefix) + "_kernel_trace.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        t = 1000
        for name, gx, gz, dur in rows:
            w.writerow({"Kernel_Name": name, "Grid_Size_X": gx, "Grid_Size_Y": 1, "Grid_Size_Z": gz,
                        "Start_Timestamp": t, "End_Timestamp": t + dur})
            t += dur + 500
    return str(prefix)


def _run(*args) -> list[str]:
    out = subprocess.run([sys.executable, "-m", "autoregressive_tts_decode_amd.prof_summary", *args], cwd=ROOT,
                         capture_output=True, text=True, check=True).stdout
    return out.splitlines()


def test_shapes_groups_by_kernel_grid_and_slices(tmp_path):
    # two frames: a 4-slice and an 8-slice launch of one GEMM, a reduction; one prompt GEMM to exclude
    rows = [("void tts::k_gemm_dec<2, 256, 1>(tts::GemmArgs)", 4096, 4, 7000),
            ("void tts::k_gemm_dec<2, 256, 1>(tts::GemmArgs)", 4096, 8, 9000),
            ("tts::k_splitk_reduce(float*, int)", 1024, 1, 4000)] * 2
    rows.append(("void tts::k_gemm_bf16<false>(tts::GemmArgs)", 65536, 1, 250000))
    lines = _run(_trace(tmp_path, rows), "--shapes", "--run-frames", "2", "--exclude", "k_gemm_bf16")
    assert lines[0] == "per frame over 2 frames: 3 launches, 20.0 us of kernels"
    body = [ln.split() for ln in lines[2:]]
    # sorted by time per frame: the 8-slice GEMM (9 us), the 4-slice one (7 us), the reduction (4 us)
    # columns: grid threads in x, grid z (the slice count), launches, average us, us per frame
    assert [b[-5:] for b in body] == [["4096", "8", "1.0", "9.00", "9.0"],
                                      ["4096", "4", "1.0", "7.00", "7.0"],
                                      ["1024", "1", "1.0", "4.00", "4.0"]]
    assert not any("k_gemm_bf16" in ln for ln in lines)


def test_shapes_needs_the_frame_count(tmp_path):
    prefix = _trace(tmp_path, [("tts::k_sample(tts::SampleArgs)", 8192, 1, 12000)])
    r = subprocess.run([sys.executable, "-m", "autoregressive_tts_decode_amd.prof_summary", prefix, "--shapes"], cwd=ROOT,
                       capture_output=True, text=True)
    assert r.returncode != 0 and "--run-frames" in r.stderr
