"""Host-side behaviour of bench.py (no GPU): the one-GPU contract and the
guard that keeps recorded HBM-traffic figures tied to the kernel source
they were taken on."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_traffic_record_names_an_existing_source():
    tr = bench.XATTN_FWD_TRAFFIC
    path = os.path.join(ROOT, tr["source"])
    assert os.path.isfile(path)
    h = bench.source_sha16(tr["source"])
    assert len(h) == 16 and all(ch in "0123456789abcdef" for ch in h)
    # the scale factors come from the 512 MiB copy and the figures are KiB per dispatch
    assert tr["fetch_kib"] > 0 and tr["write_kib"] > 0 and tr["fetch_scale"] > 0 and tr["write_scale"] > 0


def test_alu_peak_from_unit_counts():
    # 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz lane-instructions per second
    assert abs(bench.PEAK_ALU_TLANE - 256 * 4 * 16 * 2.4e9 / 1e12) < 0.05
