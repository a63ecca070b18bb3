"""bench.py contract checks that need no GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_bytes():
    # 2 x 262144 vectors x (256 B fp16 in + 48 B codes + 4 B norm) at 3 bits
    assert bench.quant_bytes(2 * 262144, 3) == 161480704
    # K and V records of 262144 (token, KV head) pairs
    assert bench.decode_bytes(262144, 3) == 27262976


def test_traffic_record_tracks_the_kernel_source(tmp_path, monkeypatch):
    rec = tmp_path / "rec.md"
    src = tmp_path / "k.hip"
    src.write_text("// the kernel\nint kernel_v1;\n")
    sha = bench.source_sha(str(src))
    rec.write_text("- code_sha256: `%s`\n- traffic_bytes_per_launch: `123`\n" % sha)
    monkeypatch.setattr(bench, "TRAFFIC_RECORD", str(rec))
    monkeypatch.setattr(bench, "QUANT_SRC", str(src))
    assert bench.read_traffic() == 123.0
    src.write_text("// the kernel, described anew\n\nint kernel_v1;  /* same code */\n")
    assert bench.read_traffic() == 123.0  # comments and blank lines do not count
    src.write_text("// the kernel\nint kernel_v2;\n")  # the code changed since the counters were taken
    assert bench.read_traffic() is None
