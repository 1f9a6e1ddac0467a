"""Host-side parts of bench.py's contract: one GPU only, profile-derived traffic
only while the profiled kernel source is unchanged, the output hash, and the
GEMM kernel naming that splits the prefill roofline."""
import json
import os
import subprocess
import sys

import numpy as np
import torch

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=300, cwd=ROOT)
    assert r.returncode != 0
    line = [l for l in r.stdout.splitlines() if l.startswith("{")][-1]
    assert "--gpus must be 1" in json.loads(line)["error"]


def test_profiled_traffic_needs_the_profiled_source(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("kernel v1\n")
    import hashlib
    sha = hashlib.sha256(src.read_bytes()).hexdigest()
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "p.txt").write_text(f"traffic_bytes_per_launch: 1234\nsource_sha256: {sha}\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.profiled_traffic("p.txt", "k.hip") == 1234
    assert bench.profiled_traffic("p.txt", "k.hip", "other_key") is None
    src.write_text("kernel v2\n")  # the kernel changed since the counters were taken
    assert bench.profiled_traffic("p.txt", "k.hip") is None
    assert bench.profiled_traffic("missing.txt", "k.hip") is None


def test_committed_profiles_name_their_source_digest():
    """Every committed summary that reports traffic records the digest it was taken from."""
    for name in os.listdir(os.path.join(ROOT, "profiles")):
        text = open(os.path.join(ROOT, "profiles", name)).read()
        if "traffic_bytes_per_launch" in text:
            assert "source_sha256:" in text, name


def test_output_hash_covers_every_byte_in_order():
    a = torch.arange(16, dtype=torch.float32)
    b = torch.zeros(4, dtype=torch.float32)
    h = bench.outputs_sha256([a, b])
    assert h == bench.outputs_sha256([a.clone(), b.clone()])
    assert h != bench.outputs_sha256([b, a])
    c = a.clone()
    c[3] = float(np.nextafter(np.float32(3), np.float32(4)))  # one ulp above 3
    assert h != bench.outputs_sha256([c, b])


def test_gemm_kernel_names_follow_the_library_rule():
    # 128 x 128 tiles when there are at least 256 of them, else the strip kernel
    assert bench.gemm_kernel_for(2048, 2048) == "gemm_kernel"            # 16 x 16 tiles
    assert bench.gemm_kernel_for(752, 8192) == "gemm_kernel"             # 6 x 64
    assert bench.gemm_kernel_for(752, 2048) == "gemm_strip_kernel"       # 6 x 16
    assert bench.gemm_kernel_for(188, 8192) == "gemm_strip_kernel"       # 2 x 64
