"""The benchmark's own arithmetic, on the CPU: the algorithmic bytes per
coordinate each stage is measured against, the kernel-source identity that
ties committed counter summaries to the code, and the one-GPU guard."""
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_stage_bytes_at_five_bits():
    # P = (5 + 0.625)/8 = 0.703125 bytes of region per coordinate; bf16 gradients
    P, meta = 0.703125, 8 / 256
    got = {k: bench.stage_bytes_per_coord(k, 5.0, 2.0, 8, True)
           for k in ("stats", "compress", "hop_grad", "hop_packed", "hop_final", "finalize")}
    assert got["stats"] == pytest.approx(2 + 15 / 256)          # 8 B/SG written by worker 0, 16 by the rest
    assert got["compress"] == pytest.approx(2 + meta + P)      # 2.734
    assert got["hop_grad"] == pytest.approx(3.4375)            # 2P + 2 + 8/256
    assert got["hop_packed"] == pytest.approx(3 * P + meta)    # 2.141
    assert got["hop_final"] == pytest.approx(3 * P + meta + 4)  # butterfly: packed own operand
    assert got["finalize"] == pytest.approx(P + meta + 4)      # 4.734
    # a ring's last hop reads the gradient as its local operand
    assert bench.stage_bytes_per_coord("hop_final", 5.0, 2.0, 8, False) == pytest.approx(2 * P + 2 + meta + 4)
    # fp32 gradients
    assert bench.dar_bytes_per_coord(5.0, 4.0) == pytest.approx(2 * P + 4 + meta)
    assert bench.stage_bytes_per_coord("allocate", 5.0, 2.0, 8, True) is None


def test_kernel_source_hash_ignores_comments(tmp_path, monkeypatch):
    src = os.path.join(ROOT, "compressed_hop_gradient_amd", "csrc")
    fake = tmp_path / "compressed_hop_gradient_amd" / "csrc"
    fake.mkdir(parents=True)
    for f in ("dq_kernels.hip", "dq_tables.h", "dq_internal.h"):
        (fake / f).write_text(open(os.path.join(src, f)).read())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_source_hash()
    k = fake / "dq_kernels.hip"
    k.write_text("// a new comment\n/* and a block\n comment */\n" + k.read_text().replace("\n", "\n\n", 3))
    assert bench.kernel_source_hash() == h0
    k.write_text(k.read_text() + "\nstatic int one_more_line = 1;\n")
    assert bench.kernel_source_hash() != h0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
