"""bench.py's host-side logic, without a GPU: the algorithmic byte counts
behind ``value`` and ``roofline.achieved``, the reader of the committed
counter summary behind ``roofline.traffic`` (used only while the kernel
sources match the ones the counters were taken on), and the refusals of
more than one GPU and of workloads an op cannot take."""
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


# Forward and backward (stage 1 + stage 2) algorithmic bytes of the RMSNorm
# workloads, worked out by hand from the byte formulas: forward
# 2*M*N*s + N*s + 4*M, backward 3*M*N*s + N*s + 4*M + 4*N.
@pytest.mark.parametrize("M,N,s,fwd,bwd", [
    (32768, 4096, 2, 537_010_176, 805_462_016),           # bf16 32768 x 4096
    (262144, 1024, 2, 1_074_792_448, 1_611_667_456),      # fp16 262144 x 1024
    (2048, 65536, 2, 537_010_176, 805_707_776),           # bf16 2048 x 65536
    (65536, 5120, 2, 1_342_449_664, 2_013_558_784),       # bf16 65536 x 5120
])
def test_rmsnorm_algorithmic_bytes(M, N, s, fwd, bwd):
    f, rows, red = bench.alg_bytes(M, N, s)
    assert f == fwd
    assert rows + red == bwd
    assert red == 4 * N  # stage 2 writes the float32 dgamma only


def test_other_ops_count_their_operands():
    M, N, s = 4, 8, 2
    # LayerNorm: beta read, mean written beside rstd, dbeta beside dgamma.
    assert bench.alg_bytes(M, N, s, "layernorm") == (2 * M * N * s + 2 * N * s + 8 * M,
                                                      3 * M * N * s + N * s + 8 * M, 8 * N)
    # Fused add: x, res read and y, h written; dy, dh, h read and dx written.
    assert bench.alg_bytes(M, N, s, "add_rmsnorm") == (4 * M * N * s + N * s + 4 * M,
                                                        4 * M * N * s + N * s + 4 * M, 4 * N)
    # Cast: 4-byte x (read) and 2-byte y (written); 2-byte dy, 4-byte x and dx.
    assert bench.alg_bytes(M, N, s, "rmsnorm_cast") == (6 * M * N + 4 * N + 4 * M,
                                                         10 * M * N + 4 * N + 4 * M, 4 * N)


def _summary(path, sha, traffic="814116866"):
    with open(path, "w") as fh:
        fh.write("# HBM traffic\n\n| a | b |\n|---|---|\n")
        fh.write(f"source_sha256: {sha}\n")
        fh.write(f"traffic_bytes_per_launch: {traffic}\n")


def test_traffic_needs_matching_sources(tmp_path, monkeypatch):
    note = tmp_path / "traffic.md"
    monkeypatch.setattr(bench, "TRAFFIC_NOTE", str(note))
    assert bench.measured_traffic("c2") is None            # no summary at all
    _summary(note, bench.kernel_source_hash())
    assert bench.measured_traffic("c2") == 814116866
    assert bench.measured_traffic("c3") is None            # counters cover c2 only
    _summary(note, "0" * 64)
    assert bench.measured_traffic("c2") is None            # kernels changed since
    _summary(note, bench.kernel_source_hash(), traffic="n/a")
    assert bench.measured_traffic("c2") is None


def test_source_hash_covers_every_kernel_source(tmp_path, monkeypatch):
    """A byte changed in any file of the library's sources changes the hash
    (checked on a copy, the tree itself is untouched)."""
    import shutil
    src = os.path.join(ROOT, "backward_rmsnorm_fwd_amd", "csrc")
    fake_root = tmp_path / "root"
    shutil.copytree(src, fake_root / "backward_rmsnorm_fwd_amd" / "csrc")
    monkeypatch.setattr(bench, "ROOT", str(fake_root))
    base = bench.kernel_source_hash()
    names = sorted(os.listdir(fake_root / "backward_rmsnorm_fwd_amd" / "csrc"))
    assert len(names) >= 8
    for name in names:
        p = fake_root / "backward_rmsnorm_fwd_amd" / "csrc" / name
        orig = p.read_bytes()
        p.write_bytes(orig + b" ")
        assert bench.kernel_source_hash() != base, name
        p.write_bytes(orig)
    assert bench.kernel_source_hash() == base


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=300)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""


@pytest.mark.parametrize("argv,needle", [
    (["--workload", "c9"], "unknown workload"),
    (["--op", "layernorm", "--workload", "c0"], "unknown workload"),
])
def test_unsupported_workloads_are_refused_before_any_gpu_work(argv, needle):
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv],
                         capture_output=True, text=True, timeout=300)
    assert res.returncode == 2
    assert needle in res.stderr
    assert res.stdout == ""


@pytest.mark.parametrize("op,workload,label", [
    ("rmsnorm", "c2", "RMSNorm fwd/bwd achieved HBM GB/s and % of peak, bf16 M=32768 N=4096"),
    ("rmsnorm", "c3", "RMSNorm fwd/bwd achieved HBM GB/s and % of peak, fp16 M=262144 N=1024"),
    ("rmsnorm", "c4", "RMSNorm fwd/bwd achieved HBM GB/s and % of peak, bf16 M=2048 N=65536"),
    ("rmsnorm", "c5", "RMSNorm fwd/bwd achieved HBM GB/s and % of peak, bf16 M=65536 N=5120"),
    ("layernorm", "c3", "LayerNorm fwd/bwd achieved HBM GB/s and % of peak, fp16 M=262144 N=1024"),
    ("layernorm", "c4", "LayerNorm fwd/bwd achieved HBM GB/s and % of peak, bf16 M=2048 N=65536"),
    ("add_rmsnorm", "c4",
     "residual add + RMSNorm fwd/bwd achieved HBM GB/s and % of peak, bf16 M=2048 N=65536"),
    ("rmsnorm_cast", "c2",
     "RMSNorm + output cast fwd/bwd achieved HBM GB/s and % of peak, fp32 M=32768 N=4096"),
])
def test_metric_names_the_workload(op, workload, label):
    assert bench.metric_for(op, workload) == label
