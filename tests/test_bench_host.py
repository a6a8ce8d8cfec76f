"""bench.py's host logic, on the CPU: the one-GPU guard, and the rule that a
committed HBM-traffic figure is reported only while the kernel sources it was
taken from are unchanged."""
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("args,world", [(["--gpus", "2"], "1"), (["--gpus", "8"], "1"), ([], "2")])
def test_more_than_one_gpu_is_refused(args, world):
    env = dict(os.environ, WORLD_SIZE=world)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], env=env, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""                  # no JSON line


def _summary(tmp_path, name, digest, traffic):
    (tmp_path / f"{name}.md").write_text(f"# {name}\n\nkernel_source_sha256_16: {digest}\n"
                                         f"traffic_bytes_per_launch: {traffic}\n")


def test_traffic_is_reported_only_for_the_current_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    k = "k_gemm_small_m_rx"
    cur = bench.kernel_sources_hash(k)
    _summary(tmp_path, "same", cur, "53533966.0")
    assert bench.load_traffic("same", k) == 53533966.0
    stale = "0" * 16 if cur != "0" * 16 else "1" * 16
    _summary(tmp_path, "stale", stale, "53533966.0")
    assert bench.load_traffic("stale", k) is None
    assert bench.load_traffic("missing", k) is None
    (tmp_path / "nohash.md").write_text("traffic_bytes_per_launch: 1.0\n")
    assert bench.load_traffic("nohash", k) is None


def test_kernel_files_follow_the_includes():
    """Every quoted include of a kernel's source, and of those headers in turn,
    is in its file list (the activation-quant helpers the small-M kernel uses
    included)."""
    import re
    for kernel in ("k_gemm_small_m_rx", "k_gemm_large_m_tiled", "k_silu_mul_quant"):
        files = bench.kernel_files(kernel)
        for rel in files:
            base = os.path.dirname(rel)
            for inc in re.findall(r'#include "([^"]+)"', open(os.path.join(bench.CSRC, rel)).read()):
                assert os.path.normpath(os.path.join(base, inc)) in files, (kernel, rel, inc)
    assert "act_quant.h" in bench.kernel_files("k_gemm_small_m_rx")
    assert "act_quant.h" not in bench.kernel_files("k_gemm_large_m_tiled")


def test_source_hash_covers_every_byte(tmp_path, monkeypatch):
    """One changed byte in a header only one kernel includes changes that
    kernel's digest and no other (the staleness rule above rests on it)."""
    src = tmp_path / "pkg" / "csrc"
    inc = tmp_path / "include"
    src.mkdir(parents=True)
    inc.mkdir()
    for kernel in ("k_gemm_small_m_rx", "k_gemm_large_m_tiled"):
        for rel in bench.kernel_files(kernel):
            dst = os.path.normpath(os.path.join(str(src), rel))
            with open(os.path.join(bench.CSRC, rel), "rb") as fh:
                data = fh.read()
            with open(dst, "wb") as out:
                out.write(data)
    small, large = "k_gemm_small_m_rx", "k_gemm_large_m_tiled"
    h_small, h_large = bench.kernel_sources_hash(small), bench.kernel_sources_hash(large)
    monkeypatch.setattr(bench, "CSRC", str(src))
    assert (bench.kernel_sources_hash(small), bench.kernel_sources_hash(large)) == (h_small, h_large)
    p = src / "act_quant.h"
    b = bytearray(p.read_bytes())
    b[len(b) // 2] ^= 0x01
    p.write_bytes(bytes(b))
    assert bench.kernel_sources_hash(small) != h_small
    assert bench.kernel_sources_hash(large) == h_large
