"""bench.py contract pieces that need no GPU: the one-GPU refusal and the rule
that HBM traffic comes from the counter summary only while the kernel's
sources are the ones the counters were taken on."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU only" in p.stderr
    assert p.stdout.strip() == ""  # no JSON line


@pytest.fixture()
def bench_mod(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    try:
        import bench
    finally:
        sys.path.remove(ROOT)
    # a private copy of the sources and a private counter summary
    csrc = tmp_path / "sparse_attention_08_amd" / "csrc"
    csrc.mkdir(parents=True)
    for files in bench.KERNEL_SOURCES.values():
        for f in files:
            src = os.path.join(ROOT, "sparse_attention_08_amd", "csrc", f)
            (csrc / f).write_bytes(open(src, "rb").read())
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    return bench


def _write_summary(bench, kernel, source_hash, nbytes):
    path = os.path.join(bench.ROOT, "profiles", "counters_prefill4k.json")
    d = {"kernels": {kernel: {"source_hash": source_hash, "hbm_bytes_per_launch": nbytes}}}
    with open(path, "w") as f:
        json.dump(d, f)


def test_traffic_follows_the_source_hash(bench_mod):
    b = bench_mod
    k = "mla_bf16_kernel"
    _write_summary(b, k, b.kernel_source_hash(k), 1234)
    assert b.traffic_from_profile(k) == 1234
    # a changed source (even one byte) makes the counters stale
    src = os.path.join(b.ROOT, "sparse_attention_08_amd", "csrc", b.KERNEL_SOURCES[k][0])
    with open(src, "ab") as f:
        f.write(b"\n")
    assert b.traffic_from_profile(k) is None
    # no summary at all
    os.remove(os.path.join(b.ROOT, "profiles", "counters_prefill4k.json"))
    assert b.traffic_from_profile(k) is None
