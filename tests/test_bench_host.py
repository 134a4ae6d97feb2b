"""Host-side contracts of bench.py (no GPU needed).

* Every workload's committed rocprofv3 summary (profiles/) was taken on the
  current kernel source: its source hash matches, so the bench line carries
  the measured HBM traffic rather than null.  A kernel change without new
  profiles fails here.
* The hash covers the kernel's own file and the shared headers, and changes
  when either does.
* --gpus N with N > 1 exits with a message before any GPU work (one GPU is
  what this benchmark measures)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("workload", sorted(bench.KERNEL_NAME))
def test_committed_profile_matches_current_source(workload):
    tag = bench.KERNEL_NAME[workload]
    traffic = bench.load_traffic(tag, workload)
    assert traffic is not None, f"profiles/ summary for {workload} missing or taken on other kernel source"
    assert traffic > 0


def test_source_hash_covers_kernel_and_headers(tmp_path, monkeypatch):
    tag = bench.KERNEL_NAME["block_window"]
    h0 = bench.kernel_source_hash(tag)
    assert h0 == bench.kernel_source_hash(tag)
    # a copy of the sources with one header byte changed hashes differently
    src = os.path.join(ROOT, "recsys_jagged_attention_amd", "csrc")
    dst = tmp_path / "recsys_jagged_attention_amd" / "csrc"
    dst.mkdir(parents=True)
    for f in (bench.KERNEL_SOURCE[tag.split("<")[0]],) + bench.KERNEL_HEADERS:
        data = open(os.path.join(src, f), "rb").read()
        if f == bench.KERNEL_HEADERS[0]:
            data += b"\n"
        (dst / f).write_bytes(data)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.kernel_source_hash(tag) != h0


@pytest.mark.parametrize("extra", [[], ["--backward"], ["--mx-quantize"]])
def test_more_than_one_gpu_is_refused(extra):
    env = dict(os.environ, HIP_VISIBLE_DEVICES="")  # (no GPU work may happen anyway)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"] + extra, cwd=ROOT,
                       env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
