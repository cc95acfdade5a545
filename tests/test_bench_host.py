"""Host-side checks of bench.py's contract that need no GPU: it refuses more
than one GPU, it reports HBM traffic only from a committed counter summary
whose kernel sources still hash the same, and its CPU baseline is the
oracle on one thread with the fields the result line carries."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_committed_traffic_matches_the_summary_and_its_sources():
    """The summary's figure when its kernel sources still hash as recorded,
    None once they differ (then the counters must be taken again)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "k_rot_qgemv1__qwen3-4b-36L-b1__hbm_traffic.md")
    lines = open(path).read().splitlines()
    want = [int(line.split(": ")[1]) for line in lines if line.startswith("traffic_bytes_per_launch:")][0]
    files = [line.split(": ", 1)[1].split() for line in lines if line.startswith("kernel_source:")][0]
    recorded = [line.split(": ", 1)[1].strip() for line in lines if line.startswith("kernel_source_sha256:")][0]
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    got = bench.committed_traffic("k_rot_qgemv1", "qwen3-4b-36L-b1")
    assert got == (want if h.hexdigest() == recorded else None)
    assert bench.committed_traffic("no_such_kernel", "no-workload") is None


def test_committed_traffic_is_null_once_a_source_changes(tmp_path, monkeypatch):
    """A copy of the tree whose kernel source differs by one byte: the
    summary's hash no longer matches and no traffic is reported."""
    prof = tmp_path / "profiles"
    prof.mkdir()
    import hashlib
    src = open(os.path.join(ROOT, "profiles", "k_rot_qgemv1__qwen3-4b-36L-b1__hbm_traffic.md")).read()
    files = [line.split(": ", 1)[1].split() for line in src.splitlines() if line.startswith("kernel_source:")][0]
    h = hashlib.sha256()
    for f in files:
        dst = tmp_path / f
        dst.parent.mkdir(parents=True, exist_ok=True)
        data = open(os.path.join(ROOT, f), "rb").read()
        dst.write_bytes(data)
        h.update(data)
    # the summary as if its counters had been taken on these very sources
    src = "\n".join(f"kernel_source_sha256: {h.hexdigest()}" if line.startswith("kernel_source_sha256:") else line
                    for line in src.splitlines())
    (prof / "k_rot_qgemv1__w__hbm_traffic.md").write_text(src)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.committed_traffic("k_rot_qgemv1", "w") is not None
    with open(tmp_path / files[0], "ab") as fh:
        fh.write(b"\n")
    assert bench.committed_traffic("k_rot_qgemv1", "w") is None


def test_cpu_baseline_fields():
    r = bench.cpu_baseline(seconds=0.2)
    assert r["kind"] == "oracle" and r["cores"] == 1 and r["unit"] == "GB/s"
    assert r["value"] > 0 and "coded bytes" in r["sample"]
