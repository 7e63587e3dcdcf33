"""bench.py's command line where no GPU is needed: a run on more than one GPU is refused
with a message (the library has no multi-GPU path), before anything touches a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2", "--steps", "1", "--warmup", "0"],
                       cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr
    assert r.stdout == ""   # no JSON line for a refused run


def test_traffic_readings_are_tied_to_the_gemm_sources(monkeypatch):
    """A stored FETCH_SIZE/WRITE_SIZE reading is reported only while the GEMM sources
    still hash to the value it was taken at; otherwise the bench reports null."""
    sys.path.insert(0, ROOT)
    import bench

    cur = bench.gemm_source_sha16()
    assert bench.TRAFFIC["fc1"].get(bench.HEADLINE) is not None
    for kind, table in bench.TRAFFIC.items():
        for w, (val, sha) in table.items():
            got, note = bench.traffic(kind, w)
            if sha == cur:
                assert got == val and sha in note
            else:
                assert got is None and sha in note and cur in note
    assert bench.traffic("fc1", "no_such_workload")[0] is None
    monkeypatch.setattr(bench, "gemm_source_sha16", lambda: "0" * 16)
    assert all(bench.traffic(k, w)[0] is None for k, t in bench.TRAFFIC.items() for w in t)
