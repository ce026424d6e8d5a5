"""bench.py's host-side contract, on the CPU: it refuses more than one GPU
before touching any, and every HBM-traffic record in profiles/ that it reads
is well formed and names source files that exist."""
import glob
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _records():
    out = []
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        for line in open(path):
            if "<!-- traffic:" in line:
                body = line.split("<!-- traffic:", 1)[1].rsplit("-->", 1)[0]
                out.append((os.path.basename(path), json.loads(body)))
    return out


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=300)
    assert r.returncode == 2, r.stderr[-2000:]
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_traffic_records_are_well_formed():
    recs = _records()
    workloads = {rec["workload"] for _, rec in recs}
    assert {"llama13b_decode", "long_fp8_decode", "prefix_cow", "chunked_prefill"} <= workloads
    for name, rec in recs:
        assert isinstance(rec["traffic_bytes_per_launch"], int) and rec["traffic_bytes_per_launch"] > 0, name
        assert len(rec["src_sha256"]) == 16 and int(rec["src_sha256"], 16) >= 0, name
        assert rec["kernel"], name
        for f in rec["src"]:
            assert os.path.exists(os.path.join(ROOT, f)), (name, f)


def test_traffic_lookup_follows_the_sources():
    """measured_traffic returns a record's bytes while its sources hash as
    recorded, and nothing for a workload it has no record of."""
    sys.path.insert(0, ROOT)
    import bench
    import hashlib
    assert bench.measured_traffic("no_such_workload", "decode_kernel") is None
    for _, rec in _records():
        h = hashlib.sha256()
        for f in rec["src"]:
            h.update(open(os.path.join(ROOT, f), "rb").read())
        want = rec["traffic_bytes_per_launch"] if h.hexdigest()[:16] == rec["src_sha256"] else None
        kernel = rec["kernel"].split()[0]
        got = bench.measured_traffic(rec["workload"], kernel)
        if want is not None:
            assert got == want, rec["workload"]
