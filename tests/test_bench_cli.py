"""The benchmark's host-side contract (no GPU): the refusal of several GPUs,
the kernel source hashes, and the traffic records kept under profiles/.

A traffic record ties rocprofv3 HBM byte counts to one kernel's sources (a
hash of their code without comments), a workload, a block size and a
partition size; the bench line reports it only while the hash matches.
"""
import glob
import json
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

RECORD = re.compile(r"traffic-record: kernel=(\S+) workload=(\S+) B=(\d+) P=(\d+) TW=(\d+) "
                    r"source_sha256=([0-9a-f]+) read_bytes=(\d+) write_bytes=(\d+)")


def records():
    out = []
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        for m in RECORD.finditer(open(path).read()):
            out.append((os.path.basename(path),) + m.groups())
    return out


def test_several_gpus_are_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_source_hashes_cover_every_kernel():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--print-source-sha"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0
    sha = json.loads(r.stdout)
    assert set(sha) == set(bench.KERNEL_SOURCES)
    assert all(re.fullmatch(r"[0-9a-f]{64}", v) for v in sha.values())
    for files in bench.KERNEL_SOURCES.values():
        for name in files:
            assert os.path.exists(os.path.join(ROOT, "paged_kv_cache_301_amd", "csrc", name)), name


def test_hash_ignores_comments_only():
    code = "int f(int x) {\n    return x + 1;  // one\n}\n/* block */\n"
    assert bench._code_only(code) == bench._code_only(code.replace("// one", "// two"))
    assert bench._code_only(code) != bench._code_only(code.replace("x + 1", "x + 2"))


def test_traffic_records_are_well_formed():
    recs = records()
    assert recs, "no traffic records under profiles/"
    seen = set()
    for path, kernel, workload, B, P, TW, sha, rb, wb in recs:
        assert kernel in bench.KERNEL_SOURCES, (path, kernel)
        assert int(rb) > 0 and int(wb) >= 0 and int(TW) in (1, 2, 4), path
        key = (kernel, workload, int(B), int(P), int(TW), sha)
        assert key not in seen, f"duplicate record {key} in {path}"
        seen.add(key)


@pytest.mark.parametrize("kernel,workload,B", [
    ("pa_valu_partitions", "mha_7b", 16),
    ("pa_mfma_partitions", "gqa_70b", 16),
    ("pa_mfma_partitions", "gqa_long", 16),
])
def test_headline_workloads_have_current_records(kernel, workload, B):
    """The decode workloads the targets name carry HBM traffic measured on the
    current kernel sources, at the partition and token-waves the automatic
    plan picks.  After
    a kernel change the records are stale until the profiles are taken again:
    reported as a skip naming the record (the bench line then reports traffic
    null), not as a failure."""
    from paged_kv_cache_301_amd import binding, workloads
    sp = workloads.SPECS[workload].replace(B=B)
    max_blocks = (sp.max_len + B - 1) // B
    p = binding.plan(sp.S, sp.Hq, sp.Hkv, sp.D, B, 1 << 20, max_blocks,
                     workloads._DTYPES[sp.dtype])
    P, TW = p["partition_tokens"], p["token_waves"]
    assert any(r[1:6] == (kernel, workload, str(B), str(P), str(TW)) for r in records()), \
        f"no record at all for {kernel} {workload} B={B} P={P} TW={TW}"
    got = bench.recorded_traffic(kernel, workload, B, P, TW)
    if got is None:
        pytest.skip(f"traffic record for {kernel} {workload} predates the current kernel "
                    "sources: profile again")
    assert got > 0


def test_prefill_roofline_picks_the_binding_floor():
    """Four new tokens per sequence on the chunked-prefill batch read 341 MB
    of K+V for 5.4 GFLOP: HBM binds.  512 new tokens: 663 GFLOP on the same
    bytes, the matrix cores bind.  Rates are in the bound's own unit."""
    import bench
    kv = 340672512
    bound, achieved, peak, unit = bench.prefill_roofline(kv, 5449187328, "bf16", 62.5e-6)
    assert (bound, peak, unit) == ("hbm", 8000.0, "GB/s")
    assert abs(achieved - kv / 62.5e-6 / 1e9) < 1e-6
    bound, achieved, peak, unit = bench.prefill_roofline(kv, 663404675072, "bf16", 950e-6)
    assert (bound, peak, unit) == ("mfma", 2500.0, "TFLOP/s")
    assert abs(achieved - 663404675072 / 950e-6 / 1e12) < 1e-9
    # the crossover: equal floors stay on the matrix cores
    assert bench.prefill_roofline(8e12, 2.5e15, "f16", 1.0)[0] == "mfma"   # one second each
    assert bench.prefill_roofline(8.1e12, 2.5e15, "f16", 1.0)[0] == "hbm"
