"""The benchmark's committed measurement records agree with the sources (CPU).

bench.py reports the decode kernel's HBM traffic from the counter records
under profiles/ only while the kernel's sources and build flags hash to the
digest stored with them; these tests fail when a decode source changes
without the counters being taken again, instead of the traffic silently
turning null in the benchmark line.
"""

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


RECORDS = [(idx, 1) for idx in sorted(bench.TRAFFIC_RECORDS)] + sorted(bench.GROUPED_TRAFFIC_RECORDS)


def _record_name(idx, group_size):
    return bench.TRAFFIC_RECORDS[idx] if group_size == 1 else bench.GROUPED_TRAFFIC_RECORDS[(idx, group_size)]


@pytest.mark.parametrize("idx,group_size", RECORDS)
def test_traffic_record_matches_the_decode_sources(idx, group_size):
    got = bench.traffic_bytes(idx, group_size)
    assert got is not None, (f"profiles/{_record_name(idx, group_size)} was taken on other decode sources or "
                             f"flags (digest now {bench.decode_source_digest()}): take the counters again")


@pytest.mark.parametrize("idx,group_size", RECORDS)
def test_traffic_is_close_to_the_algorithmic_bytes(idx, group_size):
    """The decode reads each K/V byte about once: the measured traffic per
    launch lies within a few percent above the algorithmic bytes.  With
    shared prefixes each physical row must leave memory at least once and
    no more often than the sequences that read it: unique <= traffic <=
    logical (the grouped decode, which loads a shared block once per chunk
    of sequences, included)."""
    import workloads as W
    case = W.make_case(W.CONFIGS[idx], device="cpu", H=1)      # lengths only; bytes scale with H
    H = W.CONFIGS[idx].H
    alg, uniq = case.kv_bytes * H, case.unique_kv_bytes * H
    got = bench.traffic_bytes(idx, group_size)
    assert got is not None
    if uniq < alg:
        assert uniq <= got <= alg, (idx, got, uniq, alg)
    else:
        assert 1.0 <= got / alg < 1.05, (idx, got, alg)


def _counter_summaries():
    prof = os.path.join(ROOT, "profiles")
    return sorted(f for f in os.listdir(prof)
                  if f.startswith(("paged_decode_kernel.", "paged_decode_group_kernel.")) and f.endswith(".counters.md"))


@pytest.mark.parametrize("name", _counter_summaries())
def test_counter_summaries_match_the_decode_sources(name):
    """The occupancy, LDS and L2 summaries of the decode kernel name the
    digest of the sources they were taken on; a change to a decode source
    makes them stale as it makes the traffic records stale."""
    import re
    text = open(os.path.join(ROOT, "profiles", name)).read()
    m = re.search(r"digest: `([0-9a-f]{16})`", text)
    assert m, f"{name} names no decode source digest"
    assert m.group(1) == bench.decode_source_digest(), (
        f"profiles/{name} was taken on other decode sources or flags: take the counters again")


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}), ([], {"WORLD_SIZE": "2"})])
def test_bench_refuses_more_than_one_gpu(argv, env):
    """The benchmark measures one GPU; asked for more (by flag or by a
    launcher's WORLD_SIZE) it exits with status 2 and says so, before any
    GPU work."""
    import subprocess
    e = {k: v for k, v in os.environ.items() if k != "WORLD_SIZE"}
    e.update(env)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], cwd=ROOT, env=e,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2, r.stdout + r.stderr
    assert "one GPU only" in r.stdout + r.stderr
    assert not r.stdout.strip().startswith("{"), "no benchmark line may be printed"
