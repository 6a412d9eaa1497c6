"""The benchmark's HBM-traffic figure comes from committed rocprofv3 counter
summaries (profiles/pa_decode_<workload>[_shared_mode]_traffic.md). It is
reported only for the summary's own workload, partition size and mode, and
only while the kernel sources the summary names are unchanged."""

import glob
import os
import re

import bench


def _fields(path):
    return dict(re.findall(r"^- (\w+): `([^`]*)`", open(path).read(), flags=re.M))


def test_committed_summaries_parse():
    paths = glob.glob(os.path.join(bench.PROFILES, "*_traffic.md"))
    assert paths
    for path in paths:
        f = _fields(path)
        for key in ("workload", "partition_size", "decode_source_sha256",
                    "fetch_kib_per_launch", "write_kib_per_launch", "traffic_bytes_per_launch"):
            assert key in f, f"{os.path.basename(path)}: no {key}"
        shared = path.endswith("_shared_mode_traffic.md")
        assert bench.traffic_file(f["workload"], shared) == path
        total = (float(f["fetch_kib_per_launch"]) * float(f["fetch_scale"]) +
                 float(f["write_kib_per_launch"]) * float(f["write_scale"])) * 1024
        assert abs(total - float(f["traffic_bytes_per_launch"])) < 1024
        for name in f.get("sources", " ".join(bench.DECODE_SRCS)).split():
            assert os.path.exists(os.path.join(bench.CSRC, name)), name


def _write(dirpath, workload, shared, P, sha, sources=None, scope="partials+merge"):
    lines = [f"- workload: `{workload}`", f"- partition_size: `{P}`",
             f"- decode_source_sha256: `{sha}`", "- traffic_bytes_per_launch: `12345`"]
    if scope:
        lines.append(f"- scope: `{scope}`")
    if sources:
        lines.append(f"- sources: `{sources}`")
    name = f"pa_decode_{workload}{'_shared_mode' if shared else ''}_traffic.md"
    with open(os.path.join(dirpath, name), "w") as fh:
        fh.write("# t\n\n" + "\n".join(lines) + "\n")


def test_traffic_is_tied_to_workload_mode_and_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    srcs = "pa_decode_kernel.h pa_device.h pa_prefix.hip"
    _write(tmp_path, "wl_a", False, -1, bench.decode_source_hash())
    _write(tmp_path, "wl_a", True, -1, bench.decode_source_hash(tuple(srcs.split())), srcs)
    _write(tmp_path, "wl_b", False, 512, "0" * 16)
    assert bench.committed_traffic("wl_a", -1) == 12345.0
    assert bench.committed_traffic("wl_a", -1, shared=True) == 12345.0
    assert bench.committed_traffic("wl_a", 512) is None          # other partition size
    assert bench.committed_traffic("wl_c", -1) is None           # no summary
    assert bench.committed_traffic("wl_b", 512) is None          # sources changed since
    # a summary whose hash covers fewer files than it names is stale
    _write(tmp_path, "wl_d", False, -1, bench.decode_source_hash(), srcs)
    assert bench.committed_traffic("wl_d", -1) is None
    # a split decode's figure must cover the partials kernel and the merge
    _write(tmp_path, "wl_e", False, -1, bench.decode_source_hash(), scope=None)
    assert bench.committed_traffic("wl_e", -1) is None
    _write(tmp_path, "wl_e", False, 0, bench.decode_source_hash(), scope=None)
    assert bench.committed_traffic("wl_e", 0) == 12345.0         # single pass: one kernel
