"""The counter summaries behind the benchmark's `traffic` field (no GPU
needed): rocprofv3 --pmc rows are reduced to per-kernel medians, scaled by
what the same counter reads for the copy probe of known size, and the stored
result is used only while the kernel sources are the ones it was taken on."""
import csv
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
from combine_ep_get_dispatch_amd import profiling as P  # noqa: E402
from combine_ep_get_dispatch_amd.traffic import algorithmic_bytes  # noqa: E402

FIELDS = ["Dispatch_Id", "Grid_Size", "Kernel_Name", "Workgroup_Size", "Counter_Name", "Counter_Value"]
COPY = "void moedisp::(anonymous namespace)::moedisp_probe_copy(moedisp::ProbeArgs)"
PULL = "void moedisp::(anonymous namespace)::moedisp_scatter_pull<3, 1>(moedisp::DispatchArgs)"
OTHER = "void at::native::vectorized_elementwise_kernel<16, at::native::FillFunctor<unsigned char> >(int)"


def _write_run(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "x_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Grid_Size": 1024, "Kernel_Name": name, "Workgroup_Size": 256,
                        "Counter_Name": counter, "Counter_Value": value})


def test_short_names():
    assert P.short_name(PULL) == "moedisp_scatter_pull<3,1>"
    assert P.short_name(COPY) == "moedisp_probe_copy"
    assert P.short_name(OTHER) == ""


def test_summary_scales_by_the_copy_probe(tmp_path):
    """Counters of 1 unit per 2048 B read and per 1024 B written (the probe's
    1 GiB each way gives those factors back), medians over dispatches,
    kernels that are not the library's ignored."""
    gib = 1 << 30
    f, w = str(tmp_path / "f"), str(tmp_path / "w")
    _write_run(f, "FETCH_SIZE", [(COPY, gib / 2048), (COPY, gib / 2048 + 8), (COPY, gib / 2048 - 8),
                                 (PULL, 30000), (PULL, 29000), (PULL, 31000), (OTHER, 5)])
    _write_run(w, "WRITE_SIZE", [(COPY, gib / 1024)] * 3 + [(PULL, 460000)] * 3 + [(OTHER, 7)])
    s = P.summarise(f, w, gib, "test")
    assert s["calibration"]["fetch_bytes_per_unit"] == pytest.approx(2048)
    assert s["calibration"]["write_bytes_per_unit"] == pytest.approx(1024)
    k = s["kernels"]["moedisp_scatter_pull<3,1>"]
    assert k["fetch_bytes"] == pytest.approx(30000 * 2048) and k["write_bytes"] == pytest.approx(460000 * 1024)
    assert k["dispatches"] == [3, 3]
    assert set(s["kernels"]) == {"moedisp_probe_copy", "moedisp_scatter_pull<3,1>"}
    assert s["source_sha256"] == P.source_hash()


def test_stored_traffic_only_for_the_sources_it_was_taken_on(tmp_path):
    good = tmp_path / "good.json"
    good.write_text(json.dumps({"source_sha256": P.source_hash(), "kernels": {}}))
    assert P.load_traffic(str(good)) is not None
    stale = tmp_path / "stale.json"
    stale.write_text(json.dumps({"source_sha256": "0" * 64, "kernels": {}}))
    assert P.load_traffic(str(stale)) is None
    broken = tmp_path / "broken.json"
    broken.write_text("{not json")
    assert P.load_traffic(str(broken)) is None
    assert P.load_traffic(str(tmp_path / "missing.json")) is None


def test_committed_counters_against_the_byte_model():
    """profiles/hbm_traffic.json (when it matches the sources): the copy and
    the combine at the DeepSeek-V3 shape move within 0-2% of their
    algorithmic bytes, reads and writes each."""
    d = P.load_traffic(os.path.join(ROOT, "profiles", "hbm_traffic.json"))
    if d is None:
        pytest.skip("the stored counters were taken on other kernel sources")
    B = algorithmic_bytes(4096, 7168, 256, 8, 8, 32768)
    row, R, T, k = 7168 * 2, 32768, 4096, 8
    want = {"moedisp_scatter_pull": (T * row + T * k * 4, R * row + 2 * R * 4 + T * k * 4),
            "moedisp_combine": (R * row + T * k * 4 + R * 4, T * row)}
    assert sum(want["moedisp_scatter_pull"]) + B["notify"] == B["dispatch"]
    assert sum(want["moedisp_combine"]) == B["combine"]
    for kern, (rd, wr) in want.items():
        t = P.kernel_traffic(d, kern)
        assert t is not None, kern
        assert 1.0 <= t["fetch_bytes"] / rd <= 1.04, (kern, t["fetch_bytes"], rd)
        assert 0.999 <= t["write_bytes"] / wr <= 1.02, (kern, t["write_bytes"], wr)
