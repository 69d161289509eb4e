"""Host-side logic of bench.py (CPU): the one-GPU refusal, the algorithmic byte count the roofline
divides by, the scaling of the HBM counters by the copy calibration, and that the committed counter
summary still describes the current kernel sources."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from chunked_gated_delta_amd import inputs as gen  # noqa: E402


def test_refuses_more_than_one_gpu():
    """--gpus 2 exits with a message before anything touches a GPU."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr and r.stdout == ""


def test_algorithmic_bytes_headline():
    """q, k, w, v read, o written (bf16, d = 128): 1282 bytes per token and head, plus the fp32 final
    state: 1.345 GB for B1 H16 T65536."""
    wl = gen.WORKLOADS["headline"]
    per = (3 * 128 + 2 * 128) * 2 + 2
    assert per == 1282
    assert bench.algorithmic_bytes(wl) == 16 * 65536 * per + 16 * 128 * 128 * 4 == 1345323008


def _csv(path, rows):
    with open(path, "w") as f:
        f.write('"Dispatch_Id","Kernel_Name","Counter_Name","Counter_Value"\n')
        for d, k, c, v in rows:
            f.write(f'{d},"{k}","{c}",{v}\n')


def test_summarize_pmc_scaling(tmp_path, monkeypatch):
    """Counters of the last dispatch per kernel, summed over their instances, scaled by what the
    same counters read for a 1 GiB copy."""
    f, w, cf, cw = (str(tmp_path / n) for n in ("f.csv", "w.csv", "cf.csv", "cw.csv"))
    out = str(tmp_path / "t.json")
    # two dispatches of the output pass (the last one counts), two instances in the last one
    _csv(f, [(1, "void kda::fused_kernel<true, false>(...)", "FETCH_SIZE", 10.0),
             (2, "void kda::fused_kernel<true, false>(...)", "FETCH_SIZE", 100.0),
             (2, "void kda::fused_kernel<true, false>(...)", "FETCH_SIZE", 28.0),
             (2, "void kda::seg_combine_kernel(...)", "FETCH_SIZE", 4.0)])
    _csv(w, [(2, "void kda::fused_kernel<true, false>(...)", "WRITE_SIZE", 64.0)])
    gib_kib = (1 << 30) / 1024
    _csv(cf, [(7, "__amd_rocclr_copyBuffer", "FETCH_SIZE", gib_kib / 2)])   # reads half of the copy
    _csv(cw, [(7, "__amd_rocclr_copyBuffer", "WRITE_SIZE", gib_kib)])
    monkeypatch.setattr(bench, "source_hash", lambda: "test")
    bench.summarize_pmc(f, w, cf, cw, out, "headline")
    d = json.load(open(out))
    assert d["fetch_scale"] == pytest.approx(2.0) and d["write_scale"] == pytest.approx(1.0)
    assert d["kernels"]["fused_out"]["fetch_bytes"] == pytest.approx(128 * 1024 * 2.0)
    assert d["kernels"]["fused_out"]["write_bytes"] == pytest.approx(64 * 1024)
    assert d["kernels"]["seg_combine"]["fetch_bytes"] == pytest.approx(4 * 1024 * 2.0)
    assert d["bytes_per_call"] == pytest.approx((128 * 2 + 64 + 4 * 2) * 1024)


def test_committed_traffic_tied_to_sources():
    """bench.py reports the counter bytes of profiles/traffic_headline.json only while the kernels are
    the ones the counters were taken from (same source hash), and null otherwise."""
    d = json.load(open(os.path.join(ROOT, "profiles", "traffic_headline.json")))
    if d["source_hash"] == bench.source_hash():
        assert bench.measured_traffic("headline") == d["bytes_per_call"]
    else:
        assert bench.measured_traffic("headline") is None


def test_source_hash_ignores_comments_only():
    """The hash that ties the counters to the kernels covers code, not comments: editing a comment
    keeps it, editing code (an operator, a constant) changes it."""
    base = {rel: open(os.path.join(ROOT, rel), encoding="utf-8").read() for rel in bench.KERNEL_SOURCES}
    rel = bench.KERNEL_SOURCES[1]
    h0 = bench.source_hash(lambda r: base[r])
    commented = dict(base)
    commented[rel] = "// a new comment line\n" + base[rel].replace("\n", "  /* note */\n", 1)
    assert bench.source_hash(lambda r: commented[r]) == h0
    changed = dict(base)
    changed[rel] = base[rel] + "\nconstexpr int kUnusedProbe = 1;\n"
    assert bench.source_hash(lambda r: changed[r]) != h0
