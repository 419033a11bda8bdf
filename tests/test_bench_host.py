"""Host logic of bench.py, on the CPU: the one-GPU guard, the algorithmic
bytes that the roofline divides by (against the oracle's bytes-per-token
formula, which the pages' memory tables pin), and the HBM traffic record
(counter calibration, one entry per workload, the source-hash gate)."""
import importlib.util
import json
import shutil
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", ROOT / "bench.py")
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       cwd=ROOT, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stdout + r.stderr


@pytest.mark.parametrize("wname,mname,expect", [("K4V4_32K", "K4V4", 1_107_820_544), ("K8V4_32K", "K8V4", 822_345_728),
                                               ("K4V4_32K", "K4V4_ZP", 1_107_820_544 + 32 * 8 * 32768 * 4)])
def test_split_bytes(bench, oq, wname, mname, expect):
    """Cache bytes of every attended position of every (sequence, KV head),
    plus the fp32 queries: by the oracle's formula and by hand (the
    zero-point codec: 4 bytes per group and side instead of 2)."""
    import workloads as wl
    w, m = getattr(wl, wname), getattr(wl, mname)
    g = m.group_size(w.n_kv_heads, w.head_dim)
    per_pos = oq.bytes_per_token_zp(m.k_bits, m.v_bits, w.n_kv_heads, w.head_dim, g, int(m.zero_point))
    want = w.batch * min(w.n_pos, w.capacity) * per_pos + w.batch * w.n_q_heads * w.head_dim * 4
    assert bench.split_bytes(w, m) == want == expect


def _counter_csv(path, counter, rows):
    with open(path, "w") as f:
        f.write("Kernel_Name,Counter_Name,Counter_Value\n")
        for name, kib in rows:
            f.write(f"\"{name}\",{counter},{kib}\n")


def test_traffic_record_round_trip(bench, tmp_path, monkeypatch):
    """Counters scaled by their reading for the 1 GiB copy, averaged over the
    launches; a second workload's entry joins the first; a changed kernel
    source voids the record."""
    for f in bench.TRAFFIC_SOURCES:
        (tmp_path / f).parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(ROOT / f, tmp_path / f)
    monkeypatch.setattr(bench, "ROOT", tmp_path)
    copy = "__amd_rocclr_copyBuffer"
    dec = "void kvq::decode_quant_kernel<4, 4, 128, 4, 1, false, false>(kvq::QuantParams)"
    # FETCH_SIZE reads half of the copy's 1 GiB (factor 2); WRITE_SIZE all of it
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE", [(copy, 524288), (dec, 1000), (dec, 1002), (dec, 1004)])
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE", [(copy, 1048576), (dec, 10), (dec, 10), (dec, 10)])
    assert bench.record_traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "k4v4-32k", log=lambda *a: None) == 0
    e = bench.traffic_record("k4v4-32k/k4v4")
    assert e["fetch_bytes"] == 2 * 1002 * 1024 and e["write_bytes"] == 10 * 1024
    assert e["bytes_per_launch"] == e["fetch_bytes"] + e["write_bytes"]
    assert bench.traffic_record("k8v4-32k/k8v4") is None
    _counter_csv(tmp_path / "f8.csv", "FETCH_SIZE", [(copy, 524288), (dec.replace("<4, 4", "<8, 4"), 700)])
    _counter_csv(tmp_path / "w8.csv", "WRITE_SIZE", [(copy, 1048576), (dec.replace("<4, 4", "<8, 4"), 5)])
    bench.record_traffic(str(tmp_path / "f8.csv"), str(tmp_path / "w8.csv"), "k8v4-32k", log=lambda *a: None)
    assert bench.traffic_record("k8v4-32k/k8v4")["fetch_bytes"] == 2 * 700 * 1024
    assert bench.traffic_record("k4v4-32k/k4v4") == e
    rec = json.loads((tmp_path / "profiles" / "traffic.json").read_text())
    assert set(rec["workloads"]) == {"k4v4-32k/k4v4", "k8v4-32k/k8v4"}
    with open(tmp_path / bench.TRAFFIC_SOURCES[0], "a") as f:
        f.write("\n// changed\n")
    assert bench.traffic_record("k4v4-32k/k4v4") is None


def test_committed_traffic_record_is_well_formed(bench):
    rec = json.loads((ROOT / "profiles" / "traffic.json").read_text())
    assert rec["sources"] == bench.TRAFFIC_SOURCES
    for key, e in rec["workloads"].items():
        assert e["bytes_per_launch"] == e["fetch_bytes"] + e["write_bytes"], key
        assert 1.0 <= e["ratio_to_algorithmic"] < 1.05, key
