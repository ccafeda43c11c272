"""Host logic of bench.py (CPU only): the one-GPU guard, the FLOP and peak
bookkeeping of the bench parts, and the source hash that decides whether the
committed HBM counter record still describes the kernels."""
import importlib.util
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused_before_any_device_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""


def test_part_flops_and_peaks():
    b = _bench()
    # fwd: 4·B·H·N²·d; causal halves it; the backward counts 2.5x the forward.
    assert b.part_flops("fwd") == 4 * 2 * 16 * 8192 ** 2 * 128
    assert b.part_flops("fwd_causal") == 4 * 8 * 16 * 2048 ** 2 * 128 / 2
    assert b.part_flops("bwd") == 2.5 * 4 * 4 * 16 * 4096 ** 2 * 128 / 2
    assert b.part_flops("fp8") == 4 * 4 * 16 * 4096 ** 2 * 128
    assert b.part_peak("fp8") == 2 * b.part_peak("fwd") == 5.0e3


def test_source_hash_ignores_comments_and_tracks_code(tmp_path, monkeypatch):
    b = _bench()
    csrc = tmp_path / "tiled_attention_fattn_amd" / "csrc"
    csrc.mkdir(parents=True)
    src = csrc / "k.hip"
    src.write_text("int f() { return 1; }  // one\n\n")
    monkeypatch.setattr(b, "HERE", str(tmp_path))
    monkeypatch.setitem(b.KERNEL_SOURCES, "fwd", ["k.hip"])
    h0 = b.source_hash("fwd")
    src.write_text("// a comment line\nint f() { return 1; }  // two\n")
    assert b.source_hash("fwd") == h0
    src.write_text("int f() { return 2; }\n")
    assert b.source_hash("fwd") != h0


def test_committed_traffic_record_is_well_formed():
    rec = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    cal = rec["calibration"]
    assert cal["fetch_factor"] > 0 and cal["write_factor"] > 0
    b = _bench()
    for part in b.PARTS:
        assert part in rec, part
        assert rec[part]["bytes_per_launch"] > 0
        assert len(rec[part]["source_hash"]) == 16
        assert sum(k["hbm_bytes"] for k in rec[part]["kernels"].values()) == \
            rec[part]["bytes_per_launch"]
