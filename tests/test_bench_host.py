"""Host-side pieces of bench.py: the roofline object and the measured-traffic lookup."""
import hashlib
import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _tree(tmp_path, src_text, sha):
    (tmp_path / "profiles").mkdir()
    (tmp_path / "k.hip").write_text(src_text)
    (tmp_path / "profiles" / "k_traffic.md").write_text(
        "notes\n\nkernel: er::k<1>\nsource: k.hip\nsource_sha256: %s\ntraffic_bytes_per_launch: 1234\n" % sha)


def test_traffic_reported_while_source_unchanged(tmp_path, monkeypatch):
    b = _bench()
    text = "kernel source\n"
    _tree(tmp_path, text, hashlib.sha256(text.encode()).hexdigest())
    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    assert b.measured_traffic("er::k<1>") == 1234.0
    assert b.measured_traffic("er::other") is None


def test_traffic_dropped_once_source_changes(tmp_path, monkeypatch):
    b = _bench()
    _tree(tmp_path, "edited source\n", hashlib.sha256(b"the source the counters saw\n").hexdigest())
    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    assert b.measured_traffic("er::k<1>") is None


def test_roofline_object_fields(monkeypatch):
    b = _bench()
    monkeypatch.setattr(b, "measured_traffic", lambda name: 2.0e6)
    kprof = [dict(name="er::a", launches=10, ms=1.0, bytes=4.0e9, flops=1.0e9),
             dict(name="er::k_gemm2<64, 1, 4, 64>", launches=5, ms=0.5, bytes=1.0e9, flops=1.0e9)]
    rf, detail = b.roofline_from(kprof)
    # dominant kernel: 4 GB in 1 ms -> 4000 GB/s against 8000 GB/s, HBM-bound
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s"
    assert abs(rf["achieved"] - 4000.0) < 1e-6 and abs(rf["frac"] - 0.5) < 1e-9
    assert rf["traffic"] == 2000000
    assert detail["kernel"] == "er::a" and detail["top_linear"]["kernel"].startswith("er::k_gemm2")


def test_traffic_needs_every_source_unchanged(tmp_path, monkeypatch):
    b = _bench()
    (tmp_path / "profiles").mkdir()
    (tmp_path / "a.hip").write_text("kernel\n")
    (tmp_path / "b.hip").write_text("host, edited\n")
    sha_a = hashlib.sha256(b"kernel\n").hexdigest()
    sha_b_old = hashlib.sha256(b"host\n").hexdigest()
    rec = "kernel: er::k<1>\nsource: a.hip\nsource_sha256: %s\nsource: b.hip\nsource_sha256: %s\n" \
          "traffic_bytes_per_launch: 99\n"
    (tmp_path / "profiles" / "k_traffic.md").write_text(rec % (sha_a, sha_b_old))
    monkeypatch.setattr(b, "ROOT", str(tmp_path))
    assert b.measured_traffic("er::k<1>") is None
    (tmp_path / "b.hip").write_text("host\n")
    assert b.measured_traffic("er::k<1>") == 99.0


def test_kernel_roles():
    b = _bench()
    assert b.kernel_role("er::k_skinny<3, 1, 2, 3>") == "draft"          # W4 drafter
    assert b.kernel_role("er::k_linear_mfma<2, 16, 1, 8>") == "draft"    # W8 drafter
    assert b.kernel_role("er::k_skinny<1, 1, 2, 2>") == "target"         # bf16 target (verify and AR)
    assert b.kernel_role("er::k_gemm2<64, 1, 4, 64>") == "target"
    assert b.kernel_role("er::k_wgemm<3, 8, 1, 1, 3>") == "draft"        # W4 weight-streaming GEMM
    assert b.kernel_role("er::k_wgemm<2, 4, 1, 1, 3>") == "draft"        # W8
    assert b.kernel_role("er::k_wgemm<2, 1, 4, 3>") == "target"          # bf16 (four arguments, MI first)
    assert b.kernel_role("er::k_attn_mfma<128, 4>") == "attention"
    assert b.kernel_role("er::k_attn_combine<true>") == "attention"


def test_more_than_one_gpu_is_refused():
    import json
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_bin_plan_counts_every_step_and_token_once():
    """The batch bins of the stop-length draw: at step k the live batch is #{stop - 1 > k}; every step
    falls in exactly one bin, the bins' tokens add up to the rollout's (the prefill token aside), and
    each bin's mean batch lies inside the bin."""
    import numpy as np
    b = _bench()
    stops = np.array([1, 2, 2, 5, 9, 9, 40, 300, 1000], dtype=np.int32)
    plan = b.bin_plan(stops, 512, len(stops))
    assert sum(p["plan_steps"] for p in plan) == int(stops.max()) - 1
    assert sum(p["plan_tokens"] for p in plan) == int((stops - 1).sum())
    for p in plan:
        assert p["lo"] < p["batch"] <= p["hi"]
        assert p["context"] >= 512
    # a hand count: steps 0..998 for the longest; batch 1 from step 299 to 998 (700 steps, context 512 + 648.5)
    last = plan[-1]
    assert (last["hi"], last["plan_steps"], last["plan_tokens"]) == (1, 700, 700)
    assert last["context"] == round(512 + (299 + 998) / 2)
