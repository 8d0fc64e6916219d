"""bench.py's contract, checked without a GPU: one GPU only, the method's byte
and FLOP accounting, the roofline bound, and recorded HBM traffic used only
while the kernel source it was measured on is unchanged."""

import json
import os
import subprocess
import sys
import types

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def _decode_commit_like():
    # decode_commit's sizes: T = 256 (32 requests x 8), H = 4096, L = 5,
    # 8 KV heads x 128 -> 10240 stacked rows, no bias
    return types.SimpleNamespace(T=256, H=4096, n_tot=10240, qkv_b=None, L=5, D=128,
                                 num_requests=32)


def test_algorithmic_work_of_decode_commit():
    alg = bench.algorithmic(_decode_commit_like(), written_rows=158)
    assert alg["flops"] == 2 * 256 * 10240 * 4096  # every row projected
    weight = 10240 * 4096 * 2
    hidden = 256 * 4096 * 2
    k_norm = 5 * 128 * 4
    table_rows = 256 * 128 * 4
    indices = 16 * 256 + 8 * 32
    pool_rows = 158 * 10240 * 2
    assert alg["bytes"] == weight + hidden + k_norm + table_rows + indices + pool_rows
    assert alg["bytes"] == 89_357_056


def test_bias_bytes_counted_once():
    c = _decode_commit_like()
    no_bias = bench.algorithmic(c, 100)["bytes"]
    c.qkv_b = [object()]
    assert bench.algorithmic(c, 100)["bytes"] == no_bias + 10240 * 2


def test_roofline_bound_follows_the_ridge():
    # F/B below 2.5 PFLOP/s / 8 TB/s (~312): HBM-bound, achieved in GB/s
    r = bench.roofline({"flops": 240.0e9, "bytes": 1.0e9}, 1e-3, "no_such_workload")
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert r["achieved"] == 1000.0 and r["frac"] == round(1000.0 / 8000.0, 4)
    assert r["traffic"] is None
    # above the ridge: MFMA-bound, achieved in TFLOP/s
    r = bench.roofline({"flops": 2.0e12, "bytes": 1.0e9}, 1e-3, "no_such_workload")
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["achieved"] == 2000.0 and r["frac"] == round(2000.0 / 2500.0, 4)


def test_recorded_traffic_only_for_the_current_source(tmp_path, monkeypatch):
    path = tmp_path / "traffic.json"
    sha = bench.kernel_source_hash("decode_commit")
    path.write_text(json.dumps({
        "decode_commit": {"kernel_sha": sha, "bytes_per_launch": 123},
        "prefill_8k": {"kernel_sha": "0" * 16, "bytes_per_launch": 456},
    }))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.measured_traffic("decode_commit") == 123
    assert bench.measured_traffic("prefill_8k") is None  # taken on another source
    assert bench.measured_traffic("wide_gqa_d64") is None  # never recorded


def test_executed_work_follows_the_plan():
    """Compacted commit windows project only the stored rows: the executed
    FLOPs (and so the roofline's bound) use those rows; bytes are unchanged."""
    c = _decode_commit_like()
    alg = bench.algorithmic(c, 158)
    exe = bench.executed(c, 158, {"compacts": True})
    assert exe["rows"] == 158 and exe["flops"] == 2 * 158 * 10240 * 4096
    assert exe["bytes"] == alg["bytes"]
    assert bench.executed(c, 158, {"compacts": False})["flops"] == alg["flops"]
    # wide_gqa_d64's shape: the method's count is above the ridge (MFMA), the
    # executed work below it (HBM)
    wide = types.SimpleNamespace(T=512, H=7168, n_tot=5120, qkv_b=None, L=5, D=64,
                                 num_requests=64)
    m = bench.algorithmic(wide, 276)
    e = bench.executed(wide, 276, {"compacts": True})
    assert bench.roofline(m, 50e-6, "none")["bound"] == "mfma"
    assert bench.roofline(e, 50e-6, "none")["bound"] == "hbm"


def test_spread_percentiles():
    p = bench.percentiles([1.0, 2.0, 3.0, 4.0, 5.0])
    assert p["us_median"] == 3000.0 and p["replays"] == 5
    assert p["us_p10"] == 1400.0 and p["us_p90"] == 4600.0


def test_default_run_is_every_write_config_with_prefill_headline():
    assert bench.HEADLINE == "prefill_8k" and bench.HEADLINE in bench.WRITE_CONFIGS
    assert {"tiny", "decode_commit", "prefill_8k", "biased_fp16",
            "wide_gqa_d64"} <= set(bench.WRITE_CONFIGS)


def test_weight_copies_exceed_twice_the_infinity_cache():
    """Rotating weight copies keep every step's weight out of the 256 MB
    Infinity Cache: their total exceeds twice its size, up to 64 copies."""
    mb = 1 << 20
    decode = 10240 * 4096 * 2  # decode_commit / prefill_8k stacked weight, 84 MB
    assert bench.weight_copies(decode) == 7 and 7 * decode > 2 * 256 * mb
    kv1 = 1280 * 4096 * 2
    n = bench.weight_copies(kv1)
    assert n * kv1 > 2 * 256 * mb and (n - 1) * kv1 <= 2 * 256 * mb
    assert bench.weight_copies(512 * 256 * 2) == 64  # tiny: capped
    assert bench.weight_copies(4 << 30) == 1


def test_settle_covers_the_clock_ramp():
    assert bench.SETTLE_MS >= 30.0 and bench.SETTLE_MAX_REPLAYS >= 1


def test_clock_sampler_reads_the_marked_level():
    """pp_dpm_sclk lists the clock levels and marks the current one with '*'
    (an 'S:' line when the clock sits between levels)."""
    assert bench.ClockSampler.current_mhz("S: 95Mhz *\n0: 500Mhz\n1: 2400Mhz\n") == 95
    assert bench.ClockSampler.current_mhz("0: 500Mhz\n1: 2100Mhz *\n") == 2100
    assert bench.ClockSampler.current_mhz("0: 500Mhz\n1: 2400Mhz\n") is None
