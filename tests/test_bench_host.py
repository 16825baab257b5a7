"""bench.py's host-side arithmetic and gates (no GPU): the executed-FLOP and algorithmic-byte counts it divides by,
the source-hash gate on the recorded HBM traffic, and the one-GPU refusal."""
import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_prefill_flops_of_the_benchmark_workload():
    # Causal B4 H12 N4096: B*H*N(N+1)/2 unmasked pairs, 12 d = 768 executed FLOP per pair (two Q.K^T of width d,
    # two P.V of width 2d) and 8 d = 512 for the formula count.
    pairs = bench.prefill_pairs(4, 12, 4096)
    assert pairs == 402_751_488
    assert pairs * 12 * 64 == 309_313_142_784
    assert pairs * 8 * 64 == 206_208_761_856
    # Brute force on a tiny case: count j <= i.
    assert bench.prefill_pairs(2, 3, 5) == 2 * 3 * sum(i + 1 for i in range(5))


def test_decode_bytes_of_the_benchmark_workload():
    # K1 + K2 (64 wide) and V (128 wide) read once, Q1 + Q2 read, out written, all bf16.
    B, H, L, d = 64, 16, 8192, 64
    expect = 2 * (B * H * L * (d + d + 2 * d) + B * H * 2 * d + B * H * 2 * d)
    assert bench.decode_bytes(B, H, L, d) == expect == 4_295_491_584


def _write_record(path, src_rel, digest, nbytes):
    path.write_text("# test record\n"
                    f"leg.kernel=k\nleg.source={src_rel}\nleg.source_sha256_16={digest}\n"
                    f"leg.hbm_bytes_per_launch={nbytes}\n")


def test_traffic_used_only_while_the_source_hash_matches(tmp_path, monkeypatch):
    src_rel = "differential_attention_fwd_amd/csrc/decode_bf16.hip"
    digest = hashlib.sha256(open(os.path.join(ROOT, src_rel), "rb").read()).hexdigest()[:16]
    rec = tmp_path / "traffic.txt"
    monkeypatch.setattr(bench, "PROFILE_TRAFFIC", str(rec))
    _write_record(rec, src_rel, digest, 123456789)
    assert bench.read_traffic("leg") == 123456789.0
    _write_record(rec, src_rel, "0" * 16, 123456789)        # counters taken on another version of the kernel
    assert bench.read_traffic("leg") is None
    assert bench.read_traffic("missing_leg") is None


def test_committed_traffic_record_names_existing_sources():
    keys = {}
    for line in open(os.path.join(ROOT, "profiles", "hbm_traffic.txt")):
        if "=" in line and not line.startswith("#"):
            k, v = line.strip().split("=", 1)
            keys[k] = v
    legs = {k.split(".")[0] for k in keys if k.endswith(".source")}
    assert {"prefill", "decode", "decode_multi", "decode_paged", "backward"} <= legs
    for leg in legs:
        assert os.path.exists(os.path.join(ROOT, keys[f"{leg}.source"]))
        assert float(keys[f"{leg}.hbm_bytes_per_launch"]) > 0


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], capture_output=True, text=True,
                       env={**os.environ, **env}, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_median_statistics():
    # The reported time is the median (robust to the first, slower repetitions); mean and minimum ride along.
    st = bench.med_stats([0.5, 0.3, 0.31, 0.29, 0.3])
    assert st == {"ms": 0.3, "ms_mean": 0.34, "ms_min": 0.29}
    assert bench.med_stats([2.0, 1.0]) ["ms"] == 1.5


def test_backward_flop_counts():
    # 1280 per unmasked pair: S1, S2 (2 x 2d) and dP (2 x 2d'... one dot over the 2d value channels) once, plus dV
    # (2 x 2d) and dQ1, dQ2, dK1, dK2 (4 x 2d), d = 64, 2d' = 128: 256 + 256 + 256 + 512.
    d = 64
    assert 2 * (2 * d) + 2 * (2 * d) + 2 * (2 * d) + 4 * (2 * d) == 1280
    # executed: the dQ kernel recomputes S1, S2, dP (512) and forms dQ1, dQ2 (256); dK/dV recomputes them (512)
    # and forms dV, dK1, dK2 (512)
    assert (512 + 256) + (512 + 512) == 1792
