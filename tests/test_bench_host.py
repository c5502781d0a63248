"""Host-side checks of bench.py (no GPU): the one-GPU guard, the algorithmic bytes
the HBM roofline divides by, and the rule that HBM counters taken on other kernel
sources are not reported."""
import importlib
import os
import subprocess
import sys

import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}), ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_exits_with_a_message(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], capture_output=True, text=True,
                       env={**os.environ, **env}, timeout=120)
    assert r.returncode == 2, (r.returncode, r.stderr)
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _scan_bytes(batch, L, D, N, e, gate):
    # u, delta and y (and z with the gate) once each; B and C once each; A, the skip
    # term and the bias once; the final state written once
    return batch * L * D * e * (4 if gate else 3) + 2 * batch * L * N * e + 4 * D * N + 8 * D + 4 * batch * D * N


@pytest.mark.parametrize("name,printed", [
    ("tiny_f32", 14976),                 # the five named workloads' totals, as the
    ("mamba130m_f32", 101.49e6),         # workload table states them (bytes, or MB
    ("mamba1p4b_bf16", 540.31e6),        # to two decimals)
    ("long131k_bf16", 2693.09e6),
])
def test_scan_algorithmic_bytes(name, printed):
    cfg = synth.CONFIGS[name]
    e = 4 if cfg.dtype == "f32" else 2
    got = cfg.algorithmic_bytes()
    assert got == _scan_bytes(cfg.batch, cfg.L, cfg.D, cfg.N, e, cfg.gate)
    if printed == int(printed) and printed < 1e6:
        assert got == printed
    else:
        assert round(got / 1e6, 2) == pytest.approx(printed / 1e6, abs=0.006)


def test_decode_algorithmic_bytes_per_step():
    cfg = synth.CONFIGS["decode_bf16"]
    S, D, N = cfg.batch, cfg.D, cfg.N
    # the state read and written, u, delta, z and y, B_t and C_t, A, the skip term and the bias
    want = 8 * S * D * N + S * D * 2 * 4 + 2 * S * N * 2 + 4 * D * N + 8 * D
    assert cfg.algorithmic_bytes_per_step() == want
    assert round(want / 1e6, 2) == 178.64


def test_counters_from_other_sources_are_not_reported(monkeypatch):
    sys.path.insert(0, ROOT)
    bench = importlib.import_module("bench")
    kernel = "scan_chunked_kernel"
    stored = bench.traffic_from_profiles("long131k_bf16", kernel)
    if stored is None:
        pytest.skip("the committed counters predate the current chunked-kernel source")
    assert stored > synth.CONFIGS["long131k_bf16"].algorithmic_bytes() * 0.9
    monkeypatch.setattr(bench, "src_hash", lambda k: "0" * 16)
    assert bench.traffic_from_profiles("long131k_bf16", kernel) is None
    assert bench.traffic_from_profiles("no_such_workload", kernel) is None
