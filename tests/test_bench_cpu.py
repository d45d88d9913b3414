"""bench.py's contract pieces that need no GPU: the one-GPU refusal and the
algorithmic FLOP and byte counts its roofline object divides by the
measured kernel time."""

import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import CONFIGS  # noqa: E402


def _run_bench(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, env=env, timeout=300)


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], None), (["--gpus", "8"], None),
                                      ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(args, env):
    r = _run_bench(args, env)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""          # no JSON line


def test_algorithmic_counts_prefill():
    """Closed forms for the 16K prefill layer (T=16384, K=2048, I=768,
    E=128, k=8) with every expert active: the numbers the design notes
    state per launch."""
    cfg = CONFIGS["prefill"]
    T, K, I, E, k = cfg.T, cfg.K, cfg.I, cfg.E, cfg.k
    M = T * k
    counts = np.full(E, M // E)
    a = bench.algorithmic(cfg, counts)
    assert a["gemm1_swiglu_requant"]["flops"] == 2 * M * (2 * I) * K == 824633720832
    assert a["gemm2"]["flops"] == 2 * M * K * I == 412316860416
    # bytes: e4m3 payload plus one e8m0 byte per 32 elements
    assert round(a["route_quant"]["bytes"] / 1e6, 1) == 345.5
    assert round(a["gemm1_swiglu_requant"]["bytes"] / 1e6, 1) == 795.9
    assert round(a["gemm2"]["bytes"] / 1e6, 1) == 848.3
    assert a["finalize"]["bytes"] == 2 * M * K + 8 * T * k + 2 * T * K


def test_algorithmic_weight_bytes_follow_active_experts():
    """Experts that receive no token contribute no weight bytes (the GEMMs
    never fetch them), while FLOPs depend on M only."""
    cfg = CONFIGS["prefill"]
    M = cfg.T * cfg.k
    full = np.full(cfg.E, M // cfg.E)
    half = full.copy()
    half[: cfg.E // 2] = 0
    half[cfg.E // 2:] *= 2
    a_full, a_half = bench.algorithmic(cfg, full), bench.algorithmic(cfg, half)
    w13 = cfg.E * 2 * cfg.I * cfg.K * (1 + 1 / 32)
    assert a_full["gemm1_swiglu_requant"]["flops"] == a_half["gemm1_swiglu_requant"]["flops"]
    assert np.isclose(a_full["gemm1_swiglu_requant"]["bytes"] - a_half["gemm1_swiglu_requant"]["bytes"], w13 / 2)
