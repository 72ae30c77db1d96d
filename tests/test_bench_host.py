"""Host-side logic of bench.py: the algorithmic flop count, the roofline
bound choice, and the single-GPU guard (no GPU needed)."""
import subprocess
import sys

import pytest

import bench


def test_ns_flops_formula():
    # p=2, q=3, one step: p(p+1)q + p^2(p+1) + 2p^2q = 18 + 12 + 24
    assert bench.ns_flops([(3, 2)], 1) == 54.0
    assert bench.ns_flops([(2, 3), (3, 2)], 5) == 2 * 5 * 54.0


def test_roofline_picks_the_binding_peak():
    # 2.5e12 flops take 1 ms at the bf16 peak; 8e9 bytes take 1 ms at 8 TB/s
    row = {"flops": 2.5e12, "bytes": 1e9, "ms": 2.0, "launches": 1}
    r = bench.roofline(row, "bf16")
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["frac"] == pytest.approx(0.5) and r["achieved"] == pytest.approx(1250.0)
    row = {"flops": 2.5e11, "bytes": 8e9, "ms": 4.0, "launches": 2}
    r = bench.roofline(row, "bf16")
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert r["frac"] == pytest.approx(0.25) and r["mfma_frac"] == pytest.approx(0.025)


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr


def test_gram_flops_hand_count():
    # p=2, q=3.  SYRK p(p+1)q = 18, a symmetric p x p product p^2(p+1) = 12,
    # Q X 2p^2q = 24.  One window of one step: SYRK, P, Q X.
    assert bench.gram_flops(2, 3, ns_steps=1) == 18 + 12 + 24
    # One window of 3 steps: SYRK, 3 P, 2 Q <- P Q, 2 x (P A, P (P A)), Q X.
    assert bench.gram_flops(2, 3, ns_steps=3, restarts=[]) == 18 + (3 + 2 + 4) * 12 + 24
    # Default restart [2] over 5 steps: windows of 2 and 3 steps.
    two = 18 + (2 + 1 + 2) * 12 + 24
    three = 18 + (3 + 2 + 4) * 12 + 24
    assert bench.gram_flops(2, 3) == two + three
    # restarts outside 1..steps-1 have no effect
    assert bench.gram_flops(2, 3, restarts=[0, 5, 9]) == bench.gram_flops(2, 3, restarts=[])


def test_host_gradients_reuse_the_power_law_basis():
    """bench.py --grads host keeps each matrix's power-law basis across
    steps; a gradient built from the kept basis equals the one that
    recomputes it."""
    import numpy as np
    import workloads
    for step in (0, 3):
        basis = workloads.powerlaw_basis_np(80, 48, 5, 1)
        kept = workloads.grad_np("powerlaw_t3", 80, 48, 5, step, 1, basis=basis)
        fresh = workloads.grad_np("powerlaw_t3", 80, 48, 5, step, 1)
        assert np.array_equal(kept, fresh)
