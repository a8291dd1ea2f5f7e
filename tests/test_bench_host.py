"""Host logic of the benchmark (no GPU): the per-launch byte budget adds up to the per-atom-step
figure over one step's launches, the itemised model counts what it says, and a request for more
than one GPU is refused before anything touches a device."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

AG2M = dict(N=2048000, NN=2048000 + 280731, EL=161631030, EA=110562790, K=8, M=10, D=108, H=64, T=3,
            SA=True)


def test_budget_sums_to_per_atom_step_figure():
    g = AG2M
    T, N = g["T"], g["N"]
    launches = {"aggregate": T, "net_forward": T - 1, "net_energy": 1, "net_backward": T - 1,
                "backward_layer": T, "force_gather": 1}
    per_step = sum(bench.ag2m_alg_bytes(f, g) * k for f, k in launches.items())
    rest = bench.AG2M_BYTES_PER_ATOM_STEP["integrate_ghosts_rebuild"]
    assert bench.AG2M_TOTAL == 10500
    assert per_step == pytest.approx((bench.AG2M_TOTAL - rest) * N, rel=1e-12)
    # the reverse edges' share of one launch (the line's roofline entry)
    assert bench.ag2m_alg_bytes("backward_layer", g) == pytest.approx(4000 * N / 3, rel=1e-12)
    assert bench.ag2m_alg_bytes("message_grad", g) is None


def test_itemised_model_counts():
    g = dict(N=10, NN=14, EL=100, EA=60, K=8, M=10, D=108, H=64, T=3, SA=True)
    b, f, kind = bench.kernel_model("message_grad", g)
    # segment offsets per node, transposed active map per Verlet entry, w_e per active edge,
    # dE/dc rows out per node
    assert b == 8 * 14 + 4 * 100 + 32 * 60 + 32 * 14 and kind == "hbm" and f == 8 * 60
    b, f, kind = bench.kernel_model("force_gather", g)
    assert b == 8 * 14 + 4 * 100 + 12 * 60 + 8 * 10 + 24 * 10 + 48 * 10
    b, f, kind = bench.kernel_model("net_energy", g)
    assert kind == "mfma" and f == 10 * 2 * (2 * 64 * 108 + 2 * 64 * 64 + 2 * 64)
    assert bench.kernel_model("no_such_family", g) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
