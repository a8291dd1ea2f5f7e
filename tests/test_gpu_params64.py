"""GPU parity with model parameters that fp32 cannot represent (weights, biases, C0 and radial
centres drawn in fp64 without rounding; layer and energy scales off their powers of two), through
the C ABI:
  - arithmetic mode 1 holds every parameter in fp64: compared with the oracle on the very same
    parameters;
  - modes 0 and 2 hold the parameters rounded to fp32: compared with the oracle on the rounded
    copy (tests.gpu_util.held_fp32), which is the model those modes evaluate.
Gates as everywhere: pair sets bit-exact, |dE|/|E| <= 1e-6, max|dF| <= 1e-4 RMS_F (2e-3 with bf16
networks), per-atom energies within tests.gpu_util.EI_TOL of max|E_i|."""
import numpy as np
import pytest

from molecular_dynamics_cell_amd import inputs as I
from tests import systems
from tests.gpu_util import (EI_TOL_BF16, check_ef, check_ei, gpu_model, held_fp32, oracle_ef, say,
                            unrounded_params)

pytestmark = pytest.mark.gpu

SYSTEMS = {
    "Ag4000_cfg4model": (4, lambda: systems.ag(10, seed=4)),
    "water60_T3": (2, lambda: systems.water_molecules(60, 17.0)),
    "HEA432_K12L3": (3, lambda: systems.hea(6)),
    "CHON4002_K12L3": (5, lambda: I.make_system(5, reduced=True)),
}


def _run(name, precision):
    cfg, make = SYSTEMS[name]
    s = make()
    p = unrounded_params(cfg)
    p.spec.precision = precision
    # nothing in the drawn parameters is a float32 value
    assert not np.array_equal(p.mlp[0][0]["W1"], p.mlp[0][0]["W1"].astype(np.float32))
    ref = p if precision == 1 else held_fp32(p)
    say(f"[params64] {name} n={s.n} precision={precision}")
    m = gpu_model(p, s)
    E, F, Ei = m.energy_forces(atom_energy=True)
    Eo, Fo, Eio = oracle_ef(ref, s)
    return E, F.cpu().numpy(), Ei.cpu().numpy(), Eo, Fo, Eio


@pytest.mark.parametrize("name", list(SYSTEMS))
def test_fp64_parameters_mode1(name):
    E, F, Ei, Eo, Fo, Eio = _run(name, 1)
    check_ei(Ei, Eio, label=f"{name} mode 1")
    check_ef(E, F, Eo, Fo, label=f"{name} mode 1 vs oracle on the same fp64 parameters")


@pytest.mark.parametrize("name", ["Ag4000_cfg4model", "water60_T3", "HEA432_K12L3"])
def test_fp64_parameters_mode0(name):
    E, F, Ei, Eo, Fo, Eio = _run(name, 0)
    check_ei(Ei, Eio, label=f"{name} mode 0")
    check_ef(E, F, Eo, Fo, label=f"{name} mode 0 vs oracle on the fp32-held parameters")


def test_fp64_parameters_mode2():
    E, F, Ei, Eo, Fo, Eio = _run("water60_T3", 2)
    check_ei(Ei, Eio, tol=EI_TOL_BF16, label="water60 mode 2")
    check_ef(E, F, Eo, Fo, e_tol=1e-3, f_tol=2e-3, label="water60 mode 2 vs oracle on the fp32-held parameters")

