"""GPU parity of the contraction variant (each neighbour orbital n built from the contracted
radial function sum_k C[n][k] R_k, [JACS] "REANN Architecture") against the fp64 oracle, through
the C ABI, in every arithmetic mode: per-layer orbital sums, energies and forces to the same gates
as the base model.  The base model (no contraction) is covered by test_gpu_parity."""
import numpy as np
import pytest
import torch

import oracle
from molecular_dynamics_cell_amd import inputs as I
from tests import systems
from tests.gpu_util import check_ef, gpu_model, oracle_ef, say

pytestmark = pytest.mark.gpu


CASES = {
    # name: (model cfg, system factory, arithmetic mode, force gate)
    "Ag4000_cfg4model": (4, lambda: systems.ag(10, seed=4), 0, 1e-4),
    "Ag4000_cfg4model_fp64": (4, lambda: systems.ag(10, seed=4), 1, 1e-4),
    "water60_T3": (2, lambda: systems.water_molecules(60, 17.0), 0, 1e-4),
    "HEA432_K12L3": (3, lambda: systems.hea(6), 0, 1e-4),
    "CHON4002_K12L3_fp64": (5, lambda: I.make_system(5, reduced=True), 1, 1e-4),
    "Ag108_bf16": (1, lambda: I.make_system(1), 2, 2e-3),
    # 500,000 atoms: per-edge streams of 1.7 GB, so the row kernels take their streaming path (with
    # the staged record windows), which the smaller cases do not reach
    "Ag500000_cfg4model": (4, lambda: systems.ag(50, seed=5), 0, 1e-4),
}


def _params(cfg, precision, mu_shift=False):
    p = I.make_params(cfg)
    p.spec.precision = precision
    if mu_shift:
        k = np.arange(p.spec.K)
        p.mu = np.asarray(p.mu, np.float64) + 0.08 * np.sin(1.7 * k + 0.3)
        p.mu[0] = max(p.mu[0], 0.0)
    return I.with_contraction(p, I.contraction_matrix(p.spec.K, 600 + cfg))


@pytest.mark.parametrize("name", list(CASES))
def test_contracted_energy_forces(name):
    cfg, make, precision, f_tol = CASES[name]
    s = make()
    p = _params(cfg, precision)
    say(f"[contraction] {name} n={s.n} precision={precision}")
    m = gpu_model(p, s)
    E, F, _ = m.energy_forces()
    Eo, Fo, _, dump = oracle_ef(p, s, dump=True)
    for t in range(p.spec.T):
        O = m.get_intermediate(1, t).cpu().numpy()
        err = np.abs(O - dump["O"][t]).max() / (np.abs(dump["O"][t]).max() + 1e-30)
        say(f"  O^{t}: rel max err {err:.2e}")
        assert err < 1e-4
    check_ef(E, F.cpu().numpy(), Eo, Fo, e_tol=1e-6 if precision != 2 else 1e-3, f_tol=f_tol,
             label=f"contracted {name}")


@pytest.mark.parametrize("precision", [0, 1])
def test_contracted_uneven_centres(precision):
    """Uneven centres: every primitive from its own exponential (no ratio chain), then contracted."""
    s = systems.ag(6, seed=9)
    p = _params(4, precision, mu_shift=True)
    m = gpu_model(p, s)
    E, F, _ = m.energy_forces()
    Eo, Fo, _ = oracle_ef(p, s)
    check_ef(E, F.cpu().numpy(), Eo, Fo, label=f"contracted, uneven centres, precision {precision}")


def test_identity_contraction_equals_base_model():
    """C = identity reproduces the base model's energy and forces (the contracted kernels sum
    exact zeros, so the results agree to rounding)."""
    s = systems.ag(6, seed=9)
    p = I.make_params(4)
    E0, F0, _ = gpu_model(p, s).energy_forces()
    E1, F1, _ = gpu_model(I.with_contraction(p, np.eye(p.spec.K)), s).energy_forces()
    F0, F1 = F0.cpu().numpy(), F1.cpu().numpy()
    frms = float(np.sqrt((F0 ** 2).sum(1).mean()))
    say(f"[identity] relE={abs(E1 - E0) / abs(E0):.2e} max|dF|/RMS_F={np.abs(F1 - F0).max() / frms:.2e}")
    assert abs(E1 - E0) <= 1e-7 * abs(E0)
    assert np.abs(F1 - F0).max() <= 1e-5 * frms


def test_contracted_md_one_step_and_snapshot():
    """The contracted Ag model with its own frozen scales: one velocity-Verlet step from the same
    state as the oracle's, then a 20-step run whose final state the oracle re-evaluates."""
    s = systems.ag(6, seed=9)
    p = I.make_params(4, contraction_seed=7)
    m = gpu_model(p, s)
    m.set_state(vel=torch.tensor(s.vel, device="cuda:0"))
    m.md_step(1.0, 1)
    pos, vel, _ = m.get_state()
    op, ov, _, _, _ = oracle.md(oracle.Model(p), s.pos, s.vel, s.types, s.masses, s.box, 1.0, 1)
    dp = np.abs(pos.cpu().numpy() - op).max()
    dv = np.abs(vel.cpu().numpy() - ov).max()
    say(f"[contracted md] one step: max |dx| = {dp:.2e} A, max |dv| = {dv:.2e} A/fs")
    assert dp < 1e-8 and dv < 1e-8
    st = m.md_step(1.0, 20, 10)
    say(f"[contracted md] 21 steps: T = {st['temp']:.1f} K, rebuilds = {st['rebuilds']}")
    pos, _, _ = m.get_state()
    E, F, _ = m.energy_forces()
    s2 = I.System(s.name, pos.cpu().numpy(), s.types, s.box, s.vel, s.species, s.masses)
    Eo, Fo, _ = oracle_ef(p, s2)
    check_ef(E, F.cpu().numpy(), Eo, Fo, label="contracted snapshot after 21 steps")


@pytest.mark.parametrize("precision", [0, 1])
def test_contracted_one_row_per_lane(precision):
    """Above 32,768 atoms the row kernels take one row per lane (below, a 16-lane group): the
    contracted model with uneven centres on a 37,044-atom lattice, both arithmetic modes."""
    s = systems.ag(21, seed=4)
    p = _params(4, precision, mu_shift=True)
    m = gpu_model(p, s)
    assert s.n > 32768
    E, F, _ = m.energy_forces()
    Eo, Fo, _ = oracle_ef(p, s)
    check_ef(E, F.cpu().numpy(), Eo, Fo, label=f"contracted, uneven centres, 37,044 atoms, precision {precision}")
