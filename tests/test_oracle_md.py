"""Pins of the oracle's velocity-Verlet NVE integrator (used by the paper's validation runs,
section "Strong Scaling": NVE energy conservation for several T): time reversibility,
second-order energy error, momentum conservation, and the rebuild policy."""
import numpy as np

from molecular_dynamics_cell_amd import inputs as I
from tests import systems


def test_time_reversibility(orc):
    s = systems.ag(3)
    m = orc.Model(systems.params_for(1))
    start = orc.wrap(s.pos, s.box)
    p1, v1, _, _, st = orc.md(m, start, s.vel, s.types, s.masses, s.box, 1.0, 20)
    assert st["rebuilds"] == 0
    p2, v2, _, _, _ = orc.md(m, p1, -v1, s.types, s.masses, s.box, 1.0, 20)
    diff = p2 - start
    diff -= s.box * np.round(diff / s.box)      # each run wraps its start into the box
    assert np.abs(diff).max() <= 1e-10
    assert np.abs(v2 + s.vel).max() <= 1e-10


def _energy_spread(orc, m, s, dt, n):
    _, _, ep, ek, _ = orc.md(m, s.pos, s.vel, s.types, s.masses, s.box, dt, n)
    et = ep + ek
    return et.max() - et.min()


def test_energy_error_second_order(orc):
    s = systems.ag(3)
    m = orc.Model(systems.params_for(1))
    a = _energy_spread(orc, m, s, 1.0, 30)
    b = _energy_spread(orc, m, s, 0.5, 60)
    assert 2.8 < a / b < 5.5, (a, b)


def test_momentum_conserved_and_rebuilds(orc):
    s = systems.water_molecules(30, 20.0)
    m = orc.Model(systems.params_for(2))
    p0 = (s.masses[s.types][:, None] * s.vel).sum(0)
    pos, vel, _, _, st = orc.md(m, s.pos, s.vel, s.types, s.masses, s.box, 0.5, 20,
                                rebuild_every=5)
    p1 = (s.masses[s.types][:, None] * vel).sum(0)
    scale = np.abs(s.masses[s.types][:, None] * vel).sum()
    assert np.abs(p1 - p0).max() <= 1e-12 * scale
    assert st["rebuilds"] == 4
    assert np.all((pos >= -1.0) & (pos < s.box + 1.0))


def test_maxwell_boltzmann_generator():
    s = systems.ag(10)
    ke = 0.5 * (s.masses[s.types][:, None] * s.vel ** 2).sum() / I.EV_AMU_A2_FS2
    temp = 2 * ke / ((3 * s.n - 3) * I.KB_EV)
    assert abs(temp - 300.0) < 15.0
    assert np.abs((s.masses[s.types][:, None] * s.vel).sum(0)).max() < 1e-10
