"""Velocity-Verlet MD on the GPU against the oracle: one step from an identical state, snapshot
re-evaluation after a run, rebuild policy, checkpoint/resume, NVE energy conservation."""
import numpy as np
import pytest
import torch

import oracle
from molecular_dynamics_cell_amd import inputs as I
from tests import systems
from tests.gpu_util import check_ef, gpu_model, oracle_ef, say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _start(cfg, s):
    p = I.make_params(cfg)
    m = gpu_model(p, s)
    m.set_state(vel=torch.tensor(s.vel, device=DEV))
    return p, m


def test_one_step_matches_oracle():
    s = I.make_system(1)
    p, m = _start(1, s)
    m.md_step(1.0, 1)
    pos, vel, step = m.get_state()
    assert step == 1
    op, ov, _, _, _ = oracle.md(oracle.Model(p), s.pos, s.vel, s.types, s.masses, s.box, 1.0, 1)
    dp = np.abs(pos.cpu().numpy() - op).max()
    dv = np.abs(vel.cpu().numpy() - ov).max()
    say(f"one step: max |dx| = {dp:.2e} A, max |dv| = {dv:.2e} A/fs")
    # a force error of 1e-4 RMS_F moves an Ag atom by < 1e-9 A in one 1-fs step
    assert dp < 1e-8 and dv < 1e-8


@pytest.mark.parametrize("cfg,make,dt,steps,rebuild", [
    (1, lambda: I.make_system(1), 1.0, 10, 0),
    (2, lambda: systems.water_molecules(120, 18.0), 0.5, 40, 0),
    (3, lambda: systems.hea(8), 1.0, 30, 10),
])
def test_snapshot_reevaluation(cfg, make, dt, steps, rebuild):
    """After a GPU run, the oracle re-evaluates E and F at the GPU's final positions."""
    s = make()
    p, m = _start(cfg, s)
    st = m.md_step(dt, steps, rebuild)
    say(f"cfg{cfg}: {steps} steps, rebuilds={st['rebuilds']} T={st['temp']:.1f} K")
    if rebuild:
        assert st["rebuilds"] >= steps // rebuild
    pos, _, _ = m.get_state()
    E, F, _ = m.energy_forces()
    s2 = I.System(s.name, pos.cpu().numpy(), s.types, s.box, s.vel, s.species, s.masses)
    Eo, Fo, _ = oracle_ef(p, s2)
    check_ef(E, F.cpu().numpy(), Eo, Fo, label=f"cfg{cfg} snapshot")


def test_checkpoint_resume_bitwise():
    s = I.make_system(1)
    p, m = _start(1, s)
    m.md_step(1.0, 20, 10)
    pa, va, _ = m.get_state()
    p2, m2 = _start(1, s)
    m2.md_step(1.0, 10, 10)
    pos, vel, _ = m2.get_state()
    m3 = gpu_model(p2, s)
    m3.set_state(pos=pos, vel=vel)
    m3.md_step(1.0, 10, 10)
    pb, vb, _ = m3.get_state()
    assert torch.equal(pa, pb) and torch.equal(va, vb)


def test_nve_energy_conservation():
    """100 steps of 0.25 fs.  (Later in the run, this random-init water model lets atoms fall into
    a deep attractive well; the oracle integrator shows the same at about 30 fs.)"""
    s = systems.water_molecules(120, 18.0)
    p, m = _start(2, s)
    e0 = None
    drift = []
    for _ in range(5):
        st = m.md_step(0.25, 20)
        et = st["epot"] + st["ekin"]
        e0 = et if e0 is None else e0
        drift.append(et - e0)
    ke = st["ekin"]
    say(f"NVE water (360 atoms, 100 x 0.25 fs): total-energy excursion {max(map(abs, drift)):.3e} eV, E_kin {ke:.3f} eV")
    assert max(map(abs, drift)) < 1e-3 * ke


@pytest.mark.parametrize("cfg,make,steps,rebuild,skin", [
    (1, lambda: I.make_system(1), 12, 0, None),                 # no rebuild: whole chunks
    (3, lambda: systems.hea(8), 13, 5, None),                   # chunks end before scheduled rebuilds
    (1, lambda: I.make_system(1), 12, 0, 0.02),                 # displacement rebuilds: chunks roll back
    (4, lambda: systems.ag(24, seed=3), 10, 0, None),           # 4.4M list entries: the transposed map
                                                                # is built on the second stream
])
def test_graph_replay_matches_eager(cfg, make, steps, rebuild, skin):
    """MD replayed in captured chunks gives the same state, bit for bit, as eager steps; each run
    replays the graph several times with eager rebuilds and host synchronisations in between."""
    s = make()
    p = I.make_params(cfg)
    runs = []
    for k in (0, 4):
        m = gpu_model(p, s, skin=skin)
        m.set_state(vel=torch.tensor(s.vel, device=DEV))
        m.set_graph_replay(k)
        st = m.md_step(1.0, steps, rebuild)
        pos, vel, step = m.get_state()
        runs.append((pos, vel, st["rebuilds"], step))
    say(f"cfg{cfg} rebuild_every={rebuild} skin={skin}: rebuilds eager {runs[0][2]}, replay {runs[1][2]}")
    assert runs[0][3] == runs[1][3] == steps
    assert runs[0][2] == runs[1][2]
    assert torch.equal(runs[0][0], runs[1][0]) and torch.equal(runs[0][1], runs[1][1])


def test_graph_replay_against_oracle():
    """24 steps of the 108-atom cell replayed in captured chunks of 8 with a 0.02 A skin, so that
    displacement-triggered rebuilds roll chunks back and redo them eagerly; the oracle then
    re-evaluates E and F at the final positions, and its own velocity-Verlet run from the same start
    (same skin, same rebuild rule) ends at the same positions."""
    s = I.make_system(1)
    p = I.make_params(1)
    skin = 0.02
    m = gpu_model(p, s, skin=skin)
    m.set_state(vel=torch.tensor(s.vel, device=DEV))
    m.set_graph_replay(8)
    st = m.md_step(1.0, 24)
    say(f"replayed run: {st['steps']} steps, rebuilds {st['rebuilds']}, T = {st['temp']:.1f} K")
    assert st["steps"] == 24 and st["rebuilds"] > 0
    pos, _, _ = m.get_state()
    pos = pos.cpu().numpy()
    E, F, _ = m.energy_forces()
    s2 = I.System(s.name, pos, s.types, s.box, s.vel, s.species, s.masses)
    Eo, Fo, _ = oracle_ef(p, s2)
    check_ef(E, F.cpu().numpy(), Eo, Fo, label="replayed run, final snapshot")
    op, _, _, _, ost = oracle.md(oracle.Model(p), s.pos, s.vel, s.types, s.masses, s.box, 1.0, 24, skin=skin)
    d = np.abs(oracle.wrap(op, s.box) - pos)
    d = np.minimum(d, s.box - d)          # positions wrapped at different rebuilds
    say(f"replayed run vs oracle trajectory: max |dx| = {d.max():.2e} A (oracle rebuilds {ost['rebuilds']})")
    assert d.max() < 1e-6
