"""Helpers for the GPU parity tests: run the HIP library and the fp64 oracle on the same
seeded inputs."""
import sys

import numpy as np
import torch

import oracle
from molecular_dynamics_cell_amd import binding


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def gpu_model(params, s, skin=None, subdomains=None):
    dev = torch.device("cuda:0")
    m = binding.MPNN(params, dev)
    if subdomains is not None:
        m.set_subdomains(*subdomains)
    m.build_neighbors(torch.tensor(s.pos, device=dev), torch.tensor(s.types, device=dev), s.box,
                      skin=skin)
    return m


def oracle_ef(params, s, skin=None, dump=False):
    om = oracle.Model(params)
    pos = oracle.wrap(s.pos, s.box)
    return oracle.energy_forces(om, pos, s.types, s.box, skin=skin, dump=dump)


def canonical_pairs(i, j, S, n):
    """Unique int64 code per (i, j, S) tuple, sorted."""
    code = ((np.asarray(i, np.int64) * n + np.asarray(j, np.int64)) * 27
            + (np.asarray(S[:, 0], np.int64) + 1) * 9 + (np.asarray(S[:, 1], np.int64) + 1) * 3
            + (np.asarray(S[:, 2], np.int64) + 1))
    return np.sort(code)


def check_ef(E, F, Eo, Fo, e_tol=1e-6, f_tol=1e-4, label=""):
    frms = float(np.sqrt((Fo ** 2).sum(1).mean()))
    dE = abs(E - Eo) / abs(Eo)
    dF = float(np.linalg.norm(F - Fo, axis=1).max()) / frms
    say(f"{label}: E_gpu={E:.10f} E_oracle={Eo:.10f} relE={dE:.2e} max|dF|/RMS_F={dF:.2e} RMS_F={frms:.3f}")
    assert dE <= e_tol, (label, dE)
    assert dF <= f_tol, (label, dF)


# Per-atom energies: max_i |E_i^gpu - E_i^oracle| <= EI_TOL * max_i |E_i^oracle| (fp32 and fp64
# arithmetic modes; the bf16-operand networks use the bf16 sanity bound 1e-3).  A systematic error
# of that size in every E_i would already fail the 1e-6 total-energy gate by an order of magnitude,
# so this bound is aimed at per-atom faults that cancel in the sum (a dropped or doubled edge moves
# one E_i by about 1/50 of itself).
EI_TOL = 1e-5
EI_TOL_BF16 = 1e-3


def check_ei(Ei, Eio, tol=EI_TOL, label=""):
    Ei = np.asarray(Ei, np.float64).ravel()
    Eio = np.asarray(Eio, np.float64).ravel()
    err = float(np.abs(Ei - Eio).max() / np.abs(Eio).max())
    say(f"{label}: max|dE_i|/max|E_i| = {err:.2e} (bound {tol:.0e})")
    assert err <= tol, (label, err)
    return err



from tests.params_util import held_fp32, unrounded_params  # noqa: E402,F401
