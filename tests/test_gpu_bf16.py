"""The bf16 network mode (precision 2: bf16 operands on the matrix cores, fp32 accumulation,
each operand carried as a bf16 pair) against the fp64 oracle, at the gates for bf16 networks:
max |dF| <= 2e-3 RMS_F; total energy within 1e-3 relative (a sanity bound, not a gate).  The
mode is offered for 64-wide networks on at most 128 features; wider models are refused."""
import numpy as np
import pytest
import torch

from molecular_dynamics_cell_amd import binding
from molecular_dynamics_cell_amd import inputs as I
from tests import systems
from tests.gpu_util import EI_TOL_BF16, check_ef, check_ei, gpu_model, oracle_ef, say

pytestmark = pytest.mark.gpu

CASES = {
    "Ag108_T2": (1, lambda: I.make_system(1)),
    "Ag4000_cfg4model": (4, lambda: systems.ag(10, seed=4)),
    "water60_T3": (2, lambda: systems.water_molecules(60, 17.0)),
    "water4608_full": (2, lambda: I.make_system(2)),
    "Ag2M_full": (4, lambda: I.make_system(4)),
}


@pytest.mark.parametrize("name", list(CASES))
def test_bf16_networks(name):
    cfg, make = CASES[name]
    s = make()
    p = I.make_params(cfg)
    p.spec.precision = 2
    say(f"[bf16] {name} n={s.n}")
    m = gpu_model(p, s)
    E, F, Ei = m.energy_forces(atom_energy=True)
    F = F.cpu().numpy()
    Ei = Ei.cpu().numpy()
    m.close()
    torch.cuda.empty_cache()
    Eo, Fo, Eio = oracle_ef(p, s)
    check_ei(Ei, Eio, tol=EI_TOL_BF16, label=f"{name} bf16 E_i")
    check_ef(E, F, Eo, Fo, e_tol=1e-3, f_tol=2e-3, label=f"{name} bf16")


def test_bf16_refused_for_wide_networks():
    p = I.make_params(3)      # hidden 128, 312 features
    p.spec.precision = 2
    with pytest.raises(RuntimeError):
        binding.MPNN(p, torch.device("cuda:0"))
