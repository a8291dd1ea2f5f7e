"""Freeze the per-layer density scales s_t and the energy scale of each benchmark model.

With random-init networks, |rho^t| grows roughly quadratically per layer (rho is a square of
a neighbour sum of c, and c is a network output), so the models divide rho^t by a constant
s_t.  The constants are computed ONCE by the fp64 oracle on a reduced instance (about 4,000
atoms) of the same generator and stored in molecular_dynamics_cell_amd/model_scales.json;
both the oracle and the GPU library then read them as ordinary model parameters.

  s_t      = RMS over atoms and features of rho^t (computed layer by layer, since rho^t
             depends on s_0..s_{t-1}), rounded to the nearest power of two;
  e_scale  = 0.5 eV/A divided by the RMS per-atom force norm obtained with e_scale = 1,
             rounded to the nearest power of two.
Powers of two keep the scaling exact in any floating-point precision.

Run:  python -m oracle.calibrate   (from the repository root)
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np

if __package__ in (None, ""):
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import oracle as O  # noqa: E402
from molecular_dynamics_cell_amd import inputs as I  # noqa: E402

TARGET_FRMS = 0.5


def pow2(x: float) -> float:
    return float(2.0 ** np.round(np.log2(x)))


# contraction variants with scales of their own: (config, seed of the contraction matrix)
CONTRACTED = [(4, 7)]


def calibrate(cfg: int, contraction_seed: int = None) -> dict:
    spec = I.model_spec(cfg)
    sysr = I.make_system(cfg, reduced=True)
    pos = O.wrap(sysr.pos, sysr.box)
    pl = O.pairs(pos, sysr.box, spec.rc + spec.skin)
    scales = np.ones(spec.T)

    def model(scales):
        p = I.random_params(spec, 1200 + cfg, sysr.masses, scales, 1.0)
        if contraction_seed is not None:
            p = I.with_contraction(p, I.contraction_matrix(spec.K, contraction_seed))
        return O.Model(p)

    for t in range(spec.T):
        _, _, _, dump = O.energy_forces(model(scales), pos, sysr.types, sysr.box, pair_list=pl,
                                        dump=True)
        scales[t] = pow2(float(np.sqrt(np.mean(dump["rho"][t] ** 2))))
    _, F, _ = O.energy_forces(model(scales), pos, sysr.types, sysr.box, pair_list=pl)
    frms = float(np.sqrt(np.mean(np.sum(F * F, axis=1))))
    return {"layer_scale": [float(x) for x in scales], "e_scale": pow2(TARGET_FRMS / frms),
            "calibration_atoms": int(sysr.n), "calibration_system": sysr.name}


def main():
    out = {}
    for cfg in sorted(I.CONFIGS):
        out[str(cfg)] = calibrate(cfg)
        print(cfg, out[str(cfg)], flush=True)
    for cfg, seed in CONTRACTED:
        key = I.scales_key(cfg, seed)
        out[key] = calibrate(cfg, seed)
        print(key, out[key], flush=True)
    with open(I.SCALES_FILE, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print("wrote", I.SCALES_FILE)


if __name__ == "__main__":
    main()
