"""Model parameters that fp32 cannot represent, and the copy that arithmetic modes 0 and 2 hold
(no torch, no GPU)."""
import numpy as np


def held_fp32(params):
    """The model as arithmetic modes 0 and 2 hold it: radial centres, C0, network weights and
    biases, 1/s_t, e_scale and the contraction matrix rounded to the nearest float32 (s_t enters
    only through its reciprocal)."""
    import copy

    def f32(a):
        return np.asarray(a, np.float64).astype(np.float32).astype(np.float64)

    q = copy.deepcopy(params)
    q.mu = f32(params.mu)
    q.c0 = f32(params.c0)
    q.mlp = [[{k: f32(v) for k, v in w.items()} for w in per] for per in params.mlp]
    q.layer_scale = 1.0 / f32(1.0 / np.asarray(params.layer_scale, np.float64))
    q.e_scale = float(f32(params.e_scale))
    if params.contraction is not None:
        q.contraction = f32(params.contraction)
    return q


def unrounded_params(cfg, T=None):
    """Benchmark model cfg drawn without the float32 rounding (same seed and order), with layer and
    energy scales moved off their powers of two, so that fp32 represents none of the values."""
    from molecular_dynamics_cell_amd import inputs as I
    base = I.make_params(cfg)
    spec = I.model_spec(cfg)
    if T is not None:
        spec.T = T
    sc = list(base.layer_scale) + [1.0] * spec.T
    ls = np.asarray(sc[:spec.T], np.float64) * (1.0 + np.pi * 1e-3)
    return I.random_params(spec, 1200 + cfg, base.masses, ls, base.e_scale * (1.0 + np.e * 1e-3),
                           round_f32=False)
