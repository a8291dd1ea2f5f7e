"""Seeded synthetic inputs: atomic configurations and random-init model parameters.

This module is the only code shared by the GPU path and the fp64 CPU oracle. It draws
random numbers and builds geometry; it holds none of the model's arithmetic (no basis,
no aggregation, no network, no forces).

The five systems stand in for the training/benchmark data sets of "Efficient
Parallelization of Message Passing Neural Network Potentials for Large-Scale Molecular
Dynamics" (Xia & Jiang, JACS Au; Results, "Linear Scaling with Message Passing",
"Performance on GPUs" and the graphene-formation application), which are not available:
  1  fcc Ag, 3x3x3 conventional cells (108 atoms), T=2
  2  liquid water, 1536 rigid-geometry molecules in a 35.8 A box, T=3
  3  equimolar 5-element bcc high-entropy alloy, 40^3 cells (128,000 atoms), T=3
  4  fcc Ag, 80^3 cells (2,048,000 atoms): one GPU's subdomain of a 100M-atom run, T=3
  5  reactive C2H2/O2/N2 gas at 0.5 g/cm^3 (400,002 atoms), T=3
Seeds: geometry 1000+cfg, velocities 1100+cfg, weights 1200+cfg (numpy PCG64).

Model hyper-parameters follow the paper's REANN section (Gaussian-type orbital primitives
with centre, width and angular momentum l <= L; element-wise orbital coefficients;
atomic networks per element).  Unit system: A, eV, fs, amu.
"""
from __future__ import annotations

import dataclasses
import json
import os
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SCALES_FILE = os.path.join(_HERE, "model_scales.json")

# Boltzmann constant (eV/K) and eV/amu expressed in A^2/fs^2 (CODATA values).
KB_EV = 8.617333262e-5
EV_AMU_A2_FS2 = 9.648533212e-3

MASS = {
    "H": 1.008, "C": 12.011, "N": 14.007, "O": 15.999, "Ag": 107.8682,
    "V": 50.9415, "Nb": 92.90637, "Mo": 95.95, "Ta": 180.94788, "W": 183.84,
}


@dataclass
class System:
    name: str
    pos: np.ndarray            # [n,3] float64, A (not necessarily wrapped)
    types: np.ndarray          # [n] int32 species index
    box: np.ndarray            # [3] float64, orthorhombic edge lengths, A
    vel: np.ndarray            # [n,3] float64, A/fs
    species: list              # element symbol per species index
    masses: np.ndarray         # [n_species] amu

    @property
    def n(self) -> int:
        return int(self.pos.shape[0])


@dataclass
class ModelSpec:
    n_species: int
    K: int                     # radial primitives (N_phi)
    L: int                     # max angular momentum
    T: int                     # message-passing layers
    H: int                     # hidden width of the atomic networks
    rc: float
    sigma: float = 0.5         # Gaussian standard deviation, A
    skin: float = 1.0
    precision: int = 0         # library arithmetic mode: 0 fp32 orbital sums/networks, 1 fp64
    extra: dict = field(default_factory=dict)


@dataclass
class Params:
    spec: ModelSpec
    mu: np.ndarray             # [K]
    c0: np.ndarray             # [S][K]
    mlp: list                  # mlp[t][s] = dict(W1,b1,W2,b2,W3,b3) float64
    layer_scale: np.ndarray    # [T]
    e_scale: float
    masses: np.ndarray         # [S]
    contraction: np.ndarray = None   # [K][K] contraction of the radial primitives, or None

    @property
    def D(self) -> int:
        s = self.spec
        return s.K * (s.K + 1) * (s.L + 1) // 2

    def packed_mlp(self) -> np.ndarray:
        """Flat float64 array: for t, for s: W1[H][D], b1[H], W2[H][H], b2[H], W3[out][H], b3[out]."""
        parts = []
        for t in range(self.spec.T):
            for s in range(self.spec.n_species):
                w = self.mlp[t][s]
                for key in ("W1", "b1", "W2", "b2", "W3", "b3"):
                    parts.append(np.ascontiguousarray(w[key], dtype=np.float64).ravel())
        return np.concatenate(parts)


# ----------------------------------------------------------------------------------------
# configuration table (sizes and settings of the five benchmark systems)
# ----------------------------------------------------------------------------------------
CONFIGS = {
    1: dict(name="Ag108", K=8, L=2, T=2, H=64, rc=6.0, skin=1.0, dt=1.0, steps=10,
            rebuild_every=0, temp=300.0),
    2: dict(name="water4608", K=8, L=2, T=3, H=64, rc=6.0, skin=1.0, dt=0.5, steps=100,
            rebuild_every=0, temp=300.0),
    3: dict(name="HEA128k", K=12, L=3, T=3, H=128, rc=5.0, skin=1.0, dt=1.0, steps=100,
            rebuild_every=10, temp=300.0),
    4: dict(name="Ag2M", K=8, L=2, T=3, H=64, rc=6.0, skin=1.0, dt=1.0, steps=200,
            rebuild_every=20, temp=300.0),
    5: dict(name="CHON400k", K=12, L=3, T=3, H=128, rc=6.0, skin=1.0, dt=0.25, steps=200,
            rebuild_every=5, temp=3000.0),
}


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def maxwell_boltzmann(masses_per_atom: np.ndarray, temp: float, seed: int) -> np.ndarray:
    """Velocities (A/fs) with per-component std sqrt(kB T kappa / m); centre-of-mass drift removed."""
    rng = _rng(seed)
    n = masses_per_atom.shape[0]
    sd = np.sqrt(KB_EV * temp * EV_AMU_A2_FS2 / masses_per_atom)
    v = rng.standard_normal((n, 3)) * sd[:, None]
    p = (masses_per_atom[:, None] * v).sum(axis=0)
    v -= p / masses_per_atom.sum()
    return v


def fcc(nx: int, ny: int, nz: int, a: float, jitter: float, seed: int) -> tuple:
    basis = np.array([[0, 0, 0], [0.5, 0.5, 0], [0.5, 0, 0.5], [0, 0.5, 0.5]])
    return _lattice(basis, nx, ny, nz, a, jitter, seed)


def bcc(nx: int, ny: int, nz: int, a: float, jitter: float, seed: int) -> tuple:
    basis = np.array([[0, 0, 0], [0.5, 0.5, 0.5]])
    return _lattice(basis, nx, ny, nz, a, jitter, seed)


def _lattice(basis, nx, ny, nz, a, jitter, seed):
    g = np.stack(np.meshgrid(np.arange(nx), np.arange(ny), np.arange(nz), indexing="ij"), -1)
    g = g.reshape(-1, 1, 3) + basis[None, :, :]
    pos = (g.reshape(-1, 3) * a).astype(np.float64)
    rng = _rng(seed)
    pos += rng.standard_normal(pos.shape) * jitter
    box = np.array([nx * a, ny * a, nz * a], dtype=np.float64)
    return pos, box, rng


def _random_rotations(rng: np.random.Generator, n: int) -> np.ndarray:
    """Uniform random rotation matrices from uniform unit quaternions (Shoemake's method)."""
    u1, u2, u3 = rng.random(n), rng.random(n), rng.random(n)
    q = np.stack([np.sqrt(1 - u1) * np.sin(2 * np.pi * u2),
                  np.sqrt(1 - u1) * np.cos(2 * np.pi * u2),
                  np.sqrt(u1) * np.sin(2 * np.pi * u3),
                  np.sqrt(u1) * np.cos(2 * np.pi * u3)], -1)
    x, y, z, w = q[:, 0], q[:, 1], q[:, 2], q[:, 3]
    R = np.empty((n, 3, 3))
    R[:, 0, 0] = 1 - 2 * (y * y + z * z); R[:, 0, 1] = 2 * (x * y - z * w); R[:, 0, 2] = 2 * (x * z + y * w)
    R[:, 1, 0] = 2 * (x * y + z * w); R[:, 1, 1] = 1 - 2 * (x * x + z * z); R[:, 1, 2] = 2 * (y * z - x * w)
    R[:, 2, 0] = 2 * (x * z - y * w); R[:, 2, 1] = 2 * (y * z + x * w); R[:, 2, 2] = 1 - 2 * (x * x + y * y)
    return R


def _min_image_close_pairs(pos: np.ndarray, box: np.ndarray, cutoff: float):
    from scipy.spatial import cKDTree
    wrapped = np.mod(pos, box)
    wrapped[wrapped >= box] = 0.0
    tree = cKDTree(wrapped, boxsize=box)
    return tree.query_pairs(cutoff, output_type="ndarray")


def water(n_grid: int = 12, n_mol: int = 1536, box_len: float = 35.8, seed: int = 1002) -> System:
    rng = _rng(seed)
    spacing = box_len / n_grid
    sites = np.stack(np.meshgrid(*(np.arange(n_grid),) * 3, indexing="ij"), -1).reshape(-1, 3)
    chosen = rng.choice(sites.shape[0], size=n_mol, replace=False)
    centres = (sites[chosen] + 0.5) * spacing
    o = centres + rng.uniform(-0.2, 0.2, size=centres.shape)
    box = np.array([box_len] * 3)
    for _ in range(1000):  # re-draw the jitter of molecules closer than 2.6 A (O-O)
        pairs = _min_image_close_pairs(o, box, 2.6)
        if pairs.shape[0] == 0:
            break
        bad = np.unique(pairs[:, 0])
        o[bad] = centres[bad] + rng.uniform(-0.2, 0.2, size=(bad.shape[0], 3))
    else:
        raise RuntimeError("water generator did not converge")
    roh, ang = 0.96, np.deg2rad(104.5)
    local = np.array([[0, 0, 0],
                      [roh * np.sin(ang / 2), 0, roh * np.cos(ang / 2)],
                      [-roh * np.sin(ang / 2), 0, roh * np.cos(ang / 2)]])
    R = _random_rotations(rng, n_mol)
    atoms = o[:, None, :] + np.einsum("nij,aj->nai", R, local)
    pos = atoms.reshape(-1, 3)
    types = np.tile(np.array([0, 1, 1], dtype=np.int32), n_mol)
    species = ["O", "H"]
    masses = np.array([MASS[s] for s in species])
    vel = maxwell_boltzmann(masses[types], CONFIGS[2]["temp"], 1102)
    return System("water4608", pos, types, box, vel, species, masses)


def chon(n_c2h2: int = 65772, n_o2: int = 65772, n_n2: int = 2685, density: float = 0.5,
         seed: int = 1005, temp: float = 3000.0, vel_seed: int = 1105) -> System:
    """C2H2 + O2 (1:1) + 2% N2 molecules, random orientations, min intermolecular distance 2.0 A.

    Molecules sit on randomly chosen sites of a cubic grid with a uniform +-0.3 A jitter; any
    molecule with an intermolecular contact < 2.0 A has its orientation and jitter re-drawn
    until none is left.
    """
    rng = _rng(seed)
    species = ["H", "C", "N", "O"]
    mH, mC, mN, mO = (MASS[s] for s in species)
    total_mass = n_c2h2 * (2 * mC + 2 * mH) + n_o2 * 2 * mO + n_n2 * 2 * mN
    grams = total_mass * 1.66053906660e-24
    box_len = (grams / density * 1e24) ** (1.0 / 3.0)
    box = np.array([box_len] * 3)
    # molecule templates along z (A): linear H-C#C-H (C#C 1.20, C-H 1.06), O2 1.21, N2 1.10
    c2h2 = (np.array([[0, 0, -1.66], [0, 0, -0.60], [0, 0, 0.60], [0, 0, 1.66]]), [0, 1, 1, 0])
    o2 = (np.array([[0, 0, -0.605], [0, 0, 0.605]]), [3, 3])
    n2 = (np.array([[0, 0, -0.55], [0, 0, 0.55]]), [2, 2])
    kinds = np.concatenate([np.zeros(n_c2h2, int), np.ones(n_o2, int), np.full(n_n2, 2)])
    rng.shuffle(kinds)
    n_mol = kinds.shape[0]
    n_grid = int(np.ceil(n_mol ** (1.0 / 3.0)))
    spacing = box_len / n_grid
    sites = np.stack(np.meshgrid(*(np.arange(n_grid),) * 3, indexing="ij"), -1).reshape(-1, 3)
    chosen = rng.choice(sites.shape[0], size=n_mol, replace=False)
    centres = (sites[chosen] + 0.5) * spacing
    templates = [c2h2, o2, n2]
    n_at = np.array([len(templates[k][1]) for k in kinds])
    mol_of_atom = np.repeat(np.arange(n_mol), n_at)
    first = np.concatenate([[0], np.cumsum(n_at)[:-1]])
    slot = np.arange(mol_of_atom.shape[0]) - first[mol_of_atom]
    tmpl = np.zeros((3, 4, 3))
    for k, (xyz, _) in enumerate(templates):
        tmpl[k, :xyz.shape[0]] = xyz
    types = np.concatenate([np.asarray(templates[k][1], np.int32) for k in kinds]).astype(np.int32)
    R = _random_rotations(rng, n_mol)
    jit = rng.uniform(-0.3, 0.3, size=(n_mol, 3))

    def build_pos():
        loc = tmpl[kinds[mol_of_atom], slot]
        return centres[mol_of_atom] + jit[mol_of_atom] + np.einsum("nij,nj->ni", R[mol_of_atom], loc)

    pos = build_pos()
    for _ in range(2000):
        pairs = _min_image_close_pairs(pos, box, 2.0)
        if pairs.shape[0]:
            inter = mol_of_atom[pairs[:, 0]] != mol_of_atom[pairs[:, 1]]
            pairs = pairs[inter]
        if pairs.shape[0] == 0:
            break
        bad = np.unique(mol_of_atom[pairs[:, 0]])
        R[bad] = _random_rotations(rng, bad.shape[0])
        jit[bad] = rng.uniform(-0.3, 0.3, size=(bad.shape[0], 3))
        pos = build_pos()
    else:
        raise RuntimeError("CHON generator did not converge")
    masses = np.array([MASS[s] for s in species])
    vel = maxwell_boltzmann(masses[types], temp, vel_seed)
    return System("CHON", pos, types, box, vel, species, masses)


def ag(n_cells: int, seed: int, vel_seed: int, temp: float = 300.0, a: float = 4.09,
       jitter: float = 0.05, name: str = "Ag") -> System:
    pos, box, _ = fcc(n_cells, n_cells, n_cells, a, jitter, seed)
    types = np.zeros(pos.shape[0], np.int32)
    masses = np.array([MASS["Ag"]])
    vel = maxwell_boltzmann(masses[types], temp, vel_seed)
    return System(name, pos, types, box, vel, ["Ag"], masses)


def hea(n_cells: int, seed: int = 1003, vel_seed: int = 1103, temp: float = 300.0) -> System:
    pos, box, rng = bcc(n_cells, n_cells, n_cells, 3.20, 0.08, seed)
    types = rng.integers(0, 5, size=pos.shape[0]).astype(np.int32)
    species = ["V", "Nb", "Mo", "Ta", "W"]
    masses = np.array([MASS[s] for s in species])
    vel = maxwell_boltzmann(masses[types], temp, vel_seed)
    return System(f"HEA{pos.shape[0]}", pos, types, box, vel, species, masses)


def make_system(cfg: int, reduced: bool = False) -> System:
    """The benchmark system `cfg` (1..5); `reduced=True` gives the small instance of the same
    generator used to freeze the layer scales (about 4,000 atoms)."""
    if cfg == 1:
        return ag(10 if reduced else 3, 1001, 1101, name="Ag4000" if reduced else "Ag108")
    if cfg == 2:
        return water()
    if cfg == 3:
        return hea(13 if reduced else 40)
    if cfg == 4:
        return ag(10 if reduced else 80, 1004, 1104, name="Ag4000" if reduced else "Ag2M")
    if cfg == 5:
        if reduced:
            f = 4002 / 400002
            return chon(int(round(65772 * f)), int(round(65772 * f)), max(1, int(round(2685 * f))))
        return chon()
    raise ValueError(cfg)


def model_spec(cfg: int) -> ModelSpec:
    c = CONFIGS[cfg]
    n_species = {1: 1, 2: 2, 3: 5, 4: 1, 5: 4}[cfg]
    # the reactive CHON gas has a force tail up to ~90 RMS_F, which needs the fp64 mode to meet
    # max|dF| <= 1e-4 RMS_F; the other systems meet it in fp32
    return ModelSpec(n_species=n_species, K=c["K"], L=c["L"], T=c["T"], H=c["H"], rc=c["rc"],
                     skin=c["skin"], precision=1 if cfg == 5 else 0)


def _f32(a):
    """Round to the nearest float32 value (kept as float64)."""
    return np.asarray(a, np.float64).astype(np.float32).astype(np.float64)


def random_params(spec: ModelSpec, seed: int, masses, layer_scale=None, e_scale: float = 1.0,
                  round_f32: bool = True) -> Params:
    """Random-init weights: W, b ~ N(0, 1/fan_in); C0 ~ N(0, 1).  Draw order: C0, then for
    t in 0..T-1, for s in 0..S-1: W1, b1, W2, b2, W3, b3.

    With round_f32 (the benchmark models), every drawn value (and every radial centre) is rounded
    to the nearest float32, so an fp32 implementation holds exactly the same parameters as an fp64
    one; the frozen layer and energy scales are powers of two for the same reason.  round_f32=False
    keeps the fp64 draws (the same values before rounding), for checking how each arithmetic mode
    holds parameters that fp32 cannot represent."""
    _f32 = globals()["_f32"] if round_f32 else (lambda a: np.asarray(a, np.float64))
    rng = _rng(seed)
    K, L, T, H, S = spec.K, spec.L, spec.T, spec.H, spec.n_species
    D = K * (K + 1) * (L + 1) // 2
    mu = _f32([k * spec.rc / (K - 1) for k in range(K)]) if K > 1 else np.zeros(1)
    c0 = _f32(rng.standard_normal((S, K)))
    mlp = []
    for t in range(T):
        out = K if t < T - 1 else 1
        per_s = []
        for _s in range(S):
            w = {}
            w["W1"] = _f32(rng.standard_normal((H, D)) / np.sqrt(D))
            w["b1"] = _f32(rng.standard_normal(H) / np.sqrt(D))
            w["W2"] = _f32(rng.standard_normal((H, H)) / np.sqrt(H))
            w["b2"] = _f32(rng.standard_normal(H) / np.sqrt(H))
            w["W3"] = _f32(rng.standard_normal((out, H)) / np.sqrt(H))
            w["b3"] = _f32(rng.standard_normal(out) / np.sqrt(H))
            per_s.append(w)
        mlp.append(per_s)
    if layer_scale is None:
        layer_scale = np.ones(T)
    return Params(spec, mu, c0, mlp, np.asarray(layer_scale, np.float64), float(e_scale),
                  np.asarray(masses, np.float64))


def contraction_matrix(K: int, seed: int) -> np.ndarray:
    """Random contraction of the K radial primitives into K orbitals: C[n][k] ~ N(0, 1/K),
    rounded to float32 like every other drawn parameter."""
    return _f32(_rng(seed).standard_normal((K, K)) / np.sqrt(K))


def with_contraction(params: Params, C) -> Params:
    """The same model with orbital n built from the radial function sum_k C[n][k] R_k."""
    C = np.asarray(C, np.float64)
    if C.shape != (params.spec.K, params.spec.K):
        raise ValueError("contraction must be K x K")
    return dataclasses.replace(params, contraction=C.copy())


def load_scales() -> dict:
    if not os.path.exists(SCALES_FILE):
        return {}
    with open(SCALES_FILE) as f:
        return json.load(f)


def scales_key(cfg: int, contraction_seed: int = None) -> str:
    return str(cfg) if contraction_seed is None else f"{cfg}+contraction{contraction_seed}"


def make_params(cfg: int, require_scales: bool = True, contraction_seed: int = None) -> Params:
    """Random-init parameters of benchmark model `cfg` with its frozen layer/energy scales;
    with contraction_seed, the contraction variant of the same model (C from that seed) with the
    scales frozen for it."""
    spec = model_spec(cfg)
    sysm = {1: ["Ag"], 2: ["O", "H"], 3: ["V", "Nb", "Mo", "Ta", "W"], 4: ["Ag"],
            5: ["H", "C", "N", "O"]}[cfg]
    masses = [MASS[s] for s in sysm]
    key = scales_key(cfg, contraction_seed)
    scales = load_scales().get(key)
    if scales is None:
        if require_scales:
            raise RuntimeError(f"no frozen scales for model {key} in {SCALES_FILE}")
        p = random_params(spec, 1200 + cfg, masses)
    else:
        p = random_params(spec, 1200 + cfg, masses, scales["layer_scale"], scales["e_scale"])
    if contraction_seed is not None:
        p = with_contraction(p, contraction_matrix(spec.K, contraction_seed))
    return p


def depth_variant(cfg: int, T: int) -> Params:
    """Benchmark model cfg rebuilt with T message-passing layers (same seed and draw order; the
    frozen layer scales of the T-layer model, the last one repeated for deeper layers): the models
    of the cost-against-depth measurement."""
    base = make_params(cfg)
    spec = dataclasses.replace(base.spec, T=T)
    sc = list(base.layer_scale)
    ls = [sc[min(t, len(sc) - 1)] for t in range(T)]
    return random_params(spec, 1200 + cfg, base.masses, ls, base.e_scale)


def small_spec(K=2, L=1, T=2, H=8, S=1, rc=4.0, skin=0.5, sigma=0.5) -> ModelSpec:
    return ModelSpec(n_species=S, K=K, L=L, T=T, H=H, rc=rc, sigma=sigma, skin=skin)
