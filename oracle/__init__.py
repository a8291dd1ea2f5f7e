"""fp64 CPU oracle of the REANN-style MPNN potential: TEST INFRASTRUCTURE ONLY.

Only the tests, the benchmark's `cpu_baseline` leg and `__graft_entry__.smoke()` may import
this package.  The product path (the HIP library and its binding) never does.

The C sources (orc.c / orc.h) follow "Efficient Parallelization of Message Passing Neural
Network Potentials for Large-Scale Molecular Dynamics" (Xia & Jiang): section "REANN
Architecture" (Eq. 1-2, Fig. 1) for the model and section "Parallelization Algorithm"
(Eq. 3-5, Fig. 3-4) for forces and the spatial decomposition.

Parity unpinned: agreement with the authors' own REANN code or trained models cannot be
checked (no weights, no printed values); every other function is pinned by the tests in
tests/test_oracle_*.py.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liborc.so")
_SRC = [os.path.join(_HERE, "orc.c")]
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-ffp-contract=off keeps every product/sum rounded)."""
    if force or not os.path.exists(LIB_PATH):
        cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
               "-Wall", "-Wextra", "-Wno-unused-parameter", "-o", LIB_PATH + ".tmp", *_SRC, "-lm"]
        subprocess.run(cmd, check=True, cwd=_HERE)
        os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


class _Model(C.Structure):
    _fields_ = [("S", C.c_int), ("K", C.c_int), ("L", C.c_int), ("T", C.c_int), ("H", C.c_int),
                ("rc", C.c_double), ("sigma", C.c_double),
                ("mu", C.POINTER(C.c_double)), ("c0", C.POINTER(C.c_double)),
                ("mlp", C.POINTER(C.c_double)), ("layer_scale", C.POINTER(C.c_double)),
                ("e_scale", C.c_double), ("contraction", C.POINTER(C.c_double))]


class _Dump(C.Structure):
    _fields_ = [("O", C.POINTER(C.c_double)), ("rho", C.POINTER(C.c_double)),
                ("c", C.POINTER(C.c_double)), ("GO", C.POINTER(C.c_double))]


class _Stats(C.Structure):
    _fields_ = [("epot", C.c_double), ("ekin", C.c_double), ("temp", C.c_double),
                ("rebuilds", C.c_int64), ("max_disp", C.c_double)]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = C.CDLL(LIB_PATH)
        d, i64, p = C.c_double, C.c_int64, C.c_void_p
        L.orc_wrap.argtypes = [i64, p, p, p]
        L.orc_pairs_brute.argtypes = [i64, p, p, d, i64, p, p, p]
        L.orc_pairs_brute.restype = i64
        L.orc_pairs_cell.argtypes = [i64, p, p, d, i64, p, p, p]
        L.orc_pairs_cell.restype = i64
        L.orc_energy_forces.argtypes = [C.POINTER(_Model), i64, p, p, p, i64, p, p, p, p, p, p,
                                        C.POINTER(_Dump)]
        L.orc_energy_forces_decomposed.argtypes = [C.POINTER(_Model), i64, p, p, p, d, C.c_int,
                                                   C.c_int, C.c_int, d, C.c_int, p, p]
        L.orc_md.argtypes = [C.POINTER(_Model), i64, p, p, p, p, p, d, d, C.c_int, C.c_int, p, p,
                             C.POINTER(_Stats)]
        L.orc_num_threads.restype = C.c_int
        _lib = L
    return _lib


def _ptr(a):
    return a.ctypes.data_as(C.c_void_p) if a is not None else None


class Model:
    """Keeps the contiguous float64 arrays alive for the C struct."""

    def __init__(self, params):
        s = params.spec
        self.params = params
        self.mu = np.ascontiguousarray(params.mu, np.float64)
        self.c0 = np.ascontiguousarray(params.c0, np.float64)
        self.mlp = np.ascontiguousarray(params.packed_mlp(), np.float64)
        self.scale = np.ascontiguousarray(params.layer_scale, np.float64)
        self.T, self.K, self.L, self.n_species = s.T, s.K, s.L, s.n_species
        self.M = (s.L + 1) * (s.L + 2) * (s.L + 3) // 6
        self.D = s.K * (s.K + 1) * (s.L + 1) // 2
        dp = C.POINTER(C.c_double)
        self.contraction = (None if params.contraction is None else
                            np.ascontiguousarray(params.contraction, np.float64).reshape(s.K, s.K))
        self.struct = _Model(s.n_species, s.K, s.L, s.T, s.H, s.rc, s.sigma,
                             self.mu.ctypes.data_as(dp), self.c0.ctypes.data_as(dp),
                             self.mlp.ctypes.data_as(dp), self.scale.ctypes.data_as(dp),
                             float(params.e_scale),
                             None if self.contraction is None else self.contraction.ctypes.data_as(dp))


def wrap(pos, box):
    pos = np.ascontiguousarray(pos, np.float64)
    box = np.ascontiguousarray(box, np.float64)
    out = np.empty_like(pos)
    lib().orc_wrap(pos.shape[0], _ptr(pos), _ptr(box), _ptr(out))
    return out


def pairs(pos_wrapped, box, rcut, method="cell"):
    """(i, j, S[3]) int32 arrays of every pair closer than rcut (positions already wrapped)."""
    pos = np.ascontiguousarray(pos_wrapped, np.float64)
    box = np.ascontiguousarray(box, np.float64)
    fn = lib().orc_pairs_cell if method == "cell" else lib().orc_pairs_brute
    n = fn(pos.shape[0], _ptr(pos), _ptr(box), float(rcut), 0, None, None, None)
    if n < 0:
        raise ValueError("oracle pair builder rejected the input")
    pi = np.empty(n, np.int32); pj = np.empty(n, np.int32); ps = np.empty((n, 3), np.int32)
    n2 = fn(pos.shape[0], _ptr(pos), _ptr(box), float(rcut), n, _ptr(pi), _ptr(pj), _ptr(ps))
    assert n2 == n
    return pi, pj, ps


def energy_forces(model: Model, pos_wrapped, types, box, pair_list=None, skin=None, dump=False):
    """Returns (E, F[n,3], E_i[n]) and, with dump=True, a dict of per-layer intermediates."""
    pos = np.ascontiguousarray(pos_wrapped, np.float64)
    types = np.ascontiguousarray(types, np.int32)
    box = np.ascontiguousarray(box, np.float64)
    if pair_list is None:
        sk = model.params.spec.skin if skin is None else skin
        pair_list = pairs(pos, box, model.params.spec.rc + sk)
    pi, pj, ps = (np.ascontiguousarray(a, np.int32) for a in pair_list)
    n = pos.shape[0]
    E = C.c_double(0.0)
    F = np.zeros((n, 3)); Ei = np.zeros(n)
    dmp = None
    arrays = {}
    if dump:
        T, K, KM, D = model.T, model.K, model.K * model.M, model.D
        arrays = dict(O=np.zeros((T, n, KM)), rho=np.zeros((T, n, D)), c=np.zeros((T, n, K)),
                      GO=np.zeros((T, n, KM)))
        dp = C.POINTER(C.c_double)
        dmp = _Dump(*(arrays[k].ctypes.data_as(dp) for k in ("O", "rho", "c", "GO")))
    rc = lib().orc_energy_forces(C.byref(model.struct), n, _ptr(pos), _ptr(types), _ptr(box),
                                 pi.shape[0], _ptr(pi), _ptr(pj), _ptr(ps), C.byref(E), _ptr(F),
                                 _ptr(Ei), C.byref(dmp) if dmp is not None else None)
    if rc != 0:
        raise RuntimeError(f"orc_energy_forces failed ({rc})")
    if dump:
        return E.value, F, Ei, arrays
    return E.value, F, Ei


def energy_forces_decomposed(model: Model, pos_wrapped, types, box, grid=(2, 2, 2), shell=None,
                             mode=0, skin=None):
    pos = np.ascontiguousarray(pos_wrapped, np.float64)
    types = np.ascontiguousarray(types, np.int32)
    box = np.ascontiguousarray(box, np.float64)
    sk = model.params.spec.skin if skin is None else skin
    if shell is None:
        shell = model.params.spec.rc + sk
    E = C.c_double(0.0)
    F = np.zeros_like(pos)
    rc = lib().orc_energy_forces_decomposed(C.byref(model.struct), pos.shape[0], _ptr(pos),
                                            _ptr(types), _ptr(box), float(sk), int(grid[0]),
                                            int(grid[1]), int(grid[2]), float(shell), int(mode),
                                            C.byref(E), _ptr(F))
    if rc != 0:
        raise RuntimeError(f"orc_energy_forces_decomposed failed ({rc})")
    return E.value, F


def md(model: Model, pos, vel, types, masses, box, dt, n_steps, rebuild_every=0, skin=None):
    """Velocity Verlet; returns (pos, vel, epot_trace, ekin_trace, stats dict)."""
    pos = np.array(pos, np.float64, order="C", copy=True)
    vel = np.array(vel, np.float64, order="C", copy=True)
    types = np.ascontiguousarray(types, np.int32)
    masses = np.ascontiguousarray(masses, np.float64)
    box = np.ascontiguousarray(box, np.float64)
    sk = model.params.spec.skin if skin is None else skin
    ep = np.zeros(n_steps + 1); ek = np.zeros(n_steps + 1)
    st = _Stats()
    rc = lib().orc_md(C.byref(model.struct), pos.shape[0], _ptr(pos), _ptr(vel), _ptr(types),
                      _ptr(masses), _ptr(box), float(sk), float(dt), int(n_steps),
                      int(rebuild_every), _ptr(ep), _ptr(ek), C.byref(st))
    if rc != 0:
        raise RuntimeError(f"orc_md failed ({rc})")
    stats = dict(epot=st.epot, ekin=st.ekin, temp=st.temp, rebuilds=st.rebuilds,
                 max_disp=st.max_disp)
    return pos, vel, ep, ek, stats


def num_threads() -> int:
    return int(lib().orc_num_threads())
