"""Thin ctypes binding of libmpnn.so (include/mpnn.h).  Argument marshalling only: every step of
the energy/force/MD path runs in the library's HIP kernels.  torch supplies device memory and
the stream.  There is no fallback: if the library is missing, calls raise."""
from __future__ import annotations

import ctypes as C
import os
import re

import numpy as np
import torch

from . import inputs

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmpnn.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "mpnn.h")

STATUS = {0: "MPNN_OK", -1: "MPNN_E_INVALID_ARG", -2: "MPNN_E_OOM", -3: "MPNN_E_HIP",
          -4: "MPNN_E_CAPACITY", -5: "MPNN_E_SKIN", -6: "MPNN_E_NONFINITE", -7: "MPNN_E_STATE",
          -8: "MPNN_E_BOX"}


class MPNNError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


class _Params(C.Structure):
    _fields_ = [("n_species", C.c_int32), ("K", C.c_int32), ("L", C.c_int32), ("T", C.c_int32),
                ("hidden", C.c_int32), ("precision", C.c_int32), ("rc", C.c_double),
                ("sigma", C.c_double), ("mu", C.POINTER(C.c_double)), ("c0", C.POINTER(C.c_double)),
                ("mlp", C.POINTER(C.c_double)), ("layer_scale", C.POINTER(C.c_double)),
                ("e_scale", C.c_double), ("mass", C.POINTER(C.c_double)),
                ("contraction", C.POINTER(C.c_double))]


# device allocator hooks of mpnn_set_allocator
_ALLOC_FN = C.CFUNCTYPE(C.c_void_p, C.c_size_t, C.c_void_p)
_FREE_FN = C.CFUNCTYPE(None, C.c_void_p, C.c_void_p)


class MDStats(C.Structure):
    _fields_ = [("epot", C.c_double), ("ekin", C.c_double), ("temp", C.c_double),
                ("rebuilds", C.c_int64), ("max_disp", C.c_double), ("steps", C.c_int64)]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


class Info(C.Structure):
    _fields_ = [("n_local", C.c_int64), ("n_ghost", C.c_int64), ("n_edges", C.c_int64),
                ("cells", C.c_int64 * 3), ("bytes_device", C.c_int64), ("row_bucketing", C.c_int64),
                ("n_slots", C.c_int64)]


_lib = None


def lib():
    """Load libmpnn.so (torch is imported first so one HIP runtime serves both)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run `python -m molecular_dynamics_cell_amd.build`")
        L = C.CDLL(LIB_PATH)
        p, i32, i64, d = C.c_void_p, C.c_int32, C.c_int64, C.c_double
        st = C.c_int
        sig = {
            "mpnn_create": ([C.POINTER(_Params), C.POINTER(p)], st),
            "mpnn_destroy": ([p], None),
            "mpnn_set_stream": ([p, p], st),
            "mpnn_build_neighbors": ([p, p, p, i64, C.POINTER(C.c_double), d, d], st),
            "mpnn_energy_forces": ([p, p, C.POINTER(C.c_double), p, p], st),
            "mpnn_energy_forces_noalloc": ([p, p, C.POINTER(C.c_double), p, p], st),
            "mpnn_md_step": ([p, d, i32, i32, C.POINTER(MDStats)], st),
            "mpnn_set_state": ([p, p, p], st),
            "mpnn_get_state": ([p, p, p, C.POINTER(C.c_int64)], st),
            "mpnn_get_pairs": ([p, i64, C.POINTER(C.c_int64), p, p, p], st),
            "mpnn_get_intermediate": ([p, i32, i32, p], st),
            "mpnn_get_info": ([p, C.POINTER(Info)], st),
            "mpnn_set_graph_replay": ([p, i32], st),
            "mpnn_set_subdomains": ([p, i32, i32, i32], st),
            "mpnn_set_allocator": ([p, _ALLOC_FN, _FREE_FN, p], st),
            "mpnn_set_profiling": ([p, i32], st),
            "mpnn_get_profile": ([p, i32, C.POINTER(C.c_char_p), C.POINTER(C.c_double),
                                  C.POINTER(C.c_int64)], st),
            "mpnn_last_error": ([p], C.c_char_p),
        }
        for name, (args, res) in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def header_symbols() -> list:
    """Names of the functions include/mpnn.h declares."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mpnn_[a-z_]+)\s*\(", text)))


def _dptr(t: torch.Tensor):
    return C.c_void_p(t.data_ptr()) if t is not None else None


class MPNN:
    """One library context: model parameters plus one system's neighbour list and state."""

    def __init__(self, params: inputs.Params, device="cuda"):
        self.params = params
        self.device = torch.device(device)
        s = params.spec
        self.T, self.K, self.L = s.T, s.K, s.L
        self.M = (s.L + 1) * (s.L + 2) * (s.L + 3) // 6
        self._keep = [np.ascontiguousarray(a, np.float64) for a in
                      (params.mu, params.c0, params.packed_mlp(), params.layer_scale, params.masses)]
        dp = C.POINTER(C.c_double)
        mu, c0, mlp, sc, ms = (a.ctypes.data_as(dp) for a in self._keep)
        ct = None
        if params.contraction is not None:
            self._keep.append(np.ascontiguousarray(params.contraction, np.float64).reshape(s.K, s.K))
            ct = self._keep[-1].ctypes.data_as(dp)
        self._p = _Params(s.n_species, s.K, s.L, s.T, s.H, int(s.precision), s.rc, s.sigma, mu, c0, mlp, sc,
                          float(params.e_scale), ms, ct)
        h = C.c_void_p()
        self._check(lib().mpnn_create(C.byref(self._p), C.byref(h)), None)
        self.h = h
        self.n = 0
        self.set_stream(torch.cuda.current_stream(self.device))

    def _check(self, code, h="self"):
        if code != 0:
            hh = self.h if h == "self" else h
            msg = lib().mpnn_last_error(hh).decode() if hh else ""
            raise MPNNError(code, msg)

    def close(self):
        if getattr(self, "h", None):
            lib().mpnn_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def set_stream(self, stream: torch.cuda.Stream):
        self._stream = stream
        self._check(lib().mpnn_set_stream(self.h, C.c_void_p(stream.cuda_stream)))

    def use_torch_allocator(self):
        """Take the context's later device buffers from torch's caching allocator, on the
        context's stream (existing buffers stay where they are)."""
        dev, stream = self.device, self._stream

        def alloc(nbytes, user):
            try:
                return torch.cuda.caching_allocator_alloc(int(nbytes), dev, stream)
            except RuntimeError:
                return None   # NULL: the library reports out of memory

        def release(ptr, user):
            torch.cuda.caching_allocator_delete(ptr)

        self._hooks = (_ALLOC_FN(alloc), _FREE_FN(release))   # alive as long as the context
        self._check(lib().mpnn_set_allocator(self.h, self._hooks[0], self._hooks[1], None))

    def build_neighbors(self, pos: torch.Tensor, types: torch.Tensor, box, rc=None, skin=None):
        pos = pos.to(self.device, torch.float64).contiguous()
        types = types.to(self.device, torch.int32).contiguous()
        b = (C.c_double * 3)(*[float(x) for x in box])
        rc = self.params.spec.rc if rc is None else rc
        skin = self.params.spec.skin if skin is None else skin
        self.n = pos.shape[0]
        self._check(lib().mpnn_build_neighbors(self.h, _dptr(pos), _dptr(types), self.n, b,
                                               float(rc), float(skin)))

    def energy_forces(self, pos: torch.Tensor = None, forces=True, atom_energy=False, energy=True):
        F = torch.empty((self.n, 3), dtype=torch.float64, device=self.device) if forces else None
        Ei = torch.empty(self.n, dtype=torch.float64, device=self.device) if atom_energy else None
        E = C.c_double(0.0)
        if pos is not None:
            pos = pos.to(self.device, torch.float64).contiguous()
        self._check(lib().mpnn_energy_forces(self.h, _dptr(pos), C.byref(E) if energy else None,
                                             _dptr(F), _dptr(Ei)))
        return E.value if energy else None, F, Ei

    def energy_forces_noalloc(self, pos: torch.Tensor = None, forces: torch.Tensor = None,
                              atom_energy: torch.Tensor = None, energy=True):
        """mpnn_energy_forces_noalloc: the caller passes the output tensors ([n][3] and [n] fp64 on
        the device, or None); the library allocates nothing."""
        E = C.c_double(0.0)
        if pos is not None:
            pos = pos.to(self.device, torch.float64).contiguous()
        for t, shape in ((forces, (self.n, 3)), (atom_energy, (self.n,))):
            if t is not None and (t.dtype != torch.float64 or tuple(t.shape) != shape or not t.is_contiguous()):
                raise ValueError(f"output must be a contiguous float64 tensor of shape {shape}")
        self._check(lib().mpnn_energy_forces_noalloc(self.h, _dptr(pos), C.byref(E) if energy else None,
                                                     _dptr(forces), _dptr(atom_energy)))
        return E.value if energy else None

    def md_step(self, dt, n_steps, rebuild_every=0, stats=True):
        st = MDStats()
        self._check(lib().mpnn_md_step(self.h, float(dt), int(n_steps), int(rebuild_every),
                                       C.byref(st) if stats else None))
        return st.as_dict() if stats else None

    def set_state(self, pos=None, vel=None):
        pos = pos.to(self.device, torch.float64).contiguous() if pos is not None else None
        vel = vel.to(self.device, torch.float64).contiguous() if vel is not None else None
        self._check(lib().mpnn_set_state(self.h, _dptr(pos), _dptr(vel)))

    def get_state(self):
        pos = torch.empty((self.n, 3), dtype=torch.float64, device=self.device)
        vel = torch.empty((self.n, 3), dtype=torch.float64, device=self.device)
        step = C.c_int64(0)
        self._check(lib().mpnn_get_state(self.h, _dptr(pos), _dptr(vel), C.byref(step)))
        return pos, vel, step.value

    def get_pairs(self):
        cnt = C.c_int64(0)
        self._check(lib().mpnn_get_pairs(self.h, 0, C.byref(cnt), None, None, None))
        n = cnt.value
        i = torch.empty(max(n, 1), dtype=torch.int32, device=self.device)
        j = torch.empty(max(n, 1), dtype=torch.int32, device=self.device)
        s = torch.empty((max(n, 1), 3), dtype=torch.int32, device=self.device)
        self._check(lib().mpnn_get_pairs(self.h, n, C.byref(cnt), _dptr(i), _dptr(j), _dptr(s)))
        return i[:n], j[:n], s[:n]

    def get_intermediate(self, which: int, t: int = 0):
        width = {0: self.K, 1: self.K * self.M, 2: self.K * self.M, 3: 1, 4: self.K}[which]
        out = torch.empty((self.n, width), dtype=torch.float64, device=self.device)
        self._check(lib().mpnn_get_intermediate(self.h, int(which), int(t), _dptr(out)))
        return out

    def set_graph_replay(self, steps_per_replay: int):
        """Replay MD in captured chunks of up to this many steps (0: eager)."""
        self._check(lib().mpnn_set_graph_replay(self.h, int(steps_per_replay)))

    def set_subdomains(self, px: int, py: int, pz: int):
        """Split the box into px x py x pz virtual subdomains from the next build on."""
        self._check(lib().mpnn_set_subdomains(self.h, int(px), int(py), int(pz)))

    def set_profiling(self, enable: bool):
        self._check(lib().mpnn_set_profiling(self.h, 1 if enable else 0))

    def profile(self) -> dict:
        """{kernel family: (total ms, launches)} from the library's event profiler."""
        out = {}
        idx = 0
        while True:
            name = C.c_char_p()
            ms = C.c_double()
            cnt = C.c_int64()
            if lib().mpnn_get_profile(self.h, idx, C.byref(name), C.byref(ms), C.byref(cnt)) != 0:
                break
            out[name.value.decode()] = (ms.value, cnt.value)
            idx += 1
        return out

    def info(self):
        inf = Info()
        self._check(lib().mpnn_get_info(self.h, C.byref(inf)))
        return dict(n_local=inf.n_local, n_ghost=inf.n_ghost, n_edges=inf.n_edges,
                    cells=list(inf.cells), bytes_device=inf.bytes_device, row_bucketing=inf.row_bucketing,
                    n_slots=inf.n_slots)
