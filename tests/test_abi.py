"""CPU checks of the boundary: the C-ABI library loads (no GPU needed) and exports every entry
point include/mpnn.h declares; the binding declares a signature for each of them; the oracle
library exports its C API; the package imports without a GPU."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "molecular_dynamics_cell_amd", "libmpnn.so")


@pytest.fixture(scope="module")
def mpnn_lib():
    if not os.path.exists(LIB):
        from molecular_dynamics_cell_amd import build
        build.build(verbose=False)
    import torch  # noqa: F401  (one HIP runtime for torch and the library)
    return C.CDLL(LIB)


def test_header_symbols_exported(mpnn_lib):
    from molecular_dynamics_cell_amd import binding
    syms = binding.header_symbols()
    assert len(syms) >= 14
    missing = [s for s in syms if not hasattr(mpnn_lib, s)]
    assert not missing, missing


def test_binding_covers_header():
    from molecular_dynamics_cell_amd import binding
    src = open(binding.__file__).read()
    for s in binding.header_symbols():
        assert f'"{s}"' in src, s


def test_header_is_plain_c():
    text = open(os.path.join(ROOT, "include", "mpnn.h")).read()
    assert 'extern "C"' in text
    code = re.sub(r"/\*.*?\*/", "", text, flags=re.S)      # declarations only, not comments
    for banned in ("torch", "at::", "hip_runtime", "std::"):
        assert banned not in code


def test_oracle_exports():
    import oracle
    L = oracle.lib()
    hdr = open(os.path.join(ROOT, "oracle", "orc.h")).read()
    for name in re.findall(r"\b(orc_[a-z_]+)\s*\(", hdr):
        assert hasattr(L, name), name


def test_no_oracle_in_product_path():
    """The HIP package never imports the oracle."""
    pkg = os.path.join(ROOT, "molecular_dynamics_cell_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "orc.h" not in text and "liborc" not in text, f


def test_create_rejects_bad_params(mpnn_lib):
    """mpnn_create validates its arguments before touching the device (runs without a GPU)."""
    import numpy as np
    from molecular_dynamics_cell_amd import binding
    from molecular_dynamics_cell_amd import inputs as I
    p = I.random_params(I.small_spec(K=2, L=1, T=2, H=64), 3, [1.0])
    dp = C.POINTER(C.c_double)
    keep = [np.ascontiguousarray(a, np.float64) for a in
            (p.mu, p.c0, p.packed_mlp(), p.layer_scale, p.masses, np.eye(2))]
    ptr = [a.ctypes.data_as(dp) for a in keep]

    def create(precision=0, K=2, contraction=ptr[5]):
        s = p.spec
        prm = binding._Params(s.n_species, K, s.L, s.T, s.H, precision, s.rc, s.sigma, *ptr[:4],
                              float(p.e_scale), ptr[4], contraction)
        h = C.c_void_p()
        fn = mpnn_lib.mpnn_create
        fn.argtypes = [C.POINTER(binding._Params), C.POINTER(C.c_void_p)]
        fn.restype = C.c_int
        return fn(C.byref(prm), C.byref(h))

    assert create(precision=3) == -1              # unknown arithmetic mode
    assert create(K=5) == -1                      # unsupported (K, L)
    keep[5][0, 1] = np.nan
    assert create(contraction=ptr[5]) == -1       # non-finite contraction entry
