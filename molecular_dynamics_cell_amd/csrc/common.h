// Shared device/host definitions of the MPNN library (gfx950).  Nothing here is part of the
// public ABI (include/mpnn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mpnn {

// 1 eV/(A amu) in A/fs^2 and the Boltzmann constant in eV/K (CODATA 2018).
constexpr double kAccel = 9.648533212e-3;
constexpr double kBoltzmann = 8.617333262e-5;
constexpr double kPi = 3.14159265358979323846;

constexpr int kBlock = 256;  // threads per block of the one-thread-per-item kernels

inline unsigned grid_for(int64_t n, int block = kBlock) {
    return (unsigned)((n + block - 1) / block > 0 ? (n + block - 1) / block : 1);
}

// ------------------------------------------------------------------------------------------
// Compile-time structure of the orbital basis (paper, "REANN Architecture": primitives with
// angular momenta lx+ly+lz = l <= L; Eq. 1 weights l!/(lx! ly! lz!)).
// ------------------------------------------------------------------------------------------
constexpr int n_mono(int L) { return (L + 1) * (L + 2) * (L + 3) / 6; }
constexpr int n_feat(int K, int L) { return K * (K + 1) * (L + 1) / 2; }
constexpr int fact(int k) { return k <= 1 ? 1 : k * fact(k - 1); }

template <int L>
struct Mono {
    static constexpr int M = n_mono(L);
    int lx[M], ly[M], lz[M], l[M];
    float w[M];
    constexpr Mono() : lx(), ly(), lz(), l(), w() {
        int m = 0;
        for (int ll = 0; ll <= L; ++ll)
            for (int x = ll; x >= 0; --x)
                for (int y = ll - x; y >= 0; --y) {
                    lx[m] = x; ly[m] = y; lz[m] = ll - x - y; l[m] = ll;
                    w[m] = (float)(fact(ll) / (fact(x) * fact(y) * fact(ll - x - y)));
                    ++m;
                }
    }
};

// Feature q <-> (a, b, l): q = l*K(K+1)/2 + row-major rank of (a, b), a <= b, in the upper
// triangle.  first[l] = first monomial of angular momentum l.
template <int K, int L>
struct Feat {
    static constexpr int D = n_feat(K, L);
    unsigned char a[D], b[D], l[D];
    unsigned char first[L + 2];
    constexpr Feat() : a(), b(), l(), first() {
        int q = 0;
        for (int ll = 0; ll <= L; ++ll)
            for (int x = 0; x < K; ++x)
                for (int y = x; y < K; ++y) {
                    a[q] = (unsigned char)x; b[q] = (unsigned char)y; l[q] = (unsigned char)ll;
                    ++q;
                }
        int m = 0;
        for (int ll = 0; ll <= L + 1; ++ll) {
            first[ll] = (unsigned char)m;
            m += (ll + 1) * (ll + 2) / 2;
        }
    }
};

// ------------------------------------------------------------------------------------------
// fp64 helpers that are never contracted into FMAs, so pair distances are bit-identical to a
// plain left-to-right evaluation of (dx*dx + dy*dy) + dz*dz.
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ double d2_exact(double dx, double dy, double dz) {
    return __dadd_rn(__dadd_rn(__dmul_rn(dx, dx), __dmul_rn(dy, dy)), __dmul_rn(dz, dz));
}

// Per-context model tables living in device memory (read with uniform loads).
struct ModelDev {
    float mu[16];
    float c0[16 * 16];      // [S][K]
    float inv_scale[8];     // 1 / s_t
    float e_scale;
    float neg_half_inv_s2;  // -1 / (2 sigma^2)
    float inv_s2;           // 1 / sigma^2
    float rc, inv_rc, pi_over_rc;
    double rc2;             // rc^2 (fp64, for the active-edge test)
    double mass[16];        // amu per species
};

// Periodic image shift code 0..26 <-> (sx, sy, sz) in {-1,0,1}^3; 13 is the identity.
__host__ __device__ inline void shift_of(int code, int &sx, int &sy, int &sz) {
    sx = code / 9 - 1;
    sy = (code / 3) % 3 - 1;
    sz = code % 3 - 1;
}

}  // namespace mpnn
