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

// XCD-aware launches: the hardware deals consecutive workgroups round-robin to the 8 XCDs, each
// with its own L2.  Launch a multiple of 8 groups and let group b work on logical block
// (b % 8) * (groups / 8) + b / 8, so every XCD sweeps one contiguous (spatially compact) range
// of the cell-ordered atoms.
constexpr int kXcds = 8;
inline unsigned grid_xcd(int64_t n, int block = kBlock) {
    const int64_t g = ((n + block - 1) / block + kXcds - 1) / kXcds * kXcds;
    return (unsigned)(g > 0 ? g : kXcds);
}
__device__ __forceinline__ int64_t xcd_block() {
    const int64_t per = gridDim.x / kXcds;
    return (int64_t)(blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
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
    int mx[M], my[M], mz[M];   // index of the monomial with one power of x (y, z) fewer, or -1
    float w[M];
    // position of x^a y^b z^c in the order below: degree, then a descending, then b descending
    static constexpr int index(int a, int b, int c) {
        const int ll = a + b + c;
        return ll * (ll + 1) * (ll + 2) / 6 + (ll - a) * (ll - a + 1) / 2 + (ll - a - b);
    }
    constexpr Mono() : lx(), ly(), lz(), l(), mx(), my(), mz(), w() {
        int m = 0;
        for (int ll = 0; ll <= L; ++ll)
            for (int x = ll; x >= 0; --x)
                for (int y = ll - x; y >= 0; --y) {
                    const int z = ll - x - y;
                    lx[m] = x; ly[m] = y; lz[m] = z; l[m] = ll;
                    mx[m] = x ? index(x - 1, y, z) : -1;
                    my[m] = y ? index(x, y - 1, z) : -1;
                    mz[m] = z ? index(x, y, z - 1) : -1;
                    w[m] = (float)(fact(ll) / (fact(x) * fact(y) * fact(z)));
                    ++m;
                }
    }
};

template <int L>
constexpr bool mono_index_consistent() {
    constexpr Mono<L> mo;
    for (int m = 0; m < Mono<L>::M; ++m) {
        if (Mono<L>::index(mo.lx[m], mo.ly[m], mo.lz[m]) != m) return false;
        if (mo.lx[m] && mo.lx[mo.mx[m]] != mo.lx[m] - 1) return false;
        if (mo.ly[m] && mo.ly[mo.my[m]] != mo.ly[m] - 1) return false;
        if (mo.lz[m] && mo.lz[mo.mz[m]] != mo.lz[m] - 1) return false;
    }
    return true;
}
static_assert(mono_index_consistent<1>() && mono_index_consistent<2>() && mono_index_consistent<3>(),
              "monomial index map");

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

// Feature q (order: l-major, then the upper-triangle rank of (a, b), a <= b) -> (l, a, b);
// q past the last feature gives l > L (zero padding).
struct FeatIdx {
    int l, a, b;
};
constexpr FeatIdx feat_idx(int K, int q) {
    const int P = K * (K + 1) / 2;
    int r = q % P, x = 0;
    while (r >= K - x) {
        r -= K - x;
        ++x;
    }
    return FeatIdx{q / P, x, x + r};
}

// ------------------------------------------------------------------------------------------
// Per-atom vectors of the networks (orbital coefficients O, density features rho/s, dE/drho)
// are stored column-tiled: element q of atom i at ((q / 16) np + i) 16 + q % 16, where np is
// the atom count rounded up to whole 256-row blocks.  Sixteen columns of consecutive atoms form
// one contiguous run, so a block writes a tile with full-line stores and a network tile reads
// 64 contiguous bytes per atom.
// ------------------------------------------------------------------------------------------
constexpr int pad16(int w) { return (w + 15) / 16 * 16; }

// Node records: per node and layer, the position (3 doubles in an 8-float header) followed by the
// K message coefficients, padded to a multiple of 8 floats (64 bytes for K <= 8), so one
// neighbour's position and messages share a cache line in the row kernels' gathers.
constexpr int rec_stride(int K) { return 8 + (K + 7) / 8 * 8; }
constexpr int kRecC = 8;   // float offset of c inside a record
inline int64_t pad_rows(int64_t n) { return (n + kBlock - 1) / kBlock * kBlock; }
__host__ __device__ __forceinline__ int64_t tiled(int64_t np, int64_t i, int q) {
    return ((int64_t)(q >> 4) * np + i) * 16 + (q & 15);
}

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
    double c0_64[16 * 16];  // [S][K] in fp64 (arithmetic mode 1 holds every parameter in fp64)
    double e_scale64;
    float inv_scale[8];     // 1 / s_t
    float e_scale;
    float neg_half_inv_s2;  // -1 / (2 sigma^2)
    float inv_s2;           // 1 / sigma^2
    float rc, inv_rc, pi_over_rc;
    float exp2_coef;        // -log2(e) / (2 sigma^2): R_k = exp2(exp2_coef (d - mu_k)^2)
    float dfc_scale;        // -pi / (2 rc): df_c/dd = dfc_scale sin(pi d / rc)
    double rc2;             // rc^2 (fp64, for the active-edge test)
    double mass[16];        // amu per species
    // fp64 constants of the aggregation basis
    double mu64[16];        // radial centres
    double g_a0;            // -1 / (2 sigma^2)
    double g_e;             // delta / sigma^2, delta = mu_1 - mu_0
    double g_c[16];         // exp(-delta_k (mu_k + mu_{k+1}) / (2 sigma^2)), delta_k = mu_{k+1} - mu_k
    double g_eps[16];       // (delta_k - delta) / sigma^2
    double g_ce[16];        // g_c[k] g_eps[k]
    double inv_rc64;        // 1 / rc
    double half_pi_over_rc; // pi / (2 rc)
    // contraction variant: orbital n uses the radial function sum_k C[n][k] R_k (row stride K)
    double C64[16 * 16];
    float C32[16 * 16];
};

// Sliced-ELLPACK neighbour storage: rows are grouped in slabs of 64 consecutive (cell-ordered)
// atoms; entry j of row i lives at slab_off[i / 64] + 64 j + i % 64, so the 64 lanes of a wave
// that each walk one row touch 64 consecutive words per step.
constexpr int kSlab = 64;
__host__ __device__ inline int64_t sell_base(const int64_t *slab_off, int64_t i) {
    return slab_off[i / kSlab] + (i % kSlab);
}

// Periodic image shift code 0..26 <-> (sx, sy, sz) in {-1,0,1}^3; 13 is the identity.
__host__ __device__ inline void shift_of(int code, int &sx, int &sy, int &sz) {
    sx = code / 9 - 1;
    sy = (code / 3) % 3 - 1;
    sz = code % 3 - 1;
}

}  // namespace mpnn
