// Edge kernels: the fused edge basis (Gaussian radial x cosine cutoff x scaled Cartesian
// monomial), the per-receiver orbital aggregation of Eq. 1, the reverse pass of Eq. 4-5
// (dE/dc of every sender, dE/dr of every edge) and the deterministic force gather of Eq. 3;
// plus the per-layer ghost refresh that stands in for the paper's ghost-message exchange
// (section "Parallelization Algorithm", Fig. 4a) and its reverse, the ghost->owner sum of
// gradient components (Fig. 4b).
//
// Every reduction has a fixed order (one thread owns one output row and walks its list), so
// results are bitwise reproducible and no floating-point atomics are used.
#include <algorithm>
#include <cmath>
#include <type_traits>
#include <utility>

#include "impl.h"

namespace mpnn {

namespace {

// sin and cos of theta = (pi/2) v for v in [0, 1], from their Taylor series (error terms
// theta^15/15! and theta^14/14!, below 1e-8 on [0, pi/2]); pi/2 is split into two floats so the
// argument carries no rounding bias.
__device__ __forceinline__ void sincos_half_pi(float v, float &s, float &c) {
    const float t = fmaf(v, 1.57079637f, v * -4.37113900e-8f);
    const float t2 = t * t;
    s = t * fmaf(t2, fmaf(t2, fmaf(t2, fmaf(t2, fmaf(t2, fmaf(t2, 1.0f / 6227020800.0f, -1.0f / 39916800.0f),
                                                     1.0f / 362880.0f), -1.0f / 5040.0f), 1.0f / 120.0f),
                             -1.0f / 6.0f), 1.0f);
    c = fmaf(t2, fmaf(t2, fmaf(t2, fmaf(t2, fmaf(t2, fmaf(t2, 1.0f / 479001600.0f, -1.0f / 3628800.0f),
                                                 1.0f / 40320.0f), -1.0f / 720.0f), 1.0f / 24.0f), -0.5f), 1.0f);
}

// Edge basis of one edge for the reverse pass (forces only), fp32, from the fp64 displacement:
// hardware exp2 of a pre-scaled argument for the Gaussians, the hardware square root and reciprocal
// for d and 1/d (one ulp each, about 1e-7 relative in an edge's force terms; the correctly rounded
// forms cost 1.2 % more time in the reverse pass), and the cutoff written as
// f_c = (1 + cos(pi v))/2 = cos^2(pi v/2), f_c' = -(pi/rc) sin(pi v/2) cos(pi v/2), which has no
// cancellation near rc.  (In the orbital sums, which set the energy, the hardware sqrt and cos/sin
// shifted the total energy by several 1e-6 relative; those use BasisHP below.)
// CT: the contraction variant, orbital n from sum_k C[n][k] R_k (and its derivative), in fp32.
template <int K, int L, bool CT = false>
struct Basis {
    static constexpr int M = n_mono(L);
    float Rf[K], Rd[K], A[M];   // R_k f_c, its derivative along d, monomials of r / rc
    float inv_d, rx, ry, rz;

    __device__ __forceinline__ void eval(double dx, double dy, double dz, const ModelDev *__restrict__ md,
                                         const float *mu) {
        constexpr Mono<L> mono;
        rx = (float)dx; ry = (float)dy; rz = (float)dz;
        const float d = __builtin_amdgcn_sqrtf(rx * rx + ry * ry + rz * rz);
        inv_d = __builtin_amdgcn_rcpf(d);
        // x / rc as a refined quotient (no bias from rounding 1/rc)
        const float rc = md->rc, ir = md->inv_rc;
        auto div_rc = [rc, ir](float x) {
            const float q = x * ir;
            return fmaf(fmaf(-q, rc, x), ir, q);
        };
        float sh, ch;
        sincos_half_pi(div_rc(d), sh, ch);
        const float fc = ch * ch;
        const float dfc = 2.0f * md->dfc_scale * sh * ch;
        const float c2 = md->exp2_coef, is2fc = md->inv_s2 * fc;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            // dR_k/dd = -(d - mu_k) R_k / s^2
            const float x = d - mu[k];
            const float R = __builtin_amdgcn_exp2f(c2 * x * x);
            Rf[k] = R * fc;
            Rd[k] = R * fmaf(-x, is2fc, dfc);
        }
        if constexpr (CT) {
            float cf[K], cd[K];
#pragma unroll
            for (int q = 0; q < K; ++q) {
                float x = 0.0f, y = 0.0f;
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    const float w = md->C32[q * K + k];
                    x = fmaf(w, Rf[k], x);
                    y = fmaf(w, Rd[k], y);
                }
                cf[q] = x;
                cd[q] = y;
            }
#pragma unroll
            for (int q = 0; q < K; ++q) {
                Rf[q] = cf[q];
                Rd[q] = cd[q];
            }
        }
        const float qx = div_rc(rx), qy = div_rc(ry), qz = div_rc(rz);
        float ux[L + 1], uy[L + 1], uz[L + 1];
        ux[0] = uy[0] = uz[0] = 1.0f;
#pragma unroll
        for (int p = 1; p <= L; ++p) {
            ux[p] = ux[p - 1] * qx;
            uy[p] = uy[p - 1] * qy;
            uz[p] = uz[p - 1] * qz;
        }
#pragma unroll
        for (int m = 0; m < M; ++m) A[m] = ux[mono.lx[m]] * uy[mono.ly[m]] * uz[mono.lz[m]];
    }
};

// The fp32 edge basis for half of the radial channels (the channel-split reverse pass): mu holds
// the lane's K/2 centres; monomials, 1/d and the displacement as in Basis.
template <int K, int L>
struct BasisHalf {
    static constexpr int KH = K / 2, M = n_mono(L);
    float Rf[KH], Rd[KH], A[M];
    float inv_d, rx, ry, rz;

    __device__ __forceinline__ void eval(double dx, double dy, double dz, const ModelDev *__restrict__ md,
                                         const float (&mu)[KH]) {
        constexpr Mono<L> mono;
        rx = (float)dx; ry = (float)dy; rz = (float)dz;
        const float d = sqrtf(rx * rx + ry * ry + rz * rz);
        inv_d = 1.0f / d;
        const float rc = md->rc, ir = md->inv_rc;
        auto div_rc = [rc, ir](float x) {
            const float q = x * ir;
            return fmaf(fmaf(-q, rc, x), ir, q);
        };
        float sh, ch;
        sincos_half_pi(div_rc(d), sh, ch);
        const float fc = ch * ch;
        const float dfc = 2.0f * md->dfc_scale * sh * ch;
        const float c2 = md->exp2_coef, is2fc = md->inv_s2 * fc;
#pragma unroll
        for (int k = 0; k < KH; ++k) {
            const float x = d - mu[k];
            const float R = __builtin_amdgcn_exp2f(c2 * x * x);
            Rf[k] = R * fc;
            Rd[k] = R * fmaf(-x, is2fc, dfc);
        }
        const float qx = div_rc(rx), qy = div_rc(ry), qz = div_rc(rz);
        float ux[L + 1], uy[L + 1], uz[L + 1];
        ux[0] = uy[0] = uz[0] = 1.0f;
#pragma unroll
        for (int p = 1; p <= L; ++p) {
            ux[p] = ux[p - 1] * qx;
            uy[p] = uy[p - 1] * qy;
            uz[p] = uz[p - 1] * qz;
        }
#pragma unroll
        for (int m = 0; m < M; ++m) A[m] = ux[mono.lx[m]] * uy[mono.ly[m]] * uz[mono.lz[m]];
    }
};

// e^x in fp64 for x <= 709: x = n ln 2 + r with ln 2 in two parts (Cody and Waite), so r is exact
// to rounding and |r| <= ln 2 / 2; e^r from its Taylor series to r^11 (truncation below 7e-15
// relative; SHORT: to r^8, below 3e-10, for factors that are rounded to fp32 afterwards), scaled
// by 2^n.  Arguments below -745 give 0 (the fp64 result underflows there).
template <bool SHORT = false>
__device__ __forceinline__ double exp_fp64(double x) {
    x = fmax(x, -745.0);
    const double n = rint(x * 1.4426950408889634);
    double r = fma(n, -6.93147180369123816490e-01, x);
    r = fma(n, -1.90821492927058770002e-10, r);
    double p;
    if constexpr (SHORT) {
        p = 1.0 / 40320.0;                // 1/8!
    } else {
        p = 1.0 / 39916800.0;             // 1/11!
        p = fma(p, r, 1.0 / 3628800.0);   // 1/10!
        p = fma(p, r, 1.0 / 362880.0);
        p = fma(p, r, 1.0 / 40320.0);
    }
    p = fma(p, r, 1.0 / 5040.0);
    p = fma(p, r, 1.0 / 720.0);
    p = fma(p, r, 1.0 / 120.0);
    p = fma(p, r, 1.0 / 24.0);
    p = fma(p, r, 1.0 / 6.0);
    p = fma(p, r, 0.5);
    p = fma(p, r, 1.0);
    p = fma(p, r, 1.0);
    return ldexp(p, (int)n);
}

// Aggregation factors accurate to about half an fp32 ulp each, so that every product
// c_k R_k f_c A_m entering an orbital sum carries a single rounding: the Gaussians, the cutoff and
// the monomials are evaluated in fp64 and rounded once.  The Gaussians follow from the ratio of
// neighbouring centres, R_{k+1} / R_k = exp(delta_k d / s^2) exp(-delta_k (mu_k + mu_{k+1}) / (2 s^2))
// with delta_k = mu_{k+1} - mu_k; writing delta_k = delta + (delta_k - delta), the first factor is
// one exponential E = exp(delta d / s^2) times 1 + (delta_k - delta) d / s^2 (the next term is below
// 2e-10 where the chain is used), so an edge needs two fp64 exponentials.  Centres too uneven or
// widths too narrow for it (see the model set-up) take one exponential per channel (CHAIN false).  The cutoff is cos^2(pi d / (2 rc)) from the
// Taylor series of cos to the t^18 term (truncation below 1e-14 on [0, pi/2]).
// K0, KB: only the radial channels K0 .. K0 + KB - 1 (the chain starts from a direct
// exponential at mu_K0).  CT: the contraction variant, orbital n = K0 + j from
// sum_k C[n][k] R_k f_c over all K primitives, summed in fp64 before the one rounding.
template <int K, int L, typename S = float, int K0 = 0, int KB = K, bool CHAIN = true, bool CT = false>
struct BasisHP {
    static constexpr int M = n_mono(L);
    S P[KB];  // c_k R_k f_c, k = K0 + index
    S A[M];

    template <class CV>
    __device__ __forceinline__ void eval(double dx, double dy, double dz, const CV *__restrict__ cv,
                                         const ModelDev *__restrict__ md) {
        constexpr Mono<L> mono;
        // factors kept in fp32 (S = float) need series only to ~1e-10: cos to t^14 (truncation below
        // 7e-11 on [0, pi/2]) and exponentials to r^8; the fp64 orbital sums keep the long series
        constexpr bool F32 = std::is_same<S, float>::value;
        const double d = sqrt(fma(dx, dx, fma(dy, dy, dz * dz)));
        const double t = d * md->half_pi_over_rc, t2 = t * t;
        double cs;
        if constexpr (F32) {
            cs = -1.0 / 87178291200.0;                         // -1/14!
        } else {
            cs = -1.0 / 6402373705728000.0;                    // -1/18!
            cs = fma(cs, t2, 1.0 / 20922789888000.0);          // 1/16!
            cs = fma(cs, t2, -1.0 / 87178291200.0);            // -1/14!
        }
        cs = fma(cs, t2, 1.0 / 479001600.0);                   // 1/12!
        cs = fma(cs, t2, -1.0 / 3628800.0);                    // -1/10!
        cs = fma(cs, t2, 1.0 / 40320.0);                       // 1/8!
        cs = fma(cs, t2, -1.0 / 720.0);                        // -1/6!
        cs = fma(cs, t2, 1.0 / 24.0);                          // 1/4!
        cs = fma(cs, t2, -0.5);
        cs = fma(cs, t2, 1.0);
        const double fc = cs * cs;
        if constexpr (CT) {
            double Rf[K];
            if constexpr (CHAIN) {
                const double x0 = d - md->mu64[0];
                double r = exp_fp64<F32>(md->g_a0 * x0 * x0) * fc;
                const double E = exp_fp64<F32>(md->g_e * d);
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    Rf[k] = r;
                    if (k + 1 < K) r *= E * fma(md->g_ce[k], d, md->g_c[k]);
                }
            } else {
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    const double x = d - md->mu64[k];
                    Rf[k] = exp(md->g_a0 * x * x) * fc;
                }
            }
#pragma unroll
            for (int j = 0; j < KB; ++j) {
                const int q = K0 + j;
                double a = 0.0;
#pragma unroll
                for (int k = 0; k < K; ++k) a = fma(md->C64[q * K + k], Rf[k], a);
                P[j] = (S)((double)cv[q] * a);
            }
        } else if constexpr (CHAIN) {
            // the chain runs on R_k f_c: P_k = c_k (R_k f_c), next = this E (g_c + g_c g_eps d)
            const double x0 = d - md->mu64[K0];
            double Rf = exp_fp64<F32>(md->g_a0 * x0 * x0) * fc;
            const double E = exp_fp64<F32>(md->g_e * d);
#pragma unroll
            for (int j = 0; j < KB; ++j) {
                const int k = K0 + j;
                P[j] = (S)((double)cv[k] * Rf);
                if (j + 1 < KB) Rf *= E * fma(md->g_ce[k], d, md->g_c[k]);
            }
        } else {
            // centres too uneven or widths too narrow for the chain: one exponential per channel
#pragma unroll
            for (int j = 0; j < KB; ++j) {
                const int k = K0 + j;
                const double x = d - md->mu64[k];
                P[j] = (S)((double)cv[k] * exp(md->g_a0 * x * x) * fc);
            }
        }
        // monomials of r / rc: fp32 products of the once-rounded components (S = float), else fp64
        using U = std::conditional_t<F32, float, double>;
        const U ux = (U)(dx * md->inv_rc64), uy = (U)(dy * md->inv_rc64), uz = (U)(dz * md->inv_rc64);
        U px[L + 1], py[L + 1], pz[L + 1];
        px[0] = py[0] = pz[0] = (U)1;
#pragma unroll
        for (int q = 1; q <= L; ++q) {
            px[q] = px[q - 1] * ux;
            py[q] = py[q - 1] * uy;
            pz[q] = pz[q - 1] * uz;
        }
#pragma unroll
        for (int m = 0; m < M; ++m) A[m] = (S)(px[mono.lx[m]] * py[mono.ly[m]] * pz[mono.lz[m]]);
    }
};

// Density feature q of one atom from its orbital coefficients held in registers (Eq. 1 outer
// sum): rho[(a,b),l] = sum over the monomials m of degree l of w_m O[a,m] O[b,m], accumulated in
// fp64.  Q is a template argument, so every register index is resolved at compile time; Q past
// the last feature is 0.
template <int K, int L, int Q>
__device__ __forceinline__ double feature_q(const float (&O)[K][n_mono(L)]) {
    constexpr FeatIdx f = feat_idx(K, Q);
    if constexpr (f.l > L) {
        return 0.0;
    } else {
        constexpr Mono<L> mono;
        constexpr int m0 = f.l * (f.l + 1) * (f.l + 2) / 6, m1 = m0 + (f.l + 1) * (f.l + 2) / 2;
        double acc = 0.0;
#pragma unroll
        for (int m = m0; m < m1; ++m) acc = fma((double)mono.w[m] * O[f.a][m], (double)O[f.b][m], acc);
        return acc;
    }
}

template <int K, int L, int KT, class SC, int... J>
__device__ __forceinline__ void feature_tile(const float (&O)[K][n_mono(L)], SC s, float (&v)[16],
                                             std::integer_sequence<int, J...>) {
    ((v[J] = (float)(feature_q<K, L, 16 * KT + J>(O) * s)), ...);
}

// Lane groups: the sender-major gathers, and the row kernels on small systems, give one node 16
// lanes; lane q takes entries q, q+16, ... of the node's list, and the 16 partial sums are
// combined by a fixed butterfly, after which every lane of the group holds the same bits (each
// step adds two operands in either order), so the result is reproducible.
constexpr int kGatherLanes = 16;
constexpr int kRecWin = 512;   // nodes per staged record window of the row kernels

// A node record (position, then K messages when WANT_C) from src, an LDS window slot or the record
// array; the row kernels call it on two separate paths so that each compiles to loads of its own
// memory space (one pointer into either space would make generic loads, which are slower for both).
template <int K, bool WANT_C, class P>
__device__ __forceinline__ void read_record(const P *src, double &px, double &py, double &pz, float (&cr)[K]) {
    const double2 xy = reinterpret_cast<const double2 *>(src)[0];
    px = xy.x;
    py = xy.y;
    pz = reinterpret_cast<const double *>(src)[2];
    if constexpr (WANT_C) {
        const float *cv = reinterpret_cast<const float *>(src) + kRecC;
#pragma unroll
        for (int k = 0; k < K; ++k) cr[k] = cv[k];
    }
}

template <class T>
__device__ __forceinline__ T group_sum16(T x) {
#pragma unroll
    for (int o = kGatherLanes / 2; o > 0; o >>= 1) x += __shfl_xor(x, o, kGatherLanes);
    return x;
}

// Column C of a row's orbital sums / density features, written by the lane q = C % 16 of the
// row's group (lane-group rows; register indices stay compile-time constants).
template <int K, int L, int C>
__device__ __forceinline__ void store_o_col(const float (&O)[K][n_mono(L)], float *__restrict__ dst, int64_t np,
                                            int64_t i, int q) {
    constexpr int M = n_mono(L);
    if (q != C % 16) return;
    float v = 0.0f;
    if constexpr (C < K * M) v = O[C / M][C % M];
    dst[tiled(np, i, C)] = v;
}
template <int K, int L, int Q>
__device__ __forceinline__ void store_feature_col(const float (&O)[K][n_mono(L)], float s, float *__restrict__ dst,
                                                  int64_t np, int64_t i, int q) {
    if (q != Q % 16) return;
    dst[tiled(np, i, Q)] = (float)(feature_q<K, L, Q>(O) * s);
}
template <int K, int L, int... C>
__device__ __forceinline__ void store_o_cols(const float (&O)[K][n_mono(L)], float *dst, int64_t np, int64_t i, int q,
                                             std::integer_sequence<int, C...>) {
    (store_o_col<K, L, C>(O, dst, np, i, q), ...);
}
template <int K, int L, int... Q>
__device__ __forceinline__ void store_feature_cols(const float (&O)[K][n_mono(L)], float s, float *dst, int64_t np,
                                                   int64_t i, int q, std::integer_sequence<int, Q...>) {
    (store_feature_col<K, L, Q>(O, s, dst, np, i, q), ...);
}

// One 16-column tile of the block's 256 rows: thread t holds the 16 values of row i0 + t; the
// tile is staged through LDS (rows padded to 80 bytes) and written as one contiguous 16 KB run,
// 1 KB per store instruction.  All threads of the block call it.
__device__ __forceinline__ void store_tile(const float (&v)[16], float4 *__restrict__ lds, float *__restrict__ dst,
                                           int slot) {
    const int t = threadIdx.x;
    float4 *row = lds + 5 * slot;   // the row's place in the block (rows may be held out of order)
    row[0] = float4{v[0], v[1], v[2], v[3]};
    row[1] = float4{v[4], v[5], v[6], v[7]};
    row[2] = float4{v[8], v[9], v[10], v[11]};
    row[3] = float4{v[12], v[13], v[14], v[15]};
    __syncthreads();
    float4 *out = reinterpret_cast<float4 *>(dst);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int f = p * kBlock + t;
        out[f] = lds[5 * (f >> 2) + (f & 3)];
    }
    __syncthreads();
}

template <int K, int L, int KT>
__device__ __forceinline__ void store_o_tile(const float (&O)[K][n_mono(L)], float4 *lds, float *dst, int slot) {
    constexpr int M = n_mono(L);
    float v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int q = 16 * KT + j;
        v[j] = q < K * M ? O[q / M][q % M] : 0.0f;
    }
    store_tile(v, lds, dst, slot);
}

template <int K, int L, int... KT>
__device__ __forceinline__ void store_o_rows(const float (&O)[K][n_mono(L)], float4 *lds, float *base, int64_t np,
                                             int slot, std::integer_sequence<int, KT...>) {
    (store_o_tile<K, L, KT>(O, lds, base + (int64_t)KT * np * 16, slot), ...);
}

template <int K, int L, int KT, class SC>
__device__ __forceinline__ void store_feature_tile(const float (&O)[K][n_mono(L)], SC s, float4 *lds, float *dst,
                                                   int slot) {
    float v[16];
    feature_tile<K, L, KT>(O, s, v, std::make_integer_sequence<int, 16>{});
    store_tile(v, lds, dst, slot);
}

template <int K, int L, class SC, int... KT>
__device__ __forceinline__ void store_feature_rows(const float (&O)[K][n_mono(L)], SC s, float4 *lds, float *base,
                                                   int64_t np, int slot, std::integer_sequence<int, KT...>) {
    (store_feature_tile<K, L, KT>(O, s, lds, base + (int64_t)KT * np * 16, slot), ...);
}

// Chain rule through the features: dE/dO[c,m] = w_m sum_b (1 + [b == c]) dE/drho[(b,c), l_m] O[b,m],
// from the atom's column-tiled dE/drho and O rows; one template instance per feature Q, so the
// register indices of G are compile-time constants.
template <int K, int L, int Q>
__device__ __forceinline__ void go_term(const float *__restrict__ grho, const float *__restrict__ O, int64_t np,
                                        int64_t i, float (&G)[K][n_mono(L)]) {
    constexpr int M = n_mono(L);
    constexpr FeatIdx f = feat_idx(K, Q);
    constexpr Mono<L> mono;
    constexpr int m0 = f.l * (f.l + 1) * (f.l + 2) / 6, m1 = m0 + (f.l + 1) * (f.l + 2) / 2;
    const float g = grho[tiled(np, i, Q)];
#pragma unroll
    for (int m = m0; m < m1; ++m) {
        const float wg = mono.w[m] * g;
        G[f.a][m] += wg * O[tiled(np, i, f.b * M + m)];
        G[f.b][m] += wg * O[tiled(np, i, f.a * M + m)];
    }
}

template <int K, int L, int... Q>
__device__ __forceinline__ void go_terms(const float *__restrict__ grho, const float *__restrict__ O, int64_t np,
                                         int64_t i, float (&G)[K][n_mono(L)], std::integer_sequence<int, Q...>) {
    (go_term<K, L, Q>(grho, O, np, i, G), ...);
}

template <int K, int L>
__device__ __forceinline__ void assemble_go_row(const float *__restrict__ grho, const float *__restrict__ O,
                                                int64_t np, int64_t i, float (&G)[K][n_mono(L)]) {
#pragma unroll
    for (int k = 0; k < K; ++k)
#pragma unroll
        for (int m = 0; m < n_mono(L); ++m) G[k][m] = 0.0f;
    go_terms<K, L>(grho, O, np, i, G, std::make_integer_sequence<int, n_feat(K, L)>{});
}

// The same for the channels H K/2 .. (H+1) K/2 - 1 only (the channel-split reverse pass): the
// terms that touch those channels, in the same order, so the entries equal the full assembly's.
template <int K, int L, int H, int Q>
__device__ __forceinline__ void go_term_half(const float *__restrict__ grho, const float *__restrict__ O, int64_t np,
                                             int64_t i, float (&G)[K / 2][n_mono(L)]) {
    constexpr int M = n_mono(L), KH = K / 2;
    constexpr FeatIdx f = feat_idx(K, Q);
    constexpr bool in_a = f.a / KH == H, in_b = f.b / KH == H;
    if constexpr (in_a || in_b) {
        constexpr Mono<L> mono;
        constexpr int m0 = f.l * (f.l + 1) * (f.l + 2) / 6, m1 = m0 + (f.l + 1) * (f.l + 2) / 2;
        const float g = grho[tiled(np, i, Q)];
#pragma unroll
        for (int m = m0; m < m1; ++m) {
            const float wg = mono.w[m] * g;
            if constexpr (in_a) G[f.a - KH * H][m] += wg * O[tiled(np, i, f.b * M + m)];
            if constexpr (in_b) G[f.b - KH * H][m] += wg * O[tiled(np, i, f.a * M + m)];
        }
    }
}

template <int K, int L, int H, int... Q>
__device__ __forceinline__ void assemble_go_half(const float *__restrict__ grho, const float *__restrict__ O,
                                                 int64_t np, int64_t i, float (&G)[K / 2][n_mono(L)],
                                                 std::integer_sequence<int, Q...>) {
#pragma unroll
    for (int k = 0; k < K / 2; ++k)
#pragma unroll
        for (int m = 0; m < n_mono(L); ++m) G[k][m] = 0.0f;
    (go_term_half<K, L, H, Q>(grho, O, np, i, G), ...);
}

// Ordinary or nontemporal (streamed past the caches) accesses.  Nontemporal accesses pay where the
// per-edge streams are far larger than the caches and their rows are written in order; on small
// systems (which fit in the caches) and with bucketed rows (scattered partial lines) they cost, so
// the library picks them per build (Context::nt).
template <bool NT, class T>
__device__ __forceinline__ T ld_s(const T *p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}
template <bool NT, class T>
__device__ __forceinline__ void st_s(T v, T *p) {
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// Entries a0 .. a0 + kIdxStage - 1 of this thread's row of a slab-layout index list (one row per
// thread, na >= 1 entries: the active senders, or the Verlet entries for the compaction), staged in
// the thread's own LDS column: the batch's loads are in flight together, so the row loop's chain
// (index, then the sender's record or position) waits on memory once per edge instead of twice.
// Entries past na repeat the row's last one and are never read.
constexpr int kIdxStage = 16;
template <bool NT>
__device__ __forceinline__ void stage_indices(int32_t (*stage)[kBlock], const int32_t *__restrict__ act_n,
                                              int64_t b0, int a0, int na) {
    int32_t t[kIdxStage];
#pragma unroll
    for (int u = 0; u < kIdxStage; ++u) t[u] = ld_s<NT>(&act_n[b0 + kSlab * min(a0 + u, na - 1)]);
#pragma unroll
    for (int u = 0; u < kIdxStage; ++u) stage[u][threadIdx.x] = t[u];
}

// Per-step active list: the Verlet entries of each row with d^2 < rc^2 (fp64, the same
// expression as the build), compacted in row order into the row's leading slots (sender node of
// active entry a at slot base + 64 a), plus one activity bit per Verlet entry (word j/32, bit j%32
// of the row's mask).  Per-edge outputs live in active slots, so the row kernels write them
// coalesced; the transposed active map (k_transpose_active, once per evaluation) finds the active
// slot of an entry by counting the set bits before it, with the active counts of the row's first
// words in one extra word per row (the masks are 32x smaller than a per-entry slot map and stay in
// cache).  The test
// first uses the fp32 positions (one 16-byte load per entry): d^2 from them is within `band` of
// the fp64 value (a bound from the coordinate range, see compact_active), so only entries inside
// rc^2 -/+ band, a vanishing fraction, repeat it in fp64.
// Row taken by this thread of a 256-row block starting at i0: with row bucketing (row_perm set),
// the block's rows in descending active count, else in order; positions past the last row keep
// their own index, which the caller skips.
__device__ __forceinline__ int64_t block_row(int64_t i0, int64_t n, const int32_t *__restrict__ row_perm) {
    const int64_t i = i0 + threadIdx.x;
    return (row_perm && i < n) ? (int64_t)row_perm[i] : i;
}

// Compaction of row i (see k_compact below); returns its active count.  win: the fp32 positions of
// nodes wlo .. wlo + nwin - 1 staged in LDS (nwin = 0: none).
template <bool NT>
__device__ __forceinline__ int compact_row(int64_t i, int64_t n, const double *__restrict__ pos,
                                           const float4 *__restrict__ pos32, const int64_t *__restrict__ slab_off,
                                           const int32_t *__restrict__ len, const int32_t *__restrict__ nbr,
                                           double rc2, float lo, float hi, int mw, uint32_t *__restrict__ amask,
                                           int32_t *__restrict__ act_n, int32_t (*stage)[kBlock],
                                           const float4 *win, int64_t wlo, int64_t nwin) {
    const float4 pi = pos32[i];
    const int64_t b = sell_base(slab_off, i);
    const int nl = len[i];
    int o = 0;
    uint32_t bits = 0, pre = 0;
    // eight entries per step: their index and position loads are all in flight together (four:
    // 16 % slower; sixteen: 2.2x slower)
    constexpr int U = 8;
    static_assert(kIdxStage % U == 0, "whole steps per staged batch");
    for (int j0 = 0; j0 < nl; j0 += U) {
        // the Verlet indices arrive through the thread's LDS column, kIdxStage at a time
        if (j0 % kIdxStage == 0) stage_indices<NT>(stage, nbr, b, j0, nl);
        int32_t v[U];
        float4 pv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = j0 + u < nl ? stage[j0 % kIdxStage + u][threadIdx.x] : (int32_t)i;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            // one generic load per entry (LDS window or global): here the eight loads of a step
            // stay in flight together, which separate paths would break up (0.45 vs 0.51 ms)
            const int64_t wv = v[u] - wlo;
            pv[u] = (wv >= 0 && wv < nwin) ? win[wv] : pos32[v[u]];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = j0 + u;
            if (j >= nl) break;
            const float dx = pv[u].x - pi.x, dy = pv[u].y - pi.y, dz = pv[u].z - pi.z;
            const float d2f = dx * dx + dy * dy + dz * dz;
            bool act = d2f < lo;
            if (!act && d2f < hi) {
                const double xi = pos[3 * i], yi = pos[3 * i + 1], zi = pos[3 * i + 2];
                const int64_t w = v[u];
                act = d2_exact(__dsub_rn(pos[3 * w], xi), __dsub_rn(pos[3 * w + 1], yi),
                               __dsub_rn(pos[3 * w + 2], zi)) < rc2;
            }
            if (act) {
                act_n[b + kSlab * o] = v[u];
                ++o;
                bits |= 1u << (j & 31);
            }
            if ((j & 31) == 31 || j == nl - 1) {
                amask[(int64_t)(j >> 5) * n + i] = bits;
                bits = 0;
                if ((j >> 5) < 3) pre |= (uint32_t)o << (8 * (j >> 5));   // active entries before the next word
            }
        }
    }
    amask[(int64_t)mw * n + i] = pre;
    return o;
}

template <bool NT>
__global__ __launch_bounds__(256) void k_compact(int64_t n, int64_t NN, const double *__restrict__ pos,
                                                 const float4 *__restrict__ pos32,
                                                 const int64_t *__restrict__ slab_off,
                                                 const int32_t *__restrict__ len,
                                                 const int32_t *__restrict__ nbr, double rc2, float lo, float hi,
                                                 int mw, uint32_t *__restrict__ amask, int32_t *__restrict__ act_n,
                                                 int32_t *__restrict__ nact, int32_t *__restrict__ row_perm) {
    const int64_t i0 = xcd_block() * blockDim.x, i = i0 + threadIdx.x;
    __shared__ int32_t stage[kIdxStage][kBlock];
    // the fp32 positions of a node window around the block's rows (see k_aggregate)
    constexpr int WIN = 2 * kRecWin;
    __shared__ float4 win[WIN];
    int64_t wlo = i0 + kBlock / 2 - WIN / 2;
    wlo = wlo < 0 ? 0 : wlo;
    const int64_t nwin = NN - wlo < WIN ? (NN - wlo > 0 ? NN - wlo : 0) : WIN;
    for (int64_t p = threadIdx.x; p < nwin; p += kBlock) win[p] = pos32[wlo + p];
    __syncthreads();
    const int na = i < n ? compact_row<NT>(i, n, pos, pos32, slab_off, len, nbr, rc2, lo, hi, mw, amask, act_n, stage,
                                           win, wlo, nwin)
                         : -1;
    if (i < n) nact[i] = na;
    if (row_perm) {
        // the block's rows by descending active count (ties by row), so the waves of the row
        // kernels take rows of similar length; rank = rows that come before this one
        __shared__ int32_t cnt[kBlock];
        cnt[threadIdx.x] = na;
        __syncthreads();
        if (i < n) {
            int r = 0;
            for (int j = 0; j < kBlock; ++j) {
                const int x = cnt[j];
                r += (x > na) || (x == na && j < (int)threadIdx.x);
            }
            row_perm[i0 + r] = (int32_t)i;
        }
    }
}

// The same compaction with one 16-lane group per row (small systems): each step tests 16 entries,
// one per lane, and the group's activity bits (a ballot) give every active entry its rank, so the
// active list keeps the row's entry order as above.
__global__ __launch_bounds__(256) void k_compact_groups(int64_t n, const double *__restrict__ pos,
                                                        const float4 *__restrict__ pos32,
                                                        const int64_t *__restrict__ slab_off,
                                                        const int32_t *__restrict__ len,
                                                        const int32_t *__restrict__ nbr, double rc2, float lo,
                                                        float hi, int mw, uint32_t *__restrict__ amask,
                                                        int32_t *__restrict__ act_n, int32_t *__restrict__ nact) {
    const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kGatherLanes;
    const int q = (int)(threadIdx.x % kGatherLanes);
    const int shift = (int)(threadIdx.x % 64) & ~(kGatherLanes - 1);   // the group's lanes in the wave
    if (i >= n) return;   // a group shares its row, so its 16 lanes leave together
    const float4 pi = pos32[i];
    const int64_t b = sell_base(slab_off, i);
    const int nl = len[i];
    int o = 0;
    uint32_t lo_bits = 0, pre = 0;
    for (int j0 = 0; j0 < nl; j0 += kGatherLanes) {
        const int j = j0 + q;
        bool act = false;
        int32_t v = 0;
        if (j < nl) {
            v = nbr[b + kSlab * j];
            const float4 pv = pos32[v];
            const float dx = pv.x - pi.x, dy = pv.y - pi.y, dz = pv.z - pi.z;
            const float d2f = dx * dx + dy * dy + dz * dz;
            act = d2f < lo;
            if (!act && d2f < hi) {
                const double xi = pos[3 * i], yi = pos[3 * i + 1], zi = pos[3 * i + 2];
                act = d2_exact(__dsub_rn(pos[3 * (int64_t)v], xi), __dsub_rn(pos[3 * (int64_t)v + 1], yi),
                               __dsub_rn(pos[3 * (int64_t)v + 2], zi)) < rc2;
            }
        }
        const uint32_t bits = (uint32_t)(__ballot(act) >> shift) & 0xFFFFu;
        if (act) act_n[b + kSlab * (o + __popc(bits & ((1u << q) - 1u)))] = v;
        o += __popc(bits);
        // 32-entry activity words: entries j0 .. j0 + 15 are the low or the high half
        if ((j0 & 31) == 0) {
            lo_bits = bits;
            if (q == 0 && j0 + kGatherLanes >= nl) amask[(int64_t)(j0 >> 5) * n + i] = lo_bits;
        } else if (q == 0) {
            amask[(int64_t)(j0 >> 5) * n + i] = lo_bits | (bits << 16);
        }
        // a word ends with its second half or with the row
        if (((j0 & 31) == 16 || j0 + kGatherLanes >= nl) && (j0 >> 5) < 3) pre |= (uint32_t)o << (8 * (j0 >> 5));
    }
    if (q == 0) {
        nact[i] = o;
        amask[(int64_t)mw * n + i] = pre;
    }
}

// O^t_i[k,m] = sum over active neighbours v of c^t_v[k] R_k f_c A_m (Eq. 1 inner sum), and the
// atom's density features from it; both leave through LDS-staged, column-tiled stores.
// LANES = 1: one row per lane, 256-row blocks (row bucketing applies) with LDS-staged tile stores;
// LANES = 16 (small systems): one row per lane group, the group's partial sums combined by
// group_sum16 and the row's columns written by its lanes.
// C0U (layer 0 of a one-species model): every neighbour's message is C0 of the species, taken from
// the model constants, so only the position part of each node record is gathered.
// WIN > 0 (one row per lane): the records of nodes lo .. lo + WIN - 1, a window of node indices
// centred on the block's rows, are staged in LDS once per block, and the edges whose sender falls
// in it read the record there; the rest read it from global memory.  Rows are in cell order, so
// most senders of a block lie in such a window.
template <int K, int L, bool CHAIN, bool CT, bool NT, int LANES, bool C0U = false, int WIN = 0>
__global__ __launch_bounds__(256) void k_aggregate(int64_t n, int64_t NN, int64_t np, const double *__restrict__ pos,
                                                   const int64_t *__restrict__ slab_off,
                                                   const int32_t *__restrict__ nact,
                                                   const int32_t *__restrict__ act_n, const float *__restrict__ c,
                                                   const ModelDev *__restrict__ md, float inv_scale,
                                                   const int32_t *__restrict__ row_perm,
                                                   float *__restrict__ O, float *__restrict__ feat) {
    static_assert(LANES == 1 || LANES == kGatherLanes, "one lane or one lane group per row");
    static_assert(WIN == 0 || LANES == 1, "record window with one row per lane only");
    constexpr int M = n_mono(L), KMT = pad16(K * M) / 16, DT = pad16(n_feat(K, L)) / 16;
    constexpr int RQ = rec_stride(K) / 4;       // float4 per record
    constexpr int RQL = C0U ? 2 : RQ;           // staged per record: the position part, or all
    constexpr int SHQ = WIN * RQL > 5 * kBlock ? WIN * RQL : 5 * kBlock;
    __shared__ float4 shm[LANES == 1 ? SHQ : 1];   // the window, then the tile stores' staging
    int64_t i, i0 = 0, lo = 0, nwin = 0;
    int q = 0;
    if constexpr (LANES == 1) {
        i0 = xcd_block() * kBlock;
        if (i0 >= n) return;                       // whole block past the end (grid rounded to 8 XCDs)
        i = block_row(i0, n, row_perm);
        if constexpr (WIN > 0) {
            lo = i0 + kBlock / 2 - WIN / 2;
            lo = lo < 0 ? 0 : lo;
            nwin = NN - lo < WIN ? NN - lo : WIN;
            const float4 *src = reinterpret_cast<const float4 *>(c) + lo * RQ;
            for (int64_t p = threadIdx.x; p < nwin * RQL; p += kBlock)
                shm[p] = RQL == RQ ? src[p] : src[(p / RQL) * RQ + p % RQL];
            __syncthreads();
        }
    } else {
        i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / LANES;
        q = (int)(threadIdx.x % LANES);
    }
    float acc[K][M];
#pragma unroll
    for (int k = 0; k < K; ++k)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[k][m] = 0.0f;
    // one row per thread: indices staged kIdxStage at a time; lane groups: one span, direct loads
    constexpr int SPAN = LANES == 1 ? kIdxStage : (1 << 24);
    __shared__ int32_t stage[LANES == 1 ? kIdxStage : 1][kBlock];
    float c0u[K];
    if constexpr (C0U) {
#pragma unroll
        for (int k = 0; k < K; ++k) c0u[k] = md->c0[k];
    }
    if (i < n) {
        const double xi = pos[3 * i], yi = pos[3 * i + 1], zi = pos[3 * i + 2];
        const int64_t b0 = sell_base(slab_off, i);
        const int na = nact[i];
        for (int a0 = q; a0 < na; a0 += SPAN) {
            if constexpr (LANES == 1) stage_indices<NT>(stage, act_n, b0, a0, na);
            const int a1 = min(a0 + SPAN, na);
            for (int a = a0; a < a1; a += LANES) {
                const int64_t v = LANES == 1 ? stage[a - a0][threadIdx.x] : ld_s<NT>(&act_n[b0 + kSlab * a]);
                BasisHP<K, L, float, 0, K, CHAIN, CT> b;
                const int64_t wv = v - lo;
                double px, py, pz;
                float cr[K];
                if (WIN > 0 && wv >= 0 && wv < nwin)
                    read_record<K, !C0U>(shm + wv * RQL, px, py, pz, cr);   // staged record
                else
                    read_record<K, !C0U>(c + v * rec_stride(K), px, py, pz, cr);   // the record array
                if constexpr (C0U) {
#pragma unroll
                    for (int k = 0; k < K; ++k) cr[k] = c0u[k];
                }
                __builtin_amdgcn_sched_barrier(0);   // the whole record is requested before the basis starts
                b.eval(px - xi, py - yi, pz - zi, cr, md);
#pragma unroll
                for (int k = 0; k < K; ++k)
#pragma unroll
                    for (int m = 0; m < M; ++m) acc[k][m] = fmaf(b.P[k], b.A[m], acc[k][m]);
            }
        }
    }
    if constexpr (LANES == 1) {
        if constexpr (WIN > 0) __syncthreads();   // every thread is done with the window
        // rows n..np-1 of the last block are padding: written, never read
        store_o_rows<K, L>(acc, shm, O + i0 * 16, np, (int)(i - i0), std::make_integer_sequence<int, KMT>{});
        store_feature_rows<K, L>(acc, inv_scale, shm, feat + i0 * 16, np, (int)(i - i0),
                                 std::make_integer_sequence<int, DT>{});
    } else {
#pragma unroll
        for (int k = 0; k < K; ++k)
#pragma unroll
            for (int m = 0; m < M; ++m) acc[k][m] = group_sum16(acc[k][m]);
        if (i < n) {
            store_o_cols<K, L>(acc, O, np, i, q, std::make_integer_sequence<int, 16 * KMT>{});
            store_feature_cols<K, L>(acc, inv_scale, feat, np, i, q, std::make_integer_sequence<int, 16 * DT>{});
        }
    }
}

// Orbital sums in fp64 (the accurate mode): channels k in [P KB, (P+1) KB) of O^t_i, with the
// basis factors and their products kept in fp64 and one rounding when O is stored.  The K = 12,
// L = 3 orbital block is too large for fp64 registers in one pass, so it takes several passes over
// the edges (KB M a multiple of 16, so each pass owns whole 16-column tiles of the O rows).
// C0 (layer 0): the neighbour's coefficients are the fp64 parameters C0[species] (node types),
// not the fp32 copies in the node records.
template <int K, int L, int KB, int P, bool CHAIN, bool CT, bool C0>
__global__ __launch_bounds__(256) void k_aggregate64(int64_t n, int64_t np, const double *__restrict__ pos,
                                                     const int64_t *__restrict__ slab_off,
                                                     const int32_t *__restrict__ nact,
                                                     const int32_t *__restrict__ act_n, const float *__restrict__ c,
                                                     const ModelDev *__restrict__ md,
                                                     const int32_t *__restrict__ types,
                                                     const int32_t *__restrict__ row_perm, float *__restrict__ O) {
    constexpr int M = n_mono(L), Q0 = P * KB * M;
    constexpr int T0 = Q0 / 16, T1 = (KB == K ? pad16(K * M) : Q0 + KB * M) / 16;
    static_assert(KB == K || (KB * M) % 16 == 0, "a pass must own whole 16-column tiles");
    __shared__ float4 lds[5 * kBlock];
    const int64_t i0 = xcd_block() * kBlock;
    if (i0 >= n) return;
    const int64_t i = block_row(i0, n, row_perm);
    double acc[KB][M];
#pragma unroll
    for (int k = 0; k < KB; ++k)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[k][m] = 0.0;
    __shared__ int32_t stage[kIdxStage][kBlock];
    if (i < n) {
        const double xi = pos[3 * i], yi = pos[3 * i + 1], zi = pos[3 * i + 2];
        const int64_t b0 = sell_base(slab_off, i);
        const int na = nact[i];
        for (int a0 = 0; a0 < na; a0 += kIdxStage) {
            stage_indices<false>(stage, act_n, b0, a0, na);
            const int a1 = min(a0 + kIdxStage, na);
            for (int a = a0; a < a1; ++a) {
                const int64_t v = stage[a - a0][threadIdx.x];
                BasisHP<K, L, double, P * KB, KB, CHAIN, CT> b;   // this pass's radial channels only
                const float *rv = c + v * rec_stride(K);   // node record: position, then messages
                const double *pv = reinterpret_cast<const double *>(rv);
                if constexpr (C0) b.eval(pv[0] - xi, pv[1] - yi, pv[2] - zi, md->c0_64 + types[v] * K, md);
                else b.eval(pv[0] - xi, pv[1] - yi, pv[2] - zi, rv + kRecC, md);
#pragma unroll
                for (int k = 0; k < KB; ++k)
#pragma unroll
                    for (int m = 0; m < M; ++m) acc[k][m] = fma(b.P[k], b.A[m], acc[k][m]);
            }
        }
    }
#pragma unroll
    for (int kt = T0; kt < T1; ++kt) {
        float v[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int q = 16 * kt + j - Q0;
            v[j] = (q < KB * M && P * KB + q / M < K) ? (float)acc[q / M][q % M] : 0.0f;
        }
        store_tile(v, lds, O + (int64_t)kt * np * 16 + i0 * 16, (int)(i - i0));
    }
}

// Density features from stored (column-tiled) O rows, fp64 sums; used after the fp64 passes.
template <int K, int L>
__global__ __launch_bounds__(256) void k_features(int64_t n, int64_t np, const float *__restrict__ O,
                                                  double inv_scale, float *__restrict__ feat) {
    constexpr int M = n_mono(L), DT = pad16(n_feat(K, L)) / 16;
    __shared__ float4 lds[5 * kBlock];
    const int64_t i0 = (int64_t)blockIdx.x * kBlock;
    if (i0 >= n) return;
    const int64_t i = i0 + threadIdx.x;   // rows n..np-1 read and write padding
    float o[K][M];
#pragma unroll
    for (int k = 0; k < K; ++k)
#pragma unroll
        for (int m = 0; m < M; ++m) o[k][m] = O[tiled(np, i, k * M + m)];
    store_feature_rows<K, L>(o, inv_scale, lds, feat + i0 * 16, np, (int)threadIdx.x,
                             std::make_integer_sequence<int, DT>{});
}

// Reverse pass of layer t over one receiver row per thread (Eq. 4 as a VJP), with
// G = dE/dO^t_i formed from dE/drho^t_i and held in registers for the whole row.  For every active edge e = (i <- v):
//   u_k = sum_m G[k,m] A_m,       w_e[k] = u_k R_k f_c        (dE/dc^t_v contribution, t >= 1)
//   s = sum_k c_v[k] u_k (R'_k f_c + R_k f'_c),  Q_m = sum_k c_v[k] R_k f_c G[k,m]
//   dE/dr_e += s r/d + sum_m Q_m dA_m/dr              (accumulated over layers)
// The receiver-side force sum is accumulated in fp64 per row.  The per-edge outputs (w_e and
// dE/dr_e, 3.5 + 1.3 GB per launch on the 2M-atom subdomain) are written with nontemporal stores
// (NT): they are read back only by later kernels, and keeping them out of the caches leaves room for
// the node records this pass gathers (4.7 % faster than ordinary stores, measured there); the
// streamed active indices and the dE/dr_e read back for accumulation are loaded the same way
// (another 1.2 %).
// The VJP of one active edge e (see k_backward_layer): writes w_e (WANT_W) and returns dE/dr_e.
template <int K, int L, bool WANT_W, bool NT, class B>
__device__ __forceinline__ void edge_vjp(const B &b, const float *cv, const float (&G)[K][n_mono(L)], float ir,
                                         float *__restrict__ we, float (&g)[3]) {
    constexpr int M = n_mono(L);
    constexpr Mono<L> mono;
    float s = 0.0f, Q[M];
#pragma unroll
    for (int m = 0; m < M; ++m) Q[m] = 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
        float u = 0.0f;
#pragma unroll
        for (int m = 0; m < M; ++m) u += G[k][m] * b.A[m];
        if (WANT_W) st_s<NT>(u * b.Rf[k], &we[k]);
        s = fmaf(cv[k] * u, b.Rd[k], s);
        const float P = cv[k] * b.Rf[k];
#pragma unroll
        for (int m = 0; m < M; ++m) Q[m] += P * G[k][m];
    }
    // angular part: dA_m/dx = lx x^(lx-1) y^ly z^lz / rc^lx..., i.e. lx times the monomial
    // with one power of x fewer, over rc (likewise y, z)
    float ga[3] = {0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int m = 0; m < M; ++m) {
        if (mono.lx[m]) ga[0] = fmaf((float)mono.lx[m] * Q[m], b.A[mono.mx[m]], ga[0]);
        if (mono.ly[m]) ga[1] = fmaf((float)mono.ly[m] * Q[m], b.A[mono.my[m]], ga[1]);
        if (mono.lz[m]) ga[2] = fmaf((float)mono.lz[m] * Q[m], b.A[mono.mz[m]], ga[2]);
    }
    // plus the radial part along r / d
    const float sd = s * b.inv_d;
    g[0] = fmaf(sd, b.rx, ga[0] * ir);
    g[1] = fmaf(sd, b.ry, ga[1] * ir);
    g[2] = fmaf(sd, b.rz, ga[2] * ir);
}

// C0U: layer 0 of a one-species model (see k_aggregate): the messages come from the model constants,
// folded into the row's dE/dO (no per-edge message products).
// WIN > 0: a window of node records staged in LDS per block, as in k_aggregate.
template <int K, int L, bool FIRST, bool WANT_W, bool CT, bool NT, int LANES, bool C0U = false, int WIN = 0>
__global__ __launch_bounds__(256) void k_backward_layer(int64_t n, int64_t NN, int64_t np, const double *__restrict__ pos,
                                                        const int64_t *__restrict__ slab_off,
                                                        const int32_t *__restrict__ nact,
                                                        const int32_t *__restrict__ act_n, const float *__restrict__ c,
                                                        const float *__restrict__ Grho, const float *__restrict__ Ot,
                                                        const ModelDev *__restrict__ md,
                                                        const int32_t *__restrict__ row_perm,
                                                        float *__restrict__ w, float *__restrict__ gedge,
                                                        double *__restrict__ Frecv) {
    static_assert(LANES == 1 || LANES == kGatherLanes, "one lane or one lane group per row");
    static_assert(WIN == 0 || LANES == 1, "record window with one row per lane only");
    constexpr int M = n_mono(L);
    constexpr int RQ = rec_stride(K) / 4, RQL = C0U ? 2 : RQ;
    __shared__ float4 shm[WIN > 0 ? WIN * RQL : 1];
    int64_t i, lo = 0, nwin = 0;
    int q = 0;
    if constexpr (LANES == 1) {
        const int64_t i0 = xcd_block() * blockDim.x;
        if (i0 >= n) return;   // whole block past the end
        if constexpr (WIN > 0) {
            lo = i0 + kBlock / 2 - WIN / 2;
            lo = lo < 0 ? 0 : lo;
            nwin = NN - lo < WIN ? NN - lo : WIN;
            const float4 *src = reinterpret_cast<const float4 *>(c) + lo * RQ;
            for (int64_t p = threadIdx.x; p < nwin * RQL; p += kBlock)
                shm[p] = RQL == RQ ? src[p] : src[(p / RQL) * RQ + p % RQL];
            __syncthreads();
        }
        i = block_row(i0, n, row_perm);
        if (i >= n) return;
    } else {   // lane group per row (small systems); the group's force partials meet below
        i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / LANES;
        q = (int)(threadIdx.x % LANES);
    }
    const bool row = i < n;
    const int64_t ir_ = row ? i : 0;   // idle groups past the end read row 0 and write nothing
    float mu[K];
#pragma unroll
    for (int k = 0; k < K; ++k) mu[k] = md->mu[k];
    const float ir = md->inv_rc;
    const double xi = pos[3 * ir_], yi = pos[3 * ir_ + 1], zi = pos[3 * ir_ + 2];
    float G[K][M];
    assemble_go_row<K, L>(Grho, Ot, np, ir_, G);
    if constexpr (C0U) {
        // uniform messages: C0[k] folds into the row's dE/dO once, and every edge takes c_v = 1
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const float c0k = md->c0[k];
#pragma unroll
            for (int m = 0; m < M; ++m) G[k][m] *= c0k;
        }
    }
    double F[3] = {0.0, 0.0, 0.0};
    const int64_t b0 = sell_base(slab_off, ir_);
    const int na = row ? nact[ir_] : 0;
    for (int a = q; a < na; a += LANES) {
        const int64_t e = b0 + kSlab * a;   // active slot: per-edge outputs are stored here
        const int64_t v = ld_s<NT>(&act_n[e]);
        // dE/dr_e accumulates over layers (written by the first reverse layer, added to after); the
        // earlier layers' value is requested before the edge's arithmetic
        float gp[3] = {0.0f, 0.0f, 0.0f};
        if constexpr (!FIRST) {
#pragma unroll
            for (int d = 0; d < 3; ++d) gp[d] = ld_s<NT>(&gedge[3 * e + d]);
        }
        const int64_t wv = v - lo;
        double px, py, pz;
        float cv[K];
        if (WIN > 0 && wv >= 0 && wv < nwin)
            read_record<K, !C0U>(shm + wv * RQL, px, py, pz, cv);   // staged record
        else
            read_record<K, !C0U>(c + v * rec_stride(K), px, py, pz, cv);   // the record array
        if constexpr (C0U) {
#pragma unroll
            for (int k = 0; k < K; ++k) cv[k] = 1.0f;
        }
        Basis<K, L, CT> b;
        b.eval(__dsub_rn(px, xi), __dsub_rn(py, yi), __dsub_rn(pz, zi), md, mu);
        float g[3];
        edge_vjp<K, L, WANT_W, NT>(b, cv, G, ir, w + e * K, g);
#pragma unroll
        for (int d = 0; d < 3; ++d) st_s<NT>(FIRST ? g[d] : gp[d] + g[d], &gedge[3 * e + d]);
        F[0] += (double)g[0];
        F[1] += (double)g[1];
        F[2] += (double)g[2];
    }
    if constexpr (LANES > 1) {
#pragma unroll
        for (int c = 0; c < 3; ++c) F[c] = group_sum16(F[c]);
        if (!row || q != 0) return;
    }
    if (FIRST) {
        Frecv[3 * i] = F[0]; Frecv[3 * i + 1] = F[1]; Frecv[3 * i + 2] = F[2];
    } else {
        Frecv[3 * i] += F[0]; Frecv[3 * i + 1] += F[1]; Frecv[3 * i + 2] += F[2];
    }
}

// The reverse pass with each row's radial channels split over two adjacent lanes (the 12-channel
// models: the full dE/dO block, 12 x 20 values, with the basis and the running sums exceeds the
// registers of one lane, which then runs one wave per SIMD and spills).  Lane h holds channels
// h K/2 .. (h+1) K/2 - 1 of dE/dO, evaluates the radial factors of those channels, writes their
// w_e, and the two halves' dE/dr_e terms meet by one exchange (the sum of two operands, so both
// lanes hold the same bits).  Same outputs and layout as k_backward_layer.
template <int K, int L, bool FIRST, bool WANT_W, bool NT>
__global__ __launch_bounds__(256, 2) void k_backward_split(int64_t n, int64_t np, const double *__restrict__ pos,
                                                        const int64_t *__restrict__ slab_off,
                                                        const int32_t *__restrict__ nact,
                                                        const int32_t *__restrict__ act_n, const float *__restrict__ c,
                                                        const float *__restrict__ Grho, const float *__restrict__ Ot,
                                                        const ModelDev *__restrict__ md,
                                                        const int32_t *__restrict__ row_perm,
                                                        float *__restrict__ w, float *__restrict__ gedge,
                                                        double *__restrict__ Frecv) {
    static_assert(K % 2 == 0, "two channel halves");
    constexpr int M = n_mono(L), KH = K / 2;
    constexpr Mono<L> mono;
    const int64_t p = xcd_block() * (kBlock / 2) + threadIdx.x / 2;   // row position
    const int h = (int)(threadIdx.x & 1);                               // channel half
    if (p >= n) return;   // both lanes of a row leave together
    const int64_t i = row_perm ? (int64_t)row_perm[p] : p;
    float mu[KH];
#pragma unroll
    for (int k = 0; k < KH; ++k) mu[k] = md->mu[KH * h + k];
    const float ir = md->inv_rc;
    const double xi = pos[3 * i], yi = pos[3 * i + 1], zi = pos[3 * i + 2];
    float G[KH][M];
    if (h == 0) assemble_go_half<K, L, 0>(Grho, Ot, np, i, G, std::make_integer_sequence<int, n_feat(K, L)>{});
    else assemble_go_half<K, L, 1>(Grho, Ot, np, i, G, std::make_integer_sequence<int, n_feat(K, L)>{});
    double F[3] = {0.0, 0.0, 0.0};
    const int64_t b0 = sell_base(slab_off, i);
    const int na = nact[i];
    for (int a = 0; a < na; ++a) {
        const int64_t e = b0 + kSlab * a;
        const int64_t v = ld_s<NT>(&act_n[e]);
        // the earlier layers' dE/dr_e (lane h = 0 accumulates), requested before the arithmetic
        float gp[3] = {0.0f, 0.0f, 0.0f};
        if (!FIRST && h == 0) {
#pragma unroll
            for (int d = 0; d < 3; ++d) gp[d] = ld_s<NT>(&gedge[3 * e + d]);
        }
        const float *rv = c + v * rec_stride(K);
        const double *pv = reinterpret_cast<const double *>(rv);
        BasisHalf<K, L> b;
        b.eval(__dsub_rn(pv[0], xi), __dsub_rn(pv[1], yi), __dsub_rn(pv[2], zi), md, mu);
        const float *cv = rv + kRecC + KH * h;
        float s = 0.0f, Q[M];
#pragma unroll
        for (int m = 0; m < M; ++m) Q[m] = 0.0f;
#pragma unroll
        for (int k = 0; k < KH; ++k) {
            float u = 0.0f;
#pragma unroll
            for (int m = 0; m < M; ++m) u += G[k][m] * b.A[m];
            if (WANT_W) st_s<NT>(u * b.Rf[k], &w[e * K + KH * h + k]);
            s = fmaf(cv[k] * u, b.Rd[k], s);
            const float P = cv[k] * b.Rf[k];
#pragma unroll
            for (int m = 0; m < M; ++m) Q[m] += P * G[k][m];
        }
        float ga[3] = {0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int m = 0; m < M; ++m) {
            if (mono.lx[m]) ga[0] = fmaf((float)mono.lx[m] * Q[m], b.A[mono.mx[m]], ga[0]);
            if (mono.ly[m]) ga[1] = fmaf((float)mono.ly[m] * Q[m], b.A[mono.my[m]], ga[1]);
            if (mono.lz[m]) ga[2] = fmaf((float)mono.lz[m] * Q[m], b.A[mono.mz[m]], ga[2]);
        }
        const float sd = s * b.inv_d;
        float g[3] = {fmaf(sd, b.rx, ga[0] * ir), fmaf(sd, b.ry, ga[1] * ir), fmaf(sd, b.rz, ga[2] * ir)};
#pragma unroll
        for (int q = 0; q < 3; ++q) g[q] += __shfl_xor(g[q], 1);   // the other channel half
        if (h == 0) {
#pragma unroll
            for (int d = 0; d < 3; ++d) st_s<NT>(FIRST ? g[d] : gp[d] + g[d], &gedge[3 * e + d]);
        }
        F[0] += (double)g[0];
        F[1] += (double)g[1];
        F[2] += (double)g[2];
    }
    if (h != 0) return;
    if (FIRST) {
        Frecv[3 * i] = F[0]; Frecv[3 * i + 1] = F[1]; Frecv[3 * i + 2] = F[2];
    } else {
        Frecv[3 * i] += F[0]; Frecv[3 * i + 1] += F[1]; Frecv[3 * i + 2] += F[2];
    }
}

// Sender-major gathers use kGatherLanes lanes per node (see group_sum16 above).

// dE/dc^t of every node v (local or ghost): the w_e of the active edges v sends (Eq. 4 first
// term, gathered without atomics).  t_act holds the active slot of each transposed entry for this
// step (k_transpose_active), so the gather reads it sequentially.
template <int K>
__global__ __launch_bounds__(256) void k_gather_w(int64_t NN, const int64_t *__restrict__ t_off,
                                                  const int32_t *__restrict__ t_act, const float *__restrict__ w,
                                                  float *__restrict__ Gc) {
    const int64_t v = (xcd_block() * blockDim.x + threadIdx.x) / kGatherLanes;
    const int q = threadIdx.x % kGatherLanes;
    const bool ok = v < NN;
    float acc[K];
#pragma unroll
    for (int k = 0; k < K; ++k) acc[k] = 0.0f;
    if (ok) {
        const int64_t s1 = t_off[v + 1];
        // two entries per lane per step, so both lookups are in flight together
        for (int64_t s = t_off[v] + q; s < s1; s += 2 * kGatherLanes) {
            const bool two = s + kGatherLanes < s1;
            const int32_t a0 = t_act[s];
            const int32_t a1 = two ? t_act[s + kGatherLanes] : -1;
            float w0[K], w1[K];
#pragma unroll
            for (int k = 0; k < K; ++k) w0[k] = w1[k] = 0.0f;
            if (a0 >= 0) {
                const float *p = w + (int64_t)a0 * K;
#pragma unroll
                for (int k = 0; k < K; ++k) w0[k] = p[k];
            }
            if (a1 >= 0) {
                const float *p = w + (int64_t)a1 * K;
#pragma unroll
                for (int k = 0; k < K; ++k) w1[k] = p[k];
            }
#pragma unroll
            for (int k = 0; k < K; ++k) acc[k] += w0[k] + w1[k];
        }
    }
#pragma unroll
    for (int k = 0; k < K; ++k) acc[k] = group_sum16(acc[k]);
    if (ok && q == 0)
#pragma unroll
        for (int k = 0; k < K; ++k) Gc[v * K + k] = acc[k];
}

// t_act: the active slot (or -1) of every transposed entry under this step's compaction.  Each
// entry holds its receiver row and column, packed as (row << jb) | column.  The active slot is the
// row base plus 64 times the active entries before the entry: the set bits below it in its
// activity word plus, for rows of at most four words, the count of the earlier words that the
// compaction stores in the row's extra mask word (longer rows add the earlier words' bits up).  Each thread takes kTPer
// entries a block apart and requests all their lookups (row base, activity and count words) before
// using any, so the build keeps few waves busy while it runs beside the forward layers.
constexpr int kTPer = 4;
__global__ __launch_bounds__(256) void k_transpose_active(int64_t E, int64_t n, int jb, int mw,
                                                          const uint32_t *__restrict__ t_ent,
                                                          const int64_t *__restrict__ slab_off,
                                                          const uint32_t *__restrict__ amask,
                                                          int32_t *__restrict__ t_act) {
    const int64_t s0 = (int64_t)blockIdx.x * (kBlock * kTPer) + threadIdx.x;
    uint32_t ent[kTPer];
#pragma unroll
    for (int p = 0; p < kTPer; ++p) {
        const int64_t s = s0 + (int64_t)p * kBlock;
        ent[p] = s < E ? t_ent[s] : 0u;   // past the end: row 0, column 0, not stored
    }
    int64_t r[kTPer], b[kTPer];
    int j[kTPer];
#pragma unroll
    for (int p = 0; p < kTPer; ++p) {
        r[p] = ent[p] >> jb;
        j[p] = (int)(ent[p] & ((1u << jb) - 1u));
        b[p] = sell_base(slab_off, r[p]);
    }
    uint32_t word[kTPer], pre[kTPer];
#pragma unroll
    for (int p = 0; p < kTPer; ++p) {
        word[p] = amask[(int64_t)(j[p] >> 5) * n + r[p]];
        pre[p] = mw <= 4 ? amask[(int64_t)mw * n + r[p]] : 0u;
    }
#pragma unroll
    for (int p = 0; p < kTPer; ++p) {
        const int64_t s = s0 + (int64_t)p * kBlock;
        if (s >= E) continue;
        const int bit = j[p] & 31;
        int32_t slot = -1;
        if ((word[p] >> bit) & 1u) {
            int a = __popc(word[p] & ((1u << bit) - 1u));
            if (j[p] >= 32) {
                if (mw <= 4) {
                    a += (int)((pre[p] >> (8 * ((j[p] >> 5) - 1))) & 0xFFu);
                } else {
                    for (int q = 0; q < (j[p] >> 5); ++q) a += __popc(amask[(int64_t)q * n + r[p]]);
                }
            }
            slot = (int32_t)(b[p] + (int64_t)kSlab * a);
        }
        t_act[s] = slot;
    }
}

// Ghost -> owner sum of dE/dc (the reverse ghost exchange), ghosts of an owner in order.
__global__ void k_fold_ghost_grad(int64_t n, int K, const int64_t *__restrict__ ghost_off,
                                  float *__restrict__ Gc) {
    const int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (o >= n || ghost_off[o] == ghost_off[o + 1]) return;   // most atoms have no ghost image
    for (int k = 0; k < K; ++k) {
        float s = Gc[o * K + k];
        for (int64_t g = ghost_off[o]; g < ghost_off[o + 1]; ++g) s += Gc[(n + g) * K + k];
        Gc[o * K + k] = s;
    }
}

// Owner -> ghost copy of the messages c^t (the forward ghost exchange).
__global__ void k_ghost_feat(int64_t G, int64_t n, int K, const int32_t *__restrict__ owner,
                             float *__restrict__ rec) {
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= G * K) return;
    const int64_t g = q / K;
    const int k = (int)(q - g * K);
    const int rs = rec_stride(K);
    rec[(n + g) * rs + kRecC + k] = rec[(int64_t)owner[g] * rs + kRecC + k];
}

// F_i = sum_{edges received by i} dE/dr_e - sum_{active edges sent by i or by its ghost images}
// dE/dr_e (r_e = r_sender - r_receiver), in fp64; 16 lanes per atom as in the gathers above.
__global__ __launch_bounds__(256) void k_force_gather(int64_t n, const int32_t *__restrict__ perm,
                                                      const int64_t *__restrict__ t_off,
                                                      const int32_t *__restrict__ t_act,
                                                      const int64_t *__restrict__ ghost_off,
                                                      const double *__restrict__ Frecv, const float *__restrict__ gedge,
                                                      double *__restrict__ F, double *__restrict__ Fcaller) {
    const int64_t i = (xcd_block() * blockDim.x + threadIdx.x) / kGatherLanes;
    const int q = threadIdx.x % kGatherLanes;
    const bool ok = i < n;
    double f[3] = {0.0, 0.0, 0.0};
    if (ok) {
        const int64_t g0 = ghost_off[i], g1 = ghost_off[i + 1];
        for (int64_t vv = -1; vv < g1 - g0; ++vv) {       // the atom itself, then its ghost images
            const int64_t v = vv < 0 ? i : n + g0 + vv;
            const int64_t s1 = t_off[v + 1];
            for (int64_t s = t_off[v] + q; s < s1; s += 2 * kGatherLanes) {
                const bool two = s + kGatherLanes < s1;
                const int32_t a0 = t_act[s], a1 = two ? t_act[s + kGatherLanes] : -1;
                float g0[3] = {0.f, 0.f, 0.f}, g1[3] = {0.f, 0.f, 0.f};
                if (a0 >= 0)
                    for (int c = 0; c < 3; ++c) g0[c] = gedge[3 * (int64_t)a0 + c];
                if (a1 >= 0)
                    for (int c = 0; c < 3; ++c) g1[c] = gedge[3 * (int64_t)a1 + c];
                for (int c = 0; c < 3; ++c) f[c] -= (double)g0[c] + (double)g1[c];
            }
        }
    }
#pragma unroll
    for (int a = 0; a < 3; ++a) f[a] = group_sum16(f[a]);
    if (ok && q == 0) {
        for (int a = 0; a < 3; ++a) {
            const double v = Frecv[3 * i + a] + f[a];
            F[3 * i + a] = v;
            if (Fcaller) Fcaller[3 * (int64_t)perm[i] + a] = v;
        }
    }
}

// dE/dO^t rows of every atom (for inspection; the reverse pass forms them in registers).
template <int K, int L>
__global__ __launch_bounds__(256) void k_assemble_go(int64_t n, int64_t np, const float *__restrict__ Grho,
                                                     const float *__restrict__ Ot, float *__restrict__ out) {
    constexpr int M = n_mono(L);
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    float G[K][M];
    assemble_go_row<K, L>(Grho, Ot, np, i, G);
#pragma unroll
    for (int k = 0; k < K; ++k)
#pragma unroll
        for (int m = 0; m < M; ++m) out[i * (K * M) + k * M + m] = G[k][m];
}

const int32_t *row_perm(const Context &cx) { return cx.bucket ? cx.row_perm.as<int32_t>() : nullptr; }

template <int K, int L, int KB, int P, bool CH, bool CT>
void launch_agg64(Context &cx, const float *ct, float *Ot, bool c0) {
    if (c0)
        k_aggregate64<K, L, KB, P, CH, CT, true><<<grid_xcd(cx.n), kBlock, 0, cx.stream>>>(
            cx.n, cx.np, cx.pos.as<double>(), cx.slab_off.as<int64_t>(), cx.nact.as<int32_t>(), cx.act_n.as<int32_t>(),
            ct, cx.model.as<ModelDev>(), cx.types.as<int32_t>(), row_perm(cx), Ot);
    else
        k_aggregate64<K, L, KB, P, CH, CT, false><<<grid_xcd(cx.n), kBlock, 0, cx.stream>>>(
            cx.n, cx.np, cx.pos.as<double>(), cx.slab_off.as<int64_t>(), cx.nact.as<int32_t>(), cx.act_n.as<int32_t>(),
            ct, cx.model.as<ModelDev>(), nullptr, row_perm(cx), Ot);
}

#define MPNN_DISPATCH_KL(K_, L_, CALL)                                                 \
    do {                                                                               \
        if ((K_) == 8 && (L_) == 2) { constexpr int KK = 8, LL = 2; CALL; }            \
        else if ((K_) == 12 && (L_) == 3) { constexpr int KK = 12, LL = 3; CALL; }     \
        else if ((K_) == 2 && (L_) == 1) { constexpr int KK = 2, LL = 1; CALL; }       \
        else if ((K_) == 4 && (L_) == 2) { constexpr int KK = 4, LL = 2; CALL; }       \
        else return Status::err(MPNN_E_INVALID_ARG, "unsupported (K, L)");              \
    } while (0)

}  // namespace

Status compact_active(Context &cx) {
    ProfScope ps_(cx, kProfCompact);
    if (cx.n == 0) return Status::ok();
    // |d^2(fp32 positions) - d^2(fp64)| bound: coordinates stay within [-c, c], c = largest box
    // edge + rc + 2 skin (ghost shell and drift), so each rounded coordinate is off by at most
    // eps = c 2^-24, a difference by 2 eps + 2^-24 |dx|, and d^2 <= rc^2 by
    // 4 sqrt(3) eps rc + 4 2^-23 rc^2 (+ second-order terms); the band is twice that.
    const double c = std::max(cx.box[0], std::max(cx.box[1], cx.box[2])) + cx.rc + 2.0 * cx.skin;
    const double eps = c * std::ldexp(1.0, -24);
    const double band = 2.0 * (4.0 * std::sqrt(3.0) * eps * cx.rc + 4.0 * std::ldexp(1.0, -23) * cx.rc * cx.rc) + 1e-9;
    const double rc2 = cx.rc * cx.rc;
    const float lo = (float)(rc2 - band), hi = (float)(rc2 + band);
    auto launch = [&](auto nt) {
        k_compact<decltype(nt)::value><<<grid_xcd(cx.n), kBlock, 0, cx.stream>>>(
            cx.n, cx.NN, cx.pos.as<double>(), cx.pos32.as<float4>(), cx.slab_off.as<int64_t>(), cx.row_len.as<int32_t>(),
            cx.nbr.as<int32_t>(), rc2, lo, hi, cx.mw, cx.amask.as<uint32_t>(), cx.act_n.as<int32_t>(),
            cx.nact.as<int32_t>(), cx.bucket ? cx.row_perm.as<int32_t>() : nullptr);
    };
    if (cx.lane_groups)
        k_compact_groups<<<grid_for(cx.n * kGatherLanes), kBlock, 0, cx.stream>>>(
            cx.n, cx.pos.as<double>(), cx.pos32.as<float4>(), cx.slab_off.as<int64_t>(), cx.row_len.as<int32_t>(),
            cx.nbr.as<int32_t>(), rc2, lo, hi, cx.mw, cx.amask.as<uint32_t>(), cx.act_n.as<int32_t>(),
            cx.nact.as<int32_t>());
    else if (cx.nt) launch(std::true_type{});
    else launch(std::false_type{});
    MPNN_HIP(hipGetLastError());
    return Status::ok();
}

Status aggregate(Context &cx, int t) {
    ProfScope ps_(cx, kProfAggregate);
    if (cx.n == 0) return Status::ok();
    const float *ct = cx.c.as<float>() + (int64_t)t * cx.NN * rec_stride(cx.K);
    float *Ot = cx.O.as<float>() + (int64_t)t * cx.np * pad16(cx.K * cx.M);
    float *Ft = cx.feat.as<float>() + (int64_t)t * cx.np * cx.DP;
    // layer 0 of a one-species model: the messages are the model's C0 (uniform)
    const bool c0u = t == 0 && cx.S == 1 && !cx.contracted;
    if (cx.precision != 1) {   // fp32 orbital sums (fp32 and bf16 networks)
#define MPNN_AGG32_NT(CH, CT, NT, U)                                                                            \
    MPNN_DISPATCH_KL(cx.K, cx.L, (k_aggregate<KK, LL, CH, CT, NT, 1, U, NT ? (U ? 2 * kRecWin : kRecWin) : 0><<<grid_xcd(cx.n), kBlock, 0, cx.stream>>>( \
                                      cx.n, cx.NN, cx.np, cx.pos.as<double>(), cx.slab_off.as<int64_t>(),          \
                                      cx.nact.as<int32_t>(), cx.act_n.as<int32_t>(), ct, cx.model.as<ModelDev>(), \
                                      cx.inv_scale_host[t], row_perm(cx), Ot, Ft)))
#define MPNN_AGG32_LG(CH, CT, U)                                                                                \
    MPNN_DISPATCH_KL(cx.K, cx.L, (k_aggregate<KK, LL, CH, CT, false, kGatherLanes, U><<<grid_for(cx.n * kGatherLanes), \
                                                                                   kBlock, 0, cx.stream>>>(      \
                                      cx.n, cx.NN, cx.np, cx.pos.as<double>(), cx.slab_off.as<int64_t>(),          \
                                      cx.nact.as<int32_t>(), cx.act_n.as<int32_t>(), ct, cx.model.as<ModelDev>(), \
                                      cx.inv_scale_host[t], nullptr, Ot, Ft)))
#define MPNN_AGG32(CH, CT)                                                                                      \
    do {                                                                                                        \
        if (!(CT) && c0u) {                                                                                     \
            if (cx.lane_groups) MPNN_AGG32_LG(CH, false, true);                                                 \
            else if (cx.nt) MPNN_AGG32_NT(CH, false, true, true);                                               \
            else MPNN_AGG32_NT(CH, false, false, true);                                                         \
        } else if (cx.lane_groups) MPNN_AGG32_LG(CH, CT, false);                                                \
        else if (cx.nt) MPNN_AGG32_NT(CH, CT, true, false);                                                     \
        else MPNN_AGG32_NT(CH, CT, false, false);                                                               \
    } while (0)
        if (cx.contracted) {
            if (cx.chain) MPNN_AGG32(true, true);
            else MPNN_AGG32(false, true);
        } else {
            if (cx.chain) MPNN_AGG32(true, false);
            else MPNN_AGG32(false, false);
        }
#undef MPNN_AGG32
#undef MPNN_AGG32_NT
#undef MPNN_AGG32_LG
        MPNN_HIP(hipGetLastError());
        return Status::ok();
    }
#define MPNN_AGG64(KK, LL, KB, P)                                                                               \
    if (cx.contracted) {                                                                                        \
        if (cx.chain) launch_agg64<KK, LL, KB, P, true, true>(cx, ct, Ot, t == 0);                                      \
        else launch_agg64<KK, LL, KB, P, false, true>(cx, ct, Ot, t == 0);                                              \
    } else {                                                                                                    \
        if (cx.chain) launch_agg64<KK, LL, KB, P, true, false>(cx, ct, Ot, t == 0);                                     \
        else launch_agg64<KK, LL, KB, P, false, false>(cx, ct, Ot, t == 0);                                             \
    }
    if (cx.K == 12 && cx.L == 3) {
        MPNN_AGG64(12, 3, 4, 0);
        MPNN_AGG64(12, 3, 4, 1);
        MPNN_AGG64(12, 3, 4, 2);
    } else if (cx.K == 8 && cx.L == 2) {
        MPNN_AGG64(8, 2, 8, 0);
    } else if (cx.K == 4 && cx.L == 2) {
        MPNN_AGG64(4, 2, 4, 0);
    } else if (cx.K == 2 && cx.L == 1) {
        MPNN_AGG64(2, 1, 2, 0);
    } else {
        return Status::err(MPNN_E_INVALID_ARG, "unsupported (K, L)");
    }
#undef MPNN_AGG64
    MPNN_HIP(hipGetLastError());
    MPNN_DISPATCH_KL(cx.K, cx.L, (k_features<KK, LL><<<(unsigned)(cx.np / kBlock), kBlock, 0, cx.stream>>>(
                                      cx.n, cx.np, Ot, cx.inv_scale64_host[t], Ft)));
    MPNN_HIP(hipGetLastError());
    return Status::ok();
}

Status refresh_ghost_features(Context &cx, int t) {
    ProfScope ps_(cx, kProfGhostFeat);
    if (cx.G == 0) return Status::ok();
    float *ct = cx.c.as<float>() + (int64_t)t * cx.NN * rec_stride(cx.K);
    k_ghost_feat<<<grid_for(cx.G * cx.K), kBlock, 0, cx.stream>>>(cx.G, cx.n, cx.K, cx.ghost_owner.as<int32_t>(), ct);
    MPNN_HIP(hipGetLastError());
    return Status::ok();
}

Status backward_layer(Context &cx, int t) {
    ProfScope ps_(cx, kProfBackwardLayer);
    if (cx.n == 0) return Status::ok();
    const float *ct = cx.c.as<float>() + (int64_t)t * cx.NN * rec_stride(cx.K);
    const float *Gt = cx.grho.as<float>() + (int64_t)t * cx.np * cx.DP;
    const float *Ot = cx.O.as<float>() + (int64_t)t * cx.np * pad16(cx.K * cx.M);
    const bool first = (t == cx.T - 1), want_w = (t >= 1);
    const bool c0u = t == 0 && cx.S == 1 && !cx.contracted;   // layer-0 messages uniform (see aggregate)
#define MPNN_BWD(FIRST_, W_)                                                                               \
    do {                                                                                                   \
        if (cx.contracted) MPNN_BWD_CT(FIRST_, W_, true);                                                  \
        else MPNN_BWD_CT(FIRST_, W_, false);                                                               \
    } while (0)
#define MPNN_BWD_CT(FIRST_, W_, CT_)                                                                       \
    do {                                                                                                   \
        if (!CT_ && cx.K == 12) {                                                                          \
            if (cx.nt) MPNN_BWD_SPLIT(FIRST_, W_, true);                                                   \
            else MPNN_BWD_SPLIT(FIRST_, W_, false);                                                        \
        } else if (!(CT_) && !(W_) && c0u) {                                                              \
            if (cx.lane_groups) MPNN_BWD_LG(FIRST_, false, false, true);                                   \
            else if (cx.nt) MPNN_BWD_NT(FIRST_, false, false, true, true);                                 \
            else MPNN_BWD_NT(FIRST_, false, false, false, true);                                           \
        } else if (cx.lane_groups) MPNN_BWD_LG(FIRST_, W_, CT_, false);                                    \
        else if (cx.nt) MPNN_BWD_NT(FIRST_, W_, CT_, true, false);                                         \
        else MPNN_BWD_NT(FIRST_, W_, CT_, false, false);                                                   \
    } while (0)
#define MPNN_BWD_SPLIT(FIRST_, W_, NT_)                                                                    \
    k_backward_split<12, 3, FIRST_, W_, NT_><<<grid_xcd(2 * cx.n), kBlock, 0, cx.stream>>>(                \
        cx.n, cx.np, cx.pos.as<double>(), cx.slab_off.as<int64_t>(), cx.nact.as<int32_t>(), cx.act_n.as<int32_t>(), \
        ct, Gt, Ot, cx.model.as<ModelDev>(), row_perm(cx), cx.w.as<float>(), cx.gedge.as<float>(),          \
        cx.Frecv.as<double>())
#define MPNN_BWD_LG(FIRST_, W_, CT_, U_)                                                                   \
    MPNN_DISPATCH_KL(cx.K, cx.L, (k_backward_layer<KK, LL, FIRST_, W_, CT_, false, kGatherLanes, U_>       \
                                  <<<grid_for(cx.n * kGatherLanes), kBlock, 0, cx.stream>>>(                 \
                                      cx.n, cx.NN, cx.np, cx.pos.as<double>(), cx.slab_off.as<int64_t>(), cx.nact.as<int32_t>(), \
                                      cx.act_n.as<int32_t>(), ct, Gt, Ot,                                          \
                                      cx.model.as<ModelDev>(), nullptr, cx.w.as<float>(), cx.gedge.as<float>(), \
                                      cx.Frecv.as<double>())))
#define MPNN_BWD_NT(FIRST_, W_, CT_, NT_, U_)                                                              \
    MPNN_DISPATCH_KL(cx.K, cx.L, (k_backward_layer<KK, LL, FIRST_, W_, CT_, NT_, 1, U_, NT_ ? (U_ ? 2 * kRecWin : 3 * kRecWin / 2) : 0><<<grid_xcd(cx.n), kBlock, 0, cx.stream>>>( \
                                      cx.n, cx.NN, cx.np, cx.pos.as<double>(), cx.slab_off.as<int64_t>(), cx.nact.as<int32_t>(), \
                                      cx.act_n.as<int32_t>(), ct, Gt, Ot,                                          \
                                      cx.model.as<ModelDev>(), row_perm(cx), cx.w.as<float>(), cx.gedge.as<float>(), \
                                      cx.Frecv.as<double>())))
    if (first && want_w) MPNN_BWD(true, true);
    else if (first) MPNN_BWD(true, false);
    else if (want_w) MPNN_BWD(false, true);
    else MPNN_BWD(false, false);
#undef MPNN_BWD
#undef MPNN_BWD_CT
#undef MPNN_BWD_NT
#undef MPNN_BWD_LG
#undef MPNN_BWD_SPLIT
    MPNN_HIP(hipGetLastError());
    return Status::ok();
}

Status assemble_go(Context &cx, int t, float *out) {
    if (cx.n == 0) return Status::ok();
    const float *Gt = cx.grho.as<float>() + (int64_t)t * cx.np * cx.DP;
    const float *Ot = cx.O.as<float>() + (int64_t)t * cx.np * pad16(cx.K * cx.M);
    MPNN_DISPATCH_KL(cx.K, cx.L, (k_assemble_go<KK, LL><<<grid_for(cx.n), kBlock, 0, cx.stream>>>(cx.n, cx.np, Gt, Ot,
                                                                                                 out)));
    MPNN_HIP(hipGetLastError());
    return Status::ok();
}

Status fork_transpose(Context &cx) {
    hipStream_t s = cx.stream;
    if (cx.side) {
        if (!cx.side_stream) return Status::err(MPNN_E_STATE, "side stream not created");
        MPNN_HIP(hipEventRecord(cx.side_ev[0], cx.stream));
        MPNN_HIP(hipStreamWaitEvent(cx.side_stream, cx.side_ev[0], 0));
        s = cx.side_stream;
    }
    if (cx.E > 0) {
        k_transpose_active<<<grid_for((cx.E + kTPer - 1) / kTPer), kBlock, 0, s>>>(
            cx.E, cx.n, cx.tjb, cx.mw, cx.t_eid.as<uint32_t>(), cx.slab_off.as<int64_t>(),
            cx.amask.as<uint32_t>(), cx.t_act.as<int32_t>());
        MPNN_HIP(hipGetLastError());
    }
    if (cx.side) MPNN_HIP(hipEventRecord(cx.side_ev[1], cx.side_stream));
    return Status::ok();
}

Status join_transpose(Context &cx) {
    if (cx.side) MPNN_HIP(hipStreamWaitEvent(cx.stream, cx.side_ev[1], 0));
    return Status::ok();
}

Status backward_messages(Context &cx, int t) {
    if (cx.n == 0) return Status::ok();
    float *Gct = cx.Gc.as<float>() + (int64_t)t * cx.NN * cx.K;   // dE/dc^t, kept per layer
    {
        ProfScope ps_(cx, kProfMessageGrad);
        const unsigned gg = grid_xcd(cx.NN * kGatherLanes);
#define MPNN_GW(KK)                                                                                 \
    k_gather_w<KK><<<gg, kBlock, 0, cx.stream>>>(cx.NN, cx.t_off.as<int64_t>(), cx.t_act.as<int32_t>(), \
                                                 cx.w.as<float>(), Gct)
        switch (cx.K) {
            case 2: MPNN_GW(2); break;
            case 4: MPNN_GW(4); break;
            case 8: MPNN_GW(8); break;
            case 12: MPNN_GW(12); break;
            default: return Status::err(MPNN_E_INVALID_ARG, "unsupported K");
        }
#undef MPNN_GW
        MPNN_HIP(hipGetLastError());
    }
    ProfScope ps_(cx, kProfGhostFold);
    k_fold_ghost_grad<<<grid_for(cx.n), kBlock, 0, cx.stream>>>(cx.n, cx.K, cx.ghost_off.as<int64_t>(),
                                                                 Gct);
    MPNN_HIP(hipGetLastError());
    return Status::ok();
}

Status force_gather(Context &cx, double *F_caller) {
    ProfScope ps_(cx, kProfForceGather);
    if (cx.n == 0) return Status::ok();
    k_force_gather<<<grid_xcd(cx.n * kGatherLanes), kBlock, 0, cx.stream>>>(
        cx.n, cx.perm.as<int32_t>(), cx.t_off.as<int64_t>(), cx.t_act.as<int32_t>(),
        cx.ghost_off.as<int64_t>(), cx.Frecv.as<double>(), cx.gedge.as<float>(),
        cx.F.as<double>(), F_caller);
    MPNN_HIP(hipGetLastError());
    return Status::ok();
}

}  // namespace mpnn
