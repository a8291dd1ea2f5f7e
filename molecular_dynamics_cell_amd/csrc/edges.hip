// Edge kernels: the fused edge basis (Gaussian radial x cosine cutoff x scaled Cartesian
// monomial), the per-receiver orbital aggregation of Eq. 1, the reverse pass of Eq. 4-5
// (dE/dc of every sender, dE/dr of every edge) and the deterministic force gather of Eq. 3;
// plus the per-layer ghost refresh that stands in for the paper's ghost-message exchange
// (section "Parallelization Algorithm", Fig. 4a) and its reverse, the ghost->owner sum of
// gradient components (Fig. 4b).
//
// Every reduction has a fixed order (one thread owns one output row and walks its list), so
// results are bitwise reproducible and no floating-point atomics are used.
#include "impl.h"

namespace mpnn {

namespace {

// Edge basis of one edge, fp32, from the fp64 displacement.
template <int K, int L>
struct Basis {
    static constexpr int M = n_mono(L);
    float R[K], fc, A[M];
    float d, inv_d, v;  // v = d / rc
    float rx, ry, rz;
    float ux[L + 1], uy[L + 1], uz[L + 1];

    __device__ __forceinline__ void eval(double dx, double dy, double dz, const ModelDev *__restrict__ md,
                                         const float *mu) {
        constexpr Mono<L> mono;
        rx = (float)dx; ry = (float)dy; rz = (float)dz;
        d = sqrtf(rx * rx + ry * ry + rz * rz);
        inv_d = 1.0f / d;
        // x / rc as a refined quotient (no bias from rounding 1/rc), cos(pi d/rc) via cospi
        const float rc = md->rc, ir = md->inv_rc;
        auto div_rc = [rc, ir](float x) {
            const float q = x * ir;
            return fmaf(fmaf(-q, rc, x), ir, q);
        };
        v = div_rc(d);
        fc = 0.5f * (1.0f + cospif(v));
        const float nh = md->neg_half_inv_s2;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            float x = d - mu[k];
            R[k] = expf(nh * x * x);
        }
        const float qx = div_rc(rx), qy = div_rc(ry), qz = div_rc(rz);
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

template <int K, int L>
__global__ __launch_bounds__(256) void k_aggregate(int64_t n, const double *__restrict__ pos,
                                                   const int64_t *__restrict__ row_off,
                                                   const int32_t *__restrict__ nbr, const float *__restrict__ c,
                                                   const ModelDev *__restrict__ md, float *__restrict__ O) {
    constexpr int M = n_mono(L);
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    float mu[K];
#pragma unroll
    for (int k = 0; k < K; ++k) mu[k] = md->mu[k];
    const double rc2 = md->rc2;
    const double xi = pos[3 * i], yi = pos[3 * i + 1], zi = pos[3 * i + 2];
    float acc[K][M];
#pragma unroll
    for (int k = 0; k < K; ++k)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[k][m] = 0.0f;
    const int64_t e1 = row_off[i + 1];
    for (int64_t e = row_off[i]; e < e1; ++e) {
        const int64_t v = nbr[e];
        const double dx = __dsub_rn(pos[3 * v], xi), dy = __dsub_rn(pos[3 * v + 1], yi),
                     dz = __dsub_rn(pos[3 * v + 2], zi);
        if (!(d2_exact(dx, dy, dz) < rc2)) continue;
        Basis<K, L> b;
        b.eval(dx, dy, dz, md, mu);
        const float *cv = c + v * K;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            const float P = cv[k] * b.R[k] * b.fc;
#pragma unroll
            for (int m = 0; m < M; ++m) acc[k][m] += P * b.A[m];
        }
    }
    float *o = O + i * (K * M);
#pragma unroll
    for (int k = 0; k < K; ++k)
#pragma unroll
        for (int m = 0; m < M; ++m) o[k * M + m] = acc[k][m];
}

// dE/dc^t of every node v (sender side): sum over the edges v sends of u_k R_k f_c, with
// u_k = sum_m dE/dO_i[k,m] A_m of the receiving row i (Eq. 4, first term, as a VJP).
template <int K, int L>
__global__ __launch_bounds__(256) void k_message_grad(int64_t NN, const double *__restrict__ pos,
                                                      const int64_t *__restrict__ t_off,
                                                      const int32_t *__restrict__ t_recv,
                                                      const float *__restrict__ GO, const ModelDev *__restrict__ md,
                                                      float *__restrict__ Gc) {
    constexpr int M = n_mono(L);
    const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (v >= NN) return;
    float mu[K];
#pragma unroll
    for (int k = 0; k < K; ++k) mu[k] = md->mu[k];
    const double rc2 = md->rc2;
    const double xv = pos[3 * v], yv = pos[3 * v + 1], zv = pos[3 * v + 2];
    float acc[K];
#pragma unroll
    for (int k = 0; k < K; ++k) acc[k] = 0.0f;
    const int64_t s1 = t_off[v + 1];
    for (int64_t s = t_off[v]; s < s1; ++s) {
        const int64_t i = t_recv[s];
        // same operands and order as the receiver-side test: r = x_sender - x_receiver
        const double dx = __dsub_rn(xv, pos[3 * i]), dy = __dsub_rn(yv, pos[3 * i + 1]),
                     dz = __dsub_rn(zv, pos[3 * i + 2]);
        if (!(d2_exact(dx, dy, dz) < rc2)) continue;
        Basis<K, L> b;
        b.eval(dx, dy, dz, md, mu);
        const float *gi = GO + i * (K * M);
#pragma unroll
        for (int k = 0; k < K; ++k) {
            float u = 0.0f;
#pragma unroll
            for (int m = 0; m < M; ++m) u += gi[k * M + m] * b.A[m];
            acc[k] += u * b.R[k] * b.fc;
        }
    }
#pragma unroll
    for (int k = 0; k < K; ++k) Gc[v * K + k] = acc[k];
}

// Ghost -> owner sum of dE/dc (the reverse ghost exchange), ghosts of an owner in order.
__global__ void k_fold_ghost_grad(int64_t n, int K, const int64_t *__restrict__ ghost_off,
                                  float *__restrict__ Gc) {
    const int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (o >= n) return;
    for (int k = 0; k < K; ++k) {
        float s = Gc[o * K + k];
        for (int64_t g = ghost_off[o]; g < ghost_off[o + 1]; ++g) s += Gc[(n + g) * K + k];
        Gc[o * K + k] = s;
    }
}

// Owner -> ghost copy of the messages c^t (the forward ghost exchange).
__global__ void k_ghost_feat(int64_t G, int64_t n, int K, const int32_t *__restrict__ owner,
                             float *__restrict__ c) {
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= G * K) return;
    const int64_t g = q / K;
    const int k = (int)(q - g * K);
    c[(n + g) * K + k] = c[(int64_t)owner[g] * K + k];
}

// dE/dr_e of every edge summed over the T layers (Eq. 4, both terms), one receiver row per
// thread; layer-outer so dE/dO^t of the row stays in registers.  Writes the per-edge vectors
// and the receiver-side force sum (fp64).
template <int K, int L>
__global__ __launch_bounds__(256) void k_edge_forces(int64_t n, int T, int64_t NN, const double *__restrict__ pos,
                                                     const int64_t *__restrict__ row_off,
                                                     const int32_t *__restrict__ nbr, const float *__restrict__ c,
                                                     const float *__restrict__ GO, const ModelDev *__restrict__ md,
                                                     float *__restrict__ gedge, double *__restrict__ Frecv) {
    constexpr int M = n_mono(L);
    constexpr Mono<L> mono;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    float mu[K];
#pragma unroll
    for (int k = 0; k < K; ++k) mu[k] = md->mu[k];
    const double rc2 = md->rc2;
    const float inv_s2 = md->inv_s2, ir = md->inv_rc;
    const float dfc_scale = -0.5f * md->pi_over_rc;
    const double xi = pos[3 * i], yi = pos[3 * i + 1], zi = pos[3 * i + 2];
    const int64_t e0 = row_off[i], e1 = row_off[i + 1];
    double F[3] = {0.0, 0.0, 0.0};
    for (int t = 0; t < T; ++t) {
        float G[K][M];
        const float *gi = GO + ((int64_t)t * n + i) * (K * M);
#pragma unroll
        for (int k = 0; k < K; ++k)
#pragma unroll
            for (int m = 0; m < M; ++m) G[k][m] = gi[k * M + m];
        const float *ct = c + (int64_t)t * NN * K;
        for (int64_t e = e0; e < e1; ++e) {
            const int64_t v = nbr[e];
            const double dx = __dsub_rn(pos[3 * v], xi), dy = __dsub_rn(pos[3 * v + 1], yi),
                         dz = __dsub_rn(pos[3 * v + 2], zi);
            float g[3] = {0.0f, 0.0f, 0.0f};
            if (d2_exact(dx, dy, dz) < rc2) {
                Basis<K, L> b;
                b.eval(dx, dy, dz, md, mu);
                const float dfc = dfc_scale * sinpif(b.v);
                const float *cv = ct + v * K;
                float s = 0.0f, Q[M];
#pragma unroll
                for (int m = 0; m < M; ++m) Q[m] = 0.0f;
#pragma unroll
                for (int k = 0; k < K; ++k) {
                    float u = 0.0f;
#pragma unroll
                    for (int m = 0; m < M; ++m) u += G[k][m] * b.A[m];
                    const float dR = -(b.d - mu[k]) * inv_s2 * b.R[k];
                    s += cv[k] * u * (dR * b.fc + b.R[k] * dfc);
                    const float P = cv[k] * b.R[k] * b.fc;
#pragma unroll
                    for (int m = 0; m < M; ++m) Q[m] += P * G[k][m];
                }
                // radial part along r/d, angular part through dA_m/dr
                g[0] = s * b.rx * b.inv_d;
                g[1] = s * b.ry * b.inv_d;
                g[2] = s * b.rz * b.inv_d;
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    const int lx = mono.lx[m], ly = mono.ly[m], lz = mono.lz[m];
                    if (lx) g[0] += Q[m] * (float)lx * b.ux[lx - 1] * b.uy[ly] * b.uz[lz] * ir;
                    if (ly) g[1] += Q[m] * (float)ly * b.ux[lx] * b.uy[ly - 1] * b.uz[lz] * ir;
                    if (lz) g[2] += Q[m] * (float)lz * b.ux[lx] * b.uy[ly] * b.uz[lz - 1] * ir;
                }
            }
            float *ge = gedge + 3 * e;
            if (t == 0) {
                ge[0] = g[0]; ge[1] = g[1]; ge[2] = g[2];
            } else {
                ge[0] += g[0]; ge[1] += g[1]; ge[2] += g[2];
            }
            F[0] += (double)g[0];
            F[1] += (double)g[1];
            F[2] += (double)g[2];
        }
    }
    Frecv[3 * i] = F[0];
    Frecv[3 * i + 1] = F[1];
    Frecv[3 * i + 2] = F[2];
}

// F_i = sum_{edges received by i} dE/dr_e - sum_{edges sent by i or by its ghost images} dE/dr_e
// (r_e = r_sender - r_receiver), in fp64, in the fixed order of the transposed lists.
__global__ void k_force_gather(int64_t n, const int32_t *__restrict__ perm, const int64_t *__restrict__ t_off,
                               const int32_t *__restrict__ t_eid, const int64_t *__restrict__ ghost_off,
                               const double *__restrict__ Frecv, const float *__restrict__ gedge,
                               double *__restrict__ F, double *__restrict__ Fcaller) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    double f[3] = {Frecv[3 * i], Frecv[3 * i + 1], Frecv[3 * i + 2]};
    for (int64_t s = t_off[i]; s < t_off[i + 1]; ++s) {
        const int64_t e = t_eid[s];
        f[0] -= (double)gedge[3 * e];
        f[1] -= (double)gedge[3 * e + 1];
        f[2] -= (double)gedge[3 * e + 2];
    }
    for (int64_t g = ghost_off[i]; g < ghost_off[i + 1]; ++g) {
        const int64_t v = n + g;
        for (int64_t s = t_off[v]; s < t_off[v + 1]; ++s) {
            const int64_t e = t_eid[s];
            f[0] -= (double)gedge[3 * e];
            f[1] -= (double)gedge[3 * e + 1];
            f[2] -= (double)gedge[3 * e + 2];
        }
    }
    for (int a = 0; a < 3; ++a) F[3 * i + a] = f[a];
    if (Fcaller) {
        const int64_t c = perm[i];
        for (int a = 0; a < 3; ++a) Fcaller[3 * c + a] = f[a];
    }
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

Status aggregate(Context &cx, int t) {
    ProfScope ps_(cx, kProfAggregate);
    if (cx.n == 0) return Status::ok();
    const float *ct = cx.c.as<float>() + (int64_t)t * cx.NN * cx.K;
    float *Ot = cx.O.as<float>() + (int64_t)t * cx.n * cx.K * cx.M;
    MPNN_DISPATCH_KL(cx.K, cx.L, (k_aggregate<KK, LL><<<grid_for(cx.n), kBlock, 0, cx.stream>>>(
                                      cx.n, cx.pos.as<double>(), cx.row_off.as<int64_t>(), cx.nbr.as<int32_t>(),
                                      ct, cx.model.as<ModelDev>(), Ot)));
    MPNN_HIP(hipGetLastError());
    return Status::ok();
}

Status refresh_ghost_features(Context &cx, int t) {
    ProfScope ps_(cx, kProfGhostFeat);
    if (cx.G == 0) return Status::ok();
    float *ct = cx.c.as<float>() + (int64_t)t * cx.NN * cx.K;
    k_ghost_feat<<<grid_for(cx.G * cx.K), kBlock, 0, cx.stream>>>(cx.G, cx.n, cx.K, cx.ghost_owner.as<int32_t>(), ct);
    MPNN_HIP(hipGetLastError());
    return Status::ok();
}

Status backward_messages(Context &cx, int t) {
    if (cx.n == 0) return Status::ok();
    const float *GOt = cx.GO.as<float>() + (int64_t)t * cx.n * cx.K * cx.M;
    {
        ProfScope ps_(cx, kProfMessageGrad);
        MPNN_DISPATCH_KL(cx.K, cx.L, (k_message_grad<KK, LL><<<grid_for(cx.NN), kBlock, 0, cx.stream>>>(
                                          cx.NN, cx.pos.as<double>(), cx.t_off.as<int64_t>(), cx.t_recv.as<int32_t>(),
                                          GOt, cx.model.as<ModelDev>(), cx.Gc.as<float>())));
        MPNN_HIP(hipGetLastError());
    }
    ProfScope ps_(cx, kProfGhostFold);
    k_fold_ghost_grad<<<grid_for(cx.n), kBlock, 0, cx.stream>>>(cx.n, cx.K, cx.ghost_off.as<int64_t>(),
                                                                 cx.Gc.as<float>());
    MPNN_HIP(hipGetLastError());
    return Status::ok();
}

Status force_edges(Context &cx) {
    ProfScope ps_(cx, kProfEdgeForces);
    if (cx.n == 0) return Status::ok();
    MPNN_DISPATCH_KL(cx.K, cx.L, (k_edge_forces<KK, LL><<<grid_for(cx.n), kBlock, 0, cx.stream>>>(
                                      cx.n, cx.T, cx.NN, cx.pos.as<double>(), cx.row_off.as<int64_t>(),
                                      cx.nbr.as<int32_t>(), cx.c.as<float>(), cx.GO.as<float>(),
                                      cx.model.as<ModelDev>(), cx.gedge.as<float>(), cx.Frecv.as<double>())));
    MPNN_HIP(hipGetLastError());
    return Status::ok();
}

Status force_gather(Context &cx, double *F_caller) {
    ProfScope ps_(cx, kProfForceGather);
    if (cx.n == 0) return Status::ok();
    k_force_gather<<<grid_for(cx.n), kBlock, 0, cx.stream>>>(cx.n, cx.perm.as<int32_t>(), cx.t_off.as<int64_t>(),
                                                            cx.t_eid.as<int32_t>(), cx.ghost_off.as<int64_t>(),
                                                            cx.Frecv.as<double>(), cx.gedge.as<float>(),
                                                            cx.F.as<double>(), F_caller);
    MPNN_HIP(hipGetLastError());
    return Status::ok();
}

}  // namespace mpnn
