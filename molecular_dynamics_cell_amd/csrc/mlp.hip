// Atom-wise networks (paper, Eq. 2 and Fig. 1c: per-element atomic NNs mapping the density
// features rho^t to the next messages c^{t+1}, and after T layers to the atomic energy E_i),
// their vector-Jacobian products (Eq. 5), and the rho -> O chain rule of Eq. 1.
//
// Layout on the matrix cores (gfx950, v_mfma_f32_16x16x4f32, wave64):
//   one wave handles 16 atoms of one species; every product is computed transposed,
//   Y^T [rows x 16 atoms] = W [rows x cols] * X^T [cols x 16 atoms], so the accumulator of a
//   16x16 tile (lane l holds rows 4*(l/16)+r, r = 0..3, of atom l%16) is directly the B operand
//   of the next product when the k-steps of column tile ct visit inputs 16ct + 4*(l/16) + r.
//   Weights are pre-packed in exactly that A-operand order, one float4 per lane per 4 k-steps.
// The density features are formed on the fly from the 16 atoms' O rows staged in LDS; the
// first layer's B operand is feature q = 16ct + 4*(l/16) + r of atom l%16.
#include <cmath>
#include <vector>

#include "impl.h"

namespace mpnn {

namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ floatx4 mfma4(float a, float b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }
__device__ __forceinline__ float silu_grad(float z) {
    const float sg = 1.0f / (1.0f + expf(-z));
    return sg * (1.0f + z * (1.0f - sg));
}

// acc[rt] += sum_ct W[rt][ct] * b[ct] (4 k-steps per column tile)
template <int RT, int CT>
__device__ __forceinline__ void gemm(const float4 *__restrict__ W, const float (&b)[CT][4], floatx4 (&acc)[RT],
                                     int lane) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const float4 a = W[(rt * CT + ct) * 64 + lane];
            acc[rt] = mfma4(a.x, b[ct][0], acc[rt]);
            acc[rt] = mfma4(a.y, b[ct][1], acc[rt]);
            acc[rt] = mfma4(a.z, b[ct][2], acc[rt]);
            acc[rt] = mfma4(a.w, b[ct][3], acc[rt]);
        }
}

constexpr int kMaxSpecies = 16;

struct NetArgs {
    const float *O;        // O^t [n][K*M]
    const float *W;        // packed weights of (t, species 0); species s at W + s*stride
    int64_t stride;
    int64_t oW1, oW2, oW3, oW1t, oW2t, oW3t, ob1, ob2, ob3;
    int S;
    float inv_scale, e_scale;
    const int32_t *sp_list;
    int64_t sp_off[kMaxSpecies + 1];
    int32_t tile_start[kMaxSpecies + 1];
    float *c_next;         // forward: c^{t+1} [*][K]
    float *Ei;             // energy: E_i [n]
    const float *Gc;       // backward: dE/dc^{t+1} [*][K]
    float *GO;             // energy/backward: dE/dO^t [n][K*M]
};

enum { kForward = 0, kEnergy = 1, kBackward = 2 };

template <int K, int L, int H, int MODE>
__global__ __launch_bounds__(64) void k_net(const NetArgs a) {
    constexpr int M = n_mono(L), KM = K * M, D = n_feat(K, L);
    constexpr int DT = (D + 15) / 16, HT = H / 16;
    constexpr int OS = KM + 1, GS = D + 1;
    constexpr int P = K * (K + 1) / 2;
    constexpr Mono<L> mono;
    __shared__ float sO[16 * OS];
    __shared__ float sG[MODE == kForward ? 1 : 16 * GS];

    const int lane = threadIdx.x, col = lane & 15, grp = lane >> 4;
    const int tile = blockIdx.x;
    int s = 0;
    while (s + 1 < a.S && tile >= a.tile_start[s + 1]) ++s;
    const int64_t base = (int64_t)(tile - a.tile_start[s]) * 16;
    const int64_t cnt = a.sp_off[s + 1] - a.sp_off[s];
    const int32_t *list = a.sp_list + a.sp_off[s];
    const int64_t me = (base + col < cnt) ? (int64_t)list[base + col] : -1;
    const float *W = a.W + (int64_t)s * a.stride;

    // stage the 16 O rows, scaled by sqrt(w_m) so that rho = sum_m O~[a,m] O~[b,m]
    for (int idx = lane; idx < 16 * KM; idx += 64) {
        const int q = idx / KM, r = idx - q * KM;
        const int64_t at = (base + q < cnt) ? (int64_t)list[base + q] : -1;
        const float w = mono.w[r % M];
        sO[q * OS + r] = at >= 0 ? a.O[at * KM + r] * sqrtf(w) : 0.0f;
    }
    __syncthreads();

    // layer 1: Z1 = W1 rho~ + b1, features generated per k-step
    floatx4 z1[HT];
#pragma unroll
    for (int rt = 0; rt < HT; ++rt) z1[rt] = floatx4{0.f, 0.f, 0.f, 0.f};
    const float4 *W1 = reinterpret_cast<const float4 *>(W + a.oW1);
    const float *so = sO + col * OS;
    for (int ct = 0; ct < DT; ++ct) {
        float bf[1][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = 16 * ct + 4 * grp + i;
            float v = 0.0f;
            if (q < D) {
                const int l = q / P;
                int r = q - l * P, x = 0;
                while (r >= K - x) { r -= K - x; ++x; }
                const int y = x + r;
                const int m0 = l * (l + 1) * (l + 2) / 6, m1 = m0 + (l + 1) * (l + 2) / 2;
                for (int m = m0; m < m1; ++m) v += so[x * M + m] * so[y * M + m];
            }
            bf[0][i] = v * a.inv_scale;
        }
#pragma unroll
        for (int rt = 0; rt < HT; ++rt) {
            const float4 w = W1[(rt * DT + ct) * 64 + lane];
            z1[rt] = mfma4(w.x, bf[0][0], z1[rt]);
            z1[rt] = mfma4(w.y, bf[0][1], z1[rt]);
            z1[rt] = mfma4(w.z, bf[0][2], z1[rt]);
            z1[rt] = mfma4(w.w, bf[0][3], z1[rt]);
        }
    }
    const float *b1 = W + a.ob1, *b2 = W + a.ob2, *b3 = W + a.ob3;
    float h1[HT][4];
#pragma unroll
    for (int rt = 0; rt < HT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            z1[rt][i] += b1[16 * rt + 4 * grp + i];
            h1[rt][i] = silu(z1[rt][i]);
        }
    // layer 2
    floatx4 z2[HT];
#pragma unroll
    for (int rt = 0; rt < HT; ++rt) z2[rt] = floatx4{0.f, 0.f, 0.f, 0.f};
    gemm<HT, HT>(reinterpret_cast<const float4 *>(W + a.oW2), h1, z2, lane);
    float h2[HT][4];
#pragma unroll
    for (int rt = 0; rt < HT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            z2[rt][i] += b2[16 * rt + 4 * grp + i];
            h2[rt][i] = silu(z2[rt][i]);
        }

    if constexpr (MODE != kBackward) {
        // output layer: 16 padded output rows (K messages or 1 energy)
        floatx4 y[1] = {floatx4{0.f, 0.f, 0.f, 0.f}};
        gemm<1, HT>(reinterpret_cast<const float4 *>(W + a.oW3), h2, y, lane);
        if constexpr (MODE == kForward) {
            if (me >= 0)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int k = 4 * grp + i;
                    if (k < K) a.c_next[me * K + k] = y[0][i] + b3[k];
                }
        } else {
            if (grp == 0 && me >= 0) a.Ei[me] = a.e_scale * (y[0][0] + b3[0]);
        }
    }
    if constexpr (MODE != kForward) {

    // ---- vector-Jacobian product back to rho~ ----
    float gy[1][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int k = 4 * grp + i;
        if (MODE == kEnergy) gy[0][i] = (k == 0) ? a.e_scale : 0.0f;
        else gy[0][i] = (k < K && me >= 0) ? a.Gc[me * K + k] : 0.0f;
    }
    floatx4 g2[HT];
#pragma unroll
    for (int rt = 0; rt < HT; ++rt) g2[rt] = floatx4{0.f, 0.f, 0.f, 0.f};
    gemm<HT, 1>(reinterpret_cast<const float4 *>(W + a.oW3t), gy, g2, lane);
    float gz2[HT][4];
#pragma unroll
    for (int rt = 0; rt < HT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) gz2[rt][i] = g2[rt][i] * silu_grad(z2[rt][i]);
    floatx4 g1[HT];
#pragma unroll
    for (int rt = 0; rt < HT; ++rt) g1[rt] = floatx4{0.f, 0.f, 0.f, 0.f};
    gemm<HT, HT>(reinterpret_cast<const float4 *>(W + a.oW2t), gz2, g1, lane);
    float gz1[HT][4];
#pragma unroll
    for (int rt = 0; rt < HT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) gz1[rt][i] = g1[rt][i] * silu_grad(z1[rt][i]);
    // d E / d rho = (W1^T gz1) / s_t, one 16-row tile at a time into LDS
    const float4 *W1t = reinterpret_cast<const float4 *>(W + a.oW1t);
    for (int rt = 0; rt < DT; ++rt) {
        floatx4 gr = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ct = 0; ct < HT; ++ct) {
            const float4 w = W1t[(rt * HT + ct) * 64 + lane];
            gr = mfma4(w.x, gz1[ct][0], gr);
            gr = mfma4(w.y, gz1[ct][1], gr);
            gr = mfma4(w.z, gz1[ct][2], gr);
            gr = mfma4(w.w, gz1[ct][3], gr);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = 16 * rt + 4 * grp + i;
            if (q < D) sG[col * GS + q] = gr[i] * a.inv_scale;
        }
    }
    __syncthreads();
    // dE/dO[c,m] = sqrt(w_m) * sum_b (1 + [b == c]) dE/drho[(min,max), l_m] O~[b,m]
    if (me < 0) return;
    const float *sg = sG + col * GS;
    float *go = a.GO + me * KM;
    for (int o = grp; o < KM; o += 4) {
        const int c = o / M, m = o - c * M;
        const int l = mono.l[m];
        float acc = 0.0f;
#pragma unroll
        for (int b = 0; b < K; ++b) {
            const int x = c < b ? c : b, y = c < b ? b : c;
            const int q = l * P + x * K - x * (x - 1) / 2 + (y - x);
            const float coef = (b == c) ? 2.0f : 1.0f;
            acc += coef * sg[q] * so[b * M + m];
        }
        go[o] = acc * sqrtf(mono.w[m]);
    }
    }  // MODE != kForward
}

NetArgs make_args(Context &cx, int t) {
    NetArgs a{};
    a.W = cx.weights.as<float>() + (int64_t)t * cx.S * cx.net.stride;
    a.stride = (int64_t)cx.net.stride;
    a.oW1 = cx.net.W1; a.oW2 = cx.net.W2; a.oW3 = cx.net.W3;
    a.oW1t = cx.net.W1t; a.oW2t = cx.net.W2t; a.oW3t = cx.net.W3t;
    a.ob1 = cx.net.b1; a.ob2 = cx.net.b2; a.ob3 = cx.net.b3;
    a.S = cx.S;
    a.sp_list = cx.sp_list.as<int32_t>();
    int64_t off = 0;
    int32_t tiles = 0;
    for (int s = 0; s <= cx.S; ++s) {
        a.sp_off[s] = off;
        a.tile_start[s] = tiles;
        if (s < cx.S) {
            off += cx.sp_count[s];
            tiles += (int32_t)((cx.sp_count[s] + 15) / 16);
        }
    }
    a.O = cx.O.as<float>() + (int64_t)t * cx.n * cx.K * cx.M;
    a.e_scale = (float)cx.e_scale;
    return a;
}

#define MPNN_DISPATCH_NET(MODE_, A_)                                                                   \
    do {                                                                                               \
        const unsigned tiles = (unsigned)(A_).tile_start[cx.S];                                        \
        if (tiles == 0) return Status::ok();                                                           \
        if (cx.K == 8 && cx.L == 2 && cx.H == 64) k_net<8, 2, 64, MODE_><<<tiles, 64, 0, cx.stream>>>(A_);         \
        else if (cx.K == 8 && cx.L == 2 && cx.H == 128) k_net<8, 2, 128, MODE_><<<tiles, 64, 0, cx.stream>>>(A_);  \
        else if (cx.K == 12 && cx.L == 3 && cx.H == 128) k_net<12, 3, 128, MODE_><<<tiles, 64, 0, cx.stream>>>(A_);\
        else if (cx.K == 12 && cx.L == 3 && cx.H == 64) k_net<12, 3, 64, MODE_><<<tiles, 64, 0, cx.stream>>>(A_);  \
        else if (cx.K == 2 && cx.L == 1 && cx.H == 64) k_net<2, 1, 64, MODE_><<<tiles, 64, 0, cx.stream>>>(A_);    \
        else if (cx.K == 4 && cx.L == 2 && cx.H == 64) k_net<4, 2, 64, MODE_><<<tiles, 64, 0, cx.stream>>>(A_);    \
        else return Status::err(MPNN_E_INVALID_ARG, "unsupported (K, L, H)");                          \
        MPNN_HIP(hipGetLastError());                                                                   \
    } while (0)

// A-operand packing of W [R][C] (row-major, fp64) for Y^T = W X^T: for row tile rt, column tile
// ct, lane l, component i: W[16 rt + l%16][16 ct + 4 (l/16) + i] (zero outside R x C).
void pack_a(const double *W, int R, int C, int Rp, int Cp, bool transpose, float *out) {
    const int RT = Rp / 16, CT = Cp / 16;
    for (int rt = 0; rt < RT; ++rt)
        for (int ct = 0; ct < CT; ++ct)
            for (int l = 0; l < 64; ++l)
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * rt + (l & 15), c = 16 * ct + 4 * (l >> 4) + i;
                    double v = 0.0;
                    if (r < R && c < C) v = transpose ? W[(size_t)c * R + r] : W[(size_t)r * C + c];
                    out[(((size_t)rt * CT + ct) * 64 + l) * 4 + i] = (float)v;
                }
}

}  // namespace

Status pack_weights(Context &cx, const double *mlp) {
    const int H = cx.H, D = cx.D, DP = cx.DP, K = cx.K;
    NetLayout &nl = cx.net;
    size_t o = 0;
    nl.W1 = o; o += (size_t)H * DP;
    nl.W2 = o; o += (size_t)H * H;
    nl.W3 = o; o += (size_t)16 * H;
    nl.W1t = o; o += (size_t)DP * H;
    nl.W2t = o; o += (size_t)H * H;
    nl.W3t = o; o += (size_t)H * 16;
    nl.b1 = o; o += H;
    nl.b2 = o; o += H;
    nl.b3 = o; o += 16;
    nl.stride = (o + 63) / 64 * 64;
    std::vector<float> host((size_t)cx.T * cx.S * nl.stride, 0.0f);
    const double *p = mlp;
    for (int t = 0; t < cx.T; ++t) {
        const int out = t < cx.T - 1 ? K : 1;
        for (int s = 0; s < cx.S; ++s) {
            float *blk = host.data() + ((size_t)t * cx.S + s) * nl.stride;
            const double *W1 = p, *b1 = W1 + (size_t)H * D, *W2 = b1 + H, *b2 = W2 + (size_t)H * H;
            const double *W3 = b2 + H, *b3 = W3 + (size_t)out * H;
            p = b3 + out;
            pack_a(W1, H, D, H, DP, false, blk + nl.W1);
            pack_a(W2, H, H, H, H, false, blk + nl.W2);
            pack_a(W3, out, H, 16, H, false, blk + nl.W3);
            pack_a(W1, D, H, DP, H, true, blk + nl.W1t);
            pack_a(W2, H, H, H, H, true, blk + nl.W2t);
            pack_a(W3, H, out, H, 16, true, blk + nl.W3t);
            for (int h = 0; h < H; ++h) {
                blk[nl.b1 + h] = (float)b1[h];
                blk[nl.b2 + h] = (float)b2[h];
            }
            for (int k = 0; k < out; ++k) blk[nl.b3 + k] = (float)b3[k];
        }
    }
    MPNN_TRY(cx.grow(cx.weights, host.size() * sizeof(float)));
    MPNN_HIP(hipMemcpy(cx.weights.p, host.data(), host.size() * sizeof(float), hipMemcpyHostToDevice));
    return Status::ok();
}

Status mlp_forward(Context &cx, int t) {
    ProfScope ps_(cx, kProfNetForward);
    NetArgs a = make_args(cx, t);
    a.c_next = cx.c.as<float>() + (int64_t)(t + 1) * cx.NN * cx.K;
    a.inv_scale = cx.inv_scale_host[t];
    MPNN_DISPATCH_NET(kForward, a);
    return Status::ok();
}

Status mlp_energy(Context &cx) {
    ProfScope ps_(cx, kProfNetEnergy);
    const int t = cx.T - 1;
    NetArgs a = make_args(cx, t);
    a.inv_scale = cx.inv_scale_host[t];
    a.Ei = cx.Ei.as<float>();
    a.GO = cx.GO.as<float>() + (int64_t)t * cx.n * cx.K * cx.M;
    MPNN_DISPATCH_NET(kEnergy, a);
    return Status::ok();
}

Status mlp_backward(Context &cx, int t) {
    ProfScope ps_(cx, kProfNetBackward);
    NetArgs a = make_args(cx, t);
    a.inv_scale = cx.inv_scale_host[t];
    a.Gc = cx.Gc.as<float>();
    a.GO = cx.GO.as<float>() + (int64_t)t * cx.n * cx.K * cx.M;
    MPNN_DISPATCH_NET(kBackward, a);
    return Status::ok();
}

}  // namespace mpnn
