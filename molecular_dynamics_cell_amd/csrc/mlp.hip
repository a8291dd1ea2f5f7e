// Atom-wise networks (paper, Eq. 2 and Fig. 1c: per-element atomic NNs mapping the density
// features rho^t to the next messages c^{t+1}, and after T layers to the atomic energy E_i) and
// their vector-Jacobian products (Eq. 5), on the matrix cores.
//
// Layout (gfx950, v_mfma_f32_16x16x4f32, wave64): one wave handles CT tiles of 16 atoms of one
// species; every product is computed transposed, Y^T [rows x atoms] = W [rows x cols] X^T, so the
// accumulator of a 16x16 tile (lane l holds rows 4*(l/16)+r, r = 0..3, of atom l%16) is directly
// the B operand of the next product when the k-steps of column tile kt visit inputs
// 16 kt + 4 (l/16) + r.  Weights are pre-packed in exactly that A-operand order (one float4 per
// lane per 4 k-steps).  The density features arrive from the aggregation kernel column-tiled (16
// features of one atom contiguous), so the first product's B operand is one float4 load per lane
// per column tile; the VJP leaves dE/drho in the same layout for the reverse edge pass, which forms
// dE/dO from it.
#include <cmath>
#include <cstring>
#include <type_traits>
#include <vector>

#include "impl.h"

namespace mpnn {

namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ floatx4 mfma4(float a, float b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// logistic function from the hardware exp2 of a two-part product z log2(e) (so the argument carries
// no rounding bias) and the hardware reciprocal with one Newton step.  The exponent is capped at
// 126 so 1 + 2^y stays finite (the Newton step would turn an infinite one into NaN); below
// z = -87 the result is then 2^-126 instead of e^z, both zero for every use here.
__device__ __forceinline__ float sigmoid(float z) {
    const float y = fminf(fmaf(z, -1.44269502f, z * -1.92596299e-8f), 126.0f);
    const float d = 1.0f + __builtin_amdgcn_exp2f(y);
    const float r = __builtin_amdgcn_rcpf(d);
    return fmaf(fmaf(-d, r, 1.0f), r, r);
}

// acc[rt][c] += W[rt][kt] x[c] for every row tile rt of a matrix packed with KT column tiles:
// one float4 of weights per lane feeds 4 k-steps of each of the CT atom tiles.  The matrix cores
// sum each 16-input chunk from zero in fp32 and the chunk is added to an fp64 accumulator, so no
// fp32 sum runs over more than 16 products (long fp32 chains lose several 1e-7 relative on
// these products).
template <int RT, int CT>
__device__ __forceinline__ void gemm_chunk(const float4 &w, const float (&x)[CT][4], double (&acc)[CT][4]) {
#pragma unroll
    for (int c = 0; c < CT; ++c) {
        floatx4 t = mfma4(w.x, x[c][0], floatx4{0.f, 0.f, 0.f, 0.f});
        t = mfma4(w.y, x[c][1], t);
        t = mfma4(w.z, x[c][2], t);
        t = mfma4(w.w, x[c][3], t);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[c][i] += (double)t[i];
    }
}

template <int RT, int CT>
__device__ __forceinline__ void gemm_step(const float4 *__restrict__ W, int KT, int kt, const float (&x)[CT][4],
                                          double (&acc)[RT][CT][4], int lane) {
    // 128-wide networks: one scheduling region per chunk column, which keeps the compiler from
    // hoisting the weight loads of every column at once (hundreds of registers); the 64-wide
    // ones may prefetch the next column's weights
    if constexpr (RT >= 8) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) gemm_chunk<RT, CT>(W[(rt * KT + kt) * 64 + lane], x, acc[rt]);
}

// accumulators start from the bias of their output row (row 16 rt + 4 grp + i)
template <int RT, int CT>
__device__ __forceinline__ void init_bias(double (&acc)[RT][CT][4], const float *__restrict__ b, int grp) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const double v = (double)b[16 * rt + 4 * grp + i];
#pragma unroll
            for (int c = 0; c < CT; ++c) acc[rt][c][i] = v;
        }
}

template <int RT, int CT>
__device__ __forceinline__ void zero(double (&acc)[RT][CT][4]) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[rt][c][i] = 0.0;
}

constexpr int kMaxSpecies = 16;

struct NetArgs {
    const float *F;        // rho^t / s_t, column-tiled [np][DP]
    const float *W;        // packed weights of (t, species 0); species s at W + s*stride
    const double *W64;     // the same in fp64 (accurate mode)
    const uint16_t *W16;   // bf16 operand blocks of (t, species 0) (bf16 mode); species s at W16 + s*stride16
    int64_t stride16, o16W1, o16W2, o16W3, o16W1t, o16W2t, o16lo;
    int64_t stride;
    int64_t oW1, oW2, oW3, oW1t, oW2t, oW3t, ob1, ob2, ob3;
    int S;
    float inv_scale, e_scale;   // fp32 parameters (modes 0 and 2)
    double e_scale64;           // fp64 parameter (mode 1)
    const int32_t *sp_list;
    int64_t sp_off[kMaxSpecies + 1];
    int32_t tile_start[kMaxSpecies + 1];
    float *c_next;         // forward: c^{t+1} of node v at c_next[v * rec_stride(K) + k]
    double *Ei;            // energy: E_i [n]
    const float *Gc;       // backward: dE/dc^{t+1} [*][K]
    float *Grho;           // energy/backward: dE/drho^t, column-tiled [np][DP]
    int64_t np;
    float *dact;           // fp32 message networks: silu' of both hidden layers, [species-list position][2H]
};

enum { kForward = 0, kEnergy = 1, kBackward = 2 };

template <int K, int L, int H, int MODE, int CT, bool SAVE = false>
__global__ __launch_bounds__(64, 2) void k_net(const NetArgs a) {
    static_assert(!SAVE || MODE == kForward, "only the forward network saves silu'");
    constexpr int D = n_feat(K, L), DP = (D + 15) / 16 * 16;
    constexpr int DT = DP / 16, HT = H / 16;
    const int lane = threadIdx.x, col = lane & 15, grp = lane >> 4;
    const int tile = blockIdx.x;
    int s = 0;
    while (s + 1 < a.S && tile >= a.tile_start[s + 1]) ++s;
    const int64_t base = (int64_t)(tile - a.tile_start[s]) * (16 * CT);
    const int64_t cnt = a.sp_off[s + 1] - a.sp_off[s];
    const int32_t *list = a.sp_list + a.sp_off[s];
    int64_t me[CT];
#pragma unroll
    for (int c = 0; c < CT; ++c) me[c] = (base + 16 * c + col < cnt) ? (int64_t)list[base + 16 * c + col] : -1;
    const float *W = a.W + (int64_t)s * a.stride;
    const float *b1 = W + a.ob1, *b2 = W + a.ob2, *b3 = W + a.ob3;
    // SAVE: this lane's silu' values go to the atom's row of dact (rows 16 rt + 4 grp .. + 3 of
    // each layer as one float4), for the reverse network of the same layer
    float *dsave[CT];
#pragma unroll
    for (int c = 0; c < CT; ++c)
        dsave[c] = (SAVE && me[c] >= 0) ? a.dact + (a.sp_off[s] + base + 16 * c + col) * (2 * H) : nullptr;

    // layer 1: Z1 = W1 rho~ + b1
    double z1[HT][CT][4];
    init_bias(z1, b1, grp);
    {
        const float4 *W1 = reinterpret_cast<const float4 *>(W + a.oW1);
        auto load_x = [&](int kt, float (&x)[CT][4]) {
#pragma unroll
            for (int c = 0; c < CT; ++c) {
                float4 f = float4{0.f, 0.f, 0.f, 0.f};
                if (me[c] >= 0) f = *reinterpret_cast<const float4 *>(a.F + tiled(a.np, me[c], 16 * kt + 4 * grp));
                x[c][0] = f.x; x[c][1] = f.y; x[c][2] = f.z; x[c][3] = f.w;
            }
        };
        if constexpr (HT < 8) {
            // 64-wide networks on one atom tile: the next column's features (from HBM) are
            // requested after this column's weights (from L2), so the products wait for the
            // weights only (with two tiles the registers would cost a wave per SIMD).  The loads
            // are unconditional (padding lanes read row 0 and drop it, the last step re-reads its
            // own column), so the wait counts stay exact
            auto load_all = [&](int kt, float (&x)[CT][4]) {
#pragma unroll
                for (int c = 0; c < CT; ++c) {
                    const int64_t r = me[c] >= 0 ? me[c] : 0;
                    float4 f = *reinterpret_cast<const float4 *>(a.F + tiled(a.np, r, 16 * kt + 4 * grp));
                    if (me[c] < 0) f = float4{0.f, 0.f, 0.f, 0.f};
                    x[c][0] = f.x; x[c][1] = f.y; x[c][2] = f.z; x[c][3] = f.w;
                }
            };
            float x[CT][4];
            load_all(0, x);
#pragma unroll 1
            for (int kt = 0; kt < DT; ++kt) {
                float4 w[HT];
#pragma unroll
                for (int rt = 0; rt < HT; ++rt) w[rt] = W1[(rt * DT + kt) * 64 + lane];
                float xn[CT][4];
                load_all(kt + 1 < DT ? kt + 1 : kt, xn);
#pragma unroll
                for (int rt = 0; rt < HT; ++rt) gemm_chunk<HT, CT>(w[rt], x, z1[rt]);
#pragma unroll
                for (int c = 0; c < CT; ++c)
#pragma unroll
                    for (int i = 0; i < 4; ++i) x[c][i] = xn[c][i];
            }
        } else {
#pragma unroll 1
            for (int kt = 0; kt < DT; ++kt) {
                float x[CT][4];
                load_x(kt, x);
                gemm_step<HT, CT>(W1, DT, kt, x, z1, lane);
            }
        }
    }
    // H1 = silu(Z1); the backward pass keeps only silu'(Z1) = s (1 + z (1 - s))
    // silu'(Z1) is parked in LDS (one word per lane per value, conflict-free) until the reverse pass
    // needs it, which keeps the 128-wide reverse networks within their register budget
    __shared__ float sd1[MODE == kForward ? 1 : HT * CT * 4][64];
    float h1[HT][CT][4], ds[4];
#pragma unroll
    for (int rt = 0; rt < HT; ++rt)
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float z = (float)z1[rt][c][i];
                const float sg = sigmoid(z);
                h1[rt][c][i] = z * sg;
                if constexpr (MODE != kForward) sd1[(rt * CT + c) * 4 + i][lane] = sg * (1.0f + z * (1.0f - sg));
                if constexpr (SAVE) ds[i] = sg * (1.0f + z * (1.0f - sg));
                if (SAVE && i == 3 && dsave[c])
                    *reinterpret_cast<float4 *>(dsave[c] + 16 * rt + 4 * grp) = float4{ds[0], ds[1], ds[2], ds[3]};
            }
    // layer 2
    double z2[HT][CT][4];
    __builtin_amdgcn_sched_barrier(0);
    init_bias(z2, b2, grp);
    {
        const float4 *W2 = reinterpret_cast<const float4 *>(W + a.oW2);
#pragma unroll
        for (int kt = 0; kt < HT; ++kt) gemm_step<HT, CT>(W2, HT, kt, h1[kt], z2, lane);
    }
    float h2[HT][CT][4], d2[MODE == kForward ? 1 : HT][CT][4];
#pragma unroll
    for (int rt = 0; rt < HT; ++rt)
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float z = (float)z2[rt][c][i];
                const float sg = sigmoid(z);
                h2[rt][c][i] = z * sg;
                if constexpr (MODE != kForward) d2[rt][c][i] = sg * (1.0f + z * (1.0f - sg));
                if constexpr (SAVE) ds[i] = sg * (1.0f + z * (1.0f - sg));
                if (SAVE && i == 3 && dsave[c])
                    *reinterpret_cast<float4 *>(dsave[c] + H + 16 * rt + 4 * grp) = float4{ds[0], ds[1], ds[2], ds[3]};
            }

    if constexpr (MODE != kBackward) {
        // output layer: 16 padded output rows (K messages or 1 energy)
        double y[1][CT][4];
        init_bias(y, b3, grp);
        const float4 *W3 = reinterpret_cast<const float4 *>(W + a.oW3);
#pragma unroll
        for (int kt = 0; kt < HT; ++kt) gemm_step<1, CT>(W3, HT, kt, h2[kt], y, lane);
#pragma unroll
        for (int c = 0; c < CT; ++c) {
            if (me[c] < 0) continue;
            if constexpr (MODE == kForward) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int k = 4 * grp + i;
                    if (k < K) a.c_next[me[c] * rec_stride(K) + k] = (float)y[0][c][i];
                }
            } else {
                if (grp == 0) a.Ei[me[c]] = (double)a.e_scale * y[0][c][0];
            }
        }
    }
    if constexpr (MODE != kForward) {
        // ---- vector-Jacobian product back to rho ----
        // dE/dy: e_scale on output 0 for the energy network, dE/dc^{t+1} of the atom otherwise
        float gy[CT][4];
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int k = 4 * grp + i;
                if constexpr (MODE == kEnergy) gy[c][i] = (k == 0) ? a.e_scale : 0.0f;
                else gy[c][i] = (k < K && me[c] >= 0) ? a.Gc[me[c] * K + k] : 0.0f;
            }
        // a single 16-input chunk (the output width): fp32 from the matrix cores is enough
        floatx4 g2[HT][CT];
        __builtin_amdgcn_sched_barrier(0);
        {
            const float4 *W3t = reinterpret_cast<const float4 *>(W + a.oW3t);
#pragma unroll
            for (int rt = 0; rt < HT; ++rt) {
                const float4 w = W3t[rt * 64 + lane];
#pragma unroll
                for (int c = 0; c < CT; ++c) {
                    floatx4 t = mfma4(w.x, gy[c][0], floatx4{0.f, 0.f, 0.f, 0.f});
                    t = mfma4(w.y, gy[c][1], t);
                    t = mfma4(w.z, gy[c][2], t);
                    g2[rt][c] = mfma4(w.w, gy[c][3], t);
                }
            }
        }
        float gz2[HT][CT][4];
#pragma unroll
        for (int rt = 0; rt < HT; ++rt)
#pragma unroll
            for (int c = 0; c < CT; ++c)
#pragma unroll
                for (int i = 0; i < 4; ++i) gz2[rt][c][i] = g2[rt][c][i] * d2[rt][c][i];
        double g1[HT][CT][4];
        zero(g1);
        {
            const float4 *W2t = reinterpret_cast<const float4 *>(W + a.oW2t);
#pragma unroll
            for (int kt = 0; kt < HT; ++kt) gemm_step<HT, CT>(W2t, HT, kt, gz2[kt], g1, lane);
        }
        float gz1[HT][CT][4];
#pragma unroll
        for (int rt = 0; rt < HT; ++rt)
#pragma unroll
            for (int c = 0; c < CT; ++c)
#pragma unroll
                for (int i = 0; i < 4; ++i) gz1[rt][c][i] = (float)g1[rt][c][i] * sd1[(rt * CT + c) * 4 + i][lane];
        // dE/drho = (W1^T dE/dZ1) / s_t, one 16-row tile at a time, stored as float4 row pieces
        const float4 *W1t = reinterpret_cast<const float4 *>(W + a.oW1t);
#pragma unroll 1
        for (int rt = 0; rt < DT; ++rt) {
            double gr[1][CT][4];
            zero(gr);
#pragma unroll
            for (int kt = 0; kt < HT; ++kt) gemm_step<1, CT>(W1t + (size_t)rt * HT * 64, HT, kt, gz1[kt], gr, lane);
#pragma unroll
            for (int c = 0; c < CT; ++c)
                if (me[c] >= 0)
                    *reinterpret_cast<float4 *>(a.Grho + tiled(a.np, me[c], 16 * rt + 4 * grp)) =
                        float4{(float)(gr[0][c][0] * a.inv_scale), (float)(gr[0][c][1] * a.inv_scale),
                               (float)(gr[0][c][2] * a.inv_scale), (float)(gr[0][c][3] * a.inv_scale)};
        }
    }
}

// The reverse message network from the silu' values its forward pass saved (fp32 mode): the same
// vector-Jacobian product as k_net's reverse mode, without recomputing the two hidden layers, so
// half the matrix work.  The saved values are bitwise those the recomputation would give (same
// products in the same order), so the results are too.
template <int K, int L, int H>
__global__ __launch_bounds__(64, 2) void k_net_vjp(const NetArgs a) {
    constexpr int D = n_feat(K, L), DP = (D + 15) / 16 * 16;
    constexpr int DT = DP / 16, HT = H / 16;
    const int lane = threadIdx.x, col = lane & 15, grp = lane >> 4;
    const int tile = blockIdx.x;
    int s = 0;
    while (s + 1 < a.S && tile >= a.tile_start[s + 1]) ++s;
    const int64_t base = (int64_t)(tile - a.tile_start[s]) * 16;
    const int64_t cnt = a.sp_off[s + 1] - a.sp_off[s];
    const bool valid = base + col < cnt;
    const int64_t me = valid ? (int64_t)a.sp_list[a.sp_off[s] + base + col] : -1;
    const float *dl = a.dact + (valid ? (a.sp_off[s] + base + col) * (2 * H) : 0);
    const float *W = a.W + (int64_t)s * a.stride;
    float gy[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int k = 4 * grp + i;
        gy[i] = (k < K && me >= 0) ? a.Gc[me * K + k] : 0.0f;
    }
    // dE/dZ2 = (W3^T dE/dy) silu'(Z2): a single 16-input chunk, fp32 from the matrix cores
    float gz2[HT][1][4];
    {
        const float4 *W3t = reinterpret_cast<const float4 *>(W + a.oW3t);
#pragma unroll
        for (int rt = 0; rt < HT; ++rt) {
            const float4 w = W3t[rt * 64 + lane];
            const float4 d = valid ? *reinterpret_cast<const float4 *>(dl + H + 16 * rt + 4 * grp)
                                   : float4{0.f, 0.f, 0.f, 0.f};
            floatx4 t = mfma4(w.x, gy[0], floatx4{0.f, 0.f, 0.f, 0.f});
            t = mfma4(w.y, gy[1], t);
            t = mfma4(w.z, gy[2], t);
            t = mfma4(w.w, gy[3], t);
            gz2[rt][0][0] = t[0] * d.x; gz2[rt][0][1] = t[1] * d.y;
            gz2[rt][0][2] = t[2] * d.z; gz2[rt][0][3] = t[3] * d.w;
        }
    }
    // dE/dZ1 = (W2^T dE/dZ2) silu'(Z1)
    double g1[HT][1][4];
    zero(g1);
    {
        const float4 *W2t = reinterpret_cast<const float4 *>(W + a.oW2t);
#pragma unroll
        for (int kt = 0; kt < HT; ++kt) gemm_step<HT, 1>(W2t, HT, kt, gz2[kt], g1, lane);
    }
    float gz1[HT][1][4];
#pragma unroll
    for (int rt = 0; rt < HT; ++rt) {
        const float4 d = valid ? *reinterpret_cast<const float4 *>(dl + 16 * rt + 4 * grp) : float4{0.f, 0.f, 0.f, 0.f};
        gz1[rt][0][0] = (float)g1[rt][0][0] * d.x; gz1[rt][0][1] = (float)g1[rt][0][1] * d.y;
        gz1[rt][0][2] = (float)g1[rt][0][2] * d.z; gz1[rt][0][3] = (float)g1[rt][0][3] * d.w;
    }
    // dE/drho = (W1^T dE/dZ1) / s_t, one 16-row tile at a time, stored as float4 row pieces
    const float4 *W1t = reinterpret_cast<const float4 *>(W + a.oW1t);
#pragma unroll 1
    for (int rt = 0; rt < DT; ++rt) {
        double gr[1][1][4];
        zero(gr);
#pragma unroll
        for (int kt = 0; kt < HT; ++kt) gemm_step<1, 1>(W1t + (size_t)rt * HT * 64, HT, kt, gz1[kt], gr, lane);
        if (me >= 0)
            *reinterpret_cast<float4 *>(a.Grho + tiled(a.np, me, 16 * rt + 4 * grp)) =
                float4{(float)(gr[0][0][0] * a.inv_scale), (float)(gr[0][0][1] * a.inv_scale),
                       (float)(gr[0][0][2] * a.inv_scale), (float)(gr[0][0][3] * a.inv_scale)};
    }
}

// ---- accurate mode: the same networks with fp64 operands on the fp64 matrix cores ----
// v_mfma_f64_16x16x4f64 takes its A and B operands like the fp32 instruction (lane l: A row l%16,
// B column l%16, k-step l/16) but returns row (l/16) + 4 r of column l%16 in accumulator item r
// (the fp32 one returns row 4 (l/16) + r).  Fed back as the next B operand, item r of a 16-row
// tile kt is then input 16 kt + 4 r + l/16, so the weights multiplying hidden activations are
// packed in that interleaved order; W1, whose B operand is a float4 of stored features
// (inputs 16 kt + 4 (l/16) + r), keeps the fp32 order.  Products and sums are exact to fp64
// rounding and the activations stay in fp64 between layers; only the stored messages, energies
// and dE/drho are rounded to fp32.
typedef double doublex4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ doublex4 mfma64(double a, double b, doublex4 c) {
    return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

template <int RT>
__device__ __forceinline__ void gemm64_step(const double *__restrict__ W, int KT, int kt, const double (&x)[4],
                                            doublex4 (&acc)[RT], int lane) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const double2 *w = reinterpret_cast<const double2 *>(W + ((size_t)(rt * KT + kt) * 64 + lane) * 4);
        const double2 w01 = w[0], w23 = w[1];
        acc[rt] = mfma64(w01.x, x[0], acc[rt]);
        acc[rt] = mfma64(w01.y, x[1], acc[rt]);
        acc[rt] = mfma64(w23.x, x[2], acc[rt]);
        acc[rt] = mfma64(w23.y, x[3], acc[rt]);
    }
}

// accumulator item r of lane group grp holds output row 16 rt + grp + 4 r
template <int RT>
__device__ __forceinline__ void init64(doublex4 (&acc)[RT], const double *__restrict__ b, int grp) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[rt][i] = b ? b[16 * rt + grp + 4 * i] : 0.0;
}

template <int K, int L, int H, int MODE>
__global__ __launch_bounds__(64, 2) void k_net64(const NetArgs a) {
    constexpr int D = n_feat(K, L), DP = (D + 15) / 16 * 16;
    constexpr int DT = DP / 16, HT = H / 16;
    const int lane = threadIdx.x, col = lane & 15, grp = lane >> 4;
    const int tile = blockIdx.x;
    int s = 0;
    while (s + 1 < a.S && tile >= a.tile_start[s + 1]) ++s;
    const int64_t base = (int64_t)(tile - a.tile_start[s]) * 16;
    const int64_t cnt = a.sp_off[s + 1] - a.sp_off[s];
    const int64_t me = (base + col < cnt) ? (int64_t)a.sp_list[a.sp_off[s] + base + col] : -1;
    const double *W = a.W64 + (int64_t)s * a.stride;
    // silu' of the first hidden layer, parked in LDS for the reverse pass (the second stays in
    // registers), so two waves fit per SIMD
    __shared__ double sd[MODE == kForward ? 1 : HT * 4][64];

    doublex4 z1[HT];
    init64(z1, W + a.ob1, grp);
#pragma unroll 1
    for (int kt = 0; kt < DT; ++kt) {
        float4 f = float4{0.f, 0.f, 0.f, 0.f};
        if (me >= 0) f = *reinterpret_cast<const float4 *>(a.F + tiled(a.np, me, 16 * kt + 4 * grp));
        const double x[4] = {f.x, f.y, f.z, f.w};
        gemm64_step<HT>(W + a.oW1, DT, kt, x, z1, lane);
    }
    double h1[HT][4];
#pragma unroll
    for (int rt = 0; rt < HT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const double z = z1[rt][i], sg = 1.0 / (1.0 + exp(-z));
            h1[rt][i] = z * sg;
            if constexpr (MODE != kForward) sd[rt * 4 + i][lane] = sg * (1.0 + z * (1.0 - sg));
        }
    doublex4 z2[HT];
    __builtin_amdgcn_sched_barrier(0);
    init64(z2, W + a.ob2, grp);
#pragma unroll
    for (int kt = 0; kt < HT; ++kt) gemm64_step<HT>(W + a.oW2, HT, kt, h1[kt], z2, lane);
    double h2[HT][4], d2[MODE == kForward ? 1 : HT][4];
#pragma unroll
    for (int rt = 0; rt < HT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const double z = z2[rt][i], sg = 1.0 / (1.0 + exp(-z));
            h2[rt][i] = z * sg;
            if constexpr (MODE != kForward) d2[rt][i] = sg * (1.0 + z * (1.0 - sg));
        }
    if constexpr (MODE != kBackward) {
        doublex4 y[1];
        init64(y, W + a.ob3, grp);
#pragma unroll
        for (int kt = 0; kt < HT; ++kt) gemm64_step<1>(W + a.oW3, HT, kt, h2[kt], y, lane);
        if (me >= 0) {
            if constexpr (MODE == kForward) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int k = grp + 4 * i;
                    if (k < K) a.c_next[me * rec_stride(K) + k] = (float)y[0][i];
                }
            } else {
                if (grp == 0) a.Ei[me] = a.e_scale64 * y[0][0];
            }
        }
    }
    if constexpr (MODE != kForward) {
        double gy[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int k = grp + 4 * i;
            if constexpr (MODE == kEnergy) gy[i] = (k == 0) ? a.e_scale64 : 0.0;
            else gy[i] = (k < K && me >= 0) ? (double)a.Gc[me * K + k] : 0.0;
        }
        doublex4 g2[HT];
        __builtin_amdgcn_sched_barrier(0);
        init64<HT>(g2, nullptr, grp);
        gemm64_step<HT>(W + a.oW3t, 1, 0, gy, g2, lane);
        double gz2[HT][4];
#pragma unroll
        for (int rt = 0; rt < HT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) gz2[rt][i] = g2[rt][i] * d2[rt][i];
        doublex4 g1[HT];
        init64<HT>(g1, nullptr, grp);
#pragma unroll
        for (int kt = 0; kt < HT; ++kt) gemm64_step<HT>(W + a.oW2t, HT, kt, gz2[kt], g1, lane);
        double gz1[HT][4];
#pragma unroll
        for (int rt = 0; rt < HT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) gz1[rt][i] = g1[rt][i] * sd[rt * 4 + i][lane];
        const double inv_scale = a.inv_scale;
#pragma unroll 1
        for (int rt = 0; rt < DT; ++rt) {
            doublex4 gr[1];
            init64<1>(gr, nullptr, grp);
#pragma unroll
            for (int kt = 0; kt < HT; ++kt)
                gemm64_step<1>(W + a.oW1t + (size_t)rt * HT * 64 * 4, HT, kt, gz1[kt], gr, lane);
            if (me >= 0)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    a.Grho[tiled(a.np, me, 16 * rt + grp + 4 * i)] = (float)(gr[0][i] * inv_scale);
        }
    }
}

// ---- bf16 mode: bf16 operands, fp32 accumulation on v_mfma_f32_16x16x32_bf16 ----
// Every fp32 operand (features, hidden activations, weights) enters as a pair of bf16 values, its
// rounding and the rounding of the remainder, and each product takes three instructions; one bf16
// per operand leaves errors of about 1e-2 of the atomic energies and forces on random networks.
// One instruction contracts 32 inputs, 8 per lane for each operand; a lane supplies the same 8
// input indices to A and B, so the products pair up whatever order the hardware sums them in.
// Lane group g = l/16 takes inputs 32 q + 4 g + j (j < 4) and 32 q + 16 + 4 g + (j - 4) (j >= 4) of
// block q: these are the accumulator items the lane holds for the 16-row tiles 2q and 2q+1, so
// hidden activations feed the next product without leaving the lane, and the stored features are
// two float4 loads (column tiles 2q and 2q+1).  Weights are packed in that order, 8 bf16 per lane.
// Features and activations are rounded to bf16 (to nearest even) where they enter a product;
// biases, accumulators, activation functions and every stored result stay fp32.  The output
// layer's VJP (16 inputs: the messages or the energy) runs in fp32, as in the fp32 networks.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ floatx4 mfma_bf16(const bf16x8 &a, const bf16x8 &b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 to_bf16x8(const float (&lo)[4], const float (&hi)[4]) {
    return bf16x8{(__bf16)lo[0], (__bf16)lo[1], (__bf16)lo[2], (__bf16)lo[3],
                  (__bf16)hi[0], (__bf16)hi[1], (__bf16)hi[2], (__bf16)hi[3]};
}

// One operand of 8 inputs as a bf16 pair: h = bf16(x), l = bf16(x - h), so x = h + l to about
// 2^-17 relative.
struct BOp {
    bf16x8 h;
    bf16x8 l;
};

__device__ __forceinline__ BOp make_op(const float (&lo)[4], const float (&hi)[4]) {
    BOp o;
    o.h = to_bf16x8(lo, hi);
    float rl[4], rh[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        rl[i] = lo[i] - (float)o.h[i];
        rh[i] = hi[i] - (float)o.h[4 + i];
    }
    o.l = to_bf16x8(rl, rh);
    return o;
}

// acc[rt][c] += W[rt][q] x[c] for a matrix packed with QT blocks of 32 columns, as
// Wl xh + Wh xl + Wh xh (the weights' remainder plane sits lo_off elements after the leading one;
// the dropped Wl xl term is below 2^-16 of the product)
template <int RT, int CT>
__device__ __forceinline__ void gemm_bf16(const uint16_t *__restrict__ W, int64_t lo_off, int QT, int q,
                                          const BOp (&x)[CT], floatx4 (&acc)[RT][CT], int lane) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const size_t o = ((size_t)(rt * QT + q) * 64 + lane) * 8;
        const bf16x8 wh = *reinterpret_cast<const bf16x8 *>(W + o);
        const bf16x8 wl = *reinterpret_cast<const bf16x8 *>(W + lo_off + o);
#pragma unroll
        for (int c = 0; c < CT; ++c) {
            acc[rt][c] = mfma_bf16(wl, x[c].h, acc[rt][c]);
            acc[rt][c] = mfma_bf16(wh, x[c].l, acc[rt][c]);
            acc[rt][c] = mfma_bf16(wh, x[c].h, acc[rt][c]);
        }
    }
}

template <int RT, int CT>
__device__ __forceinline__ void init_bias4(floatx4 (&acc)[RT][CT], const float *__restrict__ b, int grp) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float v = b ? b[16 * rt + 4 * grp + i] : 0.0f;
#pragma unroll
            for (int c = 0; c < CT; ++c) acc[rt][c][i] = v;
        }
}

template <int K, int L, int H, int MODE, int CT>
__global__ __launch_bounds__(64) void k_net16(const NetArgs a) {
    constexpr int D = n_feat(K, L), DP = (D + 15) / 16 * 16;
    constexpr int DT = DP / 16, HT = H / 16, DQ = (DT + 1) / 2, HQ = H / 32;
    const int lane = threadIdx.x, col = lane & 15, grp = lane >> 4;
    const int tile = blockIdx.x;
    int s = 0;
    while (s + 1 < a.S && tile >= a.tile_start[s + 1]) ++s;
    const int64_t base = (int64_t)(tile - a.tile_start[s]) * (16 * CT);
    const int64_t cnt = a.sp_off[s + 1] - a.sp_off[s];
    const int32_t *list = a.sp_list + a.sp_off[s];
    int64_t me[CT];
#pragma unroll
    for (int c = 0; c < CT; ++c) me[c] = (base + 16 * c + col < cnt) ? (int64_t)list[base + 16 * c + col] : -1;
    const float *Wf = a.W + (int64_t)s * a.stride;        // biases and the fp32 output-layer VJP
    const uint16_t *Wb = a.W16 + (int64_t)s * a.stride16;

    // layer 1: Z1 = W1 rho~ + b1
    floatx4 z1[HT][CT];
    init_bias4(z1, Wf + a.ob1, grp);
#pragma unroll 1
    for (int q = 0; q < DQ; ++q) {
        BOp x[CT];
#pragma unroll
        for (int c = 0; c < CT; ++c) {
            float lo[4] = {0.f, 0.f, 0.f, 0.f}, hi[4] = {0.f, 0.f, 0.f, 0.f};
            if (me[c] >= 0) {
                const float4 f = *reinterpret_cast<const float4 *>(a.F + tiled(a.np, me[c], 32 * q + 4 * grp));
                lo[0] = f.x; lo[1] = f.y; lo[2] = f.z; lo[3] = f.w;
                if (2 * q + 1 < DT) {
                    const float4 h = *reinterpret_cast<const float4 *>(a.F + tiled(a.np, me[c], 32 * q + 16 + 4 * grp));
                    hi[0] = h.x; hi[1] = h.y; hi[2] = h.z; hi[3] = h.w;
                }
            }
            x[c] = make_op(lo, hi);
        }
        gemm_bf16<HT, CT>(Wb + a.o16W1, a.o16lo, DQ, q, x, z1, lane);
    }
    __shared__ float sd1[MODE == kForward ? 1 : HT * CT * 4][64];
    float h1[HT][CT][4];
#pragma unroll
    for (int rt = 0; rt < HT; ++rt)
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float z = z1[rt][c][i];
                const float sg = sigmoid(z);
                h1[rt][c][i] = z * sg;
                if constexpr (MODE != kForward) sd1[(rt * CT + c) * 4 + i][lane] = sg * (1.0f + z * (1.0f - sg));
            }
    // layer 2
    floatx4 z2[HT][CT];
    init_bias4(z2, Wf + a.ob2, grp);
#pragma unroll
    for (int q = 0; q < HQ; ++q) {
        BOp x[CT];
#pragma unroll
        for (int c = 0; c < CT; ++c) x[c] = make_op(h1[2 * q][c], h1[2 * q + 1][c]);
        gemm_bf16<HT, CT>(Wb + a.o16W2, a.o16lo, HQ, q, x, z2, lane);
    }
    float h2[HT][CT][4], d2[MODE == kForward ? 1 : HT][CT][4];
#pragma unroll
    for (int rt = 0; rt < HT; ++rt)
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float z = z2[rt][c][i];
                const float sg = sigmoid(z);
                h2[rt][c][i] = z * sg;
                if constexpr (MODE != kForward) d2[rt][c][i] = sg * (1.0f + z * (1.0f - sg));
            }

    if constexpr (MODE != kBackward) {
        floatx4 y[1][CT];
        init_bias4(y, Wf + a.ob3, grp);
#pragma unroll
        for (int q = 0; q < HQ; ++q) {
            BOp x[CT];
#pragma unroll
            for (int c = 0; c < CT; ++c) x[c] = make_op(h2[2 * q][c], h2[2 * q + 1][c]);
            gemm_bf16<1, CT>(Wb + a.o16W3, a.o16lo, HQ, q, x, y, lane);
        }
#pragma unroll
        for (int c = 0; c < CT; ++c) {
            if (me[c] < 0) continue;
            if constexpr (MODE == kForward) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int k = 4 * grp + i;
                    if (k < K) a.c_next[me[c] * rec_stride(K) + k] = y[0][c][i];
                }
            } else {
                if (grp == 0) a.Ei[me[c]] = (double)a.e_scale * (double)y[0][c][0];
            }
        }
    }
    if constexpr (MODE != kForward) {
        float gy[CT][4];
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int k = 4 * grp + i;
                if constexpr (MODE == kEnergy) gy[c][i] = (k == 0) ? a.e_scale : 0.0f;
                else gy[c][i] = (k < K && me[c] >= 0) ? a.Gc[me[c] * K + k] : 0.0f;
            }
        float gz2[HT][CT][4];
        {
            const float4 *W3t = reinterpret_cast<const float4 *>(Wf + a.oW3t);
#pragma unroll
            for (int rt = 0; rt < HT; ++rt) {
                const float4 w = W3t[rt * 64 + lane];
#pragma unroll
                for (int c = 0; c < CT; ++c) {
                    floatx4 t = mfma4(w.x, gy[c][0], floatx4{0.f, 0.f, 0.f, 0.f});
                    t = mfma4(w.y, gy[c][1], t);
                    t = mfma4(w.z, gy[c][2], t);
                    t = mfma4(w.w, gy[c][3], t);
#pragma unroll
                    for (int i = 0; i < 4; ++i) gz2[rt][c][i] = t[i] * d2[rt][c][i];
                }
            }
        }
        floatx4 g1[HT][CT];
        init_bias4<HT, CT>(g1, nullptr, grp);
#pragma unroll
        for (int q = 0; q < HQ; ++q) {
            BOp x[CT];
#pragma unroll
            for (int c = 0; c < CT; ++c) x[c] = make_op(gz2[2 * q][c], gz2[2 * q + 1][c]);
            gemm_bf16<HT, CT>(Wb + a.o16W2t, a.o16lo, HQ, q, x, g1, lane);
        }
        BOp xb[HQ][CT];
#pragma unroll
        for (int q = 0; q < HQ; ++q)
#pragma unroll
            for (int c = 0; c < CT; ++c) {
                float lo[4], hi[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    lo[i] = g1[2 * q][c][i] * sd1[((2 * q) * CT + c) * 4 + i][lane];
                    hi[i] = g1[2 * q + 1][c][i] * sd1[((2 * q + 1) * CT + c) * 4 + i][lane];
                }
                xb[q][c] = make_op(lo, hi);
            }
        // dE/drho = (W1^T dE/dZ1) / s_t, one 16-row tile at a time
#pragma unroll 1
        for (int rt = 0; rt < DT; ++rt) {
            floatx4 gr[1][CT];
            init_bias4<1, CT>(gr, nullptr, grp);
#pragma unroll
            for (int q = 0; q < HQ; ++q)
                gemm_bf16<1, CT>(Wb + a.o16W1t + (size_t)rt * HQ * 64 * 8, a.o16lo, HQ, q, xb[q], gr, lane);
#pragma unroll
            for (int c = 0; c < CT; ++c)
                if (me[c] >= 0)
                    *reinterpret_cast<float4 *>(a.Grho + tiled(a.np, me[c], 16 * rt + 4 * grp)) =
                        float4{gr[0][c][0] * a.inv_scale, gr[0][c][1] * a.inv_scale, gr[0][c][2] * a.inv_scale,
                               gr[0][c][3] * a.inv_scale};
        }
    }
}

// atom tiles per wave: two for the 64-wide forward network (each weight load feeds both); one
// elsewhere (measured: the reverse networks lose more to occupancy than they gain)
constexpr int tiles_per_wave(int H, int mode) { return (mode == kForward && H == 64) ? 2 : 1; }
constexpr int kBf16Tiles = 2;   // atom tiles per wave of the bf16 networks (measured: 1 and 4 slower)

NetArgs make_args(Context &cx, int t, int mode) {
    NetArgs a{};
    a.W = cx.weights.as<float>() + (int64_t)t * cx.S * cx.net.stride;
    a.W64 = cx.precision == 1 ? cx.weights64.as<double>() + (int64_t)t * cx.S * cx.net.stride : nullptr;
    a.stride = (int64_t)cx.net.stride;
    a.W16 = cx.precision == 2 ? cx.weights16.as<uint16_t>() + (int64_t)t * cx.S * cx.net16.stride : nullptr;
    a.stride16 = (int64_t)cx.net16.stride;
    a.o16W1 = cx.net16.W1; a.o16W2 = cx.net16.W2; a.o16W3 = cx.net16.W3;
    a.o16W1t = cx.net16.W1t; a.o16W2t = cx.net16.W2t; a.o16lo = cx.net16.b1;
    a.oW1 = cx.net.W1; a.oW2 = cx.net.W2; a.oW3 = cx.net.W3;
    a.oW1t = cx.net.W1t; a.oW2t = cx.net.W2t; a.oW3t = cx.net.W3t;
    a.ob1 = cx.net.b1; a.ob2 = cx.net.b2; a.ob3 = cx.net.b3;
    a.S = cx.S;
    a.sp_list = cx.sp_list.as<int32_t>();
    const int per = 16 * (cx.precision == 0 ? tiles_per_wave(cx.H, mode) : cx.precision == 2 ? kBf16Tiles : 1);
    int64_t off = 0;
    int32_t tiles = 0;
    for (int s = 0; s <= cx.S; ++s) {
        a.sp_off[s] = off;
        a.tile_start[s] = tiles;
        if (s < cx.S) {
            off += cx.sp_count[s];
            tiles += (int32_t)((cx.sp_count[s] + per - 1) / per);
        }
    }
    a.np = cx.np;
    a.F = cx.feat.as<float>() + (int64_t)t * cx.np * cx.DP;
    a.Grho = cx.grho.as<float>() + (int64_t)t * cx.np * cx.DP;
    a.e_scale = (float)cx.e_scale;
    a.e_scale64 = cx.e_scale;
    a.inv_scale = cx.inv_scale_host[t];
    return a;
}

#define MPNN_NET(K_, L_, H_, MODE_, A_)                                                          \
    do {                                                                                         \
        if (cx.precision == 1) k_net64<K_, L_, H_, MODE_><<<tiles, 64, 0, cx.stream>>>(A_);     \
        else if (cx.precision == 2) k_net16<K_, L_, H_, MODE_, kBf16Tiles><<<tiles, 64, 0, cx.stream>>>(A_); \
        else if ((A_).dact && MODE_ == kBackward) k_net_vjp<K_, L_, H_><<<tiles, 64, 0, cx.stream>>>(A_); \
        else if ((A_).dact)                                                                      \
            k_net<K_, L_, H_, MODE_, tiles_per_wave(H_, MODE_), MODE_ == kForward><<<tiles, 64, 0, cx.stream>>>(A_); \
        else k_net<K_, L_, H_, MODE_, tiles_per_wave(H_, MODE_)><<<tiles, 64, 0, cx.stream>>>(A_); \
    } while (0)

#define MPNN_DISPATCH_NET(MODE_, A_)                                                                    \
    do {                                                                                                \
        const unsigned tiles = (unsigned)(A_).tile_start[cx.S];                                         \
        if (tiles == 0) return Status::ok();                                                            \
        if (cx.K == 8 && cx.L == 2 && cx.H == 64) MPNN_NET(8, 2, 64, MODE_, A_);                        \
        else if (cx.K == 8 && cx.L == 2 && cx.H == 128) MPNN_NET(8, 2, 128, MODE_, A_);                 \
        else if (cx.K == 12 && cx.L == 3 && cx.H == 128) MPNN_NET(12, 3, 128, MODE_, A_);               \
        else if (cx.K == 12 && cx.L == 3 && cx.H == 64) MPNN_NET(12, 3, 64, MODE_, A_);                 \
        else if (cx.K == 2 && cx.L == 1 && cx.H == 64) MPNN_NET(2, 1, 64, MODE_, A_);                   \
        else if (cx.K == 4 && cx.L == 2 && cx.H == 64) MPNN_NET(4, 2, 64, MODE_, A_);                   \
        else return Status::err(MPNN_E_INVALID_ARG, "unsupported (K, L, H)");                           \
        MPNN_HIP(hipGetLastError());                                                                    \
    } while (0)

// A-operand packing of W [R][C] (row-major, fp64) for Y^T = W X^T: for row tile rt, column tile
// ct, lane l, component i: W[16 rt + l%16][16 ct + 4 (l/16) + i] (zero outside R x C).
// interleaved: column 16 ct + 4 i + l/16 instead (the fp64 accumulator order, for the fp64
// weights that multiply hidden activations)
template <typename T>
void pack_a(const double *W, int R, int C, int Rp, int Cp, bool transpose, T *out, bool interleaved = false) {
    const int RT = Rp / 16, CT = Cp / 16;
    for (int rt = 0; rt < RT; ++rt)
        for (int ct = 0; ct < CT; ++ct)
            for (int l = 0; l < 64; ++l)
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * rt + (l & 15);
                    const int c = interleaved ? 16 * ct + 4 * i + (l >> 4) : 16 * ct + 4 * (l >> 4) + i;
                    double v = 0.0;
                    if (r < R && c < C) v = transpose ? W[(size_t)c * R + r] : W[(size_t)r * C + c];
                    out[(((size_t)rt * CT + ct) * 64 + l) * 4 + i] = (T)v;
                }
}

// bf16 operand packing of W [R][C] for the bf16 networks: for row tile rt, 32-column block q,
// lane l, element j: W[16 rt + l%16][32 q + 16 (j/4) + 4 (l/16) + j%4] (zero outside R x C),
// rounded to the nearest bf16 (ties to even; the weights are finite)
uint16_t bf16_bits(double v) {
    const float f = (float)v;
    uint32_t u;
    std::memcpy(&u, &f, sizeof(u));
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// part 0: the bf16 rounding of each weight; part 1: the bf16 rounding of what part 0 leaves
void pack_bf16(const double *W, int R, int C, int Rp, int Cp, bool transpose, uint16_t *out, int part) {
    const int RT = Rp / 16, QT = Cp / 32;
    for (int rt = 0; rt < RT; ++rt)
        for (int q = 0; q < QT; ++q)
            for (int l = 0; l < 64; ++l)
                for (int j = 0; j < 8; ++j) {
                    const int r = 16 * rt + (l & 15);
                    const int c = 32 * q + 16 * (j >> 2) + 4 * (l >> 4) + (j & 3);
                    double v = 0.0;
                    if (r < R && c < C) v = transpose ? W[(size_t)c * R + r] : W[(size_t)r * C + c];
                    const uint16_t hb = bf16_bits(v);
                    uint16_t bits = hb;
                    if (part == 1) {
                        const uint32_t u = (uint32_t)hb << 16;
                        float h;
                        std::memcpy(&h, &u, sizeof(h));
                        bits = bf16_bits(v - (double)h);
                    }
                    out[(((size_t)rt * QT + q) * 64 + l) * 8 + j] = bits;
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
    auto fill = [&](auto *host) {
        using T = std::remove_pointer_t<decltype(host)>;
        constexpr bool il = std::is_same<T, double>::value;   // fp64 weights: interleaved order
        const double *p = mlp;
        for (int t = 0; t < cx.T; ++t) {
            const int out = t < cx.T - 1 ? K : 1;
            for (int s = 0; s < cx.S; ++s) {
                T *blk = host + ((size_t)t * cx.S + s) * nl.stride;
                const double *W1 = p, *b1 = W1 + (size_t)H * D, *W2 = b1 + H, *b2 = W2 + (size_t)H * H;
                const double *W3 = b2 + H, *b3 = W3 + (size_t)out * H;
                p = b3 + out;
                pack_a(W1, H, D, H, DP, false, blk + nl.W1);
                pack_a(W2, H, H, H, H, false, blk + nl.W2, il);
                pack_a(W3, out, H, 16, H, false, blk + nl.W3, il);
                pack_a(W1, D, H, DP, H, true, blk + nl.W1t, il);
                pack_a(W2, H, H, H, H, true, blk + nl.W2t, il);
                pack_a(W3, H, out, H, 16, true, blk + nl.W3t, il);
                for (int h = 0; h < H; ++h) {
                    blk[nl.b1 + h] = (T)b1[h];
                    blk[nl.b2 + h] = (T)b2[h];
                }
                for (int k = 0; k < out; ++k) blk[nl.b3 + k] = (T)b3[k];
            }
        }
    };
    const size_t count = (size_t)cx.T * cx.S * nl.stride;
    std::vector<float> host(count, 0.0f);
    fill(host.data());
    MPNN_TRY(cx.grow(cx.weights, host.size() * sizeof(float)));
    MPNN_HIP(hipMemcpy(cx.weights.p, host.data(), host.size() * sizeof(float), hipMemcpyHostToDevice));
    if (cx.precision == 2) {
        NetLayout &nb = cx.net16;
        const int DQ32 = (DP + 31) / 32 * 32;
        size_t q = 0;
        nb.W1 = q; q += (size_t)H * DQ32;
        nb.W2 = q; q += (size_t)H * H;
        nb.W3 = q; q += (size_t)16 * H;
        nb.W1t = q; q += (size_t)DP * H;
        nb.W2t = q; q += (size_t)H * H;
        nb.b1 = (q + 63) / 64 * 64;                       // offset of the remainder plane
        nb.stride = 2 * nb.b1;
        std::vector<uint16_t> host16((size_t)cx.T * cx.S * nb.stride, 0);
        const double *p = mlp;
        for (int t = 0; t < cx.T; ++t) {
            const int out = t < cx.T - 1 ? K : 1;
            for (int s = 0; s < cx.S; ++s) {
                uint16_t *blk = host16.data() + ((size_t)t * cx.S + s) * nb.stride;
                const double *W1 = p, *b1 = W1 + (size_t)H * D, *W2 = b1 + H, *b2 = W2 + (size_t)H * H;
                const double *W3 = b2 + H, *b3 = W3 + (size_t)out * H;
                p = b3 + out;
                for (int part = 0; part < 2; ++part) {
                    uint16_t *b = blk + part * nb.b1;
                    pack_bf16(W1, H, D, H, DQ32, false, b + nb.W1, part);
                    pack_bf16(W2, H, H, H, H, false, b + nb.W2, part);
                    pack_bf16(W3, out, H, 16, H, false, b + nb.W3, part);
                    pack_bf16(W1, D, H, DP, H, true, b + nb.W1t, part);
                    pack_bf16(W2, H, H, H, H, true, b + nb.W2t, part);
                }
            }
        }
        MPNN_TRY(cx.grow(cx.weights16, host16.size() * sizeof(uint16_t)));
        MPNN_HIP(hipMemcpy(cx.weights16.p, host16.data(), host16.size() * sizeof(uint16_t), hipMemcpyHostToDevice));
    }
    if (cx.precision == 1) {
        std::vector<double> host64(count, 0.0);
        fill(host64.data());
        MPNN_TRY(cx.grow(cx.weights64, host64.size() * sizeof(double)));
        MPNN_HIP(hipMemcpy(cx.weights64.p, host64.data(), host64.size() * sizeof(double), hipMemcpyHostToDevice));
    }
    return Status::ok();
}

// silu' rows of message layer t saved by its forward network for its reverse network (fp32 mode;
// the other modes recompute them)
static float *saved_act(Context &cx, int t) {
    if (cx.precision != 0) return nullptr;
    return cx.dact.as<float>() + (int64_t)t * cx.n * 2 * cx.H;
}

Status mlp_forward(Context &cx, int t) {
    ProfScope ps_(cx, kProfNetForward);
    NetArgs a = make_args(cx, t, kForward);
    a.c_next = cx.c.as<float>() + (int64_t)(t + 1) * cx.NN * rec_stride(cx.K) + kRecC;
    a.dact = saved_act(cx, t);
    MPNN_DISPATCH_NET(kForward, a);
    return Status::ok();
}

Status mlp_energy(Context &cx) {
    ProfScope ps_(cx, kProfNetEnergy);
    NetArgs a = make_args(cx, cx.T - 1, kEnergy);
    a.Ei = cx.Ei.as<double>();
    MPNN_DISPATCH_NET(kEnergy, a);
    return Status::ok();
}

Status mlp_backward(Context &cx, int t) {
    ProfScope ps_(cx, kProfNetBackward);
    NetArgs a = make_args(cx, t, kBackward);
    a.Gc = cx.Gc.as<float>() + (int64_t)(t + 1) * cx.NN * cx.K;
    a.dact = saved_act(cx, t);
    MPNN_DISPATCH_NET(kBackward, a);
    return Status::ok();
}

}  // namespace mpnn
