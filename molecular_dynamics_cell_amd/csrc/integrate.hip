// Velocity-Verlet NVE integration in metal units (the paper validates REANN-MPI by NVE energy
// conservation, section "Strong Scaling"), fixed-order fp64 reductions for the energies, the
// skin test that triggers a neighbour rebuild, and caller-order <-> cell-order copies.
#include <cmath>
#include <cstring>
#include <mutex>
#include <string>

#include <algorithm>

#include "impl.h"

namespace mpnn {

namespace {

constexpr int kRedThreads = 256;
constexpr int kRedItems = 8;

// Stage 1: block b sums items [b*2048, (b+1)*2048) in a fixed tree; stage 2: one block sums the
// block partials the same way.  The result depends only on n, never on scheduling.
template <class F>
__device__ double block_sum(F item, int64_t n) {
    __shared__ double sh[kRedThreads];
    const int64_t base = (int64_t)blockIdx.x * kRedThreads * kRedItems + (int64_t)threadIdx.x * kRedItems;
    double s = 0.0;
    for (int k = 0; k < kRedItems; ++k)
        if (base + k < n) s += item(base + k);
    sh[threadIdx.x] = s;
    __syncthreads();
    for (int w = kRedThreads / 2; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) sh[threadIdx.x] += sh[threadIdx.x + w];
        __syncthreads();
    }
    return sh[0];
}

__global__ void k_sum_part(int64_t n, const double *__restrict__ x, double *__restrict__ part) {
    double s = block_sum([&](int64_t i) { return x[i]; }, n);
    if (threadIdx.x == 0) part[blockIdx.x] = s;
}

// One block: thread t sums x[t], x[t+256], ... in order, then a fixed tree over the threads.
__global__ void k_sum_double(int64_t n, const double *__restrict__ x, double *__restrict__ out) {
    __shared__ double sh[kRedThreads];
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < n; i += kRedThreads) s += x[i];
    sh[threadIdx.x] = s;
    __syncthreads();
    for (int w = kRedThreads / 2; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) sh[threadIdx.x] += sh[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) out[0] = sh[0];
}

__global__ void k_kinetic(int64_t n, const double *__restrict__ vel, const int32_t *__restrict__ types,
                          const ModelDev *__restrict__ md, double *__restrict__ part) {
    double s = block_sum(
        [&](int64_t i) {
            const double v2 = vel[3 * i] * vel[3 * i] + vel[3 * i + 1] * vel[3 * i + 1] + vel[3 * i + 2] * vel[3 * i + 2];
            return 0.5 * md->mass[types[i]] * v2 / kAccel;
        },
        n);
    if (threadIdx.x == 0) part[blockIdx.x] = s;
}

Status reduce_to_host(Context &cx, double *part, int64_t blocks, double *host) {
    double *out = part + blocks;
    k_sum_double<<<1, kRedThreads, 0, cx.stream>>>(blocks, part, out);
    MPNN_HIP(hipGetLastError());
    MPNN_HIP(hipMemcpyAsync(host, out, sizeof(double), hipMemcpyDeviceToHost, cx.stream));
    MPNN_HIP(hipStreamSynchronize(cx.stream));
    return Status::ok();
}

}  // namespace

int64_t red_blocks(int64_t n) {
    const int64_t per = (int64_t)kRedThreads * kRedItems;
    int64_t b = (n + per - 1) / per;
    return b > 0 ? b : 1;
}

namespace {

// v += (dt/2) a F / m; x += dt v; flag an atom that moved more than skin/2 since the build.
// First half-kick and drift of every atom, and the largest displacement since the last build
// (grid-stride loop; one atomic per block, so a 2M-atom step issues about 2K atomics instead of
// one per wave on the same word).
__global__ __launch_bounds__(256) void k_kick_drift(int64_t n, double dt, double half_skin2,
                                                    const int32_t *__restrict__ types,
                                                    const ModelDev *__restrict__ md, const double *__restrict__ F,
                                                    double *__restrict__ vel, double *__restrict__ pos,
                                                    const double *__restrict__ ref,
                                                    unsigned long long *__restrict__ flag) {
    double d2max = 0.0;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const double a = 0.5 * dt * kAccel / md->mass[types[i]];
        double d2 = 0.0;
        for (int c = 0; c < 3; ++c) {
            const double v = vel[3 * i + c] + a * F[3 * i + c];
            vel[3 * i + c] = v;
            const double x = pos[3 * i + c] + dt * v;
            pos[3 * i + c] = x;
            const double dd = x - ref[3 * i + c];
            d2 += dd * dd;
        }
        // a NaN displacement must trip the rebuild test: map it to +inf
        d2max = fmax(d2max, d2 == d2 ? d2 : INFINITY);
    }
    // block maximum (non-negative doubles order like their bit patterns)
    unsigned long long bits = (unsigned long long)__double_as_longlong(d2max);
    for (int o = 32; o > 0; o >>= 1) {
        const unsigned long long other = __shfl_xor(bits, o);
        bits = other > bits ? other : bits;
    }
    __shared__ unsigned long long wmax[kBlock / 64];
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = bits;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < (int)(blockDim.x >> 6); ++w) bits = wmax[w] > bits ? wmax[w] : bits;
        if (__longlong_as_double((long long)bits) > half_skin2) atomicOr(&flag[0], 1ull);
        atomicMax(&flag[1], bits);
    }
}

__global__ void k_skin_check(int64_t n, double half_skin2, const double *__restrict__ pos,
                             const double *__restrict__ ref, unsigned long long *__restrict__ flag) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    double d2 = 0.0;
    for (int c = 0; c < 3; ++c) {
        const double dd = pos[3 * i + c] - ref[3 * i + c];
        d2 += dd * dd;
    }
    if (!(d2 <= half_skin2)) atomicOr(&flag[0], 1ull);  // also catches NaN
    if (d2 == d2) atomicMax(&flag[1], (unsigned long long)__double_as_longlong(d2));
}

__global__ void k_kick(int64_t n, double dt, const int32_t *__restrict__ types, const ModelDev *__restrict__ md,
                       const double *__restrict__ F, double *__restrict__ vel) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const double a = 0.5 * dt * kAccel / md->mass[types[i]];
    for (int c = 0; c < 3; ++c) vel[3 * i + c] += a * F[3 * i + c];
}

__global__ void k_unpermute3(int64_t n, const int32_t *__restrict__ perm, const double *__restrict__ in,
                             double *__restrict__ out) {
    const int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (s >= n) return;
    const int64_t c = perm[s];
    for (int a = 0; a < 3; ++a) out[3 * c + a] = in[3 * s + a];
}

__global__ void k_permute_in3(int64_t n, const int32_t *__restrict__ perm, const double *__restrict__ in,
                              double *__restrict__ out) {
    const int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (s >= n) return;
    const int64_t c = perm[s];
    for (int a = 0; a < 3; ++a) out[3 * s + a] = in[3 * c + a];
}

__global__ void k_unpermute1(int64_t n, const int32_t *__restrict__ perm, const double *__restrict__ in,
                             double *__restrict__ out) {
    const int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (s < n) out[perm[s]] = in[s];
}

__global__ void k_unpermute_float(int64_t n, int width, int64_t np, const int32_t *__restrict__ perm,
                                  const float *__restrict__ in, double *__restrict__ out) {
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= n * width) return;
    const int64_t s = q / width;
    const int w = (int)(q - s * width);
    out[(int64_t)perm[s] * width + w] = (double)in[np > 0 ? tiled(np, s, w) : q];
}

}  // namespace

// E = sum_i E_i ([JACS] "Parallelization Algorithm", Eq. 3) in a fixed tree: block partials in
// part[0 .. red_blocks(n)), the total at part[red_blocks(n)] (no allocation, no host transfer: it runs
// inside every evaluation, also in a captured graph).  part = nullptr: the context's reduction
// buffer, sized at the neighbour build.
Status energy_reduce(Context &cx, double *part) {
    ProfScope ps_(cx, kProfReduce);
    if (cx.n == 0) return Status::ok();
    const int64_t b = red_blocks(cx.n);
    if (!part) {
        if (cx.red.bytes < sizeof(double) * (size_t)(b + 1)) return Status::err(MPNN_E_STATE, "reduction buffer not sized");
        part = cx.red.as<double>();
    }
    k_sum_part<<<(unsigned)b, kRedThreads, 0, cx.stream>>>(cx.n, cx.Ei.as<double>(), part);
    MPNN_HIP(hipGetLastError());
    k_sum_double<<<1, kRedThreads, 0, cx.stream>>>(b, part, part + b);
    MPNN_HIP(hipGetLastError());
    return Status::ok();
}

// The energy of the last evaluation (energy_reduce's result in `part`, nullptr = the context's
// buffer) copied to the host.
Status energy_sum(Context &cx, double *E_host, const double *part) {
    if (cx.n == 0) {
        *E_host = 0.0;
        return Status::ok();
    }
    if (!part) part = cx.red.as<double>();
    MPNN_HIP(hipMemcpyAsync(E_host, part + red_blocks(cx.n), sizeof(double), hipMemcpyDeviceToHost, cx.stream));
    MPNN_HIP(hipStreamSynchronize(cx.stream));
    return Status::ok();
}

// ---- fixed device scratch for mpnn_energy_forces_noalloc ----
// The reduction partials of the evaluations that may not allocate live in this file-scope device
// array: kStaticPartials block partials and the total, i.e. systems of up to
// kStaticPartials * 2,048 atoms.  Every GPU holds its own copy until the process ends; host code
// uses only the address hipGetSymbolAddress reports for the current device (the array's name is a
// host-side stand-in, not a device address).
static __device__ __align__(256) double scratch[kStaticPartials + 1];
namespace {
constexpr int kMaxDevices = 64;
double *g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mu;
}  // namespace

Status static_scratch(double **out) {
    int dev = 0;
    MPNN_HIP(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices) return Status::err(MPNN_E_INVALID_ARG, "device index out of range");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return Status::err(MPNN_E_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
        g_scratch_ptr[dev] = static_cast<double *>(p);
    }
    *out = g_scratch_ptr[dev];
    return Status::ok();
}

Status kinetic_energy(Context &cx, double *ke_host) {
    ProfScope ps_(cx, kProfReduce);
    if (cx.n == 0) {
        *ke_host = 0.0;
        return Status::ok();
    }
    // the second half of the reduction buffer (the first holds the potential energy's partials)
    const int64_t b = red_blocks(cx.n);
    if (cx.red.bytes < sizeof(double) * (size_t)(2 * b + 2)) return Status::err(MPNN_E_STATE, "reduction buffer not sized");
    double *part = cx.red.as<double>() + b + 1;
    k_kinetic<<<(unsigned)b, kRedThreads, 0, cx.stream>>>(cx.n, cx.vel.as<double>(), cx.types.as<int32_t>(),
                                                          cx.model.as<ModelDev>(), part);
    MPNN_HIP(hipGetLastError());
    return reduce_to_host(cx, part, b, ke_host);
}

Status kick_drift(Context &cx, double dt) {
    ProfScope ps_(cx, kProfKickDrift);
    if (cx.n == 0) return Status::ok();
    const double hs = 0.5 * cx.skin;
    const unsigned blocks = (unsigned)std::min<int64_t>((cx.n + kBlock - 1) / kBlock, 2048);
    k_kick_drift<<<blocks, kBlock, 0, cx.stream>>>(cx.n, dt, hs * hs, cx.types.as<int32_t>(),
                                                           cx.model.as<ModelDev>(), cx.F.as<double>(),
                                                           cx.vel.as<double>(), cx.pos.as<double>(),
                                                           cx.ref.as<double>(), cx.flag.as<unsigned long long>());
    MPNN_HIP(hipGetLastError());
    return Status::ok();
}

Status skin_check(Context &cx) {
    if (cx.n == 0) return Status::ok();
    const double hs = 0.5 * cx.skin;
    k_skin_check<<<grid_for(cx.n), kBlock, 0, cx.stream>>>(cx.n, hs * hs, cx.pos.as<double>(), cx.ref.as<double>(),
                                                           cx.flag.as<unsigned long long>());
    MPNN_HIP(hipGetLastError());
    return Status::ok();
}

Status kick(Context &cx, double dt) {
    ProfScope ps_(cx, kProfKick);
    if (cx.n == 0) return Status::ok();
    k_kick<<<grid_for(cx.n), kBlock, 0, cx.stream>>>(cx.n, dt, cx.types.as<int32_t>(), cx.model.as<ModelDev>(),
                                                     cx.F.as<double>(), cx.vel.as<double>());
    MPNN_HIP(hipGetLastError());
    return Status::ok();
}

Status reset_skin_flag(Context &cx) {
    MPNN_HIP(hipMemsetAsync(cx.flag.p, 0, sizeof(unsigned long long) * 2, cx.stream));
    return Status::ok();
}

Status read_skin_flag(Context &cx, bool *exceeded, double *max_disp) {
    unsigned long long h[2] = {0, 0};
    MPNN_HIP(hipMemcpyAsync(h, cx.flag.p, sizeof h, hipMemcpyDeviceToHost, cx.stream));
    MPNN_HIP(hipStreamSynchronize(cx.stream));
    *exceeded = h[0] != 0;
    double d2;
    std::memcpy(&d2, &h[1], sizeof d2);
    *max_disp = d2 > 0 ? sqrt(d2) : 0.0;
    return Status::ok();
}

Status unpermute_vec3(Context &cx, const double *sorted, double *caller) {
    if (cx.n == 0) return Status::ok();
    k_unpermute3<<<grid_for(cx.n), kBlock, 0, cx.stream>>>(cx.n, cx.perm.as<int32_t>(), sorted, caller);
    MPNN_HIP(hipGetLastError());
    return Status::ok();
}

Status permute_in_vec3(Context &cx, const double *caller, double *sorted) {
    if (cx.n == 0) return Status::ok();
    k_permute_in3<<<grid_for(cx.n), kBlock, 0, cx.stream>>>(cx.n, cx.perm.as<int32_t>(), caller, sorted);
    MPNN_HIP(hipGetLastError());
    return Status::ok();
}

__global__ void k_unpermute_rows(int64_t n, int width, int stride, const int32_t *__restrict__ perm,
                                 const float *__restrict__ in, double *__restrict__ out) {
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= n * width) return;
    const int64_t s = q / width;
    const int w = (int)(q - s * width);
    out[(int64_t)perm[s] * width + w] = (double)in[s * stride + w];
}

Status unpermute_rows(Context &cx, const float *sorted, int width, int stride, double *caller) {
    if (cx.n == 0) return Status::ok();
    k_unpermute_rows<<<grid_for(cx.n * width), kBlock, 0, cx.stream>>>(cx.n, width, stride, cx.perm.as<int32_t>(),
                                                                      sorted, caller);
    MPNN_HIP(hipGetLastError());
    return Status::ok();
}

Status unpermute_scalar(Context &cx, const double *sorted, double *caller) {
    if (cx.n == 0) return Status::ok();
    k_unpermute1<<<grid_for(cx.n), kBlock, 0, cx.stream>>>(cx.n, cx.perm.as<int32_t>(), sorted, caller);
    MPNN_HIP(hipGetLastError());
    return Status::ok();
}

Status unpermute_float(Context &cx, const float *sorted, int width, int64_t np, double *caller) {
    if (cx.n == 0) return Status::ok();
    k_unpermute_float<<<grid_for(cx.n * width), kBlock, 0, cx.stream>>>(cx.n, width, np, cx.perm.as<int32_t>(),
                                                                       sorted, caller);
    MPNN_HIP(hipGetLastError());
    return Status::ok();
}

}  // namespace mpnn
