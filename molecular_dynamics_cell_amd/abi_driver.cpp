// Stand-alone user of the C ABI (include/mpnn.h) with no Python and no torch: reads a model and a
// system from a binary file, runs one energy/force evaluation and a few velocity-Verlet steps on
// the GPU through the library, and writes the results.  Device memory comes from the HIP
// runtime directly.  Used by the tests to show the boundary works on its own.
//
// Input (little endian): int32 n_species, K, L, T, hidden, precision; double rc, sigma,
// e_scale, skin, dt; int32 md_steps, rebuild_every; int64 n, n_mlp; double box[3], mu[K],
// c0[S*K], mlp[n_mlp], layer_scale[T], mass[S]; double pos[n*3], vel[n*3]; int32 types[n].
// Output: double E; double F[n*3]; double E_after, ekin_after; int64 rebuilds;
// double pos_after[n*3], vel_after[n*3].
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <vector>

#include "mpnn.h"

namespace {

template <class T>
bool get(FILE *f, T *p, size_t n = 1) { return fread(p, sizeof(T), n, f) == n; }

template <class T>
void put(FILE *f, const T *p, size_t n = 1) { fwrite(p, sizeof(T), n, f); }

int fail(const char *what, mpnn_ctx *ctx = nullptr) {
    fprintf(stderr, "abi_driver: %s%s%s\n", what, ctx ? ": " : "", ctx ? mpnn_last_error(ctx) : "");
    return 1;
}

}  // namespace

int main(int argc, char **argv) {
    if (argc != 3) return fail("usage: abi_driver <input> <output>");
    FILE *f = fopen(argv[1], "rb");
    if (!f) return fail("cannot open input");
    int32_t hdr[6], steps = 0, rebuild_every = 0;
    double rc, sigma, e_scale, skin, dt, box[3];
    int64_t n = 0, n_mlp = 0;
    bool ok = get(f, hdr, 6) && get(f, &rc) && get(f, &sigma) && get(f, &e_scale) && get(f, &skin) &&
              get(f, &dt) && get(f, &steps) && get(f, &rebuild_every) && get(f, &n) && get(f, &n_mlp) &&
              get(f, box, 3);
    if (!ok) return fail("short header");
    const int S = hdr[0], K = hdr[1], T = hdr[3];
    std::vector<double> mu(K), c0((size_t)S * K), mlp((size_t)n_mlp), scale(T), mass(S);
    std::vector<double> pos((size_t)n * 3), vel((size_t)n * 3);
    std::vector<int32_t> types((size_t)n);
    ok = get(f, mu.data(), mu.size()) && get(f, c0.data(), c0.size()) && get(f, mlp.data(), mlp.size()) &&
         get(f, scale.data(), scale.size()) && get(f, mass.data(), mass.size()) &&
         get(f, pos.data(), pos.size()) && get(f, vel.data(), vel.size()) && get(f, types.data(), types.size());
    fclose(f);
    if (!ok) return fail("short body");

    mpnn_params p{};
    p.n_species = S; p.K = K; p.L = hdr[2]; p.T = T; p.hidden = hdr[4]; p.precision = hdr[5];
    p.rc = rc; p.sigma = sigma; p.mu = mu.data(); p.c0 = c0.data(); p.mlp = mlp.data();
    p.layer_scale = scale.data(); p.e_scale = e_scale; p.mass = mass.data();
    mpnn_ctx *ctx = nullptr;
    if (mpnn_create(&p, &ctx) != MPNN_OK) return fail("mpnn_create");

    double *d_pos = nullptr, *d_vel = nullptr, *d_F = nullptr;
    int32_t *d_types = nullptr;
    const size_t n1 = n > 0 ? (size_t)n : 1;
    if (hipMalloc(&d_pos, sizeof(double) * 3 * n1) != hipSuccess || hipMalloc(&d_vel, sizeof(double) * 3 * n1) != hipSuccess ||
        hipMalloc(&d_F, sizeof(double) * 3 * n1) != hipSuccess || hipMalloc(&d_types, sizeof(int32_t) * n1) != hipSuccess)
        return fail("hipMalloc");
    if (hipMemcpy(d_pos, pos.data(), sizeof(double) * 3 * n, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(d_vel, vel.data(), sizeof(double) * 3 * n, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(d_types, types.data(), sizeof(int32_t) * n, hipMemcpyHostToDevice) != hipSuccess)
        return fail("upload");

    if (mpnn_build_neighbors(ctx, d_pos, d_types, n, box, rc, skin) != MPNN_OK) return fail("build", ctx);
    double E = 0.0;
    if (mpnn_energy_forces(ctx, nullptr, &E, d_F, nullptr) != MPNN_OK) return fail("energy_forces", ctx);
    std::vector<double> F((size_t)n * 3);
    if (hipMemcpy(F.data(), d_F, sizeof(double) * 3 * n, hipMemcpyDeviceToHost) != hipSuccess) return fail("download");
    if (mpnn_set_state(ctx, nullptr, d_vel) != MPNN_OK) return fail("set_state", ctx);
    mpnn_md_stats st{};
    if (mpnn_md_step(ctx, dt, steps, rebuild_every, &st) != MPNN_OK) return fail("md_step", ctx);
    int64_t step = 0;
    if (mpnn_get_state(ctx, d_pos, d_vel, &step) != MPNN_OK) return fail("get_state", ctx);
    if (hipMemcpy(pos.data(), d_pos, sizeof(double) * 3 * n, hipMemcpyDeviceToHost) != hipSuccess ||
        hipMemcpy(vel.data(), d_vel, sizeof(double) * 3 * n, hipMemcpyDeviceToHost) != hipSuccess)
        return fail("download");
    mpnn_destroy(ctx);
    (void)hipFree(d_pos); (void)hipFree(d_vel); (void)hipFree(d_F); (void)hipFree(d_types);

    FILE *o = fopen(argv[2], "wb");
    if (!o) return fail("cannot open output");
    put(o, &E); put(o, F.data(), F.size()); put(o, &st.epot); put(o, &st.ekin); put(o, &st.rebuilds);
    put(o, pos.data(), pos.size()); put(o, vel.data(), vel.size());
    fclose(o);
    printf("abi_driver: n=%lld E=%.10f after %d steps: epot=%.10f ekin=%.10f rebuilds=%lld\n", (long long)n, E, steps,
           st.epot, st.ekin, (long long)st.rebuilds);
    return 0;
}
