/* mpnn.h -- C ABI of the REANN-style message-passing interatomic potential on MI355X (gfx950).
 *
 * The library evaluates the energy and forces of the model described in "Efficient
 * Parallelization of Message Passing Neural Network Potentials for Large-Scale Molecular
 * Dynamics" (Xia & Jiang; [JACS] below), section "REANN Architecture", Eq. 1 (embedded-atom density from
 * Gaussian-type orbital sums), Eq. 2 (messages c^t from atomic networks) and Fig. 1, with
 * forces from the reverse pass of section "Parallelization Algorithm", Eq. 3-5, on one GPU's
 * subdomain: the local atoms plus a ghost shell of periodic images, refreshed per layer
 * (Fig. 4a) and folded back to the owners in the reverse pass (Fig. 4b).
 *
 * Model (the readings this library implements):
 *   R_k(d)  = exp(-(d - mu_k)^2 / (2 sigma^2))             k = 0..K-1
 *   f_c(d)  = (1 + cos(pi d / rc)) / 2 for d < rc, else 0
 *   A_m(r)  = (x/rc)^lx (y/rc)^ly (z/rc)^lz, lx+ly+lz = l <= L, ordered by l, then lx
 *             descending, then ly descending; w_m = l! / (lx! ly! lz!)
 *   O_i[k,m] = sum_{j in N_c(i)} c_j[k] R_k(d_ij) f_c(d_ij) A_m(r_ij),  r_ij = r_j - r_i
 *   rho_i[(a,b),l] = sum_{|m|=l} w_m O_i[a,m] O_i[b,m], 0 <= a <= b < K, index
 *             l*K(K+1)/2 + (row-major rank of (a,b) in the upper triangle)
 *   c^0_i = C0[species_i]; c^{t+1}_i = MLP^t_{s_i}(rho^t_i / s_t) for t < T-1;
 *   E_i = e_scale * MLP^{T-1}_{s_i}(rho^{T-1}_i / s_{T-1}); E = sum_i E_i (fp64)
 *   MLP(x) = W3 silu(W2 silu(W1 x + b1) + b2) + b3, silu(x) = x / (1 + exp(-x))
 *   F_i = -dE/dr_i.
 *   (Contraction variant, mpnn_params.contraction: R_k replaced by sum_k' C[k][k'] R_k'.)
 *
 * Units: A, eV, fs, amu.  Arithmetic: positions, velocities and forces fp64, energy and force
 * sums fp64; the rest per mpnn_params.precision (0: fp32 orbital sums of fp64-evaluated basis
 * factors and fp32 networks on the matrix cores, 1: fp64 orbital sums and networks, 2: as 0
 * with bf16-pair network operands).
 *
 * Conventions for every call:
 *   - Array arguments are DEVICE pointers (e.g. torch tensors on the same GPU), read or
 *     written on the context's stream; scalars and `box` are host values.
 *   - The caller owns every array it passes; the library never frees caller memory.  The
 *     context owns its device scratch (hipMalloc, or the hooks of mpnn_set_allocator) and
 *     releases it in mpnn_destroy.
 *   - Atom arrays are in the caller's order; the library keeps its own locality (cell) order
 *     internally and converts on the way in and out.
 *   - Every call returns mpnn_status; on error mpnn_last_error() describes it and the
 *     context stays usable (a failed build leaves no neighbour list).
 *   - One context must not be used from two threads at once.  Results are deterministic:
 *     no floating-point atomics are used anywhere.
 */
#ifndef MPNN_H
#define MPNN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct mpnn_ctx mpnn_ctx;

typedef enum {
    MPNN_OK = 0,
    MPNN_E_INVALID_ARG = -1, /* null pointer, bad size, unsupported (K, L, H) combination */
    MPNN_E_OOM = -2,         /* device allocation failed */
    MPNN_E_HIP = -3,         /* a HIP runtime call or kernel launch failed */
    MPNN_E_CAPACITY = -4,    /* more than 2^31-1 neighbour entries or nodes */
    MPNN_E_SKIN = -5,        /* positions moved more than skin/2 and auto-rebuild is off */
    MPNN_E_NONFINITE = -6,   /* non-finite position or energy */
    MPNN_E_STATE = -7,       /* call order (e.g. energy before mpnn_build_neighbors) */
    MPNN_E_BOX = -8          /* box edge not larger than rc + skin */
} mpnn_status;

/* Model parameters, all host arrays, copied by mpnn_create (the caller keeps ownership).
 * Supported shapes: (K, L) in {(2,1), (4,2), (8,2), (12,3)}, hidden in {64, 128},
 * 1 <= T <= 8, 1 <= n_species <= 16. */
typedef struct {
    int32_t n_species;
    int32_t K;                  /* radial primitives (N_phi in the paper) */
    int32_t L;                  /* maximum angular momentum */
    int32_t T;                  /* message-passing layers */
    int32_t hidden;             /* width H of both hidden layers */
    int32_t precision;          /* arithmetic mode, which also fixes how the parameters are held:
                                   0: fp32 orbital sums and fp32 networks (fp64 accumulation of
                                      16-product chunks).  Parameters are held as fp32: mpnn_create
                                      rounds mu, c0, every network weight and bias, 1/s_t, e_scale
                                      and the contraction matrix to the nearest fp32 value, and the
                                      model evaluated is the one with those rounded parameters.
                                   1: fp64 orbital sums and fp64 networks, for force distributions
                                      with heavy tails (slower).  Every parameter is held in fp64
                                      exactly as passed (the per-layer messages and features are
                                      stored in fp32 between kernels; the reverse pass runs in fp32
                                      with fp64 force sums).
                                   2: as 0 (parameters rounded to fp32), with the networks on the
                                      bf16 matrix cores: every operand (features, weights, hidden
                                      activations) is carried as a pair of bf16 values (the bf16
                                      rounding and the bf16 rounding of the remainder), fp32
                                      accumulation; only for hidden = 64 and D <= 128
                                      (MPNN_E_INVALID_ARG otherwise); forces within 2e-3 of the RMS
                                      force of the fp64 model */
    double rc;                  /* cutoff radius, A */
    double sigma;               /* Gaussian standard deviation, A */
    const double *mu;           /* [K] radial centres, A */
    const double *c0;           /* [n_species][K] layer-0 orbital coefficients */
    const double *mlp;          /* for t in 0..T-1, for s in 0..S-1: W1[H][D], b1[H], W2[H][H],
                                   b2[H], W3[out][H], b3[out]; out = K for t < T-1, 1 for t = T-1;
                                   D = K(K+1)(L+1)/2 */
    const double *layer_scale;  /* [T] s_t */
    double e_scale;
    const double *mass;         /* [n_species] amu */
    const double *contraction;  /* [K][K] row-major or NULL.  NULL: orbital k of a neighbour uses
                                   the primitive radial Gaussian R_k (the base model).  Otherwise
                                   the contraction variant ([JACS] "REANN Architecture", where a
                                   neighbour's orbitals are built as linear combinations of the
                                   primitive Gaussians): orbital n uses sum_k C[n][k] R_k(d),
                                   one matrix for every species and layer, multiplied by the
                                   element-wise coefficient c_j[n] as before.  Non-finite entries:
                                   MPNN_E_INVALID_ARG. */
} mpnn_params;

typedef struct {
    double epot;                /* potential energy after the last step, eV */
    double ekin;                /* kinetic energy, eV */
    double temp;                /* 2 ekin / ((3N-3) kB), K */
    int64_t rebuilds;           /* neighbour-list rebuilds during the call */
    double max_disp;            /* largest displacement since a build seen in the call, A */
    int64_t steps;              /* total steps taken by this context */
} mpnn_md_stats;

typedef struct {
    int64_t n_local;            /* atoms */
    int64_t n_ghost;            /* ghost images in the shell(s) of width rc + skin */
    int64_t n_edges;            /* Verlet-list entries (d < rc + skin), receivers local */
    int64_t cells[3];           /* interior cells per axis of one subdomain (side >= rc + skin) */
    int64_t bytes_device;       /* device memory held by the context */
    int64_t row_bucketing;      /* 1: the neighbour slabs are less than 85 % full (ragged rows), so
                                   every step the row kernels take each 256-row block's rows in
                                   descending active count; 0: in order */
    int64_t n_slots;            /* neighbour storage slots: 64-row slabs, each as wide as its longest
                                   row (n_edges / n_slots is the slabs' fill) */
} mpnn_info;

/* Validates and copies the parameters, uploads the weights in the matrix-core layout.
 * No kernel runs.  *out receives the context (NULL on error). */
mpnn_status mpnn_create(const mpnn_params *p, mpnn_ctx **out);
void mpnn_destroy(mpnn_ctx *ctx);

/* Stream for every later call (a hipStream_t, e.g. torch.cuda.current_stream().cuda_stream);
 * NULL selects the null stream.  On long neighbour lists (4M entries or more) an evaluation also
 * runs one kernel on a second, library-owned stream of default priority, forked from and joined
 * back to this stream with events inside the same call, so work ordered on this stream before
 * and after a call stays ordered with all of it (also under graph capture). */
mpnn_status mpnn_set_stream(mpnn_ctx *ctx, void *hip_stream);

/* Device memory source for the buffers allocated from now on: alloc(bytes, user) returns device
 * memory usable on the context's stream (NULL = out of memory, MPNN_E_OOM), release(ptr, user)
 * takes back a pointer it returned; e.g. a framework's caching allocator.  Both NULL restores
 * hipMalloc / hipFree.  Buffers that already exist are kept and go back, when they are replaced
 * or the context is destroyed, to the allocator that made them, so the hooks and `user` must stay
 * valid until then.  The library synchronises its stream before handing a buffer back.  Passing
 * only one of the two hooks is MPNN_E_INVALID_ARG. */
mpnn_status mpnn_set_allocator(mpnn_ctx *ctx, void *(*alloc)(size_t bytes, void *user),
                               void (*release)(void *ptr, void *user), void *user);

/* Neighbour build for n atoms at `pos` ([n][3] fp64, device) with species `types` ([n] int32,
 * device) in the orthorhombic periodic box `box` (host, A).  Wraps positions into the box,
 * orders atoms by a Morton curve over cells of side >= rc + skin, builds the periodic-image
 * ghost shell of width rc + skin (paper: local and ghost atoms, Fig. 3a), the receiver-major
 * Verlet list of every pair with d^2 < (rc + skin)^2 evaluated in fp64 as
 * (dx*dx + dy*dy) + dz*dz, its sender-major transpose, and the per-species atom groups.
 * rc must equal the model's rc.  Velocities are reset to zero (see mpnn_set_state).
 * Errors: E_INVALID_ARG, E_BOX (box edge <= rc + skin), E_CAPACITY (more than 2^31 - 1 list entries
 * or slots, or more than 2^(32-b) atoms when the longest row holds up to 2^b entries: 33,554,432
 * atoms for rows of at most 128), E_OOM, E_HIP. */
mpnn_status mpnn_build_neighbors(mpnn_ctx *ctx, const double *pos, const int32_t *types,
                                 int64_t n, const double box[3], double rc, double skin);

/* Energy and forces ([JACS] "Parallelization Algorithm", Eq. 3: E is the sum of the local atoms'
 * energies E_i and F_k = -dE/dr_k; Eq. 4-5: the derivative runs back through every layer's density
 * features, orbital coefficients and messages; "REANN Architecture", Eq. 1-2, for the forward
 * model).  pos: NULL uses the context's current positions; otherwise new positions
 * ([n][3] fp64, device, caller order) replace them (if any atom moved more than skin/2 from
 * the last build the list is rebuilt first).  energy: host out (eV) or NULL; forces: device
 * out [n][3] fp64 (eV/A, caller order) or NULL; atom_energy: device out [n] fp64 or NULL.
 * Synchronizes the stream when `energy` is requested. */
mpnn_status mpnn_energy_forces(mpnn_ctx *ctx, const double *pos, double *energy, double *forces,
                               double *atom_energy);

/* The energy and forces of mpnn_energy_forces for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  Same arguments,
 * kernels and results (bitwise) as mpnn_energy_forces, but the call allocates nothing: every
 * buffer it uses was sized by the last neighbour build, and its one per-call scratch, the partial
 * sums of the fixed-order energy reduction, is a fixed device array of 16,385 doubles (128 KiB)
 * that the library holds on each GPU until the process ends.  Limits: at most 16,384 x 2,048 =
 * 33,554,432 atoms (MPNN_E_CAPACITY beyond); it never rebuilds the neighbour list: when new
 * positions moved an atom more than skin/2 since the last build it returns MPNN_E_SKIN (the
 * positions are taken, the forces are not computed, and the next mpnn_energy_forces or
 * mpnn_md_step rebuilds first); MPNN_E_STATE before a build.  The fixed array is shared by every
 * context on the GPU and keeps the last call's contents: calls that overlap on one GPU (two
 * contexts on different streams or threads) race and must be serialised by the caller.
 * `energy` (host out) synchronises the stream; otherwise the call only enqueues work, except that
 * new positions are checked against the skin with one stream synchronisation. */
mpnn_status mpnn_energy_forces_noalloc(mpnn_ctx *ctx, const double *pos, double *energy, double *forces,
                                       double *atom_energy);

/* n_steps velocity-Verlet steps of dt_fs (NVE; [JACS] "Strong Scaling" checks the parallel code by the
 * energy conservation of NVE runs; the integrator itself is not on the pages: half-kick, drift,
 * new forces, half-kick, a = F / m in A/fs^2 with 1 eV/(A amu) = 9.648533212e-3 A/fs^2).  After the
 * steps the total potential energy of the final state is summed in fixed order (fp64) on the
 * device; it is copied to the host only when stats is given.  The list is rebuilt every rebuild_every steps
 * (0: never by count) and whenever an atom has moved more than skin/2 since the last build.
 * stats: host out or NULL. */
mpnn_status mpnn_md_step(mpnn_ctx *ctx, double dt_fs, int32_t n_steps, int32_t rebuild_every,
                         mpnn_md_stats *stats);

/* MD state of the velocity-Verlet loop (positions and velocities, the system's phase-space point;
 * see mpnn_md_step).  Replace positions and/or velocities ([n][3] fp64, device, caller order;
 * either may be NULL).  New positions trigger a rebuild. */
mpnn_status mpnn_set_state(mpnn_ctx *ctx, const double *pos, const double *vel);

/* Current positions/velocities of the MD state ([n][3] fp64 device out, caller order; either may be
 * NULL; positions are wrapped into the box at the last rebuild) and the step counter (host out or
 * NULL). */
mpnn_status mpnn_get_state(mpnn_ctx *ctx, double *pos, double *vel, int64_t *step);

/* The Verlet list (the cutoff-sphere neighbours N_c(i) of "REANN Architecture", Eq. 1, widened by
 * the skin; with the periodic images that stand in for the ghost atoms of "Parallelization
 * Algorithm", Fig. 3a) as canonical tuples in caller ids: receiver i, sender j and image shift S
 * (r_ij = r_j + S*box - r_i for the wrapped positions of the last build).  Device outputs
 * i[cap], j[cap], shift[cap][3] (int32); *n_pairs (host) receives the total count; at most cap
 * entries are written. */
mpnn_status mpnn_get_pairs(mpnn_ctx *ctx, int64_t cap, int64_t *n_pairs, int32_t *i, int32_t *j,
                           int32_t *shift);

/* Per-atom intermediates of the last evaluation, fp64 device out in caller order:
 * which = 0: c^t [n][K]; 1: O^t [n][K*M]; 2: dE/dO^t [n][K*M]; 3: E_i [n] (t ignored);
 * 4: dE/dc^t [n][K] for 1 <= t < T (after the ghost->owner fold). */
mpnn_status mpnn_get_intermediate(mpnn_ctx *ctx, int32_t which, int32_t t, double *out);

mpnn_status mpnn_get_info(mpnn_ctx *ctx, mpnn_info *info);

/* Event profiler: enable != 0 resets the counters and records a hipEvent pair on the context's
 * stream around every kernel family launched afterwards; 0 stops recording.  Durations are
 * collected at the library's own synchronisation points.  The kernel on the second stream (see
 * mpnn_set_stream) is not among the families. */
mpnn_status mpnn_set_profiling(mpnn_ctx *ctx, int32_t enable);

/* Accumulated device time and launch count of kernel family idx (0 <= idx < number of families;
 * MPNN_E_INVALID_ARG past the end).  *name is a static string. */
mpnn_status mpnn_get_profile(mpnn_ctx *ctx, int32_t idx, const char **name, double *total_ms,
                             int64_t *launches);

/* Replay of mpnn_md_step in captured chunks: steps_per_replay > 0 records up to that many
 * velocity-Verlet steps (kick-drift, evaluation, kick) as one HIP graph and replays it, with one
 * host synchronisation per chunk instead of one per step and no per-kernel launch cost; 0 (the
 * default) runs every step eagerly.  Results are bitwise identical to the eager path.  A chunk
 * ends before every step whose list is rebuilt on schedule; when an atom moves more than skin/2
 * inside a chunk, the chunk is rolled back (positions, velocities, forces) and redone step by
 * step, rebuilding where needed.  The graph is recorded again after every rebuild and whenever
 * dt or the chunk length changes; chunks are not used while the event profiler is on. */
mpnn_status mpnn_set_graph_replay(mpnn_ctx *ctx, int32_t steps_per_replay);

/* Virtual spatial decomposition (paper, "Parallelization Algorithm", Fig. 3b and Fig. 4): from the
 * next mpnn_build_neighbors on, the box is split into px x py x pz equal subdomains (1 x 1 x 1, the
 * default, is the undecomposed box).  Each subdomain holds the atoms inside it plus its own ghost
 * shell: every image (another subdomain's atom, or a periodic image) within rc + skin of the
 * subdomain; its atoms' neighbour rows reference only its own atoms and ghosts, and after every
 * layer each ghost's messages are refreshed from its owner, the one-device stand-in for the
 * exchange between processes.  Energies and forces equal the undecomposed ones up to the order of
 * fp summation; only the ghost count (memory, refresh volume) grows.  Each of px, py, pz must be
 * in 1..16 (MPNN_E_INVALID_ARG otherwise); the build fails with MPNN_E_BOX when box / p is not
 * larger than rc + skin along an axis.  Invalidates the current list (MPNN_E_STATE until the
 * next build). */
mpnn_status mpnn_set_subdomains(mpnn_ctx *ctx, int32_t px, int32_t py, int32_t pz);

/* Text of the last error on this context ("" if none); valid until the next call. */
const char *mpnn_last_error(const mpnn_ctx *ctx);

#ifdef __cplusplus
}
#endif
#endif /* MPNN_H */
