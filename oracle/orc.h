/* Plain fp64 CPU oracle of the REANN-style MPNN potential (test infrastructure only).
 *
 * Source: "Efficient Parallelization of Message Passing Neural Network Potentials for
 * Large-Scale Molecular Dynamics" (Xia & Jiang), section "REANN Architecture" (Eq. 1, 2,
 * Fig. 1) for the forward model and section "Parallelization Algorithm" (Eq. 3-5, Fig. 3,
 * Fig. 4) for the reverse pass and the spatial decomposition.  Where that text leaves a
 * detail open, the oracle takes one plain reading (radial form, cutoff function, monomial
 * scaling, MLP shape, layer scales); the GPU library implements the same readings
 * independently.  This library is only ever loaded by the tests, the benchmark's CPU
 * baseline and the smoke check; it is never part of the product path.
 */
#ifndef ORC_H
#define ORC_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int S;                      /* species */
    int K;                      /* radial primitives N_phi */
    int L;                      /* maximum angular momentum */
    int T;                      /* message-passing layers */
    int H;                      /* hidden width of every atomic network */
    double rc;                  /* cutoff radius, A */
    double sigma;               /* Gaussian standard deviation, A */
    const double *mu;           /* [K] radial centres, A */
    const double *c0;           /* [S][K] layer-0 orbital coefficients */
    const double *mlp;          /* for t, for s: W1[H][D] b1[H] W2[H][H] b2[H] W3[out][H] b3[out]; out = K (t<T-1) or 1 */
    const double *layer_scale;  /* [T] */
    double e_scale;
    const double *contraction;  /* [K][K] or NULL.  Variant: every neighbour's orbital n uses the
                                   contracted radial function sum_k C[n][k] R_k(d) in place of
                                   R_n(d); NULL is the base model (C = identity). */
} orc_model;

/* Optional per-atom intermediates, each NULL or [T][n][...] (row-major). */
typedef struct {
    double *O;     /* [T][n][K*M]  orbital sums */
    double *rho;   /* [T][n][D]    density features before scaling */
    double *c;     /* [T][n][K]    orbital coefficients entering layer t */
    double *GO;    /* [T][n][K*M]  dE/dO */
} orc_dump;

/* r <- r - L*floor(r/L) per component (no contraction). */
void orc_wrap(int64_t n, const double *pos, const double box[3], double *out);

/* Every (i, j, S) with d^2 = |(r_j + S*box) - r_i|^2 < rcut^2 and (j,S) != (i,0), where the
 * squared norm is evaluated as (dx*dx + dy*dy) + dz*dz.  Positions must be wrapped.  Returns
 * the number of pairs (writes at most cap); -1 on bad input. */
int64_t orc_pairs_brute(int64_t n, const double *pos, const double box[3], double rcut,
                        int64_t cap, int32_t *pi, int32_t *pj, int32_t *ps);
int64_t orc_pairs_cell(int64_t n, const double *pos, const double box[3], double rcut,
                       int64_t cap, int32_t *pi, int32_t *pj, int32_t *ps);

/* Energy (eV) and forces (eV/A) from a pair list built with cutoff >= rc on wrapped
 * positions.  ei [n] and dump may be NULL.  Returns 0 on success. */
int orc_energy_forces(const orc_model *m, int64_t n, const double *pos, const int32_t *types,
                      const double box[3], int64_t n_pairs, const int32_t *pi, const int32_t *pj,
                      const int32_t *ps, double *energy, double *forces, double *ei, orc_dump *dump);

/* Same model evaluated on Px*Py*Pz virtual subdomains, each holding its local atoms plus a
 * ghost shell of width `shell`.  mode 0: per-layer owner->ghost refresh of c and ghost->owner
 * sum of dE/dc (the paper's scheme); mode 1: no refresh, every node of a subdomain is
 * evaluated from its own (possibly truncated) neighbour list.  Returns 0 on success. */
int orc_energy_forces_decomposed(const orc_model *m, int64_t n, const double *pos,
                                 const int32_t *types, const double box[3], double skin,
                                 int px, int py, int pz, double shell, int mode,
                                 double *energy, double *forces);

typedef struct {
    double epot, ekin, temp;
    int64_t rebuilds;
    double max_disp;
} orc_md_stats;

/* Velocity Verlet in metal units (A, fs, amu, eV).  pos/vel [n][3] are updated in place.
 * A neighbour list with cutoff rc+skin is rebuilt (and positions wrapped) every
 * `rebuild_every` steps (0: never by count) or when any atom has moved more than skin/2 since
 * the last build.  epot_trace/ekin_trace may be NULL or have n_steps+1 entries. */
int orc_md(const orc_model *m, int64_t n, double *pos, double *vel, const int32_t *types,
           const double *masses, const double box[3], double skin, double dt, int n_steps,
           int rebuild_every, double *epot_trace, double *ekin_trace, orc_md_stats *stats);

int orc_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
