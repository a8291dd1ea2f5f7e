/* Plain fp64 CPU oracle of the REANN-style MPNN potential (test infrastructure only: the
 * tests, the benchmark's CPU-baseline leg and the smoke check load it; the product never
 * does).  Every quantity is computed straight from its definition, in fp64, with one
 * OpenMP loop over atoms where rows are independent.  No blocking, fusion or reordering.
 *
 * Paper: "Efficient Parallelization of Message Passing Neural Network Potentials for
 * Large-Scale Molecular Dynamics" (Xia & Jiang).
 *   - Eq. 1 (section "REANN Architecture"): embedded-atom density from the square of the
 *     neighbour sum of c_j * G_j, weighted by the multinomial l!/(lx! ly! lz!).
 *   - Eq. 2: c_i^t = M_i^{t-1}(rho_i^{t-1}), 1 <= t <= T-1; the last atomic network gives E_i.
 *   - Eq. 3-5 (section "Parallelization Algorithm"): forces by the chain rule through rho, c
 *     and G; dc^0/dr = 0.
 *   - Fig. 3/Fig. 4: local atoms, ghost atoms, per-layer ghost-message refresh.
 * Readings of what the text leaves open (one plain choice each):
 *   R_k(d) = exp(-(d-mu_k)^2 / (2 sigma^2)); f_c(d) = (1 + cos(pi d / rc)) / 2 for d < rc;
 *   A_m(r) = (x/rc)^lx (y/rc)^ly (z/rc)^lz; rho[(a,b),l] = sum_{|m|=l} w_m O[a,m] O[b,m]
 *   over primitive pairs a <= b (dimension K(K+1)(L+1)/2 as the paper states);
 *   rho-tilde = rho / s_t; atomic networks D->H->H->out with SiLU, one per species and layer;
 *   E_i = e_scale * network output.
 * Contraction variant (section "REANN Architecture" builds a neighbour's orbitals G_j as linear
 * combinations of the primitive Gaussians and leaves the coefficients to its supporting
 * information): with a matrix C[K][K] shared by all species and layers, orbital n
 * uses the radial function sum_k C[n][k] R_k(d); the element-wise coefficient c_j[n] then
 * multiplies that contracted orbital.  C = identity is the base model.
 */
#include "orc.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_PI 3.14159265358979323846
#define ORC_KAPPA 9.648533212e-3 /* 1 eV/(A amu) in A/fs^2 */
#define ORC_KB 8.617333262e-5    /* eV/K */

typedef struct { int lx, ly, lz, l; double w; } mono_t;

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

static int n_mono(int L) { return (L + 1) * (L + 2) * (L + 3) / 6; }
static int n_feat(int K, int L) { return K * (K + 1) * (L + 1) / 2; }

static double factorial(int k) {
    double f = 1.0;
    for (int i = 2; i <= k; ++i) f *= i;
    return f;
}

/* Cartesian monomials ordered by l, then lx descending, then ly descending. */
static void mono_table(int L, mono_t *t) {
    int m = 0;
    for (int l = 0; l <= L; ++l)
        for (int lx = l; lx >= 0; --lx)
            for (int ly = l - lx; ly >= 0; --ly) {
                int lz = l - lx - ly;
                t[m].lx = lx; t[m].ly = ly; t[m].lz = lz; t[m].l = l;
                t[m].w = factorial(l) / (factorial(lx) * factorial(ly) * factorial(lz));
                ++m;
            }
}

/* feature index of the pair a <= b at angular momentum l */
static int feat_index(int K, int a, int b, int l) {
    return l * (K * (K + 1) / 2) + a * K - a * (a - 1) / 2 + (b - a);
}

static double ipow(double x, int p) {
    double r = 1.0;
    for (int i = 0; i < p; ++i) r *= x;
    return r;
}

/* ------------------------------------------------------------------------------------- */
/* wrap and pair lists                                                                     */
/* ------------------------------------------------------------------------------------- */

void orc_wrap(int64_t n, const double *pos, const double box[3], double *out) {
    for (int64_t i = 0; i < n; ++i)
        for (int a = 0; a < 3; ++a) {
            double r = pos[3 * i + a];
            double f = floor(r / box[a]);
            double t = box[a] * f;
            out[3 * i + a] = r - t;
        }
}

static double pair_d2(const double *pos, const double box[3], int64_t i, int64_t j,
                      const int s[3], double r[3]) {
    for (int a = 0; a < 3; ++a) {
        double img = pos[3 * j + a] + (double)s[a] * box[a];
        r[a] = img - pos[3 * i + a];
    }
    double xy = r[0] * r[0] + r[1] * r[1];
    return xy + r[2] * r[2];
}

int64_t orc_pairs_brute(int64_t n, const double *pos, const double box[3], double rcut,
                        int64_t cap, int32_t *pi, int32_t *pj, int32_t *ps) {
    if (n < 0 || rcut <= 0) return -1;
    int ns[3];
    for (int a = 0; a < 3; ++a) {
        if (!(box[a] > 0)) return -1;
        ns[a] = (int)ceil(rcut / box[a]);
    }
    const double rc2 = rcut * rcut;
    int64_t cnt = 0;
    for (int64_t i = 0; i < n; ++i)
        for (int64_t j = 0; j < n; ++j)
            for (int sx = -ns[0]; sx <= ns[0]; ++sx)
                for (int sy = -ns[1]; sy <= ns[1]; ++sy)
                    for (int sz = -ns[2]; sz <= ns[2]; ++sz) {
                        if (i == j && sx == 0 && sy == 0 && sz == 0) continue;
                        int s[3] = {sx, sy, sz};
                        double r[3];
                        if (pair_d2(pos, box, i, j, s, r) < rc2) {
                            if (cnt < cap) {
                                pi[cnt] = (int32_t)i; pj[cnt] = (int32_t)j;
                                ps[3 * cnt] = sx; ps[3 * cnt + 1] = sy; ps[3 * cnt + 2] = sz;
                            }
                            ++cnt;
                        }
                    }
    return cnt;
}

/* Periodic linked-cell list (cells of side >= rcut, at least 3 per axis; otherwise the
 * brute-force enumeration is used). */
int64_t orc_pairs_cell(int64_t n, const double *pos, const double box[3], double rcut,
                       int64_t cap, int32_t *pi, int32_t *pj, int32_t *ps) {
    int nc[3];
    for (int a = 0; a < 3; ++a) {
        if (!(box[a] > 0)) return -1;
        nc[a] = (int)floor(box[a] / rcut);
        if (nc[a] < 3) return orc_pairs_brute(n, pos, box, rcut, cap, pi, pj, ps);
    }
    int64_t ncell = (int64_t)nc[0] * nc[1] * nc[2];
    int64_t *head = (int64_t *)malloc(sizeof(int64_t) * ncell);
    int64_t *next = (int64_t *)malloc(sizeof(int64_t) * (n > 0 ? n : 1));
    int32_t *cell = (int32_t *)malloc(sizeof(int32_t) * 3 * (n > 0 ? n : 1));
    for (int64_t c = 0; c < ncell; ++c) head[c] = -1;
    /* insert in reverse so each cell lists atoms in ascending order */
    for (int64_t i = n - 1; i >= 0; --i) {
        int64_t lin = 0;
        for (int a = 0; a < 3; ++a) {
            int c = (int)floor(pos[3 * i + a] / box[a] * nc[a]);
            if (c < 0) c = 0;
            if (c >= nc[a]) c = nc[a] - 1;
            cell[3 * i + a] = c;
        }
        lin = ((int64_t)cell[3 * i] * nc[1] + cell[3 * i + 1]) * nc[2] + cell[3 * i + 2];
        next[i] = head[lin];
        head[lin] = i;
    }
    const double rc2 = rcut * rcut;
    int64_t cnt = 0;
    for (int64_t i = 0; i < n; ++i)
        for (int dx = -1; dx <= 1; ++dx)
            for (int dy = -1; dy <= 1; ++dy)
                for (int dz = -1; dz <= 1; ++dz) {
                    int c[3] = {cell[3 * i] + dx, cell[3 * i + 1] + dy, cell[3 * i + 2] + dz};
                    int s[3];
                    for (int a = 0; a < 3; ++a) {
                        s[a] = 0;
                        if (c[a] < 0) { c[a] += nc[a]; s[a] = -1; }
                        if (c[a] >= nc[a]) { c[a] -= nc[a]; s[a] = 1; }
                    }
                    int64_t lin = ((int64_t)c[0] * nc[1] + c[1]) * nc[2] + c[2];
                    for (int64_t j = head[lin]; j >= 0; j = next[j]) {
                        if (j == i && s[0] == 0 && s[1] == 0 && s[2] == 0) continue;
                        double r[3];
                        if (pair_d2(pos, box, i, j, s, r) < rc2) {
                            if (cnt < cap) {
                                pi[cnt] = (int32_t)i; pj[cnt] = (int32_t)j;
                                ps[3 * cnt] = s[0]; ps[3 * cnt + 1] = s[1]; ps[3 * cnt + 2] = s[2];
                            }
                            ++cnt;
                        }
                    }
                }
    free(head); free(next); free(cell);
    return cnt;
}

/* ------------------------------------------------------------------------------------- */
/* model pieces                                                                            */
/* ------------------------------------------------------------------------------------- */

typedef struct {
    int K, L, T, H, S, M, D;
    mono_t mt[64];
    const orc_model *m;
} ctx_t;

static int ctx_init(ctx_t *c, const orc_model *m) {
    if (!m || m->K < 1 || m->L < 0 || m->L > 5 || m->T < 1 || m->H < 1 || m->S < 1) return -1;
    c->m = m; c->K = m->K; c->L = m->L; c->T = m->T; c->H = m->H; c->S = m->S;
    c->M = n_mono(m->L); c->D = n_feat(m->K, m->L);
    mono_table(m->L, c->mt);
    return 0;
}

/* Weights of the atomic network of layer t, species s, and its output width. */
static const double *net_block(const ctx_t *c, int t, int s, int *out) {
    const double *p = c->m->mlp;
    for (int tt = 0; tt < c->T; ++tt) {
        int o = (tt < c->T - 1) ? c->K : 1;
        size_t sz = (size_t)c->H * c->D + c->H + (size_t)c->H * c->H + c->H + (size_t)o * c->H + o;
        for (int ss = 0; ss < c->S; ++ss) {
            if (tt == t && ss == s) { *out = o; return p; }
            p += sz;
        }
    }
    *out = 0;
    return NULL;
}

static double silu(double x) { return x / (1.0 + exp(-x)); }
static double silu_grad(double x) {
    double sg = 1.0 / (1.0 + exp(-x));
    return sg * (1.0 + x * (1.0 - sg));
}

/* y = W3 silu(W2 silu(W1 x + b1) + b2) + b3; z1, z2 receive the pre-activations. */
static void net_forward(const double *w, int D, int H, int out, const double *x,
                        double *z1, double *z2, double *y) {
    const double *W1 = w, *b1 = W1 + (size_t)H * D, *W2 = b1 + H, *b2 = W2 + (size_t)H * H;
    const double *W3 = b2 + H, *b3 = W3 + (size_t)out * H;
    double h1[512];
    for (int h = 0; h < H; ++h) {
        double s = b1[h];
        for (int q = 0; q < D; ++q) s += W1[(size_t)h * D + q] * x[q];
        z1[h] = s;
        h1[h] = silu(s);
    }
    for (int h = 0; h < H; ++h) {
        double s = b2[h];
        for (int k = 0; k < H; ++k) s += W2[(size_t)h * H + k] * h1[k];
        z2[h] = s;
    }
    for (int o = 0; o < out; ++o) {
        double s = b3[o];
        for (int h = 0; h < H; ++h) s += W3[(size_t)o * H + h] * silu(z2[h]);
        y[o] = s;
    }
}

/* gx = J^T gy of the network above, at pre-activations z1, z2. */
static void net_vjp(const double *w, int D, int H, int out, const double *z1, const double *z2,
                    const double *gy, double *gx) {
    const double *W1 = w, *b1 = W1 + (size_t)H * D, *W2 = b1 + H, *b2 = W2 + (size_t)H * H;
    const double *W3 = b2 + H;
    double gz2[512], gz1[512];
    for (int h = 0; h < H; ++h) {
        double s = 0.0;
        for (int o = 0; o < out; ++o) s += W3[(size_t)o * H + h] * gy[o];
        gz2[h] = s * silu_grad(z2[h]);
    }
    for (int k = 0; k < H; ++k) {
        double s = 0.0;
        for (int h = 0; h < H; ++h) s += W2[(size_t)h * H + k] * gz2[h];
        gz1[k] = s * silu_grad(z1[k]);
    }
    for (int q = 0; q < D; ++q) {
        double s = 0.0;
        for (int h = 0; h < H; ++h) s += W1[(size_t)h * D + q] * gz1[h];
        gx[q] = s;
    }
}

/* Radial Gaussians, cosine cutoff and scaled Cartesian monomials of one edge, with their
 * derivatives: dR = dR/dd, dfc = dfc/dd, dA[m][a] = dA_m/dr_a. */
static void edge_basis(const ctx_t *c, const double r[3], double d, double *R, double *dR,
                       double *fc, double *dfc, double *A, double *dA) {
    const orc_model *m = c->m;
    const double s2 = m->sigma * m->sigma;
    for (int k = 0; k < c->K; ++k) {
        double x = d - m->mu[k];
        R[k] = exp(-x * x / (2.0 * s2));
        if (dR) dR[k] = -x / s2 * R[k];
    }
    if (m->contraction) {   /* contracted radial functions and their derivatives */
        double Rc[32], dRc[32];
        for (int q = 0; q < c->K; ++q) {
            double a = 0.0, b = 0.0;
            for (int k = 0; k < c->K; ++k) {
                a += m->contraction[q * c->K + k] * R[k];
                if (dR) b += m->contraction[q * c->K + k] * dR[k];
            }
            Rc[q] = a;
            dRc[q] = b;
        }
        for (int q = 0; q < c->K; ++q) {
            R[q] = Rc[q];
            if (dR) dR[q] = dRc[q];
        }
    }
    *fc = 0.5 * (1.0 + cos(ORC_PI * d / m->rc));
    if (dfc) *dfc = -0.5 * ORC_PI / m->rc * sin(ORC_PI * d / m->rc);
    const double u[3] = {r[0] / m->rc, r[1] / m->rc, r[2] / m->rc};
    for (int q = 0; q < c->M; ++q) {
        const mono_t *t = &c->mt[q];
        double px = ipow(u[0], t->lx), py = ipow(u[1], t->ly), pz = ipow(u[2], t->lz);
        A[q] = px * py * pz;
        if (dA) {
            dA[3 * q + 0] = t->lx ? t->lx * ipow(u[0], t->lx - 1) * py * pz / m->rc : 0.0;
            dA[3 * q + 1] = t->ly ? t->ly * px * ipow(u[1], t->ly - 1) * pz / m->rc : 0.0;
            dA[3 * q + 2] = t->lz ? t->lz * px * py * ipow(u[2], t->lz - 1) / m->rc : 0.0;
        }
    }
}

/* rho[(a,b),l] = sum_{|m| = l} w_m O[a][m] O[b][m], a <= b (Eq. 1 with the pairwise product). */
static void rho_from_O(const ctx_t *c, const double *O, double *rho) {
    const int K = c->K, M = c->M;
    for (int l = 0; l <= c->L; ++l)
        for (int a = 0; a < K; ++a)
            for (int b = a; b < K; ++b) {
                double s = 0.0;
                for (int q = 0; q < M; ++q)
                    if (c->mt[q].l == l) s += c->mt[q].w * O[a * M + q] * O[b * M + q];
                rho[feat_index(K, a, b, l)] = s;
            }
}

/* GO = (d rho / d O)^T Grho (product rule on every term of rho_from_O). */
static void rho_vjp(const ctx_t *c, const double *O, const double *Grho, double *GO) {
    const int K = c->K, M = c->M;
    for (int i = 0; i < K * M; ++i) GO[i] = 0.0;
    for (int l = 0; l <= c->L; ++l)
        for (int a = 0; a < K; ++a)
            for (int b = a; b < K; ++b) {
                double g = Grho[feat_index(K, a, b, l)];
                for (int q = 0; q < M; ++q)
                    if (c->mt[q].l == l) {
                        GO[a * M + q] += g * c->mt[q].w * O[b * M + q];
                        GO[b * M + q] += g * c->mt[q].w * O[a * M + q];
                    }
            }
}

/* ------------------------------------------------------------------------------------- */
/* undecomposed periodic evaluation: the definition                                        */
/* ------------------------------------------------------------------------------------- */

/* CSR of edge ids grouped by key (receiver or sender), stable in edge order. */
static void group_edges(int64_t n, int64_t ne, const int32_t *key, int64_t *off, int64_t *ids) {
    for (int64_t i = 0; i <= n; ++i) off[i] = 0;
    for (int64_t e = 0; e < ne; ++e) off[key[e] + 1]++;
    for (int64_t i = 0; i < n; ++i) off[i + 1] += off[i];
    int64_t *cur = (int64_t *)malloc(sizeof(int64_t) * (n > 0 ? n : 1));
    for (int64_t i = 0; i < n; ++i) cur[i] = off[i];
    for (int64_t e = 0; e < ne; ++e) ids[cur[key[e]]++] = e;
    free(cur);
}

int orc_energy_forces(const orc_model *m, int64_t n, const double *pos, const int32_t *types,
                      const double box[3], int64_t ne, const int32_t *pi, const int32_t *pj,
                      const int32_t *ps, double *energy, double *forces, double *ei,
                      orc_dump *dump) {
    ctx_t cx;
    if (ctx_init(&cx, m) || n < 0 || ne < 0) return -1;
    const int K = cx.K, M = cx.M, D = cx.D, T = cx.T, H = cx.H, KM = K * M;
    for (int64_t i = 0; i < n; ++i)
        if (types[i] < 0 || types[i] >= cx.S) return -2;
    for (int64_t e = 0; e < ne; ++e)
        if (pi[e] < 0 || pi[e] >= n || pj[e] < 0 || pj[e] >= n) return -3;

    const size_t nn = (size_t)(n > 0 ? n : 1), nne = (size_t)(ne > 0 ? ne : 1);
    int64_t *roff = malloc(sizeof(int64_t) * (nn + 1)), *rids = malloc(sizeof(int64_t) * nne);
    int64_t *soff = malloc(sizeof(int64_t) * (nn + 1)), *sids = malloc(sizeof(int64_t) * nne);
    double *rv = malloc(sizeof(double) * 3 * nne), *dist = malloc(sizeof(double) * nne);
    char *act = malloc(nne);
    double *c = malloc(sizeof(double) * (size_t)T * nn * K);
    double *O = malloc(sizeof(double) * (size_t)T * nn * KM);
    double *GO = malloc(sizeof(double) * nn * KM);
    double *Grt = malloc(sizeof(double) * nn * D);
    double *Gc = malloc(sizeof(double) * nn * K);
    double *g = calloc(3 * nne, sizeof(double));
    double *Ei = malloc(sizeof(double) * nn);
    group_edges(n, ne, pi, roff, rids);
    group_edges(n, ne, pj, soff, sids);

    /* edge vectors r_e = (r_j + S box) - r_i and the active test d^2 < rc^2 */
    const double rc2 = m->rc * m->rc;
    for (int64_t e = 0; e < ne; ++e) {
        int s[3] = {ps[3 * e], ps[3 * e + 1], ps[3 * e + 2]};
        double d2 = pair_d2(pos, box, pi[e], pj[e], s, &rv[3 * e]);
        act[e] = d2 < rc2;
        dist[e] = sqrt(d2);
    }
    for (int64_t i = 0; i < n; ++i)
        for (int k = 0; k < K; ++k) c[(size_t)i * K + k] = m->c0[types[i] * K + k];

    /* forward: T aggregation passes, T-1 message networks, one energy network */
    for (int t = 0; t < T; ++t) {
        const double *ct = c + (size_t)t * nn * K;
        double *Ot = O + (size_t)t * nn * KM;
#pragma omp parallel for schedule(dynamic, 64)
        for (int64_t i = 0; i < n; ++i) {
            double R[32], fc, A[64], rho[4096], x[4096], z1[512], z2[512], y[64];
            double *Oi = Ot + (size_t)i * KM;
            for (int q = 0; q < KM; ++q) Oi[q] = 0.0;
            for (int64_t p = roff[i]; p < roff[i + 1]; ++p) {
                int64_t e = rids[p];
                if (!act[e]) continue;
                edge_basis(&cx, &rv[3 * e], dist[e], R, NULL, &fc, NULL, A, NULL);
                const double *cj = ct + (size_t)pj[e] * K;
                for (int k = 0; k < K; ++k) {
                    double P = cj[k] * R[k] * fc;
                    for (int q = 0; q < M; ++q) Oi[k * M + q] += P * A[q];
                }
            }
            rho_from_O(&cx, Oi, rho);
            if (dump && dump->rho)
                memcpy(dump->rho + ((size_t)t * n + i) * D, rho, sizeof(double) * D);
            for (int q = 0; q < D; ++q) x[q] = rho[q] / m->layer_scale[t];
            int out;
            const double *w = net_block(&cx, t, types[i], &out);
            net_forward(w, D, H, out, x, z1, z2, y);
            if (t < T - 1)
                for (int k = 0; k < K; ++k) c[((size_t)(t + 1) * nn + i) * K + k] = y[k];
            else
                Ei[i] = m->e_scale * y[0];
        }
    }
    double E = 0.0;
    for (int64_t i = 0; i < n; ++i) E += Ei[i];

    /* reverse (Eq. 3-5): seed dE/d rho-tilde^{T-1} = e_scale * J^T 1 */
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t i = 0; i < n; ++i) {
        double rho[4096], x[4096], z1[512], z2[512], y[64], gy = m->e_scale;
        rho_from_O(&cx, O + ((size_t)(T - 1) * nn + i) * KM, rho);
        for (int q = 0; q < D; ++q) x[q] = rho[q] / m->layer_scale[T - 1];
        int out;
        const double *w = net_block(&cx, T - 1, types[i], &out);
        net_forward(w, D, H, out, x, z1, z2, y);
        net_vjp(w, D, H, out, z1, z2, &gy, Grt + (size_t)i * D);
    }
    for (int t = T - 1; t >= 0; --t) {
        const double *ct = c + (size_t)t * nn * K;
        const double *Ot = O + (size_t)t * nn * KM;
#pragma omp parallel for schedule(dynamic, 64)
        for (int64_t i = 0; i < n; ++i) {
            double Grho[4096];
            for (int q = 0; q < D; ++q) Grho[q] = Grt[(size_t)i * D + q] / m->layer_scale[t];
            rho_vjp(&cx, Ot + (size_t)i * KM, Grho, GO + (size_t)i * KM);
        }
        if (dump && dump->GO) memcpy(dump->GO + (size_t)t * n * KM, GO, sizeof(double) * n * KM);
        /* dE/dr_e, accumulated over layers, one receiver row at a time */
#pragma omp parallel for schedule(dynamic, 64)
        for (int64_t i = 0; i < n; ++i) {
            double R[32], dR[32], fc, dfc, A[64], dA[192];
            const double *Gi = GO + (size_t)i * KM;
            for (int64_t p = roff[i]; p < roff[i + 1]; ++p) {
                int64_t e = rids[p];
                if (!act[e]) continue;
                const double *r = &rv[3 * e];
                double d = dist[e];
                edge_basis(&cx, r, d, R, dR, &fc, &dfc, A, dA);
                const double *cj = ct + (size_t)pj[e] * K;
                double s = 0.0, Q[64];
                for (int q = 0; q < M; ++q) Q[q] = 0.0;
                for (int k = 0; k < K; ++k) {
                    double u = 0.0;
                    for (int q = 0; q < M; ++q) u += Gi[k * M + q] * A[q];
                    s += cj[k] * u * (dR[k] * fc + R[k] * dfc);
                    double P = cj[k] * R[k] * fc;
                    for (int q = 0; q < M; ++q) Q[q] += P * Gi[k * M + q];
                }
                for (int a = 0; a < 3; ++a) {
                    double v = s * r[a] / d;
                    for (int q = 0; q < M; ++q) v += Q[q] * dA[3 * q + a];
                    g[3 * e + a] += v;
                }
            }
        }
        if (t >= 1) {
            /* dE/dc_j^t = sum over edges with sender j (any image) of u_k R_k f_c */
#pragma omp parallel for schedule(dynamic, 64)
            for (int64_t j = 0; j < n; ++j) {
                double R[32], fc, A[64];
                double *Gj = Gc + (size_t)j * K;
                for (int k = 0; k < K; ++k) Gj[k] = 0.0;
                for (int64_t p = soff[j]; p < soff[j + 1]; ++p) {
                    int64_t e = sids[p];
                    if (!act[e]) continue;
                    edge_basis(&cx, &rv[3 * e], dist[e], R, NULL, &fc, NULL, A, NULL);
                    const double *Gi = GO + (size_t)pi[e] * KM;
                    for (int k = 0; k < K; ++k) {
                        double u = 0.0;
                        for (int q = 0; q < M; ++q) u += Gi[k * M + q] * A[q];
                        Gj[k] += u * R[k] * fc;
                    }
                }
            }
            /* dE/d rho-tilde^{t-1} = J^T dE/dc^t (Eq. 5) */
            const double *Op = O + (size_t)(t - 1) * nn * KM;
#pragma omp parallel for schedule(dynamic, 64)
            for (int64_t j = 0; j < n; ++j) {
                double rho[4096], x[4096], z1[512], z2[512], y[64];
                rho_from_O(&cx, Op + (size_t)j * KM, rho);
                for (int q = 0; q < D; ++q) x[q] = rho[q] / m->layer_scale[t - 1];
                int out;
                const double *w = net_block(&cx, t - 1, types[j], &out);
                net_forward(w, D, H, out, x, z1, z2, y);
                net_vjp(w, D, H, out, z1, z2, Gc + (size_t)j * K, Grt + (size_t)j * D);
            }
        }
    }
    /* F_i = sum_{receiver i} dE/dr_e - sum_{sender i} dE/dr_e  (r_e = r_j + S box - r_i) */
    if (forces) {
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < n; ++i)
            for (int a = 0; a < 3; ++a) {
                double f = 0.0;
                for (int64_t p = roff[i]; p < roff[i + 1]; ++p) f += g[3 * rids[p] + a];
                for (int64_t p = soff[i]; p < soff[i + 1]; ++p) f -= g[3 * sids[p] + a];
                forces[3 * i + a] = f;
            }
    }
    if (energy) *energy = E;
    if (ei) memcpy(ei, Ei, sizeof(double) * n);
    if (dump && dump->O) memcpy(dump->O, O, sizeof(double) * (size_t)T * n * KM);
    if (dump && dump->c) memcpy(dump->c, c, sizeof(double) * (size_t)T * n * K);
    free(roff); free(rids); free(soff); free(sids); free(rv); free(dist); free(act);
    free(c); free(O); free(GO); free(Grt); free(Gc); free(g); free(Ei);
    return 0;
}

/* ------------------------------------------------------------------------------------- */
/* virtual spatial subdomains (Fig. 3 and Fig. 4 of the paper)                             */
/* ------------------------------------------------------------------------------------- */

typedef struct {
    int64_t nn;
    double *pos;            /* [nn][3] node positions (atom image) */
    int32_t *type, *atom;   /* [nn] */
    char *local, *hasrow;   /* [nn] */
    int64_t *roff;          /* [nn+1] */
    int32_t *nb;            /* sender node of each row entry */
    double *rv, *dist;      /* row-entry geometry */
    char *act;
    double *c, *O;          /* [T][nn][K], [T][nn][K*M] */
    double *Grt, *Gc, *GO;  /* [nn][D], [nn][K], [nn][K*M] */
    double *dEdr, *Ei;      /* [nn][3], [nn] */
} sub_t;

static int axis_slot(double x, double L, int P) {
    int q = (int)floor(x / L * P);
    if (q < 0) q = 0;
    if (q >= P) q = P - 1;
    return q;
}

static void sub_free(sub_t *s) {
    free(s->pos); free(s->type); free(s->atom); free(s->local); free(s->hasrow); free(s->roff);
    free(s->nb); free(s->rv); free(s->dist); free(s->act); free(s->c); free(s->O); free(s->Grt);
    free(s->Gc); free(s->GO); free(s->dEdr); free(s->Ei);
}

static void sub_build(const ctx_t *cx, sub_t *sd, int64_t n, const double *pos, const int32_t *types,
                      const double box[3], const int P[3], const int p[3], double shell,
                      double rlist, int rows_for_all) {
    double lo[3], hi[3];
    int ns[3];
    for (int a = 0; a < 3; ++a) {
        lo[a] = p[a] * box[a] / P[a];
        hi[a] = (p[a] + 1) * box[a] / P[a];
        ns[a] = (int)ceil(shell / box[a]) + 1;
    }
    int64_t cap = 1024, nn = 0;
    double *np_ = malloc(sizeof(double) * 3 * cap);
    int32_t *na = malloc(sizeof(int32_t) * cap);
    char *nl = malloc(cap);
    /* local atoms first (S = 0), then ghost images inside the shell */
    for (int pass = 0; pass < 2; ++pass)
        for (int64_t j = 0; j < n; ++j) {
            int own = 1;
            for (int a = 0; a < 3; ++a) own &= axis_slot(pos[3 * j + a], box[a], P[a]) == p[a];
            for (int sx = -ns[0]; sx <= ns[0]; ++sx)
                for (int sy = -ns[1]; sy <= ns[1]; ++sy)
                    for (int sz = -ns[2]; sz <= ns[2]; ++sz) {
                        int s[3] = {sx, sy, sz};
                        int zero = (sx == 0 && sy == 0 && sz == 0);
                        if (pass == 0 && !(own && zero)) continue;
                        if (pass == 1 && own && zero) continue;
                        double x[3];
                        int in = 1;
                        for (int a = 0; a < 3; ++a) {
                            x[a] = pos[3 * j + a] + (double)s[a] * box[a];
                            in &= (x[a] >= lo[a] - shell) && (x[a] < hi[a] + shell);
                        }
                        if (!in) continue;
                        if (nn == cap) {
                            cap *= 2;
                            np_ = realloc(np_, sizeof(double) * 3 * cap);
                            na = realloc(na, sizeof(int32_t) * cap);
                            nl = realloc(nl, cap);
                        }
                        memcpy(&np_[3 * nn], x, sizeof x);
                        na[nn] = (int32_t)j;
                        nl[nn] = (char)(pass == 0);
                        ++nn;
                    }
        }
    const int K = cx->K, KM = cx->K * cx->M, D = cx->D, T = cx->T;
    sd->nn = nn; sd->pos = np_; sd->atom = na; sd->local = nl;
    sd->type = malloc(sizeof(int32_t) * (nn ? nn : 1));
    sd->hasrow = malloc(nn ? nn : 1);
    for (int64_t a = 0; a < nn; ++a) {
        sd->type[a] = types[na[a]];
        sd->hasrow[a] = rows_for_all || nl[a];
    }
    /* rows: every other node within rlist (brute force over the subdomain's nodes) */
    const double r2 = rlist * rlist, rc2 = cx->m->rc * cx->m->rc;
    sd->roff = malloc(sizeof(int64_t) * (nn + 1));
    int64_t ecap = 4096, ne = 0;
    sd->nb = malloc(sizeof(int32_t) * ecap);
    sd->rv = malloc(sizeof(double) * 3 * ecap);
    sd->dist = malloc(sizeof(double) * ecap);
    sd->act = malloc(ecap);
    for (int64_t a = 0; a < nn; ++a) {
        sd->roff[a] = ne;
        if (!sd->hasrow[a]) continue;
        for (int64_t b = 0; b < nn; ++b) {
            if (b == a) continue;
            double r[3];
            for (int q = 0; q < 3; ++q) r[q] = np_[3 * b + q] - np_[3 * a + q];
            double xy = r[0] * r[0] + r[1] * r[1];
            double d2 = xy + r[2] * r[2];
            if (!(d2 < r2)) continue;
            if (ne == ecap) {
                ecap *= 2;
                sd->nb = realloc(sd->nb, sizeof(int32_t) * ecap);
                sd->rv = realloc(sd->rv, sizeof(double) * 3 * ecap);
                sd->dist = realloc(sd->dist, sizeof(double) * ecap);
                sd->act = realloc(sd->act, ecap);
            }
            sd->nb[ne] = (int32_t)b;
            memcpy(&sd->rv[3 * ne], r, sizeof r);
            sd->dist[ne] = sqrt(d2);
            sd->act[ne] = d2 < rc2;
            ++ne;
        }
    }
    sd->roff[nn] = ne;
    size_t m1 = nn ? (size_t)nn : 1;
    sd->c = calloc((size_t)T * m1 * K, sizeof(double));
    sd->O = calloc((size_t)T * m1 * KM, sizeof(double));
    sd->Grt = calloc(m1 * D, sizeof(double));
    sd->Gc = calloc(m1 * K, sizeof(double));
    sd->GO = calloc(m1 * KM, sizeof(double));
    sd->dEdr = calloc(m1 * 3, sizeof(double));
    sd->Ei = calloc(m1, sizeof(double));
    for (int64_t a = 0; a < nn; ++a)
        for (int k = 0; k < K; ++k) sd->c[a * K + k] = cx->m->c0[sd->type[a] * K + k];
}

/* one layer of aggregation + network for every node with a row */
static void sub_forward_layer(const ctx_t *cx, sub_t *sd, int t) {
    const int K = cx->K, M = cx->M, KM = K * M, D = cx->D, T = cx->T, H = cx->H;
    const int64_t nn = sd->nn;
    const size_t m1 = nn ? (size_t)nn : 1;
    const double *ct = sd->c + (size_t)t * m1 * K;
    for (int64_t a = 0; a < nn; ++a) {
        if (!sd->hasrow[a]) continue;
        double R[32], fc, A[64], rho[4096], x[4096], z1[512], z2[512], y[64];
        double *Oa = sd->O + ((size_t)t * m1 + a) * KM;
        for (int q = 0; q < KM; ++q) Oa[q] = 0.0;
        for (int64_t e = sd->roff[a]; e < sd->roff[a + 1]; ++e) {
            if (!sd->act[e]) continue;
            edge_basis(cx, &sd->rv[3 * e], sd->dist[e], R, NULL, &fc, NULL, A, NULL);
            const double *cb = ct + (size_t)sd->nb[e] * K;
            for (int k = 0; k < K; ++k) {
                double P = cb[k] * R[k] * fc;
                for (int q = 0; q < M; ++q) Oa[k * M + q] += P * A[q];
            }
        }
        rho_from_O(cx, Oa, rho);
        for (int q = 0; q < D; ++q) x[q] = rho[q] / cx->m->layer_scale[t];
        int out;
        const double *w = net_block(cx, t, sd->type[a], &out);
        net_forward(w, D, H, out, x, z1, z2, y);
        if (t < T - 1)
            for (int k = 0; k < K; ++k) sd->c[((size_t)(t + 1) * m1 + a) * K + k] = y[k];
        else
            sd->Ei[a] = cx->m->e_scale * y[0];
    }
}

/* dE/d rho-tilde^{t} = J^T gy for node a, network of layer t */
static void sub_net_vjp(const ctx_t *cx, sub_t *sd, int64_t a, int t, const double *gy) {
    const int KM = cx->K * cx->M, D = cx->D, H = cx->H;
    const size_t m1 = sd->nn ? (size_t)sd->nn : 1;
    double rho[4096], x[4096], z1[512], z2[512], y[64];
    rho_from_O(cx, sd->O + ((size_t)t * m1 + a) * KM, rho);
    for (int q = 0; q < D; ++q) x[q] = rho[q] / cx->m->layer_scale[t];
    int out;
    const double *w = net_block(cx, t, sd->type[a], &out);
    net_forward(w, D, H, out, x, z1, z2, y);
    net_vjp(w, D, H, out, z1, z2, gy, sd->Grt + (size_t)a * D);
}

/* reverse pass of layer t over every row: dE/dr of both ends and dE/dc of senders */
static void sub_backward_layer(const ctx_t *cx, sub_t *sd, int t) {
    const int K = cx->K, M = cx->M, KM = K * M, D = cx->D;
    const int64_t nn = sd->nn;
    const size_t m1 = nn ? (size_t)nn : 1;
    const double *ct = sd->c + (size_t)t * m1 * K;
    for (int64_t a = 0; a < nn * K; ++a) sd->Gc[a] = 0.0;
    for (int64_t a = 0; a < nn; ++a) {
        if (!sd->hasrow[a]) continue;
        double Grho[4096];
        for (int q = 0; q < D; ++q) Grho[q] = sd->Grt[(size_t)a * D + q] / cx->m->layer_scale[t];
        double *Ga = sd->GO + (size_t)a * KM;
        rho_vjp(cx, sd->O + ((size_t)t * m1 + a) * KM, Grho, Ga);
        for (int64_t e = sd->roff[a]; e < sd->roff[a + 1]; ++e) {
            if (!sd->act[e]) continue;
            double R[32], dR[32], fc, dfc, A[64], dA[192], Q[64], s = 0.0;
            const double *r = &sd->rv[3 * e];
            double d = sd->dist[e];
            int64_t b = sd->nb[e];
            edge_basis(cx, r, d, R, dR, &fc, &dfc, A, dA);
            const double *cb = ct + (size_t)b * K;
            for (int q = 0; q < M; ++q) Q[q] = 0.0;
            for (int k = 0; k < K; ++k) {
                double u = 0.0;
                for (int q = 0; q < M; ++q) u += Ga[k * M + q] * A[q];
                s += cb[k] * u * (dR[k] * fc + R[k] * dfc);
                sd->Gc[(size_t)b * K + k] += u * R[k] * fc;
                double P = cb[k] * R[k] * fc;
                for (int q = 0; q < M; ++q) Q[q] += P * Ga[k * M + q];
            }
            for (int q3 = 0; q3 < 3; ++q3) {
                double v = s * r[q3] / d;
                for (int q = 0; q < M; ++q) v += Q[q] * dA[3 * q + q3];
                sd->dEdr[3 * b + q3] += v;
                sd->dEdr[3 * a + q3] -= v;
            }
        }
    }
}

int orc_energy_forces_decomposed(const orc_model *m, int64_t n, const double *pos,
                                 const int32_t *types, const double box[3], double skin,
                                 int px, int py, int pz, double shell, int mode,
                                 double *energy, double *forces) {
    ctx_t cx;
    if (ctx_init(&cx, m) || n < 1 || px < 1 || py < 1 || pz < 1) return -1;
    if (mode != 0 && mode != 1) return -1;
    const int K = cx.K, D = cx.D, T = cx.T;
    const int P[3] = {px, py, pz};
    const int nsub = px * py * pz;
    sub_t *sd = calloc(nsub, sizeof(sub_t));
    for (int q = 0; q < nsub; ++q) {
        int p[3] = {q / (py * pz), (q / pz) % py, q % pz};
        sub_build(&cx, &sd[q], n, pos, types, box, P, p, shell, m->rc + skin, mode == 1);
    }
    double *catom = calloc((size_t)n * K, sizeof(double));
    double *gatom = calloc((size_t)n * K, sizeof(double));
    for (int t = 0; t < T; ++t) {
        for (int q = 0; q < nsub; ++q) sub_forward_layer(&cx, &sd[q], t);
        if (mode == 0 && t < T - 1) {
            /* owner -> ghost refresh of the new messages */
            for (int q = 0; q < nsub; ++q)
                for (int64_t a = 0; a < sd[q].nn; ++a)
                    if (sd[q].local[a])
                        memcpy(&catom[(size_t)sd[q].atom[a] * K],
                               &sd[q].c[((size_t)(t + 1) * sd[q].nn + a) * K], sizeof(double) * K);
            for (int q = 0; q < nsub; ++q)
                for (int64_t a = 0; a < sd[q].nn; ++a)
                    memcpy(&sd[q].c[((size_t)(t + 1) * sd[q].nn + a) * K],
                           &catom[(size_t)sd[q].atom[a] * K], sizeof(double) * K);
        }
    }
    double E = 0.0;
    for (int q = 0; q < nsub; ++q)
        for (int64_t a = 0; a < sd[q].nn; ++a)
            if (sd[q].local[a]) E += sd[q].Ei[a];
    /* seeds at the local atoms only */
    for (int q = 0; q < nsub; ++q)
        for (int64_t a = 0; a < sd[q].nn; ++a) {
            double gy = sd[q].local[a] ? m->e_scale : 0.0;
            if (sd[q].hasrow[a]) sub_net_vjp(&cx, &sd[q], a, T - 1, &gy);
        }
    for (int t = T - 1; t >= 0; --t) {
        for (int q = 0; q < nsub; ++q) sub_backward_layer(&cx, &sd[q], t);
        if (t == 0) break;
        if (mode == 0) {
            /* ghost -> owner sum of dE/dc^t, then the local atoms' network VJP */
            memset(gatom, 0, sizeof(double) * (size_t)n * K);
            for (int q = 0; q < nsub; ++q)
                for (int64_t a = 0; a < sd[q].nn; ++a)
                    for (int k = 0; k < K; ++k)
                        gatom[(size_t)sd[q].atom[a] * K + k] += sd[q].Gc[(size_t)a * K + k];
            for (int q = 0; q < nsub; ++q)
                for (int64_t a = 0; a < sd[q].nn; ++a)
                    if (sd[q].hasrow[a])
                        sub_net_vjp(&cx, &sd[q], a, t - 1, &gatom[(size_t)sd[q].atom[a] * K]);
        } else {
            for (int q = 0; q < nsub; ++q)
                for (int64_t a = 0; a < sd[q].nn; ++a)
                    if (sd[q].hasrow[a]) sub_net_vjp(&cx, &sd[q], a, t - 1, &sd[q].Gc[(size_t)a * K]);
        }
    }
    if (forces) {
        memset(forces, 0, sizeof(double) * 3 * n);
        for (int q = 0; q < nsub; ++q)
            for (int64_t a = 0; a < sd[q].nn; ++a)
                for (int c3 = 0; c3 < 3; ++c3)
                    forces[3 * sd[q].atom[a] + c3] -= sd[q].dEdr[3 * a + c3];
    }
    if (energy) *energy = E;
    for (int q = 0; q < nsub; ++q) sub_free(&sd[q]);
    free(sd); free(catom); free(gatom);
    (void)D;
    return 0;
}

/* ------------------------------------------------------------------------------------- */
/* velocity Verlet (NVE), metal units                                                      */
/* ------------------------------------------------------------------------------------- */

static int md_forces(const orc_model *m, int64_t n, const double *pos, const int32_t *types,
                     const double box[3], int64_t np_, const int32_t *pi, const int32_t *pj,
                     const int32_t *ps, double *E, double *F) {
    return orc_energy_forces(m, n, pos, types, box, np_, pi, pj, ps, E, F, NULL, NULL);
}

static int64_t md_build(int64_t n, const double *pos, const double box[3], double rcut,
                        int32_t **pi, int32_t **pj, int32_t **ps) {
    int64_t cnt = orc_pairs_cell(n, pos, box, rcut, 0, NULL, NULL, NULL);
    if (cnt < 0) return cnt;
    free(*pi); free(*pj); free(*ps);
    *pi = malloc(sizeof(int32_t) * (cnt ? cnt : 1));
    *pj = malloc(sizeof(int32_t) * (cnt ? cnt : 1));
    *ps = malloc(sizeof(int32_t) * 3 * (cnt ? cnt : 1));
    return orc_pairs_cell(n, pos, box, rcut, cnt, *pi, *pj, *ps);
}

static double kinetic(int64_t n, const double *vel, const int32_t *types, const double *masses) {
    double ke = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        double v2 = vel[3 * i] * vel[3 * i] + vel[3 * i + 1] * vel[3 * i + 1] + vel[3 * i + 2] * vel[3 * i + 2];
        ke += 0.5 * masses[types[i]] * v2 / ORC_KAPPA;
    }
    return ke;
}

int orc_md(const orc_model *m, int64_t n, double *pos, double *vel, const int32_t *types,
           const double *masses, const double box[3], double skin, double dt, int n_steps,
           int rebuild_every, double *epot_trace, double *ekin_trace, orc_md_stats *stats) {
    if (!m || n < 1 || n_steps < 0) return -1;
    const double rcut = m->rc + skin, half2 = 0.25 * skin * skin;
    int32_t *pi = NULL, *pj = NULL, *ps = NULL;
    double *F = malloc(sizeof(double) * 3 * n), *ref = malloc(sizeof(double) * 3 * n);
    double E = 0.0, maxd = 0.0;
    int64_t rebuilds = 0;
    orc_wrap(n, pos, box, pos);
    int64_t np_ = md_build(n, pos, box, rcut, &pi, &pj, &ps);
    if (np_ < 0) return -2;
    memcpy(ref, pos, sizeof(double) * 3 * n);
    int rc = md_forces(m, n, pos, types, box, np_, pi, pj, ps, &E, F);
    if (rc) return rc;
    if (epot_trace) epot_trace[0] = E;
    if (ekin_trace) ekin_trace[0] = kinetic(n, vel, types, masses);
    int since = 0;
    for (int step = 1; step <= n_steps; ++step) {
        double worst = 0.0;
        for (int64_t i = 0; i < n; ++i) {
            double a = 0.5 * dt * ORC_KAPPA / masses[types[i]];
            double d2 = 0.0;
            for (int c3 = 0; c3 < 3; ++c3) {
                vel[3 * i + c3] += a * F[3 * i + c3];
                pos[3 * i + c3] += dt * vel[3 * i + c3];
                double dd = pos[3 * i + c3] - ref[3 * i + c3];
                d2 += dd * dd;
            }
            if (d2 > worst) worst = d2;
        }
        if (sqrt(worst) > maxd) maxd = sqrt(worst);
        ++since;
        if ((rebuild_every > 0 && since >= rebuild_every) || worst > half2) {
            orc_wrap(n, pos, box, pos);
            np_ = md_build(n, pos, box, rcut, &pi, &pj, &ps);
            if (np_ < 0) return -2;
            memcpy(ref, pos, sizeof(double) * 3 * n);
            since = 0;
            ++rebuilds;
        }
        rc = md_forces(m, n, pos, types, box, np_, pi, pj, ps, &E, F);
        if (rc) return rc;
        for (int64_t i = 0; i < n; ++i) {
            double a = 0.5 * dt * ORC_KAPPA / masses[types[i]];
            for (int c3 = 0; c3 < 3; ++c3) vel[3 * i + c3] += a * F[3 * i + c3];
        }
        if (epot_trace) epot_trace[step] = E;
        if (ekin_trace) ekin_trace[step] = kinetic(n, vel, types, masses);
    }
    if (stats) {
        stats->epot = E;
        stats->ekin = kinetic(n, vel, types, masses);
        stats->temp = n > 1 ? 2.0 * stats->ekin / ((3.0 * n - 3.0) * ORC_KB) : 0.0;
        stats->rebuilds = rebuilds;
        stats->max_disp = maxd;
    }
    free(pi); free(pj); free(ps); free(F); free(ref);
    return 0;
}
