// Neighbour build for one GPU's subdomain (paper, section "Parallelization Algorithm",
// Fig. 3a: each process holds its local atoms (LAs) with full neighbour lists plus ghost atoms
// (GAs) inside the cutoff of its LAs; Fig. 2: one list, built once, is reused by all T layers).
// On one GPU the subdomain is by default the whole periodic box and the ghost shell is made of
// periodic images within rc + skin of the box (a Verlet skin lets the list live for several
// steps).  The box can also be split into px x py x pz equal virtual subdomains: every subdomain
// then holds its own atoms plus its own shell of images (atoms of the other subdomains and periodic
// images) within rc + skin, its atoms' rows reference only those nodes, and the per-layer ghost
// refresh plays the part of the exchange between subdomains (Fig. 3b and Fig. 4 of the paper).
//
// Pipeline (all on the device; the host reads three counts to size arrays):
//   wrap + cell key -> counting sort by Morton cell code (ties by caller id) -> sorted state
//   -> ghost images per owner (count / scan / fill) -> bin all nodes on the extended grid
//   -> receiver rows (count / scan / fill over the 27-cell stencil, fp64 distance test)
//   -> sender-major transpose (count / scan / fill / per-segment sort by edge id)
//   -> per-species atom lists for the atomic networks.
#include <algorithm>
#include <vector>

#include <hipcub/hipcub.hpp>

#include "impl.h"

namespace mpnn {

namespace {

__device__ __forceinline__ uint32_t spread3(uint32_t v) {  // 10 bits -> every third bit
    v &= 0x3ffu;
    v = (v | (v << 16)) & 0x030000ffu;
    v = (v | (v << 8)) & 0x0300f00fu;
    v = (v | (v << 4)) & 0x030c30c3u;
    v = (v | (v << 2)) & 0x09249249u;
    return v;
}

struct Grid {
    double L[3], h[3];
    double Ls[3];   // subdomain edge L / P
    int n[3];       // interior cells per axis of one subdomain
    int P[3];       // subdomains per axis
    int morton;     // 1: Morton code of the interior cell, 0: linear index
    int64_t krange; // cell keys per subdomain
    int64_t next;   // extended cells per subdomain
};

// Subdomain slot along axis a of a wrapped coordinate (0 with one subdomain per axis), and the
// faces of slot p (0 and L with one subdomain).
__device__ __forceinline__ int sub_slot(double x, const Grid &g, int a) {
    if (g.P[a] == 1) return 0;
    int p = (int)floor(__ddiv_rn(x, g.Ls[a]));
    return p < 0 ? 0 : (p >= g.P[a] ? g.P[a] - 1 : p);
}

__device__ __forceinline__ double sub_lo(int p, const Grid &g, int a) { return (double)p * g.Ls[a]; }

__device__ __forceinline__ double sub_hi(int p, const Grid &g, int a) {
    return p == g.P[a] - 1 ? g.L[a] : (double)(p + 1) * g.Ls[a];
}

__device__ __forceinline__ int sub_index(const int (&p)[3], const Grid &g) { return (p[0] * g.P[1] + p[1]) * g.P[2] + p[2]; }

__device__ __forceinline__ void sub_coords(int q, const Grid &g, int (&p)[3]) {
    p[0] = q / (g.P[1] * g.P[2]);
    p[1] = (q / g.P[2]) % g.P[1];
    p[2] = q % g.P[2];
}

__device__ __forceinline__ double wrap1(double r, double L) {
    double f = floor(__ddiv_rn(r, L));
    return __dsub_rn(r, __dmul_rn(L, f));
}

__device__ __forceinline__ int interior_cell(double x, double h, int n) {
    int c = (int)floor(__ddiv_rn(x, h));
    return c < 0 ? 0 : (c >= n ? n - 1 : c);
}

__global__ void k_wrap_key(int64_t n, const double *__restrict__ pos_in, Grid g,
                           double *__restrict__ pos_w, int32_t *__restrict__ key) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    int c[3], p[3];
    for (int a = 0; a < 3; ++a) {
        double x = wrap1(pos_in[3 * i + a], g.L[a]);
        pos_w[3 * i + a] = x;
        p[a] = sub_slot(x, g, a);
        c[a] = interior_cell(__dsub_rn(x, sub_lo(p[a], g, a)), g.h[a], g.n[a]);
    }
    // subdomain-major, then the cell order inside the subdomain
    const int64_t k = g.morton ? (int64_t)(spread3(c[0]) << 2 | spread3(c[1]) << 1 | spread3(c[2]))
                               : (int64_t)((c[0] * g.n[1] + c[1]) * g.n[2] + c[2]);
    key[i] = (int32_t)(sub_index(p, g) * g.krange + k);
}

__global__ void k_count(int64_t n, const int32_t *__restrict__ key, int32_t *__restrict__ cnt) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) atomicAdd(&cnt[key[i]], 1);
}

__global__ void k_scatter(int64_t n, const int32_t *__restrict__ key, const int64_t *__restrict__ off,
                          int32_t *__restrict__ cursor, int32_t *__restrict__ out) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) {
        int32_t k = key[i];
        out[off[k] + atomicAdd(&cursor[k], 1)] = (int32_t)i;
    }
}

// Each segment (one key) sorted ascending, which makes the scatter order-independent.
__global__ void k_sort_segments(int64_t nseg, const int64_t *__restrict__ off, int32_t *__restrict__ v) {
    int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (s >= nseg) return;
    int64_t b = off[s], e = off[s + 1];
    for (int64_t p = b + 1; p < e; ++p) {
        int32_t x = v[p];
        int64_t q = p - 1;
        while (q >= b && v[q] > x) {
            v[q + 1] = v[q];
            --q;
        }
        v[q + 1] = x;
    }
}


// Same, carrying a payload along with the key.
__global__ void k_sort_segments_kv(int64_t nseg, const int64_t *__restrict__ off,
                                   int32_t *__restrict__ k, int32_t *__restrict__ v) {
    int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (s >= nseg) return;
    int64_t b = off[s], e = off[s + 1];
    for (int64_t p = b + 1; p < e; ++p) {
        int32_t x = k[p], y = v[p];
        int64_t q = p - 1;
        while (q >= b && k[q] > x) {
            k[q + 1] = k[q];
            v[q + 1] = v[q];
            --q;
        }
        k[q + 1] = x;
        v[q + 1] = y;
    }
}

__global__ void k_gather_sorted(int64_t n, const int32_t *__restrict__ perm,
                                const double *__restrict__ pos_w, const int32_t *__restrict__ types_in,
                                const double *__restrict__ vel_in, double *__restrict__ pos,
                                double *__restrict__ ref, int32_t *__restrict__ types,
                                double *__restrict__ vel, int32_t *__restrict__ inv_perm) {
    int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (s >= n) return;
    int32_t c = perm[s];
    inv_perm[c] = (int32_t)s;
    types[s] = types_in[c];
    for (int a = 0; a < 3; ++a) {
        double x = pos_w[3 * (int64_t)c + a];
        pos[3 * s + a] = x;
        ref[3 * s + a] = x;
        vel[3 * s + a] = vel_in ? vel_in[3 * (int64_t)c + a] : 0.0;
    }
}

// An image x + s*L (s = -1, 0, 1 per axis) belongs to the shell of subdomain q when every
// component lies in [lo_q - w, hi_q + w), unless it is the atom itself in its own subdomain
// (s = 0 and q the atom's subdomain).  With one subdomain: [-w, L + w), every s except 0.
__device__ __forceinline__ bool in_shell(const double *x, int code, int q, int own, const Grid &g, double w) {
    if (code == 13 && q == own) return false;
    int s[3], p[3];
    shift_of(code, s[0], s[1], s[2]);
    sub_coords(q, g, p);
    for (int a = 0; a < 3; ++a) {
        double y = __dadd_rn(x[a], (double)s[a] * g.L[a]);
        if (!(y >= __dsub_rn(sub_lo(p[a], g, a), w) && y < __dadd_rn(sub_hi(p[a], g, a), w))) return false;
    }
    return true;
}

__device__ __forceinline__ int own_sub(const double (&x)[3], const Grid &g) {
    int p[3];
    for (int a = 0; a < 3; ++a) p[a] = sub_slot(x[a], g, a);
    return sub_index(p, g);
}

__global__ void k_ghost_count(int64_t n, const double *__restrict__ pos, Grid g, double w,
                              int32_t *__restrict__ cnt) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const double x[3] = {pos[3 * i], pos[3 * i + 1], pos[3 * i + 2]};
    const int own = own_sub(x, g), nsub = g.P[0] * g.P[1] * g.P[2];
    int c = 0;
    for (int q = 0; q < nsub; ++q)
        for (int code = 0; code < 27; ++code)
            if (in_shell(x, code, q, own, g, w)) ++c;
    cnt[i] = c;
}

__global__ void k_ghost_fill(int64_t n, const double *__restrict__ pos, Grid g, double w,
                             const int64_t *__restrict__ off, int32_t *__restrict__ owner,
                             int32_t *__restrict__ code_out, int32_t *__restrict__ sub_out) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const double x[3] = {pos[3 * i], pos[3 * i + 1], pos[3 * i + 2]};
    const int own = own_sub(x, g), nsub = g.P[0] * g.P[1] * g.P[2];
    int64_t o = off[i];
    for (int q = 0; q < nsub; ++q)
        for (int code = 0; code < 27; ++code)
            if (in_shell(x, code, q, own, g, w)) {
                owner[o] = (int32_t)i;
                code_out[o] = code;
                sub_out[o] = q;
                ++o;
            }
}

// Ghost g = image of its owner: position owner + s*L (exactly as in the distance test).
__global__ void k_ghost_pos(int64_t G, int64_t n, const int32_t *__restrict__ owner,
                            const int32_t *__restrict__ code, Grid g, double *__restrict__ pos,
                            int32_t *__restrict__ types) {
    int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= G) return;
    int32_t o = owner[k];
    int s[3];
    shift_of(code[k], s[0], s[1], s[2]);
    for (int a = 0; a < 3; ++a) pos[3 * (n + k) + a] = __dadd_rn(pos[3 * (int64_t)o + a], (double)s[a] * g.L[a]);
    if (types) types[n + k] = types[o];
}

// Every node's position for this step: a ghost takes its owner's plus S L (as k_ghost_pos; owners
// are local atoms, which this kernel does not write), then the fp32 copy for the active-edge
// pre-test and the fp64 position in the node record of every layer.
__global__ void k_node_pos(int64_t NN, int64_t n, int T, int rs, const int32_t *__restrict__ owner,
                           const int32_t *__restrict__ code, Grid g, double *__restrict__ pos,
                           float4 *__restrict__ pos32, float *__restrict__ rec) {
    const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (v >= NN) return;
    double x, y, z;
    if (v < n) {
        x = pos[3 * v]; y = pos[3 * v + 1]; z = pos[3 * v + 2];
    } else {
        const int64_t o = owner[v - n];
        int s[3];
        shift_of(code[v - n], s[0], s[1], s[2]);
        x = __dadd_rn(pos[3 * o], (double)s[0] * g.L[0]);
        y = __dadd_rn(pos[3 * o + 1], (double)s[1] * g.L[1]);
        z = __dadd_rn(pos[3 * o + 2], (double)s[2] * g.L[2]);
        pos[3 * v] = x; pos[3 * v + 1] = y; pos[3 * v + 2] = z;
    }
    pos32[v] = float4{(float)x, (float)y, (float)z, 0.0f};
    for (int t = 0; t < T; ++t) {
        double *r = reinterpret_cast<double *>(rec + ((int64_t)t * NN + v) * rs);
        r[0] = x; r[1] = y; r[2] = z;
    }
}

__device__ __forceinline__ int ext_cell(double x, double h, int n) {
    int c = (int)floor(__ddiv_rn(x, h)) + 1;
    return c < 0 ? 0 : (c > n + 1 ? n + 1 : c);
}

// Extended cell of a node in the grid of subdomain q (a local atom's own subdomain, a ghost's
// shell), subdomain-major.
__device__ __forceinline__ int64_t ext_key(const double (&x)[3], int q, const Grid &g) {
    int p[3], c[3];
    sub_coords(q, g, p);
    for (int a = 0; a < 3; ++a) c[a] = ext_cell(__dsub_rn(x[a], sub_lo(p[a], g, a)), g.h[a], g.n[a]);
    return (int64_t)q * g.next + ((int64_t)c[0] * (g.n[1] + 2) + c[1]) * (g.n[2] + 2) + c[2];
}

__global__ void k_ext_key(int64_t NN, int64_t n, const double *__restrict__ pos, const int32_t *__restrict__ gsub,
                          Grid g, int32_t *__restrict__ key) {
    int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (v >= NN) return;
    const double x[3] = {pos[3 * v], pos[3 * v + 1], pos[3 * v + 2]};
    const int q = v < n ? own_sub(x, g) : gsub[v - n];
    key[v] = (int32_t)ext_key(x, q, g);
}

// Node positions in grid-cell order (the order of cnodes) in fp32, with the node's index in the
// fourth word: the row search reads each cell's candidates as one contiguous run.
__global__ void k_cell_pos(int64_t NN, const int32_t *__restrict__ cnodes, const double *__restrict__ pos,
                           float4 *__restrict__ cp) {
    const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (p >= NN) return;
    const int64_t v = cnodes[p];
    cp[p] = float4{(float)pos[3 * v], (float)pos[3 * v + 1], (float)pos[3 * v + 2], __int_as_float((int32_t)v)};
}

// Receiver rows: every node v != i of the 27 extended cells around local atom i with
// (dx*dx + dy*dy) + dz*dz < rcut^2 in fp64.  Cells in fixed (dx, dy, dz) order, nodes of a cell
// in ascending id, so rows are deterministic.  The test runs first on the fp32 positions: d^2 from
// them is within `band` of the fp64 value (the bound of the per-step compaction, with rcut), so
// only candidates with d^2 in [lo, hi] = rcut^2 -/+ band repeat it in fp64.
template <bool FILL>
__global__ void k_rows(int64_t n, const double *__restrict__ pos, Grid g,
                       const int64_t *__restrict__ coff, const float4 *__restrict__ cp,
                       double rcut2, float lo, float hi, int32_t *__restrict__ cnt,
                       const int64_t *__restrict__ slab_off, int32_t *__restrict__ nbr) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const double xi = pos[3 * i], yi = pos[3 * i + 1], zi = pos[3 * i + 2];
    const float xf = (float)xi, yf = (float)yi, zf = (float)zi;
    // the stencil lives in the receiver's own subdomain grid, which holds only its nodes
    const double xv[3] = {xi, yi, zi};
    const int q = own_sub(xv, g);
    int p[3];
    sub_coords(q, g, p);
    const int cx = ext_cell(__dsub_rn(xi, sub_lo(p[0], g, 0)), g.h[0], g.n[0]);
    const int cy = ext_cell(__dsub_rn(yi, sub_lo(p[1], g, 1)), g.h[1], g.n[1]);
    const int cz = ext_cell(__dsub_rn(zi, sub_lo(p[2], g, 2)), g.h[2], g.n[2]);
    const int ny = g.n[1] + 2, nz = g.n[2] + 2;
    const int64_t cell0 = (int64_t)q * g.next;
    const int64_t base = FILL ? sell_base(slab_off, i) : 0;
    int64_t o = 0;
    int32_t c = 0;
    for (int dx = -1; dx <= 1; ++dx) {
        int x = cx + dx;
        if (x < 0 || x > g.n[0] + 1) continue;
        for (int dy = -1; dy <= 1; ++dy) {
            int y = cy + dy;
            if (y < 0 || y > g.n[1] + 1) continue;
            for (int dz = -1; dz <= 1; ++dz) {
                int z = cz + dz;
                if (z < 0 || z > g.n[2] + 1) continue;
                int64_t cell = cell0 + ((int64_t)x * ny + y) * nz + z;
                for (int64_t p = coff[cell]; p < coff[cell + 1]; ++p) {
                    const float4 c4 = cp[p];
                    const int32_t v = __float_as_int(c4.w);
                    if (v == (int32_t)i) continue;
                    const float dx = c4.x - xf, dy = c4.y - yf, dz = c4.z - zf;
                    const float d2f = dx * dx + dy * dy + dz * dz;
                    bool in = d2f < lo;
                    if (!in && d2f < hi)
                        in = d2_exact(__dsub_rn(pos[3 * (int64_t)v], xi), __dsub_rn(pos[3 * (int64_t)v + 1], yi),
                                      __dsub_rn(pos[3 * (int64_t)v + 2], zi)) < rcut2;
                    if (in) {
                        if (FILL) nbr[base + kSlab * (o++)] = v;
                        else ++c;
                    }
                }
            }
        }
    }
    if (!FILL) cnt[i] = c;
}

// Sort keys of the sender-major transpose: for every neighbour slot (the slab layout, padding slots
// included) the sender node, or NN for a padding slot past its row's length; values = the slot.
// Sort keys and values of every slab slot: key = the sender (NN for padding), value = the receiver
// row and the slot's column packed as (row << jb) | column, so that the per-step map build
// (k_transpose_active) reads the row without a lookup.
__global__ void k_tkeys(int64_t nslab, int64_t n, const int64_t *__restrict__ slab_off, const int32_t *__restrict__ len,
                        const int32_t *__restrict__ nbr, uint32_t NN, int jb, uint32_t *__restrict__ keys,
                        uint32_t *__restrict__ vals) {
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // (slab, lane)
    if (q >= nslab * kSlab) return;
    const int64_t s = q / kSlab, r = q % kSlab, i = q;
    const int64_t b = slab_off[s] + r, w = (slab_off[s + 1] - slab_off[s]) / kSlab;
    const int nl = i < n ? len[i] : 0;
    for (int64_t j = 0; j < w; ++j) {
        const int64_t e = b + kSlab * j;
        keys[e] = j < nl ? (uint32_t)nbr[e] : NN;
        vals[e] = ((uint32_t)i << jb) | (uint32_t)j;
    }
}

// Segment starts from the sorted keys: t_off[v] = first position whose key is >= v (t_off[NN] = E).
__global__ void k_tsegments(int64_t E, const uint32_t *__restrict__ keys, int64_t NN, int64_t *__restrict__ t_off) {
    const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (p > E) return;
    const int64_t prev = p > 0 ? (int64_t)keys[p - 1] : -1;
    const int64_t next = p < E ? (int64_t)keys[p] : NN;
    for (int64_t v = prev + 1; v <= next; ++v) t_off[v] = p;
}

// Width of each 64-row slab (its longest row), times 64.
__global__ void k_slab_width(int64_t n, int64_t nslab, const int32_t *__restrict__ len, int32_t *__restrict__ sw) {
    int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (s >= nslab) return;
    int w = 0;
    for (int64_t i = s * kSlab; i < (s + 1) * kSlab && i < n; ++i) w = len[i] > w ? len[i] : w;
    sw[s] = w * kSlab;
}


__global__ void k_flag_species(int64_t n, const int32_t *__restrict__ types, int s, int32_t *__restrict__ f) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) f[i] = types[i] == s;
}

__global__ void k_species_scatter(int64_t n, const int32_t *__restrict__ types, int s,
                                  const int64_t *__restrict__ rank, int64_t base, int32_t *__restrict__ list) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n && types[i] == s) list[base + rank[i]] = (int32_t)i;
}

__global__ void k_c0(int64_t NN, int K, const int32_t *__restrict__ types, const ModelDev *__restrict__ md,
                     float *__restrict__ rec) {
    int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (v >= NN) return;
    int s = types[v];
    const int rs = rec_stride(K);
    for (int k = 0; k < K; ++k) rec[v * rs + kRecC + k] = md->c0[s * K + k];
}

__global__ void k_validate(int64_t n, const double *__restrict__ p, const int32_t *__restrict__ types, int S,
                           int32_t *__restrict__ bad) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < 3 * n && !isfinite(p[i])) atomicOr(bad, 1);
    if (i < n && (types[i] < 0 || types[i] >= S)) atomicOr(bad, 2);
}

__global__ void k_pairs(int64_t n, const int64_t *__restrict__ row_off, const int64_t *__restrict__ slab_off,
                        const int32_t *__restrict__ nbr, const int32_t *__restrict__ perm,
                        const int32_t *__restrict__ ghost_owner, const int32_t *__restrict__ ghost_code, int64_t cap,
                        int32_t *__restrict__ pi, int32_t *__restrict__ pj, int32_t *__restrict__ ps) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const int64_t b = sell_base(slab_off, i);
    for (int64_t e = row_off[i]; e < row_off[i + 1] && e < cap; ++e) {
        int32_t v = nbr[b + kSlab * (e - row_off[i])];
        int sx = 0, sy = 0, sz = 0;
        int32_t o = v;
        if (v >= n) {
            o = ghost_owner[v - n];
            shift_of(ghost_code[v - n], sx, sy, sz);
        }
        pi[e] = perm[i];
        pj[e] = perm[o];
        ps[3 * e] = sx; ps[3 * e + 1] = sy; ps[3 * e + 2] = sz;
    }
}

Grid make_grid(const Context &cx) {
    Grid g;
    for (int a = 0; a < 3; ++a) {
        g.L[a] = cx.box[a];
        g.h[a] = cx.hcell[a];
        g.n[a] = cx.nc[a];
        g.P[a] = cx.sub[a];
        g.Ls[a] = cx.box[a] / cx.sub[a];
    }
    int mx = cx.nc[0] > cx.nc[1] ? cx.nc[0] : cx.nc[1];
    mx = mx > cx.nc[2] ? mx : cx.nc[2];
    int bits = 0;
    while ((1 << bits) < mx) ++bits;
    int64_t cells = (int64_t)cx.nc[0] * cx.nc[1] * cx.nc[2];
    g.morton = bits <= 10 && ((int64_t)1 << (3 * bits)) <= 8 * cells;
    g.krange = g.morton ? (int64_t)1 << (3 * bits) : cells;
    g.next = (int64_t)(cx.nc[0] + 2) * (cx.nc[1] + 2) * (cx.nc[2] + 2);
    return g;
}

int64_t n_sub(const Context &cx) { return (int64_t)cx.sub[0] * cx.sub[1] * cx.sub[2]; }

// cell keys over all subdomains
int64_t key_range(const Grid &g) { return g.krange * g.P[0] * g.P[1] * g.P[2]; }

template <class T>
Status fetch(Context &cx, const T *dev, T *host) {
    MPNN_HIP(hipMemcpyAsync(host, dev, sizeof(T), hipMemcpyDeviceToHost, cx.stream));
    MPNN_HIP(hipStreamSynchronize(cx.stream));
    return Status::ok();
}

// Counting sort of `n` items by key in [0, nkeys): out_off [nkeys+1] offsets, out_items the
// item ids ordered by (key, id).
Status counting_sort(Context &cx, const int32_t *key, int64_t n, int64_t nkeys, int64_t *out_off,
                     int32_t *out_items, int32_t *cnt_scratch) {
    MPNN_HIP(hipMemsetAsync(cnt_scratch, 0, sizeof(int32_t) * (size_t)nkeys, cx.stream));
    k_count<<<grid_for(n), kBlock, 0, cx.stream>>>(n, key, cnt_scratch);
    MPNN_HIP(hipGetLastError());
    MPNN_TRY(exclusive_scan(cx, cnt_scratch, nkeys, out_off));
    MPNN_HIP(hipMemsetAsync(cnt_scratch, 0, sizeof(int32_t) * (size_t)nkeys, cx.stream));
    k_scatter<<<grid_for(n), kBlock, 0, cx.stream>>>(n, key, out_off, cnt_scratch, out_items);
    MPNN_HIP(hipGetLastError());
    k_sort_segments<<<grid_for(nkeys), kBlock, 0, cx.stream>>>(nkeys, out_off, out_items);
    MPNN_HIP(hipGetLastError());
    return Status::ok();
}

}  // namespace

Status build_neighbors(Context &cx, const double *pos_caller, const int32_t *types_caller, int64_t n,
                       const double box[3], double skin, const double *vel_caller) {
    cx.built = false;
    cx.forces_valid = false;
    cx.graph_valid = false;   // buffers and launch shapes may change
    const double w = cx.rc + skin;
    for (int a = 0; a < 3; ++a) {
        const double Ls = box[a] / cx.sub[a];   // subdomain edge (the box itself by default)
        if (!(Ls > w)) return Status::err(MPNN_E_BOX, "box edge / subdomains must exceed rc + skin");
        int c = (int)floor(Ls / (w + 1e-8));
        if (c < 1) return Status::err(MPNN_E_BOX, "box edge / subdomains must exceed rc + skin");
        cx.nc[a] = c;
        cx.hcell[a] = Ls / c;
        cx.box[a] = box[a];
    }
    cx.skin = skin;
    cx.rcut = w;
    cx.n = n;
    const Grid g = make_grid(cx);
    const int64_t nkeys = key_range(g);
    const int64_t next = g.next * n_sub(cx);   // extended cells over all subdomains
    const int64_t n1 = n > 0 ? n : 1;

    // ---- wrap, Morton order, sorted state ----
    MPNN_TRY(cx.grow(cx.tmp_a, sizeof(double) * 3 * n1));            // wrapped caller-order pos
    MPNN_TRY(cx.grow(cx.tmp_b, sizeof(int32_t) * (size_t)(n1 > next ? n1 : next) * 2));
    MPNN_TRY(cx.grow(cx.tmp_c, sizeof(int32_t) * (size_t)(nkeys > next ? nkeys : next) + 64));
    MPNN_TRY(cx.grow(cx.tmp_d, sizeof(int64_t) * (size_t)((nkeys > next ? nkeys : next) + 1)));
    double *pos_w = cx.tmp_a.as<double>();
    int32_t *key = cx.tmp_b.as<int32_t>();
    int32_t *cnt = cx.tmp_c.as<int32_t>();
    int64_t *off = cx.tmp_d.as<int64_t>();
    MPNN_TRY(cx.grow(cx.perm, sizeof(int32_t) * n1));
    MPNN_TRY(cx.grow(cx.inv_perm, sizeof(int32_t) * n1));
    MPNN_TRY(cx.grow(cx.vel, sizeof(double) * 3 * n1));
    MPNN_TRY(cx.grow(cx.ref, sizeof(double) * 3 * n1));
    MPNN_TRY(cx.grow(cx.flag, sizeof(uint64_t) * 4));
    if (n > 0) {
        MPNN_HIP(hipMemsetAsync(cx.flag.p, 0, sizeof(int32_t), cx.stream));
        k_validate<<<grid_for(3 * n), kBlock, 0, cx.stream>>>(n, pos_caller, types_caller, cx.S,
                                                              cx.flag.as<int32_t>());
        MPNN_HIP(hipGetLastError());
        int32_t bad = 0;
        MPNN_TRY(fetch(cx, cx.flag.as<int32_t>(), &bad));
        if (bad & 1) return Status::err(MPNN_E_NONFINITE, "non-finite position");
        if (bad & 2) return Status::err(MPNN_E_INVALID_ARG, "species index out of range");
    }
    cx.prof_begin(kProfBuildSort);
    k_wrap_key<<<grid_for(n), kBlock, 0, cx.stream>>>(n, pos_caller, g, pos_w, key);
    MPNN_HIP(hipGetLastError());
    MPNN_TRY(counting_sort(cx, key, n, nkeys, off, cx.perm.as<int32_t>(), cnt));

    // sorted positions go straight into the node array; ghosts are appended later
    MPNN_TRY(cx.grow(cx.types, sizeof(int32_t) * n1));
    MPNN_TRY(cx.grow(cx.pos, sizeof(double) * 3 * n1));
    k_gather_sorted<<<grid_for(n), kBlock, 0, cx.stream>>>(n, cx.perm.as<int32_t>(), pos_w, types_caller,
                                                           vel_caller, cx.pos.as<double>(), cx.ref.as<double>(),
                                                           cx.types.as<int32_t>(), cx.vel.as<double>(),
                                                           cx.inv_perm.as<int32_t>());
    MPNN_HIP(hipGetLastError());

    cx.prof_end(kProfBuildSort);

    // ---- ghost shell: images within rc + skin of the box (margin 1e-9 A) ----
    cx.prof_begin(kProfBuildGhost);
    const double wg = w + 1e-9;
    MPNN_TRY(cx.grow(cx.ghost_off, sizeof(int64_t) * (n1 + 1)));
    k_ghost_count<<<grid_for(n), kBlock, 0, cx.stream>>>(n, cx.pos.as<double>(), g, wg, key);
    MPNN_HIP(hipGetLastError());
    MPNN_TRY(exclusive_scan(cx, key, n, cx.ghost_off.as<int64_t>()));
    int64_t G = 0;
    MPNN_TRY(fetch(cx, cx.ghost_off.as<int64_t>() + n, &G));
    if (n + G > INT32_MAX) return Status::err(MPNN_E_CAPACITY, "too many nodes");
    cx.G = G;
    cx.NN = n + G;
    const int64_t NN1 = cx.NN > 0 ? cx.NN : 1;
    MPNN_TRY(cx.grow(cx.ghost_owner, sizeof(int32_t) * (G > 0 ? G : 1)));
    MPNN_TRY(cx.grow(cx.ghost_code, sizeof(int32_t) * (G > 0 ? G : 1)));
    MPNN_TRY(cx.grow(cx.ghost_sub, sizeof(int32_t) * (G > 0 ? G : 1)));
    {
        // keep sorted local state while the node arrays grow
        MPNN_TRY(cx.grow_keep(cx.pos, sizeof(double) * 3 * NN1, sizeof(double) * 3 * n1));
        MPNN_TRY(cx.grow_keep(cx.types, sizeof(int32_t) * NN1, sizeof(int32_t) * n1));
    }
    k_ghost_fill<<<grid_for(n), kBlock, 0, cx.stream>>>(n, cx.pos.as<double>(), g, wg, cx.ghost_off.as<int64_t>(),
                                                        cx.ghost_owner.as<int32_t>(), cx.ghost_code.as<int32_t>(),
                                                        cx.ghost_sub.as<int32_t>());
    MPNN_HIP(hipGetLastError());
    k_ghost_pos<<<grid_for(G), kBlock, 0, cx.stream>>>(G, n, cx.ghost_owner.as<int32_t>(), cx.ghost_code.as<int32_t>(),
                                                       g, cx.pos.as<double>(), cx.types.as<int32_t>());
    MPNN_HIP(hipGetLastError());

    cx.prof_end(kProfBuildGhost);

    // ---- bin every node on the extended grid (one cell layer of ghosts per side) ----
    cx.prof_begin(kProfBuildRows);
    MPNN_TRY(cx.grow(cx.tmp_b, sizeof(int32_t) * (size_t)(NN1 > next ? NN1 : next) * 2));
    key = cx.tmp_b.as<int32_t>();
    int32_t *cnodes = key + (NN1 > next ? NN1 : next);
    k_ext_key<<<grid_for(cx.NN), kBlock, 0, cx.stream>>>(cx.NN, n, cx.pos.as<double>(), cx.ghost_sub.as<int32_t>(),
                                                         g, key);
    MPNN_HIP(hipGetLastError());
    MPNN_TRY(counting_sort(cx, key, cx.NN, next, off, cnodes, cnt));

    // ---- receiver rows ----
    const double rcut2 = w * w;
    // fp32 pre-test band (as in the per-step compaction, with rcut): coordinates within [-c, c]
    const double cmax = std::max(cx.box[0], std::max(cx.box[1], cx.box[2])) + cx.rc + 2.0 * skin;
    const double eps32 = cmax * std::ldexp(1.0, -24);
    const double band = 2.0 * (4.0 * std::sqrt(3.0) * eps32 * w + 4.0 * std::ldexp(1.0, -23) * w * w) + 1e-9;
    const float lo = (float)(rcut2 - band), hi = (float)(rcut2 + band);
    MPNN_TRY(cx.grow(cx.cellpos, sizeof(float4) * NN1));
    if (cx.NN > 0) {
        k_cell_pos<<<grid_for(cx.NN), kBlock, 0, cx.stream>>>(cx.NN, cnodes, cx.pos.as<double>(),
                                                               cx.cellpos.as<float4>());
        MPNN_HIP(hipGetLastError());
    }
    MPNN_TRY(cx.grow(cx.tmp_c, sizeof(int32_t) * (size_t)(n1 > next ? n1 : next) + 64));
    cnt = cx.tmp_c.as<int32_t>();
    MPNN_TRY(cx.grow(cx.row_off, sizeof(int64_t) * (n1 + 1)));
    k_rows<false><<<grid_for(n), kBlock, 0, cx.stream>>>(n, cx.pos.as<double>(), g, off, cx.cellpos.as<float4>(),
                                                         rcut2, lo, hi, cnt, nullptr, nullptr);
    MPNN_HIP(hipGetLastError());
    MPNN_TRY(cx.grow(cx.row_len, sizeof(int32_t) * n1));
    if (n > 0)
        MPNN_HIP(hipMemcpyAsync(cx.row_len.p, cnt, sizeof(int32_t) * n, hipMemcpyDeviceToDevice, cx.stream));
    MPNN_TRY(exclusive_scan(cx, cnt, n, cx.row_off.as<int64_t>()));
    int64_t E = 0;
    MPNN_TRY(fetch(cx, cx.row_off.as<int64_t>() + n, &E));
    if (E > INT32_MAX) return Status::err(MPNN_E_CAPACITY, "more than 2^31-1 neighbour entries");
    cx.E = E;
    // slab layout: width of a slab = its longest row
    const int64_t nslab = (n + kSlab - 1) / kSlab;
    MPNN_TRY(cx.grow(cx.slab_off, sizeof(int64_t) * (size_t)(nslab + 2)));
    k_slab_width<<<grid_for(nslab), kBlock, 0, cx.stream>>>(n, nslab, cx.row_len.as<int32_t>(), cnt);
    MPNN_HIP(hipGetLastError());
    {
        // longest row -> words of the per-step activity mask
        std::vector<int32_t> widths((size_t)nslab);
        if (nslab > 0) {
            MPNN_HIP(hipMemcpyAsync(widths.data(), cnt, sizeof(int32_t) * nslab, hipMemcpyDeviceToHost, cx.stream));
            MPNN_HIP(hipStreamSynchronize(cx.stream));
        }
        int64_t longest = 0, slots = 0;
        for (int32_t w : widths) {
            longest = std::max<int64_t>(longest, w / kSlab);
            slots += w;
        }
        cx.mw = (int)std::max<int64_t>(1, (longest + 31) / 32);
        // transposed entries hold (row, column) in 32 bits (2.05M rows of at most 128 columns:
        // 21 + 7 bits; at most 2^25 rows of 128 columns, 2^24 of 256)
        int jb = 1;
        while (((int64_t)1 << jb) < longest) ++jb;
        if (n > ((int64_t)1 << (32 - jb)))
            return Status::err(MPNN_E_CAPACITY, "too many atoms for the longest neighbour row (" + std::to_string(longest) +
                                                    " entries): at most " + std::to_string((int64_t)1 << (32 - jb)));
        cx.tjb = jb;
        // ragged rows (slabs less than 85 % full, e.g. a gas with clusters): the row kernels take
        // each block's rows by descending active count, so a wave's rows have similar lengths.  The
        // reordering scatters the rows' per-edge stores and spreads a wave over four slabs, so it
        // pays only for strongly ragged rows (the CHON gas, 83 % full: reverse pass 6 % faster; a
        // heated metal, 90 % full: 50 % slower)
        // up to 32,768 rows, one row per lane would leave most of the chip idle (at most 512
        // waves on 1,024 SIMDs) and each wave's rows run one edge after another: the row kernels
        // give every row 16 lanes instead (and need no bucketing)
        cx.lane_groups = n <= 32768;
        cx.bucket = !cx.lane_groups && slots > 0 && (double)E < 0.85 * (double)slots;
        // per-edge streams (index, w_e, dE/dr_e) several times the 256 MB last-level cache, rows in
        // order (measured: the 2M-atom Ag subdomain, 7 GB, gains 6 %; a 128,000-atom alloy, 0.45 GB,
        // loses 3 %; a 4,608-atom water box, which fits in the caches, loses 13 %)
        cx.nt = !cx.bucket && !cx.lane_groups && (double)E * 4.0 * (cx.K + 3) > 1024.0 * (1 << 20);
    }
    MPNN_TRY(exclusive_scan(cx, cnt, nslab, cx.slab_off.as<int64_t>()));
    int64_t Es = 0;
    MPNN_TRY(fetch(cx, cx.slab_off.as<int64_t>() + nslab, &Es));
    if (Es > INT32_MAX) return Status::err(MPNN_E_CAPACITY, "more than 2^31-1 neighbour slots");
    cx.E_sell = Es;
    const int64_t E1 = Es > 0 ? Es : 1;
    MPNN_TRY(cx.grow(cx.nbr, sizeof(int32_t) * E1));
    k_rows<true><<<grid_for(n), kBlock, 0, cx.stream>>>(n, cx.pos.as<double>(), g, off, cx.cellpos.as<float4>(),
                                                        rcut2, lo, hi, nullptr, cx.slab_off.as<int64_t>(),
                                                        cx.nbr.as<int32_t>());
    MPNN_HIP(hipGetLastError());
    cx.prof_end(kProfBuildRows);

    // ---- sender-major transpose: for every node, the edges it sends, in edge order ----
    cx.prof_begin(kProfBuildTranspose);
    MPNN_TRY(cx.grow(cx.t_off, sizeof(int64_t) * (NN1 + 1)));
    MPNN_TRY(cx.grow(cx.t_eid, sizeof(int32_t) * E1));
    // a stable radix sort of (sender node, slot) pairs in slot order: each sender's segment lists
    // its slots in ascending order, so the transposed order (and every sum over it) is fixed.
    // Scratch: the edge-gradient buffer (3 words per slot, written per step later) holds the keys,
    // the values and the sorted keys; the sorted values are t_eid
    MPNN_TRY(cx.grow(cx.gedge, sizeof(float) * 3 * E1));
    {
        uint32_t *keys = reinterpret_cast<uint32_t *>(cx.gedge.p), *vals = keys + E1, *skeys = vals + E1;
        const int64_t nslab_all = (n + kSlab - 1) / kSlab;
        if (Es > 0) {
            k_tkeys<<<grid_for(nslab_all * kSlab), kBlock, 0, cx.stream>>>(
                nslab_all, n, cx.slab_off.as<int64_t>(), cx.row_len.as<int32_t>(), cx.nbr.as<int32_t>(),
                (uint32_t)cx.NN, cx.tjb, keys, vals);
            MPNN_HIP(hipGetLastError());
            int bits = 1;
            while (bits < 32 && ((int64_t)1 << bits) <= cx.NN) ++bits;
            size_t temp = 0;
            MPNN_HIP(hipcub::DeviceRadixSort::SortPairs(nullptr, temp, keys, skeys, vals,
                                                        reinterpret_cast<uint32_t *>(cx.t_eid.p), (int)Es, 0, bits,
                                                        cx.stream));
            MPNN_TRY(cx.grow(cx.tmp_scan, temp));
            MPNN_HIP(hipcub::DeviceRadixSort::SortPairs(cx.tmp_scan.p, temp, keys, skeys, vals,
                                                        reinterpret_cast<uint32_t *>(cx.t_eid.p), (int)Es, 0, bits,
                                                        cx.stream));
        }
        k_tsegments<<<grid_for(E + 1), kBlock, 0, cx.stream>>>(E, skeys, cx.NN, cx.t_off.as<int64_t>());
        MPNN_HIP(hipGetLastError());
    }

    cx.prof_end(kProfBuildTranspose);

    // ---- atoms grouped by species (ascending sorted index within a species) ----
    cx.prof_begin(kProfBuildSpecies);
    MPNN_TRY(cx.grow(cx.sp_list, sizeof(int32_t) * n1));
    MPNN_TRY(cx.grow(cx.sp_off, sizeof(int64_t) * (cx.S + 1)));
    cx.sp_count.assign(cx.S, 0);
    std::vector<int64_t> sp_off(cx.S + 1, 0);
    MPNN_TRY(cx.grow(cx.tmp_d, sizeof(int64_t) * (size_t)(n1 + 1)));
    int64_t *rank = cx.tmp_d.as<int64_t>();
    for (int s = 0; s < cx.S; ++s) {
        k_flag_species<<<grid_for(n), kBlock, 0, cx.stream>>>(n, cx.types.as<int32_t>(), s, cnt);
        MPNN_HIP(hipGetLastError());
        MPNN_TRY(exclusive_scan(cx, cnt, n, rank));
        int64_t cs = 0;
        MPNN_TRY(fetch(cx, rank + n, &cs));
        k_species_scatter<<<grid_for(n), kBlock, 0, cx.stream>>>(n, cx.types.as<int32_t>(), s, rank, sp_off[s],
                                                                 cx.sp_list.as<int32_t>());
        MPNN_HIP(hipGetLastError());
        cx.sp_count[s] = cs;
        sp_off[s + 1] = sp_off[s] + cs;
    }
    MPNN_HIP(hipMemcpyAsync(cx.sp_off.p, sp_off.data(), sizeof(int64_t) * (cx.S + 1), hipMemcpyHostToDevice,
                            cx.stream));

    // ---- per-evaluation buffers and layer-0 messages ----
    const int KM = cx.K * cx.M;
    MPNN_TRY(cx.grow(cx.c, sizeof(float) * (size_t)cx.T * NN1 * rec_stride(cx.K)));
    cx.np = pad_rows(cx.n);
    const size_t np1 = (size_t)(cx.np > 0 ? cx.np : kBlock);
    MPNN_TRY(cx.grow(cx.O, sizeof(float) * (size_t)cx.T * np1 * pad16(KM)));
    MPNN_TRY(cx.grow(cx.feat, sizeof(float) * (size_t)cx.T * np1 * cx.DP));
    MPNN_TRY(cx.grow(cx.grho, sizeof(float) * (size_t)cx.T * np1 * cx.DP));
    MPNN_TRY(cx.grow(cx.Gc, sizeof(float) * (size_t)cx.T * NN1 * cx.K));
    MPNN_TRY(cx.grow(cx.pos32, sizeof(float4) * NN1));
    MPNN_TRY(cx.grow(cx.amask, sizeof(uint32_t) * (size_t)(cx.mw + 1) * n1));
    MPNN_TRY(cx.grow(cx.t_act, sizeof(int32_t) * E1));
    if (cx.precision == 0 && cx.T > 1)
        MPNN_TRY(cx.grow(cx.dact, sizeof(float) * (size_t)(cx.T - 1) * n1 * 2 * cx.H));
    MPNN_TRY(cx.grow(cx.act_n, sizeof(int32_t) * E1));
    MPNN_TRY(cx.grow(cx.nact, sizeof(int32_t) * n1));
    MPNN_TRY(cx.grow(cx.row_perm, sizeof(int32_t) * n1));
    if (cx.T > 1) MPNN_TRY(cx.grow(cx.w, sizeof(float) * (size_t)E1 * cx.K));
    MPNN_TRY(cx.grow(cx.Frecv, sizeof(double) * 3 * n1));
    MPNN_TRY(cx.grow(cx.F, sizeof(double) * 3 * n1));
    MPNN_TRY(cx.grow(cx.Ei, sizeof(double) * n1));
    MPNN_TRY(cx.grow(cx.red, sizeof(double) * (size_t)(2 * red_blocks(n1) + 2)));
    k_c0<<<grid_for(cx.NN), kBlock, 0, cx.stream>>>(cx.NN, cx.K, cx.types.as<int32_t>(), cx.model.as<ModelDev>(),
                                                    cx.c.as<float>());
    MPNN_HIP(hipGetLastError());
    cx.prof_end(kProfBuildSpecies);
    MPNN_HIP(hipStreamSynchronize(cx.stream));
    // a second stream pays where the map's build is long enough to hide (measured: the fork and join
    // cost Ag108 a third of its step inside replayed graphs)
    cx.side = cx.E >= ((int64_t)1 << 22);
    if (cx.side && !cx.side_stream) MPNN_HIP(hipStreamCreateWithFlags(&cx.side_stream, hipStreamNonBlocking));
    for (hipEvent_t &e : cx.side_ev)
        if (cx.side && !e) MPNN_HIP(hipEventCreateWithFlags(&e, hipEventDisableTiming));
    cx.built = true;
    cx.stale = false;
    cx.since_build = 0;
    return Status::ok();
}

Status refresh_ghost_positions(Context &cx) {
    ProfScope ps_(cx, kProfGhostPos);
    if (cx.NN > 0) {
        const Grid g = make_grid(cx);
        k_node_pos<<<grid_for(cx.NN), kBlock, 0, cx.stream>>>(cx.NN, cx.n, cx.T, rec_stride(cx.K),
                                                               cx.ghost_owner.as<int32_t>(), cx.ghost_code.as<int32_t>(),
                                                               g, cx.pos.as<double>(), cx.pos32.as<float4>(),
                                                               cx.c.as<float>());
        MPNN_HIP(hipGetLastError());
    }
    return Status::ok();
}

Status get_pairs(Context &cx, int64_t cap, int64_t *n_pairs, int32_t *i, int32_t *j, int32_t *s) {
    *n_pairs = cx.E;
    if (cap <= 0 || cx.E == 0) return Status::ok();
    k_pairs<<<grid_for(cx.n), kBlock, 0, cx.stream>>>(cx.n, cx.row_off.as<int64_t>(), cx.slab_off.as<int64_t>(),
                                                      cx.nbr.as<int32_t>(),
                                                      cx.perm.as<int32_t>(), cx.ghost_owner.as<int32_t>(),
                                                      cx.ghost_code.as<int32_t>(), cap, i, j, s);
    MPNN_HIP(hipGetLastError());
    return Status::ok();
}

}  // namespace mpnn
