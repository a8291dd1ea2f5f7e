// Host-side context of the MPNN library and the launchers each translation unit provides.
#pragma once

#include <string>
#include <vector>

#include "../../include/mpnn.h"
#include "common.h"

namespace mpnn {

struct Status {
    mpnn_status code = MPNN_OK;
    std::string msg;
    static Status ok() { return Status(); }
    static Status err(mpnn_status c, std::string m) {
        Status s;
        s.code = c;
        s.msg = std::move(m);
        return s;
    }
    bool bad() const { return code != MPNN_OK; }
};

#define MPNN_HIP(call)                                                                      \
    do {                                                                                    \
        hipError_t e_ = (call);                                                             \
        if (e_ != hipSuccess)                                                               \
            return ::mpnn::Status::err(MPNN_E_HIP, std::string(#call) + ": " +              \
                                                       hipGetErrorString(e_));              \
    } while (0)

#define MPNN_TRY(expr)                                                                      \
    do {                                                                                    \
        ::mpnn::Status s_ = (expr);                                                         \
        if (s_.bad()) return s_;                                                            \
    } while (0)

// Kernel families timed by the optional event profiler (mpnn_set_profiling).
enum ProfId {
    kProfBuildSort = 0, kProfBuildGhost, kProfBuildRows, kProfBuildTranspose, kProfBuildSpecies,
    kProfGhostPos, kProfCompact, kProfAggregate, kProfNetForward, kProfNetEnergy, kProfNetBackward,
    kProfGhostFeat, kProfBackwardLayer, kProfMessageGrad, kProfGhostFold, kProfForceGather,
    kProfKickDrift, kProfKick, kProfReduce, kProfCount
};
extern const char *const kProfNames[kProfCount];

// A growable device allocation.
struct Buf {
    void *p = nullptr;
    size_t bytes = 0;
    void (*free_fn)(void *, void *) = nullptr;   // the caller's release hook that owns p, if any
    void *free_user = nullptr;
    template <class T> T *as() const { return static_cast<T *>(p); }
};

// Packed per-(layer, species) network block, all float, offsets in floats.  Matrices are in
// the matrix-core A-operand order (see mlp.hip): W1 [H][DP], W2 [H][H], W3 [16][H],
// W1t [DP][H], W2t [H][H], W3t [H][16], then biases b1 [H], b2 [H], b3 [16].
struct NetLayout {
    size_t W1, W2, W3, W1t, W2t, W3t, b1, b2, b3, stride;
};

struct Context {
    // ---- model ----
    int S = 0, K = 0, L = 0, T = 0, H = 0, M = 0, D = 0, DP = 0;
    bool chain = true;  // aggregation Gaussians by the ratio chain (else one exponential each)
    bool contracted = false;  // orbitals from contracted radial functions (mpnn_params.contraction)
    int precision = 0;  // 0: fp32 orbital sums / fp32 networks; 1: fp64 orbital sums and networks;
                        // 2: fp32 orbital sums, bf16-operand networks with fp32 accumulation
    double rc = 0, sigma = 0, e_scale = 0;
    std::vector<double> mass;
    NetLayout net{};
    Buf weights;        // float, T*S blocks of net.stride
    Buf weights64;      // the same in fp64 (precision 1)
    NetLayout net16{};  // bf16 operand blocks (precision 2): W1, W2, W3, W1t, W2t and stride
    Buf weights16;      // bf16 bits, T*S blocks of net16.stride
    Buf model;          // ModelDev
    hipStream_t stream = nullptr;

    // ---- system ----
    bool built = false;
    bool forces_valid = false;  // F_sorted matches the current positions
    int64_t n = 0, G = 0, NN = 0, E = 0, E_sell = 0;
    int64_t np = 0;             // n rounded up to whole 256-row blocks (column-tiled vectors)
    int mw = 1;                 // activity-mask words per row (longest row / 32, rounded up)
    int tjb = 1;                // transposed entries hold (row << tjb) | column
    double box[3] = {0, 0, 0};
    double skin = 0, rcut = 0;
    int sub[3] = {1, 1, 1};     // virtual subdomains per axis (the next build applies them)
    int nc[3] = {0, 0, 0};      // interior cells per axis of one subdomain
    double hcell[3] = {0, 0, 0};
    int64_t step = 0;
    int since_build = 0;
    std::vector<int64_t> sp_count;  // atoms per species (host copy)

    // per-atom / per-node state (sorted, locals first then ghosts)
    Buf perm, inv_perm;             // int32 [n]: sorted -> caller, caller -> sorted
    Buf pos;                        // double [NN][3]
    Buf pos32;                      // float4 [NN]: positions rounded to fp32 (active-edge pre-test)
    Buf vel;                        // double [n][3]
    Buf ref;                        // double [n][3], positions at the last build
    Buf types;                      // int32 [NN]
    Buf ghost_owner, ghost_code;    // int32 [G]
    Buf ghost_sub;                  // int32 [G]: subdomain whose shell holds the ghost
    Buf ghost_off;                  // int64 [n+1] ghosts of each owner
    Buf row_off;                    // int64 [n+1] prefix of row lengths (canonical pair order)
    Buf row_len;                    // int32 [n] Verlet entries per row
    Buf slab_off;                   // int64 [n/64+2] start of each 64-row slab
    Buf nbr;                        // int32 [E_sell] sender node of each entry (sliced ELLPACK)
    Buf cellpos;                    // float4 [NN]: fp32 node positions in grid-cell order (build only)
    Buf t_off, t_eid;               // int64 [NN+1], uint32 [E]: sender-major segments, (row << tjb) | column of each entry
    Buf sp_list, sp_off;            // int32 [n], int64 [S+1]

    // per-evaluation buffers
    Buf c;        // float [T][NN][rec_stride(K)]: node records (position, then c^t)
    Buf O;        // float [T] x column-tiled [np][pad16(K*M)]: orbital coefficients O^t
    Buf feat;     // float [T] x column-tiled [np][DP]: density features rho^t / s_t
    Buf grho;     // float [T] x column-tiled [np][DP]: dE/drho^t
    Buf Gc;       // float [T][NN][K]  dE/dc^t (layers 1..T-1)
    Buf gedge;    // float [E][3]  dE/dr_e summed over layers
    Buf w;        // float [E][K]  per-edge dE/dc contribution of the current layer
    Buf amask;    // uint32 [mw + 1][n]: bit j%32 of word j/32 = entry j of the row is active (d < rc);
                  // word mw: byte w - 1 = active entries in words 0 .. w - 1 (w = 1, 2, 3)
    Buf act_n;    // int32 [E]: sender node of each active slot
    Buf t_act;    // int32 [E]: active slot of each transposed entry this step (-1: d >= rc)
    Buf dact;     // float [T-1][n][2H]: silu' of both hidden layers of each message network (fp32 mode)
    Buf nact;     // int32 [n] active entries per row
    Buf row_perm; // int32 [n]: per 256-row block, its rows by descending active count (bucketing)
    bool bucket = false;   // row kernels take rows in row_perm order (ragged row lengths)
    bool nt = false;       // per-edge streams far larger than the caches, rows in order: nontemporal
    bool lane_groups = false;   // small systems: the row kernels give each row a 16-lane group
    double *scratch = nullptr;  // device address of the fixed reduction array (mpnn_energy_forces_noalloc)
    bool stale = false;         // positions moved beyond skin/2 without a rebuild: the next call rebuilds
    Buf Frecv;    // double [n][3]
    Buf F;        // double [n][3] (sorted)
    Buf Ei;       // double [n]: E_i
    Buf red;      // double [2 red_blocks(n) + 2]: energy partials, E, kinetic partials, KE
    Buf flag;     // uint64 [4]: displacement flag, max displacement bits
    Buf tmp_a, tmp_b, tmp_c, tmp_d, tmp_scan;  // build scratch

    std::string last_error;
    size_t device_bytes = 0;
    // caller-supplied device allocator (mpnn_set_allocator); hipMalloc / hipFree when null
    void *(*alloc_fn)(size_t, void *) = nullptr;
    void (*free_fn)(void *, void *) = nullptr;
    void *alloc_user = nullptr;

    // ---- event profiler ----
    bool prof_on = false;

    // ---- graph replay of MD chunks ----
    int graph_steps = 0;                 // requested chunk length (0: eager)
    struct Chunk {
        int k;
        double dt;
        hipGraphExec_t exec;
    };
    std::vector<Chunk> graphs;           // recorded chunks by (length, dt)
    bool graph_valid = false;            // false after a rebuild: every recorded chunk is stale
    Buf bak_pos, bak_vel, bak_F;         // state at the start of a replayed chunk
    hipStream_t cap_stream = nullptr;    // own (non-default, default-priority) stream: graphs are
                                         // captured and replayed there, ordered by events
    hipEvent_t cap_ev[2] = {nullptr, nullptr};
    // second stream (default priority) on which the transposed active map of each evaluation is
    // built while the forward layers run; events fork it from and join it to the context's stream
    hipStream_t side_stream = nullptr;
    hipEvent_t side_ev[2] = {nullptr, nullptr};
    bool side = false;   // transposed map on the side stream (large lists), else inline after the compaction
    double prof_ms[kProfCount] = {};
    int64_t prof_launches[kProfCount] = {};
    std::vector<hipEvent_t> prof_pool;
    struct Pending { int id; hipEvent_t a, b; };
    std::vector<Pending> prof_pending;
    std::vector<hipEvent_t> prof_open;  // start event per id while a scope is open
    void prof_begin(int id);
    void prof_end(int id);
    void prof_harvest();                // after a stream synchronisation

    Buf types_caller;             // int32 [n] species in caller order (for rebuilds)
    Buf stage_pos, stage_vel;     // double [n][3] caller-order staging
    std::vector<float> inv_scale_host;     // 1 / s_t rounded to fp32 (arithmetic modes 0 and 2)
    std::vector<double> inv_scale64_host;  // 1 / s_t (mode 1)

    Status grow(Buf &b, size_t bytes);
    Status grow_keep(Buf &b, size_t bytes, size_t keep);
    void release(Buf &b);
    ~Context();
};

// Times the launches issued while it lives (no-op unless profiling is on).
struct ProfScope {
    Context &cx;
    int id;
    ProfScope(Context &c, int i) : cx(c), id(i) { cx.prof_begin(id); }
    ~ProfScope() { cx.prof_end(id); }
};

// ---- scan.hip ----
// out[0..n] = exclusive prefix sum of in[0..n-1] (int32), out[n] = total.  int64 output.
Status exclusive_scan(Context &cx, const int32_t *in, int64_t n, int64_t *out);

// ---- neighbors.hip ----
Status build_neighbors(Context &cx, const double *pos_caller, const int32_t *types_caller,
                       int64_t n, const double box[3], double skin, const double *vel_caller);
Status refresh_ghost_positions(Context &cx);
Status get_pairs(Context &cx, int64_t cap, int64_t *n_pairs, int32_t *i, int32_t *j, int32_t *s);

// ---- edges.hip ----
Status compact_active(Context &cx);               // per-step active entries (d < rc)
Status aggregate(Context &cx, int t);
Status refresh_ghost_features(Context &cx, int t);
Status backward_layer(Context &cx, int t);        // per-edge w_e and dE/dr_e of layer t
Status assemble_go(Context &cx, int t, float *out);  // dE/dO^t [n][K*M] (diagnostics)
Status backward_messages(Context &cx, int t);     // dE/dc^t of all nodes + ghost fold (reads t_act)
// t_act (the active slot of every transposed entry) for this step: on the side stream, forked from
// the context's stream after the first aggregation, for long lists (Context::side), else on the
// context's stream; join_transpose makes the context's stream wait for the side stream
Status fork_transpose(Context &cx);
Status join_transpose(Context &cx);
Status force_gather(Context &cx, double *F_caller);

// ---- mlp.hip ----
Status mlp_forward(Context &cx, int t);           // c^{t+1} from rho^t (t < T-1)
Status mlp_energy(Context &cx);                   // E_i and dE/drho^{T-1}
Status mlp_backward(Context &cx, int t);          // dE/drho^t from dE/dc^{t+1}
Status pack_weights(Context &cx, const double *mlp);

// ---- integrate.hip ----
int64_t red_blocks(int64_t n);                   // partial sums of the fixed-order reductions
// E = sum E_i on the device (every evaluation); part: partials + total, nullptr = the context's buffer
Status energy_reduce(Context &cx, double *part = nullptr);
Status energy_sum(Context &cx, double *E_host, const double *part = nullptr);  // last evaluation's E to the host
// The fixed device array that mpnn_energy_forces_noalloc reduces into (kStaticPartials partials and
// the total), as a device address for the current device (looked up once per device).
constexpr int64_t kStaticPartials = 16384;
Status static_scratch(double **out);
Status kick_drift(Context &cx, double dt);       // first half-kick + drift + skin test
Status kick(Context &cx, double dt);             // second half-kick
Status skin_check(Context &cx);                  // displacement test only
Status kinetic_energy(Context &cx, double *ke_host);
Status read_skin_flag(Context &cx, bool *exceeded, double *max_disp);
Status reset_skin_flag(Context &cx);
Status unpermute_vec3(Context &cx, const double *sorted, double *caller);
Status permute_in_vec3(Context &cx, const double *caller, double *sorted);
// one double per atom, sorted -> caller order
Status unpermute_scalar(Context &cx, const double *sorted, double *caller);
// sorted rows of `width` floats (row-major, or column-tiled with row count np when np > 0)
Status unpermute_float(Context &cx, const float *sorted, int width, int64_t np, double *caller);
// sorted rows of `width` floats at a row stride of `stride` floats
Status unpermute_rows(Context &cx, const float *sorted, int width, int stride, double *caller);

}  // namespace mpnn
