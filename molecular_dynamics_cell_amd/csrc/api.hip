// C ABI entry points (include/mpnn.h): validation, buffer management and the call sequence
// of one energy/force evaluation and of the velocity-Verlet loop.
#include <cmath>
#include <cstring>
#include <new>
#include <vector>

#include <algorithm>

#include "impl.h"

struct mpnn_ctx {
    mpnn::Context cx;
};

namespace mpnn {

Status Context::grow(Buf &b, size_t bytes) {
    if (bytes == 0) bytes = 16;
    if (b.bytes >= bytes) return Status::ok();
    if (b.p) {
        MPNN_HIP(hipStreamSynchronize(stream));
        release(b);
    }
    size_t want = bytes + bytes / 8;
    void *p = nullptr;
    if (alloc_fn) {
        p = alloc_fn(want, alloc_user);
        if (!p) return Status::err(MPNN_E_OOM, "allocator hook returned NULL for " + std::to_string(want) + " bytes");
        b.free_fn = free_fn;
        b.free_user = alloc_user;
    } else {
        if (hipMalloc(&p, want) != hipSuccess) {
            (void)hipGetLastError();
            return Status::err(MPNN_E_OOM, "hipMalloc of " + std::to_string(want) + " bytes failed");
        }
        b.free_fn = nullptr;
        b.free_user = nullptr;
    }
    b.p = p;
    b.bytes = want;
    device_bytes += want;
    return Status::ok();
}

Status Context::grow_keep(Buf &b, size_t bytes, size_t keep) {
    if (b.bytes >= bytes) return Status::ok();
    Buf nb;
    MPNN_TRY(grow(nb, bytes));
    if (b.p && keep) MPNN_HIP(hipMemcpyAsync(nb.p, b.p, keep < b.bytes ? keep : b.bytes, hipMemcpyDeviceToDevice, stream));
    MPNN_HIP(hipStreamSynchronize(stream));
    release(b);
    b = nb;
    return Status::ok();
}

const char *const kProfNames[kProfCount] = {
    "build_sort", "build_ghosts", "build_rows", "build_transpose", "build_species", "ghost_positions",
    "compact", "aggregate", "net_forward", "net_energy", "net_backward", "ghost_messages",
    "backward_layer", "message_grad", "ghost_grad_fold", "force_gather", "kick_drift", "kick", "reduce"};

void Context::prof_begin(int id) {
    if (!prof_on) return;
    if (prof_open.empty()) prof_open.assign(kProfCount, nullptr);
    hipEvent_t e = nullptr;
    if (!prof_pool.empty()) {
        e = prof_pool.back();
        prof_pool.pop_back();
    } else if (hipEventCreate(&e) != hipSuccess) {
        return;
    }
    (void)hipEventRecord(e, stream);
    prof_open[id] = e;
}

void Context::prof_end(int id) {
    if (!prof_on || prof_open.empty() || !prof_open[id]) return;
    hipEvent_t e = nullptr;
    if (!prof_pool.empty()) {
        e = prof_pool.back();
        prof_pool.pop_back();
    } else if (hipEventCreate(&e) != hipSuccess) {
        return;
    }
    (void)hipEventRecord(e, stream);
    prof_pending.push_back({id, prof_open[id], e});
    prof_open[id] = nullptr;
}

void Context::prof_harvest() {
    for (const Pending &p : prof_pending) {
        float ms = 0.0f;
        if (hipEventSynchronize(p.b) == hipSuccess && hipEventElapsedTime(&ms, p.a, p.b) == hipSuccess) {
            prof_ms[p.id] += ms;
            prof_launches[p.id] += 1;
        }
        prof_pool.push_back(p.a);
        prof_pool.push_back(p.b);
    }
    prof_pending.clear();
}

void Context::release(Buf &b) {
    if (b.p) {
        if (b.free_fn) b.free_fn(b.p, b.free_user);
        else (void)hipFree(b.p);
        device_bytes -= b.bytes;
    }
    b.p = nullptr;
    b.bytes = 0;
    b.free_fn = nullptr;
    b.free_user = nullptr;
}

Context::~Context() {
    if (stream) (void)hipStreamSynchronize(stream);
    Buf *all[] = {&weights, &weights64, &weights16, &ghost_sub, &row_perm, &model, &perm, &inv_perm, &pos, &pos32, &vel, &ref, &types, &ghost_owner, &ghost_code,
                  &ghost_off, &row_off, &row_len, &slab_off, &nbr, &cellpos, &t_off, &t_eid, &sp_list, &sp_off, &c, &O, &feat, &grho, &Gc,
                  &gedge, &w, &amask, &act_n, &t_act, &dact, &nact, &Frecv, &F, &Ei, &red, &flag, &tmp_a, &tmp_b, &tmp_c,
                  &tmp_d, &tmp_scan,
                  &types_caller, &stage_pos, &stage_vel, &bak_pos, &bak_vel, &bak_F};
    for (const Chunk &c : graphs) (void)hipGraphExecDestroy(c.exec);
    if (cap_stream) (void)hipStreamSynchronize(cap_stream);
    for (hipEvent_t e : cap_ev)
        if (e) (void)hipEventDestroy(e);
    if (cap_stream) (void)hipStreamDestroy(cap_stream);
    if (side_stream) (void)hipStreamSynchronize(side_stream);
    for (hipEvent_t e : side_ev)
        if (e) (void)hipEventDestroy(e);
    if (side_stream) (void)hipStreamDestroy(side_stream);
    for (Buf *b : all) release(*b);
    prof_harvest();
    for (hipEvent_t e : prof_pool) (void)hipEventDestroy(e);
}

namespace {

bool supported(int K, int L, int H) {
    const bool kl = (K == 8 && L == 2) || (K == 12 && L == 3) || (K == 2 && L == 1) || (K == 4 && L == 2);
    return kl && (H == 64 || H == 128);
}

// One energy/force evaluation on the current (sorted) state: paper Eq. 1-2 forward with the
// per-layer ghost refresh, then Eq. 3-5 backward with the ghost->owner folds.
Status evaluate(Context &cx, double *F_caller, double *red_part = nullptr) {
    MPNN_TRY(refresh_ghost_positions(cx));
    MPNN_TRY(compact_active(cx));
    // the transposed active map depends only on the compaction: it is built on the side stream
    // beside the forward layers after the first aggregation (which then runs alone: 0.04 ms per
    // step better on the 2.05M-atom Ag subdomain than beside it), and joined before the first
    // sender-major gather
    for (int t = 0; t < cx.T; ++t) {
        MPNN_TRY(aggregate(cx, t));
        if (t == 0) MPNN_TRY(fork_transpose(cx));
        if (t < cx.T - 1) {
            MPNN_TRY(mlp_forward(cx, t));
            MPNN_TRY(refresh_ghost_features(cx, t + 1));
        } else {
            MPNN_TRY(mlp_energy(cx));
        }
    }
    for (int t = cx.T - 1; t >= 0; --t) {
        MPNN_TRY(backward_layer(cx, t));
        if (t == cx.T - 1) MPNN_TRY(join_transpose(cx));
        if (t >= 1) {
            MPNN_TRY(backward_messages(cx, t));
            MPNN_TRY(mlp_backward(cx, t - 1));
        }
    }
    MPNN_TRY(force_gather(cx, F_caller));
    MPNN_TRY(energy_reduce(cx, red_part));
    cx.forces_valid = true;
    return Status::ok();
}

// Rebuild from the context's own state (positions and velocities carried over).
Status rebuild_from_state(Context &cx) {
    const int64_t n1 = cx.n > 0 ? cx.n : 1;
    MPNN_TRY(cx.grow(cx.stage_pos, sizeof(double) * 3 * n1));
    MPNN_TRY(cx.grow(cx.stage_vel, sizeof(double) * 3 * n1));
    MPNN_TRY(unpermute_vec3(cx, cx.pos.as<double>(), cx.stage_pos.as<double>()));
    MPNN_TRY(unpermute_vec3(cx, cx.vel.as<double>(), cx.stage_vel.as<double>()));
    double box[3] = {cx.box[0], cx.box[1], cx.box[2]};
    return build_neighbors(cx, cx.stage_pos.as<double>(), cx.types_caller.as<int32_t>(), cx.n, box, cx.skin,
                           cx.stage_vel.as<double>());
}

mpnn_status finish(mpnn_ctx *ctx, const Status &s) {
    if (ctx) ctx->cx.last_error = s.msg;
    return s.code;
}

}  // namespace
}  // namespace mpnn

using mpnn::Status;

extern "C" {

mpnn_status mpnn_create(const mpnn_params *p, mpnn_ctx **out) {
    if (!out) return MPNN_E_INVALID_ARG;
    *out = nullptr;
    if (!p || !p->mu || !p->c0 || !p->mlp || !p->layer_scale || !p->mass) return MPNN_E_INVALID_ARG;
    if (p->precision < 0 || p->precision > 2 || p->n_species < 1 || p->n_species > 16 || p->T < 1 || p->T > 8 ||
        !mpnn::supported(p->K, p->L, p->hidden) || !(p->rc > 0) || !(p->sigma > 0))
        return MPNN_E_INVALID_ARG;
    // bf16 networks only for 64-wide networks on at most 128 features, where their force error
    // was measured within 2e-3 of the RMS force (longer contractions exceed it)
    if (p->precision == 2 && (p->hidden != 64 || mpnn::n_feat(p->K, p->L) > 128)) return MPNN_E_INVALID_ARG;
    for (int t = 0; t < p->T; ++t)
        if (!(p->layer_scale[t] > 0) || !std::isfinite(p->layer_scale[t])) return MPNN_E_INVALID_ARG;
    for (int k = 0; k < p->K; ++k)
        if (!std::isfinite(p->mu[k])) return MPNN_E_INVALID_ARG;
    if (p->contraction)
        for (int q = 0; q < p->K * p->K; ++q)
            if (!std::isfinite(p->contraction[q])) return MPNN_E_INVALID_ARG;
    mpnn_ctx *ctx = new (std::nothrow) mpnn_ctx;
    if (!ctx) return MPNN_E_OOM;
    mpnn::Context &cx = ctx->cx;
    cx.S = p->n_species; cx.K = p->K; cx.L = p->L; cx.T = p->T; cx.H = p->hidden;
    cx.precision = p->precision;
    cx.M = mpnn::n_mono(cx.L);
    cx.D = mpnn::n_feat(cx.K, cx.L);
    cx.DP = (cx.D + 15) / 16 * 16;
    cx.rc = p->rc; cx.sigma = p->sigma; cx.e_scale = p->e_scale;
    cx.mass.assign(p->mass, p->mass + cx.S);
    // Parameters as the arithmetic mode holds them: mode 1 keeps every parameter in fp64; modes 0
    // and 2 hold the radial centres, C0, the contraction matrix, 1/s_t and e_scale rounded to fp32
    // (the network weights too, see pack_weights), so every part of the path, including the fp64
    // basis factors of the orbital sums, sees the same fp32 parameter values.
    const bool p64 = cx.precision == 1;
    auto held = [p64](double v) { return p64 ? v : (double)(float)v; };
    std::vector<double> mu(cx.K);
    for (int k = 0; k < cx.K; ++k) mu[k] = held(p->mu[k]);
    cx.inv_scale_host.resize(cx.T);
    cx.inv_scale64_host.resize(cx.T);
    for (int t = 0; t < cx.T; ++t) {
        cx.inv_scale_host[t] = (float)(1.0 / p->layer_scale[t]);
        cx.inv_scale64_host[t] = 1.0 / p->layer_scale[t];
    }
    mpnn::ModelDev md{};
    for (int k = 0; k < cx.K; ++k) md.mu[k] = (float)p->mu[k];
    md.e_scale64 = p->e_scale;
    for (int s = 0; s < cx.S; ++s) {
        for (int k = 0; k < cx.K; ++k) {
            md.c0[s * cx.K + k] = (float)p->c0[s * cx.K + k];
            md.c0_64[s * cx.K + k] = p->c0[s * cx.K + k];
        }
        md.mass[s] = p->mass[s];
        if (!(p->mass[s] > 0)) {
            delete ctx;
            return MPNN_E_INVALID_ARG;
        }
    }
    for (int t = 0; t < cx.T; ++t) md.inv_scale[t] = cx.inv_scale_host[t];
    md.e_scale = (float)p->e_scale;
    md.neg_half_inv_s2 = (float)(-1.0 / (2.0 * p->sigma * p->sigma));
    md.inv_s2 = (float)(1.0 / (p->sigma * p->sigma));
    md.rc = (float)p->rc;
    md.inv_rc = (float)(1.0 / p->rc);
    md.pi_over_rc = (float)(mpnn::kPi / p->rc);
    md.exp2_coef = (float)(-1.0 / (2.0 * p->sigma * p->sigma * std::log(2.0)));
    md.dfc_scale = (float)(-0.5 * mpnn::kPi / p->rc);
    md.rc2 = p->rc * p->rc;
    {
        const double s2 = p->sigma * p->sigma;
        for (int k = 0; k < cx.K; ++k) md.mu64[k] = mu[k];
        md.g_a0 = -1.0 / (2.0 * s2);
        const double delta = cx.K > 1 ? mu[1] - mu[0] : 0.0;
        md.g_e = delta / s2;
        // the chain R_{k+1} = R_k E g_c[k] (1 + g_eps[k] d) replaces exp(g_eps[k] d) by its first
        // two terms, so it needs |g_eps[k]| rc below 2e-5 (the dropped terms stay under 2e-10
        // relative; evenly spaced centres stored in fp32 give about 4e-6), and
        // E = exp(delta rc / sigma^2), R_0 = exp(-(rc - mu_0)^2 / (2 sigma^2)) must stay inside the
        // fp64 range; otherwise every channel is evaluated directly
        bool chain = true;
        for (int k = 0; k + 1 < cx.K; ++k) {
            const double dk = mu[k + 1] - mu[k];
            md.g_c[k] = std::exp(-dk * (mu[k] + mu[k + 1]) / (2.0 * s2));
            md.g_eps[k] = (dk - delta) / s2;
            md.g_ce[k] = md.g_c[k] * md.g_eps[k];
            chain = chain && std::fabs(md.g_eps[k]) * p->rc < 2e-5 && std::isfinite(md.g_c[k]) && md.g_c[k] > 0.0;
        }
        double span = 0.0;
        for (int k = 0; k < cx.K; ++k) span = std::max(span, std::fabs(p->rc - mu[k]) + std::fabs(mu[k]));
        chain = chain && std::fabs(md.g_e) * p->rc < 600.0 && span * span / (2.0 * s2) < 600.0;
        cx.chain = chain;
        md.inv_rc64 = 1.0 / p->rc;
        md.half_pi_over_rc = 0.5 * mpnn::kPi / p->rc;
    }
    cx.contracted = p->contraction != nullptr;
    if (cx.contracted)
        for (int q = 0; q < cx.K * cx.K; ++q) {
            md.C64[q] = held(p->contraction[q]);
            md.C32[q] = (float)p->contraction[q];
        }
    // the fixed reduction array of mpnn_energy_forces_noalloc, on the device current at create
    Status s = mpnn::static_scratch(&cx.scratch);
    if (!s.bad()) s = cx.grow(cx.model, sizeof md);
    if (!s.bad()) {
        if (hipMemcpy(cx.model.p, &md, sizeof md, hipMemcpyHostToDevice) != hipSuccess)
            s = Status::err(MPNN_E_HIP, "upload of model constants failed");
    }
    if (!s.bad()) s = mpnn::pack_weights(cx, p->mlp);
    if (s.bad()) {
        delete ctx;
        return s.code;
    }
    *out = ctx;
    return MPNN_OK;
}

void mpnn_destroy(mpnn_ctx *ctx) { delete ctx; }

mpnn_status mpnn_set_stream(mpnn_ctx *ctx, void *hip_stream) {
    if (!ctx) return MPNN_E_INVALID_ARG;
    ctx->cx.stream = static_cast<hipStream_t>(hip_stream);
    return mpnn::finish(ctx, Status::ok());
}

mpnn_status mpnn_build_neighbors(mpnn_ctx *ctx, const double *pos, const int32_t *types, int64_t n,
                                 const double box[3], double rc, double skin) {
    if (!ctx) return MPNN_E_INVALID_ARG;
    mpnn::Context &cx = ctx->cx;
    if (n < 0 || !box || (n > 0 && (!pos || !types)) || !(skin >= 0) || !std::isfinite(skin))
        return mpnn::finish(ctx, Status::err(MPNN_E_INVALID_ARG, "bad arguments"));
    if (!(std::fabs(rc - cx.rc) <= 1e-12 * cx.rc))
        return mpnn::finish(ctx, Status::err(MPNN_E_INVALID_ARG, "rc differs from the model's cutoff"));
    if (n > INT32_MAX) return mpnn::finish(ctx, Status::err(MPNN_E_CAPACITY, "too many atoms"));
    for (int a = 0; a < 3; ++a)
        if (!std::isfinite(box[a])) return mpnn::finish(ctx, Status::err(MPNN_E_INVALID_ARG, "bad box"));
    Status s = cx.grow(cx.types_caller, sizeof(int32_t) * (n > 0 ? n : 1));
    if (!s.bad() && n > 0) {
        if (hipMemcpyAsync(cx.types_caller.p, types, sizeof(int32_t) * n, hipMemcpyDeviceToDevice, cx.stream) !=
            hipSuccess)
            s = Status::err(MPNN_E_HIP, "copy of types failed");
    }
    if (!s.bad()) s = mpnn::build_neighbors(cx, pos, types, n, box, skin, nullptr);
    return mpnn::finish(ctx, s);
}

static Status load_positions(mpnn::Context &cx, const double *pos) {
    // new caller-order positions: rebuild if any atom left the skin, else keep the list
    const int64_t n1 = cx.n > 0 ? cx.n : 1;
    MPNN_TRY(cx.grow(cx.stage_pos, sizeof(double) * 3 * n1));
    MPNN_HIP(hipMemcpyAsync(cx.stage_pos.p, pos, sizeof(double) * 3 * cx.n, hipMemcpyDeviceToDevice, cx.stream));
    MPNN_TRY(mpnn::permute_in_vec3(cx, cx.stage_pos.as<double>(), cx.pos.as<double>()));
    MPNN_TRY(mpnn::reset_skin_flag(cx));
    MPNN_TRY(mpnn::skin_check(cx));
    bool ex = false;
    double md = 0;
    MPNN_TRY(mpnn::read_skin_flag(cx, &ex, &md));
    if (ex) MPNN_TRY(mpnn::rebuild_from_state(cx));
    cx.forces_valid = false;
    return Status::ok();
}

mpnn_status mpnn_energy_forces(mpnn_ctx *ctx, const double *pos, double *energy, double *forces,
                               double *atom_energy) {
    if (!ctx) return MPNN_E_INVALID_ARG;
    mpnn::Context &cx = ctx->cx;
    if (!cx.built) return mpnn::finish(ctx, Status::err(MPNN_E_STATE, "mpnn_build_neighbors first"));
    Status s;
    if (pos) s = load_positions(cx, pos);
    else if (cx.stale) s = mpnn::rebuild_from_state(cx);
    if (!s.bad()) cx.stale = false;
    if (!s.bad()) s = mpnn::evaluate(cx, forces);
    if (!s.bad() && atom_energy) s = mpnn::unpermute_scalar(cx, cx.Ei.as<double>(), atom_energy);
    if (!s.bad() && energy) {
        s = mpnn::energy_sum(cx, energy);
        if (!s.bad() && !std::isfinite(*energy)) s = Status::err(MPNN_E_NONFINITE, "non-finite energy");
    }
    if (cx.prof_on && !s.bad()) {
        if (hipStreamSynchronize(cx.stream) != hipSuccess) s = Status::err(MPNN_E_HIP, "stream sync failed");
        cx.prof_harvest();
    }
    return mpnn::finish(ctx, s);
}

mpnn_status mpnn_energy_forces_noalloc(mpnn_ctx *ctx, const double *pos, double *energy, double *forces,
                                       double *atom_energy) {
    if (!ctx) return MPNN_E_INVALID_ARG;
    mpnn::Context &cx = ctx->cx;
    if (!cx.built || cx.stale)
        return mpnn::finish(ctx, Status::err(MPNN_E_STATE, "needs a current neighbour list (mpnn_build_neighbors)"));
    if (!cx.scratch) return mpnn::finish(ctx, Status::err(MPNN_E_STATE, "no fixed scratch on this device"));
    if (mpnn::red_blocks(cx.n) > mpnn::kStaticPartials)
        return mpnn::finish(ctx, Status::err(MPNN_E_CAPACITY, "more atoms than the fixed scratch holds (" +
                                                                  std::to_string(mpnn::kStaticPartials * 2048) + ")"));
    auto run = [&]() -> Status {
        if (pos && cx.n > 0) {
            // the caller's array is device memory: permute it straight into the sorted state
            MPNN_TRY(mpnn::permute_in_vec3(cx, pos, cx.pos.as<double>()));
            MPNN_TRY(mpnn::reset_skin_flag(cx));
            MPNN_TRY(mpnn::skin_check(cx));
            bool ex = false;
            double md = 0;
            MPNN_TRY(mpnn::read_skin_flag(cx, &ex, &md));
            cx.forces_valid = false;
            if (ex) {
                cx.stale = true;   // the next allocating call rebuilds first
                return Status::err(MPNN_E_SKIN, "an atom moved more than skin/2 since the last build: a rebuild "
                                                "(which may allocate) is needed");
            }
        }
        MPNN_TRY(mpnn::evaluate(cx, forces, cx.scratch));
        if (atom_energy) MPNN_TRY(mpnn::unpermute_scalar(cx, cx.Ei.as<double>(), atom_energy));
        if (energy) {
            MPNN_TRY(mpnn::energy_sum(cx, energy, cx.scratch));
            if (!std::isfinite(*energy)) return Status::err(MPNN_E_NONFINITE, "non-finite energy");
        }
        // the context's own reduction buffer holds the last evaluation's energy for later calls
        if (cx.n > 0)
            MPNN_HIP(hipMemcpyAsync(cx.red.as<double>() + mpnn::red_blocks(cx.n), cx.scratch + mpnn::red_blocks(cx.n),
                                    sizeof(double), hipMemcpyDeviceToDevice, cx.stream));
        return Status::ok();
    };
    return mpnn::finish(ctx, run());
}

}  // extern "C"

namespace mpnn {

Status drop_graphs(Context &cx) {
    for (const Context::Chunk &c : cx.graphs) MPNN_HIP(hipGraphExecDestroy(c.exec));
    cx.graphs.clear();
    cx.graph_valid = true;
    return Status::ok();
}

// Record k steps (state backup, then kick-drift / evaluation / kick per step) as one graph.
Status capture_chunk(Context &cx, double dt, int k, hipGraphExec_t *out) {
    const size_t bytes = sizeof(double) * 3 * (size_t)(cx.n > 0 ? cx.n : 1);
    MPNN_TRY(cx.grow(cx.bak_pos, bytes));       // every allocation happens before the capture
    MPNN_TRY(cx.grow(cx.bak_vel, bytes));
    MPNN_TRY(cx.grow(cx.bak_F, bytes));
    if (!cx.cap_stream) MPNN_HIP(hipStreamCreateWithFlags(&cx.cap_stream, hipStreamNonBlocking));
    for (hipEvent_t &e : cx.cap_ev)
        if (!e) MPNN_HIP(hipEventCreateWithFlags(&e, hipEventDisableTiming));
    MPNN_HIP(hipStreamSynchronize(cx.stream));
    // the launchers use cx.stream: point it at the capture stream while recording
    const hipStream_t user = cx.stream;
    cx.stream = cx.cap_stream;
    const hipError_t eb = hipStreamBeginCapture(cx.stream, hipStreamCaptureModeThreadLocal);
    if (eb != hipSuccess) {
        cx.stream = user;
        MPNN_HIP(eb);
    }
    auto body = [&]() -> Status {
        const size_t b = sizeof(double) * 3 * (size_t)cx.n;
        if (cx.n > 0) {
            MPNN_HIP(hipMemcpyAsync(cx.bak_pos.p, cx.pos.p, b, hipMemcpyDeviceToDevice, cx.stream));
            MPNN_HIP(hipMemcpyAsync(cx.bak_vel.p, cx.vel.p, b, hipMemcpyDeviceToDevice, cx.stream));
            MPNN_HIP(hipMemcpyAsync(cx.bak_F.p, cx.F.p, b, hipMemcpyDeviceToDevice, cx.stream));
        }
        for (int j = 0; j < k; ++j) {
            MPNN_TRY(kick_drift(cx, dt));
            MPNN_TRY(evaluate(cx, nullptr));
            MPNN_TRY(kick(cx, dt));
        }
        return Status::ok();
    };
    const Status st = body();
    hipGraph_t g = nullptr;
    const hipError_t e = hipStreamEndCapture(cx.stream, &g);
    cx.stream = user;
    if (st.bad()) {
        if (g) (void)hipGraphDestroy(g);
        return st;
    }
    MPNN_HIP(e);
    hipGraphExec_t exec = nullptr;
    const hipError_t ei = hipGraphInstantiate(&exec, g, nullptr, nullptr, 0);
    (void)hipGraphDestroy(g);
    MPNN_HIP(ei);
    cx.graphs.push_back({k, dt, exec});
    *out = exec;
    return Status::ok();
}

// Run k steps as one replay.  *done = false: an atom crossed skin/2 inside the chunk; the state
// is restored to the chunk's start (the displacement flag recomputed for it) for an eager redo.
Status replay_chunk(Context &cx, double dt, int k, bool *done, double *max_disp) {
    if (!cx.graph_valid) MPNN_TRY(drop_graphs(cx));
    hipGraphExec_t exec = nullptr;
    for (const Context::Chunk &c : cx.graphs)
        if (c.k == k && c.dt == dt) exec = c.exec;
    if (!exec) MPNN_TRY(capture_chunk(cx, dt, k, &exec));
    // replay on the capture stream, ordered after and before the work of the context's stream
    MPNN_HIP(hipEventRecord(cx.cap_ev[0], cx.stream));
    MPNN_HIP(hipStreamWaitEvent(cx.cap_stream, cx.cap_ev[0], 0));
    MPNN_HIP(hipGraphLaunch(exec, cx.cap_stream));
    MPNN_HIP(hipEventRecord(cx.cap_ev[1], cx.cap_stream));
    MPNN_HIP(hipStreamWaitEvent(cx.stream, cx.cap_ev[1], 0));
    bool ex = false;
    MPNN_TRY(read_skin_flag(cx, &ex, max_disp));
    if (!ex) {
        *done = true;
        return Status::ok();
    }
    const size_t b = sizeof(double) * 3 * (size_t)cx.n;
    if (cx.n > 0) {
        MPNN_HIP(hipMemcpyAsync(cx.pos.p, cx.bak_pos.p, b, hipMemcpyDeviceToDevice, cx.stream));
        MPNN_HIP(hipMemcpyAsync(cx.vel.p, cx.bak_vel.p, b, hipMemcpyDeviceToDevice, cx.stream));
        MPNN_HIP(hipMemcpyAsync(cx.F.p, cx.bak_F.p, b, hipMemcpyDeviceToDevice, cx.stream));
    }
    MPNN_TRY(reset_skin_flag(cx));
    MPNN_TRY(skin_check(cx));
    *done = false;
    return Status::ok();
}

}  // namespace mpnn

extern "C" {

mpnn_status mpnn_set_graph_replay(mpnn_ctx *ctx, int32_t steps_per_replay) {
    if (!ctx || steps_per_replay < 0) return MPNN_E_INVALID_ARG;
    mpnn::Context &cx = ctx->cx;
    cx.graph_steps = steps_per_replay;
    cx.graph_valid = false;
    return mpnn::finish(ctx, Status::ok());
}

mpnn_status mpnn_set_allocator(mpnn_ctx *ctx, void *(*alloc)(size_t, void *), void (*release)(void *, void *),
                               void *user) {
    if (!ctx) return MPNN_E_INVALID_ARG;
    if ((alloc == nullptr) != (release == nullptr))
        return mpnn::finish(ctx, Status::err(MPNN_E_INVALID_ARG, "allocator and release hooks go together"));
    mpnn::Context &cx = ctx->cx;
    cx.alloc_fn = alloc;
    cx.free_fn = release;
    cx.alloc_user = user;
    return mpnn::finish(ctx, Status::ok());
}

mpnn_status mpnn_set_subdomains(mpnn_ctx *ctx, int32_t px, int32_t py, int32_t pz) {
    if (!ctx) return MPNN_E_INVALID_ARG;
    mpnn::Context &cx = ctx->cx;
    if (px < 1 || py < 1 || pz < 1 || px > 16 || py > 16 || pz > 16)
        return mpnn::finish(ctx, Status::err(MPNN_E_INVALID_ARG, "subdomains per axis must be in 1..16"));
    cx.sub[0] = px; cx.sub[1] = py; cx.sub[2] = pz;
    cx.built = false;          // the list and the ghost shell follow the decomposition
    cx.forces_valid = false;
    cx.graph_valid = false;
    return mpnn::finish(ctx, Status::ok());
}

mpnn_status mpnn_md_step(mpnn_ctx *ctx, double dt_fs, int32_t n_steps, int32_t rebuild_every,
                         mpnn_md_stats *stats) {
    if (!ctx) return MPNN_E_INVALID_ARG;
    mpnn::Context &cx = ctx->cx;
    if (!cx.built) return mpnn::finish(ctx, Status::err(MPNN_E_STATE, "mpnn_build_neighbors first"));
    if (n_steps < 0 || rebuild_every < 0 || !std::isfinite(dt_fs))
        return mpnn::finish(ctx, Status::err(MPNN_E_INVALID_ARG, "bad arguments"));
    auto run = [&]() -> Status {
        int64_t rebuilds = 0;
        double max_disp = 0.0;
        if (cx.stale) {
            MPNN_TRY(mpnn::rebuild_from_state(cx));
            cx.stale = false;
            ++rebuilds;
        }
        if (!cx.forces_valid) MPNN_TRY(mpnn::evaluate(cx, nullptr));
        MPNN_TRY(mpnn::reset_skin_flag(cx));
        int eager_left = 0;   // after a rolled-back chunk, its steps run eagerly
        for (int32_t s = 0; s < n_steps; ++s) {
            // a replayed chunk of k steps, ending before the next scheduled rebuild
            int k = 0;
            if (eager_left > 0) {
                --eager_left;
            } else if (cx.graph_steps > 0 && !cx.prof_on && cx.n > 0) {
                k = std::min<int32_t>(cx.graph_steps, n_steps - s);
                if (rebuild_every > 0) k = std::min(k, rebuild_every - 1 - cx.since_build);
            }
            if (k > 0) {
                bool done = false;
                double md = 0.0;
                MPNN_TRY(mpnn::replay_chunk(cx, dt_fs, k, &done, &md));
                if (done) {
                    max_disp = md > max_disp ? md : max_disp;
                    cx.since_build += k;
                    cx.step += k;
                    s += k - 1;
                    continue;
                }
                eager_left = k - 1;
            }
            MPNN_TRY(mpnn::kick_drift(cx, dt_fs));
            ++cx.since_build;
            bool need = rebuild_every > 0 && cx.since_build >= rebuild_every;
            bool ex = false;
            double md = 0.0;
            MPNN_TRY(mpnn::read_skin_flag(cx, &ex, &md));
            cx.prof_harvest();
            max_disp = md > max_disp ? md : max_disp;
            if (need || ex) {
                MPNN_TRY(mpnn::rebuild_from_state(cx));
                MPNN_TRY(mpnn::reset_skin_flag(cx));
                ++rebuilds;
            }
            MPNN_TRY(mpnn::evaluate(cx, nullptr));
            MPNN_TRY(mpnn::kick(cx, dt_fs));
            ++cx.step;
        }
        if (stats) {
            double ep = 0, ke = 0;
            MPNN_TRY(mpnn::energy_sum(cx, &ep));
            MPNN_TRY(mpnn::kinetic_energy(cx, &ke));
            stats->epot = ep;
            stats->ekin = ke;
            stats->temp = cx.n > 1 ? 2.0 * ke / ((3.0 * cx.n - 3.0) * mpnn::kBoltzmann) : 0.0;
            stats->rebuilds = rebuilds;
            stats->max_disp = max_disp;
            stats->steps = cx.step;
        } else {
            MPNN_HIP(hipStreamSynchronize(cx.stream));
        }
        cx.prof_harvest();
        return Status::ok();
    };
    return mpnn::finish(ctx, run());
}

mpnn_status mpnn_set_state(mpnn_ctx *ctx, const double *pos, const double *vel) {
    if (!ctx) return MPNN_E_INVALID_ARG;
    mpnn::Context &cx = ctx->cx;
    if (!cx.built) return mpnn::finish(ctx, Status::err(MPNN_E_STATE, "mpnn_build_neighbors first"));
    auto run = [&]() -> Status {
        if (pos) {
            const int64_t n1 = cx.n > 0 ? cx.n : 1;
            MPNN_TRY(cx.grow(cx.stage_pos, sizeof(double) * 3 * n1));
            MPNN_TRY(cx.grow(cx.stage_vel, sizeof(double) * 3 * n1));
            if (cx.n > 0) {
                MPNN_HIP(hipMemcpyAsync(cx.stage_pos.p, pos, sizeof(double) * 3 * cx.n, hipMemcpyDeviceToDevice,
                                        cx.stream));
                if (vel)
                    MPNN_HIP(hipMemcpyAsync(cx.stage_vel.p, vel, sizeof(double) * 3 * cx.n,
                                            hipMemcpyDeviceToDevice, cx.stream));
                else
                    MPNN_TRY(mpnn::unpermute_vec3(cx, cx.vel.as<double>(), cx.stage_vel.as<double>()));
            }
            double box[3] = {cx.box[0], cx.box[1], cx.box[2]};
            MPNN_TRY(mpnn::build_neighbors(cx, cx.stage_pos.as<double>(), cx.types_caller.as<int32_t>(), cx.n, box,
                                           cx.skin, cx.stage_vel.as<double>()));
        } else if (vel) {
            MPNN_TRY(mpnn::permute_in_vec3(cx, vel, cx.vel.as<double>()));
        }
        MPNN_HIP(hipStreamSynchronize(cx.stream));
        return Status::ok();
    };
    return mpnn::finish(ctx, run());
}

mpnn_status mpnn_get_state(mpnn_ctx *ctx, double *pos, double *vel, int64_t *step) {
    if (!ctx) return MPNN_E_INVALID_ARG;
    mpnn::Context &cx = ctx->cx;
    if (!cx.built) return mpnn::finish(ctx, Status::err(MPNN_E_STATE, "mpnn_build_neighbors first"));
    auto run = [&]() -> Status {
        if (pos) MPNN_TRY(mpnn::unpermute_vec3(cx, cx.pos.as<double>(), pos));
        if (vel) MPNN_TRY(mpnn::unpermute_vec3(cx, cx.vel.as<double>(), vel));
        if (step) *step = cx.step;
        MPNN_HIP(hipStreamSynchronize(cx.stream));
        return Status::ok();
    };
    return mpnn::finish(ctx, run());
}

mpnn_status mpnn_get_pairs(mpnn_ctx *ctx, int64_t cap, int64_t *n_pairs, int32_t *i, int32_t *j,
                           int32_t *shift) {
    if (!ctx || !n_pairs) return MPNN_E_INVALID_ARG;
    mpnn::Context &cx = ctx->cx;
    if (!cx.built) return mpnn::finish(ctx, Status::err(MPNN_E_STATE, "mpnn_build_neighbors first"));
    if (cap > 0 && (!i || !j || !shift)) return mpnn::finish(ctx, Status::err(MPNN_E_INVALID_ARG, "null output"));
    auto run = [&]() -> Status {
        MPNN_TRY(mpnn::get_pairs(cx, cap, n_pairs, i, j, shift));
        MPNN_HIP(hipStreamSynchronize(cx.stream));
        return Status::ok();
    };
    return mpnn::finish(ctx, run());
}

mpnn_status mpnn_get_intermediate(mpnn_ctx *ctx, int32_t which, int32_t t, double *out) {
    if (!ctx || !out) return MPNN_E_INVALID_ARG;
    mpnn::Context &cx = ctx->cx;
    if (!cx.built || !cx.forces_valid) return mpnn::finish(ctx, Status::err(MPNN_E_STATE, "no evaluation yet"));
    if (which != 3 && (t < 0 || t >= cx.T)) return mpnn::finish(ctx, Status::err(MPNN_E_INVALID_ARG, "bad layer"));
    if (which == 4 && cx.T < 2) return mpnn::finish(ctx, Status::err(MPNN_E_INVALID_ARG, "no message layers"));
    const int KM = cx.K * cx.M;
    auto run = [&]() -> Status {
        switch (which) {
            case 0:
                MPNN_TRY(mpnn::unpermute_rows(cx, cx.c.as<float>() + (int64_t)t * cx.NN * mpnn::rec_stride(cx.K) + mpnn::kRecC,
                                              cx.K, mpnn::rec_stride(cx.K), out));
                break;
            case 1:
                MPNN_TRY(mpnn::unpermute_float(cx, cx.O.as<float>() + (int64_t)t * cx.np * mpnn::pad16(KM), KM, cx.np, out));
                break;
            case 2:
                MPNN_TRY(cx.grow(cx.tmp_a, sizeof(float) * (size_t)(cx.n > 0 ? cx.n : 1) * KM));
                MPNN_TRY(mpnn::assemble_go(cx, t, cx.tmp_a.as<float>()));
                MPNN_TRY(mpnn::unpermute_float(cx, cx.tmp_a.as<float>(), KM, 0, out));
                break;
            case 3:
                MPNN_TRY(mpnn::unpermute_scalar(cx, cx.Ei.as<double>(), out));
                break;
            case 4:
                if (t < 1) return Status::err(MPNN_E_INVALID_ARG, "dE/dc^t exists for t >= 1");
                MPNN_TRY(mpnn::unpermute_float(cx, cx.Gc.as<float>() + (int64_t)t * cx.NN * cx.K, cx.K, 0, out));
                break;
            default:
                return Status::err(MPNN_E_INVALID_ARG, "bad selector");
        }
        MPNN_HIP(hipStreamSynchronize(cx.stream));
        return Status::ok();
    };
    return mpnn::finish(ctx, run());
}

mpnn_status mpnn_get_info(mpnn_ctx *ctx, mpnn_info *info) {
    if (!ctx || !info) return MPNN_E_INVALID_ARG;
    mpnn::Context &cx = ctx->cx;
    info->n_local = cx.n;
    info->n_ghost = cx.G;
    info->n_edges = cx.E;
    for (int a = 0; a < 3; ++a) info->cells[a] = cx.nc[a];
    info->bytes_device = (int64_t)cx.device_bytes;
    info->row_bucketing = cx.bucket ? 1 : 0;
    info->n_slots = cx.E_sell;
    return mpnn::finish(ctx, Status::ok());
}

mpnn_status mpnn_set_profiling(mpnn_ctx *ctx, int32_t enable) {
    if (!ctx) return MPNN_E_INVALID_ARG;
    mpnn::Context &cx = ctx->cx;
    if (hipStreamSynchronize(cx.stream) != hipSuccess)
        return mpnn::finish(ctx, Status::err(MPNN_E_HIP, "stream sync failed"));
    cx.prof_harvest();
    for (int i = 0; i < mpnn::kProfCount; ++i) {
        cx.prof_ms[i] = 0.0;
        cx.prof_launches[i] = 0;
    }
    cx.prof_on = enable != 0;
    return mpnn::finish(ctx, Status::ok());
}

mpnn_status mpnn_get_profile(mpnn_ctx *ctx, int32_t idx, const char **name, double *total_ms, int64_t *launches) {
    if (!ctx || idx < 0 || idx >= mpnn::kProfCount) return MPNN_E_INVALID_ARG;
    mpnn::Context &cx = ctx->cx;
    if (name) *name = mpnn::kProfNames[idx];
    if (total_ms) *total_ms = cx.prof_ms[idx];
    if (launches) *launches = cx.prof_launches[idx];
    return mpnn::finish(ctx, Status::ok());
}

const char *mpnn_last_error(const mpnn_ctx *ctx) { return ctx ? ctx->cx.last_error.c_str() : "null context"; }

}  // extern "C"
