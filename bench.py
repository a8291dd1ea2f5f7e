"""Benchmark: atom-steps/s of the MPNN energy+force+MD hot path on one MI355X.

Workload (default): fcc Ag, 80^3 conventional cells = 2,048,000 local atoms (one GPU's
subdomain of a 100M-atom run) plus the periodic-image ghost shell of width rc + skin;
T = 3 message-passing layers, K = 8 radial primitives, L = 2, MLP 2x64 SiLU, rc = 6 A,
skin = 1 A; velocity-Verlet steps of 1 fs with a neighbour rebuild every 20 steps.
One "step" = one MD step of the whole path (half-kick + drift, skin test, rebuild when due,
ghost refresh, T forward layers, energy network, reverse pass, force gather, half-kick).

Prints ONE JSON line.  Timing: warmup steps untimed, then `--steps` steps bracketed by
torch.cuda.synchronize(); inputs are resident in HBM before the timed region, and nothing else
(no profiler) runs inside it.  Per-kernel durations come from a separate pass of profiled steps
afterwards: the library's hipEvent profiler on the stream the kernels run on.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
FP32_VALU_TFLOPS = 157.3       # MI355X published fp32 vector peak
FP32_MFMA_TFLOPS = 157.3       # MI355X published dense fp32 matrix peak
MFMA_PEAK_TFLOPS = {0: FP32_MFMA_TFLOPS, 1: 78.6, 2: 2500.0}   # by arithmetic mode: fp32, fp64, bf16
DTYPE = {0: "f32", 1: "f64", 2: "f32 (bf16 MLP operands)"}
METRIC = "atom-steps/s (E+F, T=3) on 2.05M-atom Ag subdomain, 1 MI355X; % HBM roof"


# Algorithmic HBM bytes per atom-step of each part of the path on the 2.05M-atom Ag subdomain
# (K = 8, L = 2, H = 64, T = 3; 54 active and 78.9 Verlet neighbours per atom), the budget of the
# minimal design: forward edges = the Verlet index (79 x 4 B) and the O row written (320 B) per
# layer; the networks read their feature rows and write their outputs once; the reverse edge pass
# reads a transposed index and the dE/dO rows and writes 12 B of dE/dr per active edge; the force
# gather reads those back; integrator, ghost refresh and the amortised rebuild take the rest.
AG2M_BYTES_PER_ATOM_STEP = {
    "forward_edges": 2100, "networks_forward": 1300, "networks_vjp": 1300,
    "reverse_edges": 4000, "force_gather": 1500, "integrate_ghosts_rebuild": 300,
}
AG2M_TOTAL = sum(AG2M_BYTES_PER_ATOM_STEP.values())   # 10.5 KB per atom-step


def ag2m_alg_bytes(fam, g):
    """Bytes per launch of kernel family `fam` from the per-atom-step budget above (the 2.05M-atom
    Ag workload only): each family gets the parts of the path it performs, spread over its
    launches per step; None for families that the budget counts inside another part."""
    N, T = g["N"], g["T"]
    B = AG2M_BYTES_PER_ATOM_STEP
    per_launch = {
        "aggregate": B["forward_edges"] / T,
        "net_forward": B["networks_forward"] / T,
        "net_energy": B["networks_forward"] / T + B["networks_vjp"] / T,
        "net_backward": B["networks_vjp"] / T,
        # the receiver pass of the reverse edges (its sender-major gathers are inside this budget)
        "backward_layer": B["reverse_edges"] / T,
        "force_gather": B["force_gather"],
    }.get(fam)
    return None if per_launch is None else per_launch * N


def kernel_model(fam, g):
    """Itemised (bytes, flops, kind) per launch of kernel family `fam`, for any workload.

    Bytes count each array the kernel must touch once (index streams, per-atom state read or
    written, per-edge outputs); gathered neighbour data (positions, messages) is counted once
    per node, not per edge.  Flops count the contractions of the method per active edge or
    per atom (multiply-add = 2), not the basis transcendentals.  N local atoms, NN nodes,
    EL Verlet entries, EA active entries (d < rc); per-atom rows are padded to 16 floats
    (KMP = pad16(K M) orbital coefficients, DP = pad16(D) density features)."""
    N, NN, EL, EA = g["N"], g["NN"], g["EL"], g["EA"]
    K, M, D, H, T = g["K"], g["M"], g["D"], g["H"], g["T"]
    KM = K * M
    KMP, DP = (KM + 15) // 16 * 16, (D + 15) // 16 * 16
    if fam == "compact":
        # row lengths, neighbour ids, fp32 positions (per node), activity bits, active list, counts
        b = 4 * N + 4 * EL + 16 * NN + EL / 8 + 4 * EA + 4 * N
        return b, 8 * EL, "hbm"
    if fam == "aggregate":
        # counts, active list, positions and messages (per node); O and feature rows out
        b = 4 * N + 4 * EA + 24 * NN + 4 * K * NN + 4 * KMP * N + 4 * DP * N
        f = EA * (2 * KM + 2 * K)
        return b, f, "alu"
    if fam == "backward_layer":
        w_frac = (T - 1) / T                       # layers that emit dE/dc edge terms
        g_rw = (12 + 24 * (T - 1)) / T             # first layer writes dE/dr, later ones accumulate
        b = (4 * N + 4 * EA + 24 * NN + 4 * K * NN + 4 * DP * N + 4 * KMP * N
             + w_frac * 4 * K * EA + g_rw * EA + 24 * N * (2 * T - 1) / T)
        f = EA * (4 * KM + 6 * K + 6 * M)
        return b, f, "alu"
    if fam == "message_grad":
        # segment offsets (per node), the transposed active map (per Verlet entry; built once per
        # evaluation by its own kernel), w_e (per active edge), dE/dc rows out (per node)
        b = 8 * NN + 4 * EL + 4 * K * EA + 4 * K * NN
        return b, K * EA, "hbm"
    if fam == "force_gather":
        b = 8 * NN + 4 * EL + 12 * EA + 8 * N + 24 * N + 48 * N
        return b, 3 * EA, "hbm"
    SA = g.get("SA", False)   # fp32 message networks: silu' saved forward, read back in reverse
    if fam == "net_forward":
        b = 4 * DP * N + 4 * K * N + (8 * H * N if SA else 0)
        f = N * 2 * (H * D + H * H + K * H)
        return b, f, "mfma"
    if fam == "net_energy":
        b = 4 * DP * N + 4 * N + 4 * DP * N
        f = N * 2 * (2 * H * D + 2 * H * H + 2 * H)
        return b, f, "mfma"
    if fam == "net_backward":
        if SA:   # the vector-Jacobian product alone
            return 4 * K * N + 8 * H * N + 4 * DP * N, N * 2 * (H * D + H * H + K * H), "mfma"
        b = 4 * DP * N + 4 * K * N + 4 * DP * N
        f = N * 2 * (2 * H * D + 2 * H * H + K * H + K * H)
        return b, f, "mfma"
    return None


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_ag2m.json")


def csrc_digest():
    """SHA-256 over the HIP sources, to tell whether stored counter readings are current."""
    import hashlib
    d = os.path.join(ROOT, "molecular_dynamics_cell_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".h")):
            h.update(f.encode())
            with open(os.path.join(d, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()


def measured_traffic(fam, cfg, precision=0, contracted=False):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE readings (scaled
    by the copy-kernel calibration; taken on the 2.05M-atom Ag workload in fp32 mode, base model),
    or None if absent, taken on different kernel sources or for another workload, mode or model."""
    if cfg != 4 or precision != 0 or contracted or not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    k = t.get("kernels", {}).get(fam)
    if k is None or t.get("source_sha256") != csrc_digest():
        return None
    return int((k["fetch_kib"] * t["fetch_scale"] + k["write_kib"] * t["write_scale"]) * 1024)


VALU_FILE = os.path.join(ROOT, "profiles", "valu_ag2m.json")


def measured_valu(fam, cfg, precision=0, contracted=False):
    """VALU utilisation of kernel family `fam` from the committed rocprofv3 SQ counter pass on the
    2.05M-atom Ag workload (fp32 mode, base model), or None if absent or taken on other sources."""
    if cfg != 4 or precision != 0 or contracted or not os.path.exists(VALU_FILE):
        return None
    with open(VALU_FILE) as f:
        t = json.load(f)
    k = t.get("kernels", {}).get(fam)
    if k is None or t.get("source_sha256") != csrc_digest():
        return None
    return k


def roofline_for(fam, ms_avg, g, cfg=4, precision=0, contracted=False):
    """The kernel's HBM roofline: achieved = algorithmic bytes per launch (the 2.05M-atom budget
    where it applies, else the itemised model) / its average duration, against the 8 TB/s peak.
    Matrix-core kernels (the networks) report their MFMA rate against the mode's matrix peak
    instead.  `traffic` = measured HBM bytes per launch (rocprofv3 counters) when current."""
    layout_b, flops, kind = kernel_model(fam, g)
    alg = ag2m_alg_bytes(fam, g) if cfg == 4 and g["K"] == 8 and g["T"] == 3 else None
    bytes_ = alg if alg is not None else layout_b
    traffic = measured_traffic(fam, cfg, precision, contracted)
    t = ms_avg * 1e-3
    gbs = bytes_ / t / 1e9
    out = {"kernel": fam, "avg_ms": round(ms_avg, 4), "traffic": traffic,
           "algorithmic_bytes": int(bytes_),
           "bytes_basis": "per-atom-step budget" if alg is not None else "itemised model",
           "itemised_bytes": int(layout_b), "algorithmic_flops": int(flops)}
    if kind == "mfma":
        peak = MFMA_PEAK_TFLOPS[precision]
        tfs = flops / t / 1e12
        out.update({"bound": "mfma", "achieved": round(tfs, 2), "peak": peak, "unit": "TFLOP/s",
                    "frac": round(tfs / peak, 4), "hbm_GBs_at_algorithmic_bytes": round(gbs, 1)})
    else:
        out.update({"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(gbs / HBM_PEAK_GBS, 4)})
        if kind == "alu":
            out["valu_tflops_at_algorithmic_flops"] = round(flops / t / 1e12, 2)
    v = measured_valu(fam, cfg, precision, contracted)
    if v is not None:
        out["valu_busy"] = v.get("valu_busy")            # % of SIMD cycles issuing VALU (SQ counters)
        out["valu_insts_per_unit"] = v.get("valu_insts_per_unit")   # per lane-edge
        out["ta_busy"] = v.get("ta_busy")                # % of cycles the texture-address unit is busy
    return out


def _oracle_sample(cfg):
    """A bounded periodic sample of workload `cfg` with the same model (seconds of oracle work)."""
    from molecular_dynamics_cell_amd import inputs as I
    if cfg in (1, 4):
        return I.ag(10, 1004, 1104, name="Ag4000"), "fcc Ag 10^3 cells (4,000 atoms, periodic), same model and lattice"
    if cfg == 3:
        return I.hea(13), "bcc HEA 13^3 cells (4,394 atoms, periodic), same model"
    if cfg == 5:
        return I.make_system(5, reduced=True), "CHON gas, 4,002 atoms at 0.5 g/cm3, same model"
    return I.make_system(2), "the full 4,608-atom water box"


def _oracle_md_rate(cfg, budget_s):
    """atom-steps/s of the oracle's velocity-Verlet loop on the bounded sample, sized to about
    budget_s seconds; returns (rate, steps, seconds, threads, sample text)."""
    import oracle
    from molecular_dynamics_cell_amd import inputs as I
    p = I.make_params(cfg)
    s, sample = _oracle_sample(cfg)
    m = oracle.Model(p)
    rb = I.CONFIGS[cfg]["rebuild_every"]
    dt = I.CONFIGS[cfg]["dt"]
    t0 = time.perf_counter()
    oracle.md(m, s.pos, s.vel, s.types, s.masses, s.box, dt, 2, rebuild_every=rb)
    t1 = (time.perf_counter() - t0) / 3          # 2 steps plus the initial evaluation
    steps = int(max(1, min(1000, budget_s / max(t1, 1e-3))))
    t0 = time.perf_counter()
    oracle.md(m, s.pos, s.vel, s.types, s.masses, s.box, dt, steps, rebuild_every=rb)
    el = time.perf_counter() - t0
    return s.n * steps / el, steps, el, oracle.num_threads(), sample


def cpu_baseline(cfg, system=None, full=True, sample_budget_s=10.0):
    """The fp64 oracle as it stands, on this host's cores: on the full workload (one E+F, then one
    velocity-Verlet step; rate = N / time of that step) where it fits a minute, and on a bounded
    sample of the same workload with all threads and with one thread (a child process started
    with OMP_NUM_THREADS=1, which touches no GPU)."""
    import subprocess
    import oracle
    from molecular_dynamics_cell_amd import inputs as I
    out = {"unit": "atom-steps/s", "kind": "oracle"}
    rate, steps, el, thr, sample = _oracle_md_rate(cfg, sample_budget_s)
    out["sample_all_threads"] = {"value": round(rate, 1), "threads": thr,
                                 "sample": f"{sample}; {steps} velocity-Verlet steps in {el:.1f} s"}
    env = dict(os.environ, OMP_NUM_THREADS="1")
    code = ("import json, sys; sys.path.insert(0, %r); import bench; "
            "print(json.dumps(bench._oracle_md_rate(%d, %f)))" % (ROOT, cfg, sample_budget_s))
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=600)
    if r.returncode == 0:
        r1 = json.loads(r.stdout.strip().splitlines()[-1])
        out["sample_one_thread"] = {"value": round(r1[0], 1), "threads": r1[3],
                                    "sample": f"{r1[4]}; {r1[1]} velocity-Verlet steps in {r1[2]:.1f} s"}
    if full and system is not None:
        p = I.make_params(cfg)
        m = oracle.Model(p)
        s = system
        t0 = time.perf_counter()
        oracle.energy_forces(m, oracle.wrap(s.pos, s.box), s.types, s.box)
        t_ef = time.perf_counter() - t0
        print(f"cpu_baseline: oracle E+F on {s.n} atoms in {t_ef:.1f} s", file=sys.stderr, flush=True)
        t0 = time.perf_counter()
        oracle.md(m, s.pos, s.vel, s.types, s.masses, s.box, I.CONFIGS[cfg]["dt"], 1,
                  rebuild_every=I.CONFIGS[cfg]["rebuild_every"])
        t_md = time.perf_counter() - t0
        t_step = max(t_md - t_ef, 1e-9)
        out.update({"value": round(s.n / t_step, 1), "cores": oracle.num_threads(),
                    "sample": f"the full workload ({s.n} atoms): one E+F in {t_ef:.1f} s, then "
                              f"E+F + one velocity-Verlet step in {t_md:.1f} s; value = N / "
                              f"({t_md:.1f} - {t_ef:.1f}) s"})
    else:
        out.update({"value": out["sample_all_threads"]["value"], "cores": thr,
                    "sample": out["sample_all_threads"]["sample"]})
    return out


def bandwidth(gib=4, reps=10):
    """Practical HBM rates of plain device copies (torch kernels): the ceiling the
    memory-bound kernels can approach, next to the 8 TB/s published peak."""
    import torch
    d = torch.device("cuda:0")
    a = torch.ones(gib * (1 << 28), dtype=torch.float32, device=d)
    b = torch.empty_like(a)
    nbytes = a.numel() * 4

    def rate(f, moved):
        f()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            f()
        e1.record()
        torch.cuda.synchronize()
        return round(moved / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9, 1)

    return {"unit": "GB/s", "bytes": nbytes, "peak": HBM_PEAK_GBS,
            "copy_read_plus_write": rate(lambda: b.copy_(a), 2 * nbytes),
            "fill_write": rate(lambda: b.fill_(1.0), nbytes),
            "sum_read": rate(lambda: a.sum(), nbytes)}


def t_sweep(cfg=4, max_t=6, evals=10):
    """Cost of one E+F evaluation against the number of message-passing layers T (the pages' claim
    of a cost linear in T) on workload cfg (the 2.05M-atom Ag subdomain or the 4,608-atom water box)
    with random-init models of each depth (inputs.depth_variant), and, for Ag, the per-layer
    ghost-refresh volume against subdomain size (surface, not volume, scaling)."""
    import torch
    from molecular_dynamics_cell_amd import binding, inputs as I
    dev = torch.device("cuda:0")
    s = I.make_system(cfg)
    rows = []
    for T in range(1, max_t + 1):
        p = I.depth_variant(cfg, T)
        m = binding.MPNN(p, dev)
        m.build_neighbors(torch.tensor(s.pos, device=dev), torch.tensor(s.types, device=dev), s.box)
        m.energy_forces(energy=False)
        ts = []
        for _ in range(evals):
            torch.cuda.synchronize()
            a0 = time.perf_counter()
            m.energy_forces(energy=False)
            torch.cuda.synchronize()
            ts.append(time.perf_counter() - a0)
        ms = float(np.median(ts)) * 1e3
        rows.append({"T": T, "ef_ms": round(ms, 4), "atom_steps_per_s": round(s.n / ms * 1e3, 1)})
        print(f"T={T}: {ms:.4f} ms per E+F", file=sys.stderr, flush=True)
        m.close()
        torch.cuda.empty_cache()
    # linear fit ms = a + b T
    Ts = np.array([r["T"] for r in rows], float)
    ys = np.array([r["ef_ms"] for r in rows])
    b, a = np.polyfit(Ts, ys, 1)
    resid = float(np.max(np.abs(ys - (a + b * Ts)) / ys))
    halo = []
    if cfg == 4:
        p = I.make_params(4)
        for cells in (20, 40, 80):
            g = I.ag(cells, 1004, 1104, name=f"Ag{cells}")
            m = binding.MPNN(p, dev)
            m.build_neighbors(torch.tensor(g.pos, device=dev), torch.tensor(g.types, device=dev), g.box)
            info = m.info()
            halo.append({"fcc_cells": cells, "atoms": g.n, "ghosts": info["n_ghost"],
                         "ghost_fraction": round(info["n_ghost"] / g.n, 4),
                         "refresh_bytes_per_layer": info["n_ghost"] * p.spec.K * 4})
            m.close()
            torch.cuda.empty_cache()
    spec = I.make_params(cfg).spec
    return {"sweep": f"E+F cost vs layers T, {s.name} ({s.n} atoms; random-init models, K={spec.K}, "
                     f"L={spec.L}, H={spec.H})",
            "rows": rows, "fit_ms": {"fixed": round(float(a), 4), "per_layer": round(float(b), 4),
                                     "max_rel_residual": round(resid, 4)},
            "halo": halo}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed MD steps (default: the workload's run length; 200 for the Ag subdomain)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed MD steps first (default: steps / 10)")
    ap.add_argument("--config", type=int, default=4, help="benchmark system 1..5 (default 4)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sample-baseline", action="store_true",
                    help="time the oracle on the bounded sample only (not on the full workload)")
    ap.add_argument("--no-profile", action="store_true", help="skip the per-kernel event timing")
    ap.add_argument("--ef-evals", type=int, default=10)
    ap.add_argument("--precision", type=int, choices=(0, 1, 2), default=None,
                    help="arithmetic mode (0 fp32 orbital sums/networks, 1 fp64, 2 fp32 sums with bf16 "
                         "network operands); default: the workload's")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="also launch one device copy of this many MiB (counter calibration)")
    ap.add_argument("--graph-replay", type=int, default=None,
                    help="MD steps per captured replay (0: eager; default: 8 below 1,000 atoms, else 0)")
    ap.add_argument("--subdomains", type=str, default="1,1,1",
                    help="px,py,pz virtual subdomains (per-layer ghost refresh between them)")
    ap.add_argument("--bandwidth", action="store_true",
                    help="instead of the benchmark line: device copy / fill / read rates (practical HBM ceiling)")
    ap.add_argument("--contraction", type=int, default=None, metavar="SEED",
                    help="time the contraction variant of the model (a seeded random K x K contraction "
                         "of the radial primitives, with layer scales frozen for it: seed 7 on the Ag "
                         "subdomain)")
    ap.add_argument("--t-sweep", action="store_true",
                    help="instead of the benchmark line: E+F cost vs layers T and ghost volume vs size")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: measures one GPU only (the library decomposes a box into subdomains on one "
              "device; there is no multi-GPU halo exchange); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.t_sweep:
        print(json.dumps(t_sweep(args.config)))
        return
    if args.bandwidth:
        print(json.dumps(bandwidth()))
        return

    import torch
    from molecular_dynamics_cell_amd import binding, inputs as I

    dev = torch.device("cuda:0")
    cfg = args.config
    c = I.CONFIGS[cfg]
    if args.steps is None:
        # the workload's run length; the random-init water model drives molecules into a deep
        # well within 6-8 fs at dt = 0.5 fs (the oracle integrator does the same), so its timed
        # run is cut to 8 steps (4 fs)
        args.steps = 8 if cfg == 2 else c["steps"]
    if args.warmup is None:
        args.warmup = max(1, args.steps // 10)
    t_setup = time.perf_counter()
    s = I.make_system(cfg)
    p = I.make_params(cfg, contraction_seed=args.contraction)
    if args.precision is not None:
        p.spec.precision = args.precision
    contracted = p.contraction is not None
    m = binding.MPNN(p, dev)
    sub = tuple(int(x) for x in args.subdomains.split(","))
    m.set_subdomains(*sub)
    pos = torch.tensor(s.pos, device=dev)
    m.build_neighbors(pos, torch.tensor(s.types, device=dev), s.box)
    m.set_state(vel=torch.tensor(s.vel, device=dev))
    info = m.info()
    # active edges (d < rc) of the initial configuration, for the algorithmic work model
    pi, pj, ps = m.get_pairs()
    pw = pos.remainder(torch.tensor(s.box, device=dev))
    r = pw[pj.long()] + ps.double() * torch.tensor(s.box, device=dev) - pw[pi.long()]
    EA = int((r.square().sum(1) < p.spec.rc ** 2).sum().item())
    del pi, pj, ps, r, pw
    torch.cuda.empty_cache()
    print(f"setup {time.perf_counter() - t_setup:.1f} s: {info}", file=sys.stderr, flush=True)

    if args.copy_mib:
        a = torch.ones(args.copy_mib * 262144, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    # replayed chunks pay off where launch latency dominates (the 108-atom cell); the 4,608-atom
    # water run is short and rebuilds inside it, so a rolled-back chunk and re-recording cost more
    replay = args.graph_replay if args.graph_replay is not None else (8 if s.n < 1_000 else 0)
    m.set_graph_replay(replay)
    E0, _, _ = m.energy_forces()
    # warm-up covers at least one full replayed chunk, so its recording is not timed
    m.md_step(c["dt"], max(args.warmup, replay), c["rebuild_every"], stats=False)
    torch.cuda.synchronize()
    # timed region: the MD steps alone (the fp64 energy sum runs inside every step)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    st = m.md_step(c["dt"], args.steps, c["rebuild_every"], stats=False)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    # per-kernel durations: a separate pass of profiled steps (event pairs on the library's stream)
    prof = {}
    if not args.no_profile:
        m.set_profiling(True)
        m.md_step(c["dt"], max(1, min(args.steps, 20)), c["rebuild_every"], stats=False)
        torch.cuda.synchronize()
        prof = m.profile()
        m.set_profiling(False)
    st = m.md_step(c["dt"], 0, c["rebuild_every"])      # energies at the end of the run
    elapsed = t1 - t0
    value = s.n * args.steps / elapsed

    # E+F only: median of evaluations on the current state
    ef = []
    for _ in range(args.ef_evals):
        torch.cuda.synchronize()
        a0 = time.perf_counter()
        m.energy_forces(energy=False)
        torch.cuda.synchronize()
        ef.append(time.perf_counter() - a0)
    ef_rate = s.n / float(np.median(ef)) if ef else None

    g = dict(N=s.n, NN=info["n_local"] + info["n_ghost"], EL=info["n_edges"], EA=EA, K=p.spec.K,
             M=(p.spec.L + 1) * (p.spec.L + 2) * (p.spec.L + 3) // 6, D=p.D, H=p.spec.H, T=p.spec.T,
             SA=p.spec.precision == 0 and p.spec.T > 1)
    kernels = {k: {"ms_total": round(v[0], 3), "launches": v[1],
                   "ms_avg": round(v[0] / v[1], 4) if v[1] else 0.0}
               for k, v in prof.items() if v[1]}
    roof = None
    modeled = [k for k in kernels if kernel_model(k, g) is not None]
    if modeled:
        dom = max(modeled, key=lambda k: kernels[k]["ms_total"])
        roof = roofline_for(dom, kernels[dom]["ms_avg"], g, cfg, p.spec.precision, contracted)
    for k in modeled:
        kernels[k]["roofline"] = roofline_for(k, kernels[k]["ms_avg"], g, cfg, p.spec.precision, contracted)
    # whole step against the HBM roof: atom-steps/s x algorithmic bytes per atom-step / 8 TB/s
    # (the per-atom-step budget on the 2.05M-atom workload; elsewhere the sum of the itemised
    # per-launch bytes of one profiled step)
    if cfg == 4 and g["K"] == 8 and g["T"] == 3:
        bpas, basis = float(AG2M_TOTAL), "per-atom-step budget"
    elif kernels:
        nsteps = max(1, min(args.steps, 20))
        tot = sum(kernel_model(k, g)[0] * v["launches"] for k, v in kernels.items() if kernel_model(k, g))
        bpas, basis = tot / nsteps / s.n, "itemised model of the profiled steps"
    else:
        bpas, basis = None, None
    whole = None
    if bpas:
        gbs = value * bpas / 1e9
        whole = {"bytes_per_atom_step": round(bpas, 1), "bytes_basis": basis, "achieved_GBs": round(gbs, 1),
                 "peak": HBM_PEAK_GBS, "frac": round(gbs / HBM_PEAK_GBS, 4)}

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "atom-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE[p.spec.precision],
        "data": "synthetic",
        "config": {"workload": f"{s.name}: {s.n} atoms + {info['n_ghost']} ghosts, T={p.spec.T}, "
                               f"K={p.spec.K}, L={p.spec.L}, MLP 2x{p.spec.H}, rc={p.spec.rc}, "
                               f"skin={p.spec.skin}, dt={c['dt']} fs, rebuild every {c['rebuild_every']}",
                   "atoms": s.n, "ghosts": info["n_ghost"], "verlet_entries": info["n_edges"],
                   "active_edges": EA, "contraction": contracted, "parallelism": "single GPU" if sub == (1, 1, 1) else
                   "single GPU, {}x{}x{} virtual subdomains".format(*sub), "graph_replay_steps": replay},
        "roofline": roof,
        "hbm_roof_whole_step": whole,
        "ef_only_atom_steps_per_s": round(ef_rate, 1) if ef_rate else None,
        "md": {"epot_start": E0, "epot_end": st["epot"], "ekin_end": st["ekin"],
               "temp_end": st["temp"], "steps_total": st["steps"],
               # neighbour rebuilds among the profiled steps (scheduled or displacement-triggered)
               "rebuilds_profiled": kernels.get("build_rows", {}).get("launches", 0) if kernels else None},
        "kernels": kernels,
    }
    if not args.no_cpu_baseline:
        m.close()
        del m, pos
        torch.cuda.empty_cache()
        out["cpu_baseline"] = cpu_baseline(cfg, system=s, full=not args.sample_baseline)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
