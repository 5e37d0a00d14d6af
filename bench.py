"""Benchmark of the fused selective scan on one MI355X.

One step = one full pass of the scan (discretise, scan over L, C-contraction,
D skip term, final state) over one batch of synthetic input already resident in
device memory; for a backward workload, one full backward pass (every
gradient); for a training-step workload, the forward pass that also keeps the
state entering every 32-step round, then the backward pass that reads those
states instead of rebuilding them. Three input sets are rotated so that consecutive steps do not
re-read a working set left in the 256 MB last-level cache.

Prints ONE JSON line. `value` is scan elements (Bs*L*ED*N) per second;
`roofline` describes the dominant kernel against the HBM peak (algorithmic
bytes per launch over its per-launch time, measured with HIP events on the
stream it is launched on); `valu` puts the same time against the vector-ALU
issue peak; `cpu_baseline` is the fp64 oracle on the host cores over the same
workload.

`--micro valu` instead measures the vector ALU's issue rates (float32 FMA,
v_exp_f32, and the two mixed 4:1) with the probe kernels of
csrc/valu_probe.hip; the ALU cost model below rests on those rates.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# the largest single-GPU configuration: the long-sequence float32 scan (Bs 1,
# L 2^17, ED 2048, N 16), which splits the sequence across workgroups
DEFAULT_WORKLOAD = "fwd_f32_Bs1_L131072_ED2048_N16"
METRIC = "scan elements (Bs·L·ED·N)/s and achieved HBM GB/s vs MI355X peak"

# MI355X published figures
HBM_PEAK_GBPS = 8000.0
CUS, SIMDS, CLOCK_GHZ = 256, 4, 2.4
# float32 vector peak in FMA lane-ops per second: the published 157.3 TFLOP/s
# counted as two flops per FMA, i.e. 32 FMA lanes per SIMD per clock
# (256 CUs x 4 SIMDs x 32 x 2.4 GHz). `bench.py --micro valu` measures 65 T
# non-packed FMA lane-ops/s with two or more waves per SIMD, 29 T with one.
VALU_SLOTS_PER_S = CUS * SIMDS * 32 * CLOCK_GHZ * 1e9
# FMA slots one v_exp_f32 costs: that peak over the measured exp rate
# (19.3 T lane-ops/s at any occupancy): 4.07, rounded to 4
EXP_SLOTS = 4.0
# algorithmic VALU cost of one scan element: delta*A, (delta x)*B, the state
# FMA, the C FMA (4 full-rate slots) + one v_exp_f32
SLOTS_PER_ELEMENT = 4.0 + EXP_SLOTS
# bidirectional: the exp and the two multiplies are shared by both
# directions; 2 mul + exp + 2 x (state FMA + C FMA)
SLOTS_PER_ELEMENT_BIDIR = 6.0 + EXP_SLOTS
# backward: rebuild the state (delta*A, (delta x)*B, state FMA: 3, + the exp)
# and the adjoint with its terms (g FMA, k = a g, dC and dB products, sum g B,
# q = g a h_{t-1} (2), sum A q, dA += delta q: 9)
SLOTS_PER_ELEMENT_BWD = 12.0 + EXP_SLOTS
# bidirectional backward: both directions' 12, less the discretisation they
# share (delta*A, (delta x)*B: 2), and one exp
SLOTS_PER_ELEMENT_BIDIR_BWD = 22.0 + EXP_SLOTS


def alg_bytes(w):
    s = 4 if w["dtype"] == "f32" else 2
    Bs, L, ED, N = w["Bs"], w["L"], w["ED"], w["N"]
    b = Bs * L * ED * (2 * s + s) + 2 * Bs * L * N * s + 4 * ED * N + 4 * ED
    if w.get("bwd"):
        # read x, delta, dy, B, C, A, D; write dx, ddelta, dB, dC, dA, dD
        # (a training step adds the forward's bytes; the round states it
        # keeps for the backward are not counted)
        bb = Bs * L * ED * 5 * s + 4 * Bs * L * N * s + 2 * (4 * ED * N + 4 * ED)
        return bb + (b if w.get("train") else 0)
    if w.get("h_last"):
        b += 4 * Bs * ED * N
    return b


KERNEL_SOURCES = {
    "fwd": ("scan_common.h", "ssm_scan.hip"),
    "bwd": ("scan_common.h", "ssm_scan_bwd.hip"),
    "train": ("scan_common.h", "ssm_scan.hip", "ssm_scan_bwd.hip"),
    "ssd": ("scan_common.h", "ssm_ssd.hip"),
}


def kernel_family(workload):
    if workload.startswith("bwd"):
        return "bwd"
    if workload.startswith("train"):
        return "train"
    if workload.startswith("ssd"):
        return "ssd"
    return "fwd"


def kernel_source_hash(workload):
    """sha256[:16] over the HIP source files that the workload's kernels are
    built from (in the order listed in KERNEL_SOURCES)."""
    h = hashlib.sha256()
    src = os.path.join(ROOT, "state_space_model_selective_amd", "csrc")
    for name in KERNEL_SOURCES[kernel_family(workload)]:
        with open(os.path.join(src, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload, src_hash):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_sha256_16") != src_hash:
        return None
    return d.get("hbm_bytes_per_launch")


def host_cpus():
    """CPUs this process may run on (the host's core count as the scheduler
    offers it), and the host's total."""
    try:
        avail = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        avail = os.cpu_count() or 1
    return avail, os.cpu_count() or avail


def oracle_threads():
    """Threads the oracle baseline runs on: every CPU offered, at most 16 (a
    GPU machine shares its host between 8 GPUs: 16 CPUs per GPU)."""
    return min(16, host_cpus()[0])


def cpu_fields(threads):
    avail, total = host_cpus()
    return dict(cores=threads, threads=threads, host_cpus_available=avail, host_cpus_total=total)


def cpu_baseline(inp, w, budget_s=20.0):
    import numpy as np
    import oracle
    threads = oracle_threads()
    Bs, ED = w["Bs"], w["ED"]
    E_per_channel = w["L"] * w["N"] * (2 if w["bidir"] else 1)
    # time a small sample first, then size the measured sample to the budget
    probe = np.arange(0, min(Bs * ED, threads * 4), dtype=np.int64)
    t0 = time.perf_counter()
    oracle.scan(**inp, bidir=w["bidir"], chans=probe, nthreads=threads)
    dt = max(time.perf_counter() - t0, 1e-6)
    per_ch = dt / probe.size
    nch = int(min(Bs * ED, max(probe.size, budget_s / per_ch)))
    chans = None if nch >= Bs * ED else np.linspace(0, Bs * ED - 1, nch).astype(np.int64)
    # when the whole workload takes well under the budget, it is run several
    # times (at least min_s of CPU work in all) so that the rate is not one
    # short, noisy measurement
    min_s = min(10.0, budget_s)
    reps, dt = 0, 0.0
    while reps == 0 or (chans is None and dt < min_s):
        t0 = time.perf_counter()
        y_ref, _, _ = oracle.scan(**inp, bidir=w["bidir"], chans=chans, nthreads=threads)
        dt += time.perf_counter() - t0
        reps += 1
    n_eff = Bs * ED if chans is None else chans.size
    rate = reps * n_eff * E_per_channel / dt / (2 if w["bidir"] else 1)
    sample = ("all %d channels" % n_eff) if chans is None else ("%d of %d channels, every time step" % (n_eff, Bs * ED))
    if reps > 1:
        sample += ", %d runs" % reps
    return dict(value=rate, unit="scan elements/s", **cpu_fields(threads), kind="oracle",
                sample=sample + " (fp64 sequential recurrence, %.2f s)" % dt), y_ref, chans


def cpu_baseline_bwd(inp, dy, w, budget_s=20.0):
    """The oracle's backward pass (for a training step: its forward pass, then
    its backward pass) on the first batch rows of the workload (as many as fit
    the time budget, at least one)."""
    import numpy as np
    import oracle
    threads = oracle_threads()
    Bs = w["Bs"]
    train = bool(w.get("train"))

    def rows(k):
        sub = {n: (v[:k] if v.ndim == 3 else v) for n, v in inp.items()}
        return sub, dy[:k]

    def run(sub, dys):
        y = oracle.scan(**sub, bidir=bidir, nthreads=threads)[0] if train else None
        ref = oracle.scan_bwd(**sub, dy=dys, bidir=bidir, nthreads=threads)
        return ref if y is None else dict(ref, y=y)

    bidir = bool(w["bidir"])
    sub, dys = rows(1)
    t0 = time.perf_counter()
    ref = run(sub, dys)
    dt = max(time.perf_counter() - t0, 1e-6)
    k = int(min(Bs, max(1, budget_s / dt)))
    if k > 1:
        sub, dys = rows(k)
        t0 = time.perf_counter()
        ref = run(sub, dys)
        dt = time.perf_counter() - t0
    E = k * w["L"] * w["ED"] * w["N"]
    sample = ("all %d batch rows" % Bs) if k == Bs else ("%d of %d batch rows" % (k, Bs))
    what = "fp64 forward scan, then forward states + adjoint" if train else "fp64 forward states + adjoint"
    return dict(value=E / dt, unit="scan elements/s", **cpu_fields(threads), kind="oracle",
                sample=sample + " (%s, %.2f s)" % (what, dt)), ref, k


# dense fp32 matrix-core peak of the MI355X (the multi-head scan's products run there)
MFMA_F32_PEAK_TFLOPS = 157.3   # dense float32 matrix instructions
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix instructions
SSD_CHUNK = 32  # chunk length of the multi-head kernel


def ssd_flops(w):
    """Products of the chunked multi-head scan per launch: per (batch row,
    head) and chunk of Q steps, the causal C B^T (Q (Q+1)/2 N multiply-adds),
    its product with x (Q (Q+1)/2 P), C S^T (Q N P) and the state update
    (Q N P); 2 flops per multiply-add; twice that for the bidirectional scan
    (one sweep per direction)."""
    Q, P, N = SSD_CHUNK, w["P"], w["N"]
    chunks = (w["L"] + Q - 1) // Q
    per_chunk = 2 * (Q * (Q + 1) // 2 * (N + P) + 2 * Q * N * P)
    sweeps = 2 if w.get("bidir") else 1
    return sweeps * w["Bs"] * w["H"] * chunks * per_chunk


def bench_ssd(args, name):
    import numpy as np
    import torch
    import state_space_model_selective_amd as ssm
    import synth
    w = dict(synth.SSD_WORKLOADS[name])
    Bs, L, H, P, G, N = w["Bs"], w["L"], w["H"], w["P"], w["G"], w["N"]
    dev = torch.device("cuda:0")

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    bidir = bool(w.get("bidir"))
    nsets = 3
    sets, host0 = [], None
    for i in range(nsets):
        inp = synth.make_ssd_inputs(Bs, L, H, P, G, N, w["dtype"], seed=i)
        if i == 0:
            host0 = inp
        t = {k: to_dev(v) for k, v in inp.items()}
        t["y"] = torch.empty_like(t["x"])
        sets.append(t)
    stream = torch.cuda.current_stream(dev)
    # the workspace (a split sequence's range states; the bidirectional bf16
    # scan's partials) is allocated once, outside the timed region
    dcode = ssm.SSM_F32 if w["dtype"] == "f32" else ssm.SSM_BF16
    need = (ssm.ssm_ssd_bidir_workspace_bytes if bidir else ssm.ssm_ssd_workspace_bytes)(Bs, L, H, P, dcode)
    ws = torch.empty(need, dtype=torch.uint8, device=dev) if need else None

    def step(t):
        if bidir:
            ssm.ssm_ssd_bidir_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], y=t["y"], workspace=ws,
                                  stream=stream)
        else:
            ssm.ssm_ssd_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], y=t["y"], workspace=ws, stream=stream)

    for i in range(args.warmup):
        step(sets[i % nsets])
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(sets[i % nsets])
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    avg = ev0.elapsed_time(ev1) / 1e3 / args.steps
    E = Bs * L * H * P * N
    flops = ssd_flops(w)
    s = 4 if w["dtype"] == "f32" else 2
    alg_bytes = 2 * Bs * L * H * P * s + Bs * L * H * s + 2 * Bs * L * G * N * s + 8 * H

    cpu = parity = None
    if not args.no_cpu:
        import oracle
        threads = oracle_threads()

        def rows(k):
            return {n: (v[:k] if v.ndim >= 3 else v) for n, v in host0.items()}
        t1 = time.perf_counter()
        oracle.ssd(**rows(1), bidir=bidir, nthreads=threads)
        dt1 = max(time.perf_counter() - t1, 1e-6)
        k = int(min(Bs, max(1, 20.0 / dt1)))
        t1 = time.perf_counter()
        y_ref, _, _ = oracle.ssd(**rows(k), bidir=bidir, nthreads=threads)
        dtk = time.perf_counter() - t1
        cpu = dict(value=k * L * H * P * N / dtk, unit="scan elements/s", **cpu_fields(threads), kind="oracle",
                   sample=(("all %d batch rows" % Bs) if k == Bs else ("%d of %d batch rows" % (k, Bs))) +
                   " (fp64 sequential recurrence, %.2f s)" % dtk)
        step(sets[0])
        torch.cuda.synchronize()
        got = sets[0]["y"][:k].float().cpu().numpy().astype(np.float64)
        tol = 1e-4 if w["dtype"] == "f32" else 2e-2
        rel = float(np.max(np.abs(got - y_ref) / (1 + np.abs(y_ref))))
        parity = dict(max_rel_err=rel, tol=tol, passed=bool(rel <= tol))

    # float32 inputs run on the float32 matrix instructions, bf16 inputs on the
    # bf16 ones; the roofline is the resource whose time bound is the larger
    bf16 = w["dtype"] == "bf16"
    peak_mfma = MFMA_BF16_PEAK_TFLOPS if bf16 else MFMA_F32_PEAK_TFLOPS
    mfma = {"achieved_TFLOPs": flops / avg / 1e12, "peak_TFLOPs": peak_mfma,
            "frac": flops / avg / 1e12 / peak_mfma, "flops_per_launch": flops,
            "instruction": "v_mfma_f32_16x16x32_bf16" if bf16 else "v_mfma_f32_16x16x4f32"}
    hbm = {"alg_bytes_per_launch": alg_bytes, "achieved_GBps": alg_bytes / avg / 1e9, "peak_GBps": HBM_PEAK_GBPS,
           "frac": alg_bytes / avg / 1e9 / HBM_PEAK_GBPS}
    timed = (("the bidirectional multi-head scan kernel (one launch per step, both sweeps)" if bidir
              else "the multi-head scan kernel (one launch per step)") + "; products on the " +
             ("bf16 matrix instructions (float32 operands split into two bf16 parts)" if bf16
              else "float32 matrix instructions"))
    if flops / (peak_mfma * 1e12) >= alg_bytes / (HBM_PEAK_GBPS * 1e9):
        roofline = {"bound": "mfma", "achieved": mfma["achieved_TFLOPs"], "peak": peak_mfma, "unit": "TFLOP/s",
                    "frac": mfma["frac"]}
    else:
        roofline = {"bound": "hbm", "achieved": hbm["achieved_GBps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": hbm["frac"]}
    roofline.update({"traffic": load_traffic(name, kernel_source_hash(name)), "kernel_avg_us": avg * 1e6,
                     "timed": timed})

    out = {
        "metric": "multi-head scan elements (Bs·L·H·P·N)/s",
        "value": E / (wall / args.steps),
        "unit": "scan elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w["dtype"],
        "data": "synthetic (seeded counter-based generator; x,B,C,D ~ N(0,1), dt log-uniform [1e-3,1e-1], "
                "A[h] = -U(1,16)); 3 input sets rotated",
        "config": {"workload": name, "Bs": Bs, "L": L, "H": H, "P": P, "G": G, "N": N, "bidir": bidir,
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "mfma": mfma,
        "hbm": hbm,
        "kernel_source_sha256_16": kernel_source_hash(name),
        "parity": parity,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


def micro_valu(args):
    """Issue rates of the vector ALU: launches of 256-thread workgroups (one
    wave per SIMD each), 1, 2, 4 or 8 workgroups per compute unit, each thread
    running 8 independent chains; the rate is lane-operations per second of
    the kernel time (HIP events around `steps` launches on one stream)."""
    import ctypes
    import torch
    import state_space_model_selective_amd as ssm
    P = ssm.probe_lib()
    dev = torch.device("cuda:0")
    ncu = torch.cuda.get_device_properties(dev).multi_processor_count
    out = torch.empty(8 * ncu * 256, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    kinds = ((0, "fma", 4096), (1, "exp", 2048), (2, "exp_plus_4_fma", 1024), (3, "fma_dpp_operand", 4096))
    res = {}
    for wps in (1, 2, 4, 8):
        blocks = wps * ncu
        for kind, name, iters in kinds:
            nf, ne = ctypes.c_int(), ctypes.c_int()
            P.ssm_probe_valu_ops_per_iter(kind, ctypes.byref(nf), ctypes.byref(ne))
            it = max(1, iters * 2 // wps) if wps < 8 else iters
            for _ in range(max(1, args.warmup)):
                assert P.ssm_probe_valu_launch(kind, blocks, it, out.data_ptr(), stream.cuda_stream) == 0
            ev0 = torch.cuda.Event(enable_timing=True)
            ev1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            ev0.record(stream)
            for _ in range(args.steps):
                assert P.ssm_probe_valu_launch(kind, blocks, it, out.data_ptr(), stream.cuda_stream) == 0
            ev1.record(stream)
            torch.cuda.synchronize()
            t = ev0.elapsed_time(ev1) / 1e3 / args.steps
            lanes = blocks * 256 * it
            res["%s_waves_per_simd_%d" % (name, wps)] = {
                "kernel_avg_us": t * 1e6, "iters": it, "fma_lane_ops_per_s": lanes * nf.value / t,
                "exp_lane_ops_per_s": lanes * ne.value / t}
    fma = res["fma_waves_per_simd_8"]["fma_lane_ops_per_s"]
    ex = res["exp_waves_per_simd_8"]["exp_lane_ops_per_s"]
    mixed = res["exp_plus_4_fma_waves_per_simd_8"]["exp_lane_ops_per_s"]
    print(json.dumps({
        "micro": "valu",
        "compute_units": ncu,
        "rates": res,
        "fma_lane_ops_per_s": fma,
        "exp_lane_ops_per_s": ex,
        "fma_frac_of_157_3_tflops": 2 * fma / 157.3e12,
        "exp_slots_of_peak": VALU_SLOTS_PER_S / ex,
        "exp_slots_alone": fma / ex,
        "exp_slots_mixed_with_4_fma": fma / mixed - 4.0,
    }))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU-baseline leg")
    ap.add_argument("--micro", choices=["valu"], default=None,
                    help="instead of the scan, measure the vector ALU issue rates (float32 FMA, v_exp_f32, mixed)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="instead of the scan, run plain device copies of MIB MiB (a known-size reference for "
                         "the FETCH_SIZE / WRITE_SIZE counters) and print their size")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the scan shards along batch rows and channels without "
              "communication, so a multi-GPU figure would be N copies of this one. Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.micro == "valu":
        micro_valu(args)
        return

    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_per_launch": n * 4, "launches": args.steps}))
        return

    import state_space_model_selective_amd as ssm
    import synth
    from synth import WORKLOADS

    if args.workload in synth.SSD_WORKLOADS:
        bench_ssd(args, args.workload)
        return

    w = dict(WORKLOADS[args.workload])
    Bs, L, ED, N = w["Bs"], w["L"], w["ED"], w["N"]
    dev = torch.device("cuda:0")
    tdt = torch.float32 if w["dtype"] == "f32" else torch.bfloat16

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    nsets = 3
    bwd = bool(w.get("bwd"))
    train = bool(w.get("train"))
    dcode = ssm.SSM_F32 if w["dtype"] == "f32" else ssm.SSM_BF16
    host_sets, sets = [], []
    for i in range(nsets):
        inp = synth.make_inputs(Bs, L, ED, N, w["dtype"], seed=i)
        t = {k: to_dev(v) for k, v in inp.items()}
        if bwd:
            dy = synth.make_output_grad(Bs, L, ED, w["dtype"], seed=i)
            t["dy"] = to_dev(dy)
            host_sets.append((inp, dy) if i == 0 else None)
            t["out"] = {"dx": torch.empty_like(t["x"]), "ddelta": torch.empty_like(t["x"]),
                        "dA": torch.empty_like(t["A"]), "dB": torch.empty_like(t["B"]),
                        "dC": torch.empty_like(t["C"]), "dD": torch.empty_like(t["D"])}
            need = (ssm.ssm_scan_bidir_bwd_workspace_bytes if w["bidir"] else ssm.ssm_scan_bwd_workspace_bytes)(
                Bs, L, ED, N, dcode)
            if train:
                t["y"] = torch.empty((Bs, L, ED), dtype=tdt, device=dev)
                t["ck"] = torch.empty(ssm.ssm_scan_ckpt_shape(Bs, L, ED), dtype=torch.float32, device=dev)
                fneed = ssm.ssm_scan_workspace_bytes(Bs, L, ED, N, dcode, w["bidir"])
                t["fws"] = torch.empty(fneed, dtype=torch.uint8, device=dev) if fneed else None
        else:
            host_sets.append(inp if i == 0 else None)
            t["y"] = torch.empty((Bs, L, ED), dtype=tdt, device=dev)
            t["h"] = torch.empty((Bs, ED, N), dtype=torch.float32, device=dev) if w["h_last"] else None
            need = ssm.ssm_scan_workspace_bytes(Bs, L, ED, N, dcode, w["bidir"])
        t["ws"] = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
        sets.append(t)

    stream = torch.cuda.current_stream(dev)

    def step(t):
        if train:
            (ssm.ssm_scan_bidir_fwd if w["bidir"] else ssm.ssm_scan_fwd)(
                t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], y=t["y"], workspace=t["fws"], ckpt=t["ck"],
                stream=stream)
            (ssm.ssm_scan_bidir_bwd if w["bidir"] else ssm.ssm_scan_bwd)(
                t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["dy"], out=t["out"], workspace=t["ws"],
                ckpt=t["ck"], stream=stream)
        elif bwd:
            (ssm.ssm_scan_bidir_bwd if w["bidir"] else ssm.ssm_scan_bwd)(
                             t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], t["dy"], out=t["out"],
                             workspace=t["ws"], stream=stream)
        elif w["bidir"]:
            ssm.ssm_scan_bidir_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], y=t["y"], h_last=t["h"],
                                   workspace=t["ws"], stream=stream)
        else:
            ssm.ssm_scan_fwd(t["x"], t["delta"], t["A"], t["B"], t["C"], t["D"], y=t["y"], h_last=t["h"],
                             workspace=t["ws"], stream=stream)

    for i in range(args.warmup):
        step(sets[i % nsets])
    torch.cuda.synchronize()

    # timed region: K steps back to back, HIP events on the launch stream at
    # its two ends; the per-launch kernel time is the region time over K
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(sets[i % nsets])
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    avg_launch_s = ev0.elapsed_time(ev1) / 1e3 / args.steps
    ms_per_step = wall * 1e3 / args.steps

    E = Bs * L * ED * N
    value = E / (wall / args.steps)
    bytes_alg = alg_bytes(w)
    kernel_elem_rate = E / avg_launch_s
    # bidirectional: the exp and the two multiplies are shared by both
    # directions; algorithmic cost 2 mul + exp + 2 x (state FMA + C FMA) = 8
    if train:
        slots = (SLOTS_PER_ELEMENT_BIDIR + SLOTS_PER_ELEMENT_BIDIR_BWD) if w["bidir"] else \
            (SLOTS_PER_ELEMENT + SLOTS_PER_ELEMENT_BWD)
    elif bwd:
        slots = SLOTS_PER_ELEMENT_BIDIR_BWD if w["bidir"] else SLOTS_PER_ELEMENT_BWD
    else:
        slots = SLOTS_PER_ELEMENT_BIDIR if w["bidir"] else SLOTS_PER_ELEMENT
    achieved_slots = kernel_elem_rate * slots
    src_hash = kernel_source_hash(args.workload)
    traffic = load_traffic(args.workload, src_hash)

    # parity check of step 0's input set against the oracle (also the CPU baseline)
    cpu = None
    parity = None
    if not args.no_cpu and bwd:
        inp0, dy0 = host_sets[0]
        cpu, ref, k = cpu_baseline_bwd(inp0, dy0, w)
        step(sets[0])
        torch.cuda.synchronize()
        tol = 1e-4 if w["dtype"] == "f32" else 2e-2
        rel = 0.0
        names = ("y", "dx", "ddelta", "dB", "dC") if train else ("dx", "ddelta", "dB", "dC")
        for name in names:
            src = sets[0]["y"] if name == "y" else sets[0]["out"][name]
            got = src[:k].float().cpu().numpy().astype(np.float64)
            rel = max(rel, float(np.max(np.abs(got - ref[name]) / (1 + np.abs(ref[name])))))
        parity = dict(max_rel_err=rel, tol=tol, passed=bool(rel <= tol),
                      checked=", ".join(names) + " of the sampled batch rows")
    elif not args.no_cpu:
        cpu, y_ref, chans = cpu_baseline(host_sets[0], w)
        step(sets[0])
        torch.cuda.synchronize()
        y0 = sets[0]["y"].float().cpu().numpy().astype(np.float64)
        if chans is None:
            got = y0
        else:
            b_i, e_i = np.divmod(chans, ED)
            got = y0[b_i, :, e_i]
        tol = 1e-4 if w["dtype"] == "f32" else 2e-2
        rel = float(np.max(np.abs(got - y_ref) / (1 + np.abs(y_ref))))
        parity = dict(max_rel_err=rel, tol=tol, passed=bool(rel <= tol))

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "scan elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w["dtype"],
        "data": "synthetic (seeded counter-based generator; x,B,C,D ~ N(0,1), delta log-uniform [1e-3,1e-1], "
                "A[e,n] = -(n+1)" + ("; dy ~ N(0,1)" if bwd else "") + "); 3 input sets rotated",
        "config": {"workload": args.workload, "Bs": Bs, "L": L, "ED": ED, "N": N, "bidir": w["bidir"],
                   "h_last": w["h_last"], "backward": bwd, "training_step": train, "parallelism": "single GPU"},
        "roofline": {
            "bound": "hbm",
            "achieved": bytes_alg / avg_launch_s / 1e9,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": bytes_alg / avg_launch_s / 1e9 / HBM_PEAK_GBPS,
            "traffic": traffic,
            "alg_bytes_per_launch": bytes_alg,
            "kernel_avg_us": avg_launch_s * 1e6,
            "timed": (("whole training step: the forward scan's kernels (writing the round states), the backward "
                       "scan kernel (once per direction) and the two small kernels that add up the dB/dC and dA/dD "
                       "partial sums")
                      if train else
                      ("whole backward step: the scan kernel (once per direction) and the two small kernels "
                       "that add up the dB/dC and dA/dD partial sums") if bwd else
                      "the scan kernel (one launch per step)"),
        },
        # the same kernel time against the vector ALU, the resource that
        # actually bounds the scan (one exp per element; see --micro valu)
        "valu": {
            "achieved": achieved_slots / 1e12,
            "peak": VALU_SLOTS_PER_S / 1e12,
            "unit": "T VALU-slot/s",
            "frac": achieved_slots / VALU_SLOTS_PER_S,
            "slots_per_element": slots,
            "exp_slots": EXP_SLOTS,
            "peak_from": "published float32 vector 157.3 TFLOP/s = 78.6 T FMA lane-ops/s (256 CUs x 4 SIMDs x 32 x 2.4 GHz)",
        },
        "kernel_source_sha256_16": src_hash,
        "parity": parity,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
