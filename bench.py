"""Benchmark: ExTernD decomposition of a 2560 x 2560 LLM-shaped matrix on one GPU.

One step = the whole hot path over one synthetic input: the sequential
greedy ALS (k = 5120 components) followed by the block ALS (b = 64, 80
blocks) of the same matrix, mu = 2, tau = 0.7, 15 iterations.  Prints one
JSON line (rank 0) with components/s, the sequential kernel's roofline
figures and the fp64 oracle's rate on a bounded sample as a CPU baseline.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--modes seq,block]
                    [--cpu-sample N | --no-cpu]
                    [--workload gauss256|llm2560|mlp9728|layer|lowrank4096]

The other workloads print a line of the same form for their own input:
gauss256 adds the per-component energy trace, layer times the seven matrices
of one transformer layer back to back, lowrank4096 times the mu x tau sweep.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
FP32_PEAK_TFLOPS = 157.3       # MI355X fp32 (vector and MFMA), published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published

# Measured HBM traffic of one k_seq_resident launch on the 2560 x 2560
# workload: rocprofv3 FETCH_SIZE and WRITE_SIZE passes, scaled by what the
# same counters read for a plain 1 GiB copy (FETCH x 2.0, WRITE x 1.0).  It is
# reported only while the kernel's sources hash to the ones it was taken on.
SEQ_TRAFFIC_BYTES = 47515127744
SEQ_TRAFFIC_SOURCES = ["ternary_rank_weight_amd/csrc/seq_resident.hip",
                       "ternary_rank_weight_amd/csrc/device_common.hpp",
                       "ternary_rank_weight_amd/csrc/exchange.hpp"]
SEQ_TRAFFIC_SHA = "c97be5df5c9f5a50"

# Measured HBM traffic of one k_seq_persist launch on the 9728 x 2560 workload
# (mu = 3, tau = 1.0, k = 7680), scaled the same way; reported only while the
# kernel's sources hash to the ones it was taken on.
PERSIST_TRAFFIC_BYTES = 10250384020576
PERSIST_TRAFFIC_SOURCES = ["ternary_rank_weight_amd/csrc/seq_persist.hip",
                           "ternary_rank_weight_amd/csrc/device_common.hpp",
                           "ternary_rank_weight_amd/csrc/exchange.hpp"]
PERSIST_TRAFFIC_SHA = "4dbbebdf9a48a7bc"

# rocprofv3 counters of the block path on the 2560 x 2560 workload (b = 64),
# per dispatch of the combined Gram / inverse / contraction launch: MFMA busy
# cycles over active cycles x SIMDs, bf16 MFMA flops and int8 MFMA operations
# (MOPS x 512), and HBM
# bytes (FETCH x 2.0, WRITE x 1.0) against the 26.2 MB of R it must read.
# Reported only while the block sources hash to the ones they were taken on.
BLOCK_COUNTERS = {"kernel": "k_contract_with_inverse", "mfma_busy_frac": 0.0375,
                  "bf16_mfma_flops": 2.5281e9, "int8_mfma_ops": 3.220e7, "fetch_bytes": 26732544,
                  "write_bytes": 3293286, "R_bytes": 26214400}
BLOCK_COUNTER_SOURCES = ["ternary_rank_weight_amd/csrc/block.hip",
                         "ternary_rank_weight_amd/csrc/device_common.hpp",
                         "ternary_rank_weight_amd/csrc/exchange.hpp"]
BLOCK_COUNTER_SHA = "0d5d5cd91db09a88"


def _sources_sha(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def seq_traffic(workload, kernel="k_seq_resident"):
    if kernel == "k_seq_resident":
        if workload != "llm2560" or _sources_sha(SEQ_TRAFFIC_SOURCES) != SEQ_TRAFFIC_SHA:
            return None
        return SEQ_TRAFFIC_BYTES
    if kernel == "k_seq_persist":
        if workload != "mlp9728" or _sources_sha(PERSIST_TRAFFIC_SOURCES) != PERSIST_TRAFFIC_SHA:
            return None
        return PERSIST_TRAFFIC_BYTES
    return None


def block_counters(workload, b):
    if workload != "llm2560" or b != 64 or _sources_sha(BLOCK_COUNTER_SOURCES) != BLOCK_COUNTER_SHA:
        return None
    return dict(BLOCK_COUNTERS, source="profiles/block_als_b64_2560x2560.md")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--modes", default=None,
                    help="comma-separated subset of seq,block (default: seq,block; block for mlp9728)")
    ap.add_argument("--cpu-sample", type=int, default=200,
                    help="components of the oracle's sequential run timed as the CPU baseline")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-importance", dest="importance", action="store_false",
                    help="skip the importance-weighted runs")
    ap.add_argument("--no-projection", dest="projection", action="store_false",
                    help="skip the block run with the optimal ternary projection")
    ap.add_argument("--no-streaming", dest="streaming", action="store_false",
                    help="skip the streaming-versus-resident comparison of the sequential mode")
    ap.add_argument("--sweeps", type=int, default=10,
                    help="refinement sweeps measured after the block run (0: skip)")
    ap.add_argument("--workload", default="llm2560",
                    choices=["gauss256", "llm2560", "mlp9728", "layer", "lowrank4096"],
                    help="gauss256: 256x256 Gaussian, with the sequential energy trace; llm2560: "
                         "2560x2560 LLM-shaped (default); mlp9728: 9728x2560 LLM-shaped, mu=3, tau=1.0, "
                         "block b=128; layer: the seven matrices of one 4B-class layer, mu=2.5, block "
                         "b=128, back to back; lowrank4096: the mu x tau sweep on a 4096x4096 rank-256 "
                         "plus noise matrix, block b=128")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (5 launches) and "
                         "exit; its HBM counters calibrate the per-kernel traffic figures")
    return ap.parse_args()


def copy_probe(mib):
    """A plain copy kernel of known size: reads and writes mib MiB per launch."""
    import torch
    torch.cuda.set_device(0)
    src = torch.ones(mib << 18, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": mib << 20, "copy_probe_bytes_written": mib << 20,
                      "launches": 5}), flush=True)


def seq_alg_bytes(m, n, k, iterations, sum_nnz_u):
    """Bytes a streaming implementation must move for the sequential path.

    Per component: the first R^T u0 pass reads all of R (u0 is dense); each
    R v pass reads all of R; the R^T u passes of the later iterations read
    only rows where u is nonzero; the deflation rewrites the rows where the
    final u is nonzero.  Over the decomposition that is
    4 n ((iterations + k) m + sum_t nnz(u_t)), iterations being the ALS
    iterations run over all components and t running over the u vectors of
    those iterations.
    """
    return 4.0 * n * ((iterations + k) * m + sum_nnz_u)


def block_alg_flops(m, n, k, b, iters):
    """Dense-contraction flops of the block path: per block, 2*iters
    contractions R^T U / R V of 2 m n b flops plus one rank-b deflation."""
    nblocks = (k + b - 1) // b
    return 2.0 * m * n * b * (2 * iters + 1) * nblocks


def _random_codes(torch, rows, L, gen):
    """Valid 2-bit code rows (no 0b10 code, zero padding), uniformly random."""
    w = torch.randint(-2**31, 2**31 - 1, (rows, (L + 15) // 16), dtype=torch.int64,
                      device="cuda", generator=gen).to(torch.int32)
    w = w | ((w >> 1) & 0x55555555)          # a set sign bit forces the nonzero bit
    if L % 16:
        w[:, -1] &= (1 << (2 * (L % 16))) - 1
    return w.contiguous()


def measure_inference(trw, outs, m, n, reps=20):
    """y = B (diag(D) (C x)) (externd_apply) on the block run's factors and on
    a 16384 x 16384, k = 32768 set of random factors; HIP events around
    `reps` calls.  Algorithmic bytes per call: both code arrays, D, x, y."""
    import torch
    res = []
    cases = []
    if "block" in outs:
        r = outs["block"]
        cases.append((f"{m}x{n} block-ALS factors, k={r.k}", r.B2, r.C2, r.D, m, n))
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    M = N = 16384
    K = 32768
    cases.append((f"{M}x{N} random 2-bit factors, k={K}", _random_codes(torch, K, M, gen),
                  _random_codes(torch, K, N, gen), torch.randn(K, device="cuda", generator=gen) * 0.01, M, N))
    for name, B2, C2, D, mm, nn in cases:
        x = torch.randn(nn, device="cuda", generator=gen)
        k = D.numel()
        BT2 = trw.transpose_codes(B2, k, mm)   # B row by row, once per factorisation (not timed)
        ws = torch.empty(trw.apply_rows_workspace_bytes(mm, nn, k), dtype=torch.uint8, device="cuda")
        y = torch.empty(mm, dtype=torch.float32, device="cuda")
        for form, call in (("B component-major, fp32 VALU (externd_apply)",
                            lambda: trw.apply(B2, C2, D, mm, nn, x)),
                           ("B row by row, int8 MFMA, caller workspace (externd_apply_rows)",
                            lambda: trw.apply_rows(BT2, C2, D, mm, nn, x, out=y, workspace=ws))):
            for _ in range(3):
                call()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                call()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / reps
            alg = 4.0 * k * ((mm + 15) // 16 + (nn + 15) // 16) + 4.0 * (k + mm + nn)
            gbps = alg / us / 1e3
            res.append({"workload": name, "form": form, "us_per_call": round(us, 2), "alg_bytes": alg,
                        "gbps": round(gbps, 1), "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBS, 4)})
    return res


def measure_sweeps(trw, Ad, c, block, sweeps, block_ms, block_energy):
    """Refinement sweeps (§2.4) after block extraction on the same matrix:
    one run of extraction + `sweeps` sweeps between HIP events; the time per
    sweep is that run less the block extraction's mean time, over `sweeps`."""
    import torch
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    r = trw.decompose(Ad, c["mu"], c["tau"], c["iters"], block, c["seed"], trace=True, stats=True,
                      sweeps=sweeps)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    a2 = float(r.norm_a2.item())
    per_sweep = [round(1.0 - float(t) / a2, 6) for t in r.sweep_trace.cpu().numpy()]
    E = float(r.energy.item())
    return {"sweeps": sweeps, "ms_total": round(ms, 3),
            "ms_per_sweep": round((ms - block_ms) / sweeps, 3),
            "energy_extraction": round(block_energy, 6), "energy_after": round(E, 6),
            "gain_points": round(100.0 * (E - block_energy), 4),
            "energy_per_sweep": per_sweep, "visits_kept_old": r.stat("sweep_kept_old")}


def measure_importance(trw, Ad, c, block, modes, sigma=1.5):
    """Importance-weighted ALS (§2.5) on the same matrix with a synthetic
    skewed importance vector (lognormal, sigma 1.5, lambda 0): time and
    weighted energy per mode, one run each between HIP events, next to the
    plain run's time."""
    import torch
    import synthetic
    h = torch.from_numpy(synthetic.importance(Ad.shape[1], 11, sigma)).cuda()
    out = {}
    for md in modes:
        blk = 0 if md == "seq" else block
        trw.decompose(Ad, c["mu"], c["tau"], c["iters"], blk, c["seed"], importance=h)   # warm
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        r = trw.decompose(Ad, c["mu"], c["tau"], c["iters"], blk, c["seed"], importance=h)
        e1.record()
        torch.cuda.synchronize()
        out[md] = {"ms": round(e0.elapsed_time(e1), 3), "weighted_energy": round(float(r.energy.item()), 6)}
    return {"importance": f"lognormal(0, {sigma}) over the {Ad.shape[1]} input columns, lambda 0",
            "modes": out}


def measure_projection(trw, Ad, c, block):
    """Block ALS with the optimal ternary projection (§2.2) in place of T_tau
    on the same matrix: one run between HIP events, and its energy."""
    import torch
    trw.decompose(Ad, c["mu"], c["tau"], c["iters"], block, c["seed"], projection=True)   # warm
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    r = trw.decompose(Ad, c["mu"], c["tau"], c["iters"], block, c["seed"], projection=True)
    e1.record()
    torch.cuda.synchronize()
    return {"mode": f"block ALS b={trw.block_width(Ad.shape[0], Ad.shape[1], block)}",
            "ms": round(e0.elapsed_time(e1), 3), "energy": round(float(r.energy.item()), 6)}


def measure_streaming(trw, Ad, c, k=256):
    """The sequential decomposition's first k components in the streaming
    mode (R in HBM, a few kernels per half-step) and in the cooperative mode
    the shape takes (resident when R fits on chip, else persistent), on the
    same matrix: event times, components/s and the algorithmic bytes rate of
    each (the same byte model as the roofline)."""
    import torch
    m, n = Ad.shape
    mu = (k + 0.25) / min(m, n)
    out = {"components": k}
    coop = ("resident", trw.MODE_RESIDENT) if trw.resident_fits(m, n) else ("persistent", trw.MODE_PERSISTENT)
    for name, mode in (("streaming", trw.MODE_STREAMING), coop):
        trw.decompose(Ad, mu, c["tau"], c["iters"], 0, c["seed"], mode=mode)   # warm
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        r = trw.decompose(Ad, mu, c["tau"], c["iters"], 0, c["seed"], mode=mode, stats=True)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        alg = seq_alg_bytes(m, n, k, r.stat("iterations") or k * c["iters"], r.stat("sum_nnz_u"))
        gbps = alg / (ms / 1e3) / 1e9
        out[name] = {"ms": round(ms, 3), "components_per_s": round(k / (ms / 1e3), 1),
                     "gbps": round(gbps, 1), "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBS, 4),
                     "energy": round(float(r.energy.item()), 6)}
    return out


def measure_streaming_large(trw, k=64, name="mlp9728", shape=None):
    """The sequential decomposition on a shape past the resident limit
    (9728 x 2560, the LLM-shaped MLP workload, or with `shape` an LLM-shaped
    matrix of that size, e.g. 10240 x 10240, whose 419 MB exceed the 256 MB
    last-level cache; mu for its first k components, tau 0.7), in the
    persistent streaming mode and in the streaming kernel chain: event time,
    components/s, the algorithmic bytes rate (the roofline's byte model) and
    its fraction of the HBM peak."""
    import torch
    import synthetic
    c = synthetic.WORKLOADS[name]
    if shape is None:
        A = torch.from_numpy(synthetic.workload_matrix(name)).cuda()
    else:
        A = torch.from_numpy(synthetic.llm_like(shape[0], shape[1], c["seed"])).cuda()
    m, n = A.shape
    mu = (k + 0.25) / min(m, n)
    out = {"workload": f"{m}x{n} LLM-shaped, first {k} components, tau 0.7, sequential mode"}
    for label, mode in (("persistent", trw.MODE_PERSISTENT), ("streaming", trw.MODE_STREAMING)):
        trw.decompose(A, mu, 0.7, c["iters"], 0, c["seed"], mode=mode)   # warm
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        r = trw.decompose(A, mu, 0.7, c["iters"], 0, c["seed"], mode=mode, stats=True)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        alg = seq_alg_bytes(m, n, k, r.stat("iterations") or k * c["iters"], r.stat("sum_nnz_u"))
        gbps = alg / (ms / 1e3) / 1e9
        out[label] = {"ms": round(ms, 3), "components_per_s": round(k / (ms / 1e3), 1), "alg_bytes": alg,
                      "gbps": round(gbps, 1), "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBS, 4),
                      "energy": round(float(r.energy.item()), 6), "safeguard": r.stat("safeguard")}
    return out


def cpu_baseline(A, c, sample, block=0):
    """The oracle timed on a bounded sample: the first `sample` components of
    the sequential decomposition, or for block mode alone (block > 0) the
    first ceil(sample / b) blocks of the block decomposition."""
    import numpy as np
    import oracle
    cores = len(os.sched_getaffinity(0))
    m, n = A.shape
    k_all = oracle.rank_for(m, n, c["mu"])
    t = time.perf_counter()
    if block:
        b = oracle.block_width(m, n, block)
        sample = min(k_all, -(-sample // b) * b)
        r = oracle.decompose_block(A, c["mu"], c["tau"], c["iters"], block, c["seed"], k=sample)
        what = f"block decomposition (b={b})"
    else:
        r = oracle.decompose_seq(A, c["mu"], c["tau"], c["iters"], c["seed"], k=sample)
        what = "sequential decomposition"
    dt = time.perf_counter() - t
    return {"value": round(sample / dt, 3), "unit": "components/s", "cores": cores,
            "kind": "oracle",
            "sample": f"first {sample} of {k_all} components of the {what} of the same "
                      f"{m}x{n} matrix, fp64 numpy oracle ({dt:.1f} s, E after sample {r.E:.4f})"}


def run_layer(args):
    """The seven matrices of one transformer layer (q, k, v, o, gate, up,
    down), decomposed back to back on one stream in block mode; a step is the
    whole layer."""
    import numpy as np
    import torch
    import synthetic
    import ternary_rank_weight_amd as trw

    torch.cuda.set_device(0)
    c = synthetic.WORKLOADS["layer"]
    shapes = synthetic.layer_shapes()
    host = {name: synthetic.workload_matrix("layer", name) for name, _, _ in shapes}
    dev = {name: torch.from_numpy(A).cuda() for name, A in host.items()}
    outs = {}

    def step():
        for name, _, _ in shapes:
            outs[name] = trw.decompose(dev[name], c["mu"], c["tau"], c["iters"], c["block"], c["seed"],
                                       stats=True, out=outs.get(name))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print("[bench] warmup done", file=sys.stderr, flush=True)
    ev = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        step()
        e1.record()
        ev.append((e0, e1))
        print("[bench] layer launched", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    per = {}
    total_k = 0
    flops = 0.0
    for name, m, n in shapes:
        k = trw.rank(m, n, c["mu"])
        b = trw.block_width(m, n, c["block"])
        total_k += k
        fl = block_alg_flops(m, n, k, b, c["iters"])
        flops += fl
        per[name] = {"m": m, "n": n, "k": k, "b": b, "energy": round(float(outs[name].energy.item()), 6),
                     "alg_tflop": round(fl / 1e12, 3)}
    tflops = flops / (ms / 1e3) / 1e12
    cpu = None
    if not args.no_cpu and args.cpu_sample > 0:
        cpu = cpu_baseline(host["q"], c, min(args.cpu_sample, trw.rank(4096, 2560, c["mu"])), c["block"])
        cpu["sample"] += " (the layer's q matrix)"
    line = {
        "metric": "ALS components/sec + achieved HBM GB/s at 2560x2560 mu=2 tau=0.7; energy E",
        "value": round(total_k / (ms / 1e3), 2),
        "unit": "components/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "one 4B-class transformer layer as 7 LLM-shaped synthetic matrices "
                               "(q 4096x2560, k/v 1024x2560, o 2560x4096, gate/up 9728x2560, down 2560x9728), "
                               f"mu={c['mu']}, tau={c['tau']}, {c['iters']} iterations, block ALS b={c['block']}, "
                               "back to back on one stream; step = the whole layer",
                   "mu": c["mu"], "tau": c["tau"], "iters": c["iters"], "block": c["block"], "k_total": total_k,
                   "seed": c["seed"]},
        "matrices": per,
        "roofline": {"bound": "mfma", "kernel": "block ALS pipeline", "achieved": round(tflops, 3),
                     "peak": FP32_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tflops / FP32_PEAK_TFLOPS, 4),
                     "traffic": None, "alg_flops_per_step": flops},
        "cpu_baseline": cpu,
        "wall_s": round(wall, 3),
    }
    print(json.dumps(line), flush=True)


def run_lowrank(args):
    """The mu / tau sweep on the 4096 x 4096 rank-256-plus-noise matrix in
    block mode (b = 128): every (mu, tau) pair is a separate decomposition,
    reported with its energy and the zero fractions of its factors; a step is
    the whole sweep (12 decompositions back to back on one stream).  Checks
    that E does not fall as mu grows at fixed tau, and that the zero fraction
    grows with tau at fixed mu."""
    import numpy as np
    import torch
    import synthetic
    import ternary_rank_weight_amd as trw

    torch.cuda.set_device(0)
    c = synthetic.WORKLOADS["lowrank4096"]
    A = synthetic.workload_matrix("lowrank4096")
    m, n = A.shape
    Ad = torch.from_numpy(A).cuda()
    runs = [(mu, tau) for tau in c["taus"] for mu in c["mus"]]
    outs = {}

    def step(record):
        ev = {}
        for mu, tau in runs:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            outs[(mu, tau)] = trw.decompose(Ad, mu, tau, c["iters"], c["block"], c["seed"], stats=True,
                                            out=outs.get((mu, tau)))
            e1.record()
            ev[(mu, tau)] = (e0, e1)
        if record is not None:
            record.append(ev)

    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    print("[bench] warmup done", file=sys.stderr, flush=True)
    records = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(records)
        print("[bench] sweep launched", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    b = trw.block_width(m, n, c["block"])
    sweep = []
    total_k, total_ms, flops = 0, 0.0, 0.0
    for mu, tau in runs:
        r = outs[(mu, tau)]
        ms = float(np.mean([rec[(mu, tau)][0].elapsed_time(rec[(mu, tau)][1]) for rec in records]))
        k = r.k
        nb, nc = r.stat("nnz_b"), r.stat("nnz_c")
        fl = block_alg_flops(m, n, k, b, c["iters"])
        total_k += k
        total_ms += ms
        flops += fl
        sweep.append({"mu": mu, "tau": tau, "k": k, "ms": round(ms, 3),
                      "components_per_s": round(k / (ms / 1e3), 1),
                      "energy": round(float(r.energy.item()), 6),
                      "zero_fraction_B": round(1.0 - nb / (k * m), 4),
                      "zero_fraction_C": round(1.0 - nc / (k * n), 4),
                      "zero_fraction": round(1.0 - (nb + nc) / (k * (m + n)), 4),
                      "safeguard": r.stat("safeguard"), "timeouts": r.stat("timeouts"),
                      "inverse_unconverged": r.stat("inverse_unconverged")})
    by = {(e["mu"], e["tau"]): e for e in sweep}
    e_monotone = {str(tau): all(by[(a, tau)]["energy"] <= by[(bb, tau)]["energy"]
                                for a, bb in zip(c["mus"], c["mus"][1:])) for tau in c["taus"]}
    z_increasing = {str(mu): all(by[(mu, a)]["zero_fraction"] < by[(mu, bb)]["zero_fraction"]
                                 for a, bb in zip(c["taus"], c["taus"][1:])) for mu in c["mus"]}
    tflops = flops / (total_ms / 1e3) / 1e12
    cpu = None
    if not args.no_cpu and args.cpu_sample > 0:
        c1 = dict(c, mu=c["mus"][0], tau=c["taus"][0])
        cpu = cpu_baseline(A, c1, min(args.cpu_sample, trw.rank(m, n, c1["mu"])), c["block"])
        cpu["sample"] += f" (mu={c1['mu']}, tau={c1['tau']})"
    line = {
        "metric": "ALS components/sec + achieved HBM GB/s at 2560x2560 mu=2 tau=0.7; energy E",
        "value": round(total_k / (total_ms / 1e3), 2),
        "unit": "components/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{m}x{n} rank-256 structure (U diag(s) V^T, Gaussian U, V, s_i = i^-0.8) "
                               f"plus N(0, 0.005^2) noise; mu in {list(c['mus'])} x tau in {list(c['taus'])}, "
                               f"{c['iters']} iterations, block ALS b={b}; step = the 12 decompositions",
                   "m": m, "n": n, "mus": list(c["mus"]), "taus": list(c["taus"]), "iters": c["iters"],
                   "block": b, "seed": c["seed"], "k_total": total_k},
        "sweep": sweep,
        "checks": {"energy_nondecreasing_in_mu": e_monotone, "zero_fraction_increasing_in_tau": z_increasing},
        "roofline": {"bound": "mfma", "kernel": "block ALS pipeline", "achieved": round(tflops, 3),
                     "peak": FP32_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tflops / FP32_PEAK_TFLOPS, 4),
                     "traffic": None, "alg_flops_per_step": flops},
        "cpu_baseline": cpu,
        "wall_s": round(wall, 3),
    }
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the decomposition runs on one GPU; --gpus must be 1"}))
        sys.exit(2)
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.workload == "layer":
        run_layer(args)
        return
    if args.workload == "lowrank4096":
        run_lowrank(args)
        return
    import numpy as np
    import torch
    import synthetic
    import ternary_rank_weight_amd as trw

    torch.cuda.set_device(0)
    c = synthetic.WORKLOADS[args.workload]
    A = synthetic.workload_matrix(args.workload)
    m, n = A.shape
    Ad = torch.from_numpy(A).cuda()
    k = trw.rank(m, n, c["mu"])
    if args.modes is None:
        args.modes = "block" if args.workload == "mlp9728" else "seq,block"
    modes = [s for s in args.modes.split(",") if s]
    block = c.get("block", 64) or 64
    b = trw.block_width(m, n, block)

    outs = {}

    def run_step(record):
        ev = {}
        for md in modes:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            if md == "seq":
                outs[md] = trw.decompose(Ad, c["mu"], c["tau"], c["iters"], 0, c["seed"], stats=True,
                                         out=outs.get(md))
            else:
                outs[md] = trw.decompose(Ad, c["mu"], c["tau"], c["iters"], block, c["seed"],
                                         stats=True, out=outs.get(md))
            e1.record()
            ev[md] = (e0, e1)
            print(f"[bench] {md} launched", file=sys.stderr, flush=True)
        if record is not None:
            record.append(ev)

    for _ in range(args.warmup):
        run_step(None)
    torch.cuda.synchronize()
    print("[bench] warmup done", file=sys.stderr, flush=True)
    records = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run_step(records)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    per_mode = {}
    for md in modes:
        ms = [r[md][0].elapsed_time(r[md][1]) for r in records]
        res = outs[md]
        E = float(res.energy.item())
        per_mode[md] = {"ms": float(np.mean(ms)), "ms_min": float(np.min(ms)), "k": k,
                        "components_per_s": k / (float(np.mean(ms)) / 1e3), "energy": E,
                        "stats": {kk: res.stat(kk) for kk in trw.STAT}}
    step_ms = sum(per_mode[md]["ms"] for md in modes)
    total_components = k * len(modes)
    value = total_components / (step_ms / 1e3)

    roofline = None
    if "seq" in per_mode:
        s = per_mode["seq"]
        alg = seq_alg_bytes(m, n, k, s["stats"]["iterations"] or k * c["iters"], s["stats"]["sum_nnz_u"])
        achieved = alg / (s["ms"] / 1e3) / 1e9
        s["alg_bytes"] = alg
        s["gbps"] = achieved
        kernel = {0: "streaming kernel chain", 1: "k_seq_resident", 3: "k_seq_persist"}.get(
            s["stats"]["mode"], "sequential path")
        roofline = {"bound": "hbm", "kernel": kernel, "achieved": round(achieved, 1),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": seq_traffic(args.workload, kernel),
                    "traffic_unit": "bytes per launch",
                    "alg_bytes_per_launch": alg}
    if "block" in per_mode:
        bm = per_mode["block"]
        fl = block_alg_flops(m, n, k, b, c["iters"])
        bm["alg_tflops"] = fl / (bm["ms"] / 1e3) / 1e12
        bm["alg_flops"] = fl
        bm["b"] = b
        bm["counters"] = block_counters(args.workload, b)
        if roofline is None:
            # block mode alone: its dense contractions on fp32 MFMA
            roofline = {"bound": "mfma", "kernel": "block ALS pipeline",
                        "achieved": round(bm["alg_tflops"], 3), "peak": FP32_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(bm["alg_tflops"] / FP32_PEAK_TFLOPS, 4),
                        "traffic": None, "alg_flops_per_run": fl}

    trace = None
    if args.workload == "gauss256" and "seq" in modes:
        # the per-component energy trace of the sequential run (outside the timed region)
        r = trw.decompose(Ad, c["mu"], c["tau"], c["iters"], 0, c["seed"], trace=True)
        tr = r.trace.cpu().numpy()
        na2 = float(r.norm_a2.item())
        trace = {"what": "E after each component, 1 - ||R_i||^2 / ||A||^2, sequential mode",
                 "energy": [round(1.0 - float(v) / na2, 7) for v in tr]}
    inference = measure_inference(trw, outs, m, n)
    importance = None
    if args.importance:
        print("[bench] importance", file=sys.stderr, flush=True)
        importance = measure_importance(trw, Ad, c, block, modes)
    projection = None
    if "block" in per_mode and args.projection:
        print("[bench] projection", file=sys.stderr, flush=True)
        projection = measure_projection(trw, Ad, c, block)
    streaming = None
    if "seq" in per_mode and args.streaming:
        print("[bench] streaming", file=sys.stderr, flush=True)
        streaming = measure_streaming(trw, Ad, c)
        if args.workload != "mlp9728":
            print("[bench] streaming 9728x2560", file=sys.stderr, flush=True)
            streaming["large"] = measure_streaming_large(trw)
        print("[bench] streaming 10240x10240", file=sys.stderr, flush=True)
        streaming["past_cache"] = measure_streaming_large(trw, shape=(10240, 10240))
    sweeps = None
    if "block" in per_mode and args.sweeps > 0:
        print("[bench] sweeps", file=sys.stderr, flush=True)
        sweeps = measure_sweeps(trw, Ad, c, block, args.sweeps, per_mode["block"]["ms"],
                                per_mode["block"]["energy"])

    cpu = None
    if not args.no_cpu and args.cpu_sample > 0:
        cpu = cpu_baseline(A, c, min(args.cpu_sample, k), 0 if "seq" in modes else block)

    line = {
        "metric": "ALS components/sec + achieved HBM GB/s at 2560x2560 mu=2 tau=0.7; energy E",
        "value": round(value, 2),
        "unit": "components/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{m}x{n} LLM-shaped synthetic matrix (Student-t(5), bf16-rounded, "
                               f"lognormal rows, 16 outlier columns), mu={c['mu']}, tau={c['tau']}, "
                               f"{c['iters']} iterations, k={k}; step = " + " + ".join(
                                   {"seq": "sequential greedy ALS",
                                    "block": f"block ALS b={b}"}[md] for md in modes),
                   "m": m, "n": n, "mu": c["mu"], "tau": c["tau"], "iters": c["iters"], "k": k,
                   "block": b, "seed": c["seed"]},
        "modes": {md: {kk: (round(vv, 6) if isinstance(vv, float) else vv)
                       for kk, vv in per_mode[md].items()} for md in modes},
        "roofline": roofline,
        "inference": inference,
        "sweeps": sweeps,
        "importance_weighted": importance,
        "optimal_projection": projection,
        "seq_streaming_vs_resident": streaming,
        "trace": trace,
        "cpu_baseline": cpu,
        "wall_s": round(wall, 3),
    }
    print(json.dumps(line), flush=True)
    # explicit teardown before interpreter exit: every launch finished, the
    # library's outputs and inputs released, torch's cached blocks returned
    torch.cuda.synchronize()
    outs.clear()
    del Ad
    torch.cuda.empty_cache()
    torch.cuda.synchronize()


if __name__ == "__main__":
    main()
