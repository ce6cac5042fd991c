"""Write tests/golden/oracle_energies.json: the fp64 oracle's energies on the
five synthetic workloads at full size.

Calls only oracle/ and synthetic/.  Run from the repository root:
    python tests/golden/make_oracle_goldens.py [--only NAME ...]
Each entry records the workload, the knobs, E, the zero fraction and the
oracle's wall time on this host.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synthetic  # noqa: E402

OUT = os.path.join(ROOT, "tests", "golden", "oracle_energies.json")


def _entry(name, A, res, mode, mu, tau, iters, block, seed, secs, extra=None):
    e = {"name": name, "m": int(A.shape[0]), "n": int(A.shape[1]), "mode": mode, "mu": mu,
         "tau": tau, "iters": iters, "block": block, "seed": seed, "k": int(res.D.size),
         "E": float(res.E), "zero_fraction": float(oracle.zero_fraction(res.B, res.C)),
         "seconds": round(secs, 2)}
    if extra:
        e.update(extra)
    return e


def jobs():
    c = synthetic.WORKLOADS
    yield "gauss256_seq", lambda: _seq("gauss256", c["gauss256"])
    yield "llm2560_seq", lambda: _seq("llm2560", c["llm2560"])
    yield "llm2560_block64", lambda: _block("llm2560", c["llm2560"], c["llm2560"]["block"])
    yield "mlp9728_block128", lambda: _block("mlp9728", c["mlp9728"], c["mlp9728"]["block"])
    for name, _, _ in synthetic.layer_shapes():
        yield f"layer_{name}_block128", (lambda nm: (lambda: _layer(nm, c["layer"])))(name)
    for tau in c["lowrank4096"]["taus"]:
        yield f"lowrank4096_tau{tau}", (lambda tt: (lambda: _sweep(c["lowrank4096"], tt)))(tau)


def _seq(wl, c):
    A = synthetic.workload_matrix(wl)
    t = time.time()
    r = oracle.decompose_seq(A, c["mu"], c["tau"], c["iters"], c["seed"])
    return [_entry(f"{wl}_seq", A, r, "sequential", c["mu"], c["tau"], c["iters"], 0,
                   c["seed"], time.time() - t, {"sum_nnz_u": int(r.extra["sum_nnz_u"])})]


def _block(wl, c, b):
    A = synthetic.workload_matrix(wl)
    t = time.time()
    r = oracle.decompose_block(A, c["mu"], c["tau"], c["iters"], b, c["seed"])
    return [_entry(f"{wl}_block{b}", A, r, "block", c["mu"], c["tau"], c["iters"], b,
                   c["seed"], time.time() - t, {"ridge_retries": r.extra["ridge_retries"]})]


def _layer(name, c):
    A = synthetic.workload_matrix("layer", name)
    t = time.time()
    r = oracle.decompose_block(A, c["mu"], c["tau"], c["iters"], c["block"], c["seed"])
    return [_entry(f"layer_{name}_block{c['block']}", A, r, "block", c["mu"], c["tau"],
                   c["iters"], c["block"], c["seed"], time.time() - t)]


def _sweep(c, tau):
    # One run at the largest mu; smaller mu are prefixes (greedy deflation),
    # read off the per-block trace at k = mu * min(m, n) (multiples of b).
    A = synthetic.workload_matrix("lowrank4096")
    mus = c["mus"]
    t = time.time()
    r = oracle.decompose_block(A, max(mus), tau, c["iters"], c["block"], c["seed"])
    secs = time.time() - t
    out = []
    b = r.extra["b"]
    for mu in mus:
        k = oracle.rank_for(A.shape[0], A.shape[1], mu)
        assert k % b == 0
        E = 1.0 - r.trace[k // b - 1] / r.norm_a2
        zf = oracle.zero_fraction(r.B[:, :k], r.C[:k])
        out.append({"name": f"lowrank4096_tau{tau}_mu{mu}", "m": int(A.shape[0]), "n": int(A.shape[1]),
                    "mode": "block", "mu": mu, "tau": tau, "iters": c["iters"], "block": b,
                    "seed": c["seed"], "k": k, "E": float(E), "zero_fraction": float(zf),
                    "seconds": round(secs, 2)})
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--only", nargs="*")
    args = ap.parse_args()
    data = {}
    if os.path.exists(OUT):
        with open(OUT) as f:
            data = json.load(f)
    data.setdefault("source", "fp64 oracle (oracle/) on synthetic/ inputs; written by "
                              "tests/golden/make_oracle_goldens.py")
    entries = data.setdefault("entries", {})
    for name, fn in jobs():
        if args.only and not any(name.startswith(o) for o in args.only):
            continue
        t = time.time()
        for e in fn():
            entries[e["name"]] = e
            print(json.dumps(e), flush=True)
        with open(OUT, "w") as f:
            json.dump(data, f, indent=1, sort_keys=True)
        print(f"# {name} done in {time.time() - t:.1f}s", flush=True)


if __name__ == "__main__":
    main()
