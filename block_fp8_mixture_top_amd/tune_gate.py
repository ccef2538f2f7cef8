"""Measures where each path is fastest and generates the gate's per-shape table.

    python -m block_fp8_mixture_top_amd.tune_gate --shape decode   # E=256 H=2048 I=512 k=8 (GPU)
    python -m block_fp8_mixture_top_amd.tune_gate --shape large    # E=256 H=7168 I=2048 k=8 (GPU)
    python -m block_fp8_mixture_top_amd.tune_gate --emit           # CPU: table + summary from the profiles
    python -m block_fp8_mixture_top_amd.tune_gate --shape decode --paths auto   # check the built gate

A sweep times whole forwards at each token count T with the path forced to GATHER, STREAM
and MFMA (HIP-graph replays over rotating input sets of the synthetic workload) and stores
the times in profiles/gate_sweep_E<E>_H<H>_I<I>_k<k>.json, stamped with a digest of the
kernel sources. --emit turns every such profile into block_fp8_mixture_top_amd/csrc/
gate_table.inc, which the library's gate reads when moe_opts.use_measured_gate is set: for
each shape, the fastest path at each swept T (a path keeps its interval while it is within
2% of the fastest), with the boundary between two swept T at their geometric mean. It also
writes profiles/gate_sweep.md. The rule the table refines is the page's gate: gather while
tokens * top_k <= local experts * ratio (gaudi-cookbook "fp8-moe-gather", The fix); picking
a backend from measured bandwidth is FreeToken PR #662's approach (PR body).
"""

from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PROFILES = os.path.join(ROOT, "profiles")
TABLE = os.path.join(HERE, "csrc", "gate_table.inc")
PATHS = ("gather", "stream", "mfma")
PATH_IDS = {"gather": 1, "stream": 2, "mfma": 3}
HYSTERESIS = 1.02
MAX_INTERVALS = 24  # GateEntry holds this many

# (workload of the generators, token counts swept)
SHAPES = {
    "decode": ("sweep", [1, 2, 4, 8, 12, 16, 24, 32, 48, 64, 96, 128, 192, 256, 384, 512, 1024, 2048, 4096]),
    "large": ("large", [1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024]),
}


def source_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(HERE, "csrc")
    for f in sorted(os.listdir(csrc)):
        if f == "gate_table.inc":
            continue
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def profile_path(E, H, I, k) -> str:
    return os.path.join(PROFILES, f"gate_sweep_E{E}_H{H}_I{I}_k{k}.json")


def time_path(M, torch, cases, k, opts, reps):
    """Microseconds per forward over graph replays of all cases, and the path taken."""
    T, E, H, I = cases[0].T, cases[0].E, cases[0].H, cases[0].I
    dev = cases[0].hidden.device
    outs = [torch.empty((T, H), dtype=torch.bfloat16, device=dev) for _ in cases]
    ws = torch.empty(max(M.workspace_size(T, E, H, I, k, **opts), 1), dtype=torch.uint8, device=dev)

    def step(i):
        c = cases[i]
        return M.forward(c.hidden, c.logits, c.w13, c.w2, k, out=outs[i], workspace=ws, **opts)[1]

    info = step(0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(len(cases)):
            step(i)
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int(4e6))
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1000.0 / (reps * len(cases)), info["path"]


def sweep(args):
    import torch

    import block_fp8_mixture_top_amd as M
    import workloads as W

    wl, Ts = SHAPES[args.shape]
    if args.max_T:
        Ts = [t for t in Ts if t <= args.max_T]
    dev = torch.device("cuda:0")
    shp = W.SHAPES[wl]
    E, H, I, k = shp["E"], shp["H"], shp["I"], shp["top_k"]
    path = profile_path(E, H, I, k)
    prof = {"shape": dict(E=E, H=H, I=I, top_k=k), "workload": wl, "rows": {}}
    if os.path.exists(path):
        with open(path) as f:
            prof = json.load(f)
    paths = args.paths.split(",")
    digest = source_digest()
    banks = W.make_banks(wl, seed=args.seed, device=dev)
    for T in Ts:
        cases = [W.make_case(wl, T=T, seed=args.seed + 1000 + i, device=dev, banks=banks) for i in range(args.sets)]
        reps = max(2, min(100, 1000 // max(1, T // 8)))
        row = prof["rows"].get(str(T), {"T": T})
        for name in paths:
            opts = {"force_path": M.PATH_AUTO} if name == "auto" else {"force_path": PATH_IDS[name]}
            try:
                us, took = time_path(M, torch, cases, k, opts, reps)
            except M.MoeError:  # a path this shape does not support
                us, took = None, None
            row[name + "_us"] = None if us is None else round(us, 2)
            if name == "auto":
                row["auto_path"] = took
            row[name + "_digest"] = digest
        prof["rows"][str(T)] = row
        print(json.dumps(row), flush=True)
        del cases
        torch.cuda.empty_cache()
    prof["source_digest"] = digest
    os.makedirs(PROFILES, exist_ok=True)
    with open(path, "w") as f:
        json.dump(prof, f, indent=1, sort_keys=True)
        f.write("\n")


def best_paths(rows):
    """[(T, fastest forced path)] in T order, a path kept while within HYSTERESIS of the best."""
    out, prev = [], None
    for r in sorted(rows, key=lambda r: r["T"]):
        times = {p: r.get(p + "_us") for p in PATHS if r.get(p + "_us") is not None}
        if not times:
            continue
        best = min(times, key=times.get)
        if prev in times and times[prev] <= HYSTERESIS * times[best]:
            best = prev
        out.append((r["T"], best))
        prev = best
    return out


def intervals(bp):
    """[(t_max, path)]: path for T <= t_max, boundaries at the geometric mean of the swept T."""
    iv = []
    for i, (T, p) in enumerate(bp):
        if iv and iv[-1][1] == p:
            continue
        if iv:
            iv[-1] = (int(math.floor(math.sqrt(bp[i - 1][0] * T))), iv[-1][1])
        iv.append((None, p))
    if iv:
        iv[-1] = (2147483647, iv[-1][1])
    return iv


def emit_text():
    """The generated table (gate_table.inc) and the summary (gate_sweep.md)."""
    profs = []
    for path in sorted(glob.glob(os.path.join(PROFILES, "gate_sweep_E*_H*_I*_k*.json"))):
        with open(path) as f:
            profs.append((os.path.basename(path), json.load(f)))
    lines = ["// The gate's measured table: generated by block_fp8_mixture_top_amd/tune_gate.py --emit from",
             "// the sweeps under profiles/ (do not edit). path[i] (1 GATHER, 2 STREAM, 3 MFMA) is the path",
             "// measured fastest for T <= t_max[i].",
             "static const GateEntry kGateTable[] = {"]
    md = ["# Gate sweep: time per forward on each path", "",
          "Made by `python -m block_fp8_mixture_top_amd.tune_gate --shape <decode|large>` on the GPU box (times),",
          "`--paths auto` (the built gate's choice) and `--emit` (this file and `csrc/gate_table.inc`).",
          "Each time is one forward with the path forced, over HIP-graph replays of 4 input sets.", ""]
    n = 0
    for name, prof in profs:
        s = prof["shape"]
        rows = list(prof["rows"].values())
        iv = intervals(best_paths(rows))
        if not iv:
            continue
        assert len(iv) <= MAX_INTERVALS
        tm = ", ".join(str(t) for t, _ in iv)
        ps = ", ".join(str(PATH_IDS[p]) for _, p in iv)
        lines.append(f"    // {name}, workload {prof['workload']}, kernel sources {prof.get('source_digest')}")
        lines.append(f"    {{{s['E']}, {s['H']}, {s['I']}, {s['top_k']}, {len(iv)}, {{{tm}}}, {{{ps}}}}},")
        n += 1
        md += [f"## E={s['E']} H={s['H']} I={s['I']} top_k={s['top_k']} ({prof['workload']} workload)", "",
               f"Profile `profiles/{name}`, kernel sources {prof.get('source_digest')}.", "",
               "| T | GATHER µs | STREAM µs | MFMA µs | fastest | auto µs (path) | auto / fastest |",
               "|---|---|---|---|---|---|---|"]
        for r in sorted(rows, key=lambda r: r["T"]):
            times = {p: r.get(p + "_us") for p in PATHS if r.get(p + "_us") is not None}
            fast = min(times, key=times.get) if times else None
            a = r.get("auto_us")
            ratio = f"{a / times[fast]:.3f}" if a and fast else "—"
            auto = "—" if a is None else "%.1f (%s)" % (a, r.get("auto_path"))

            def cell(p):
                return "—" if r.get(p + "_us") is None else "%.1f" % r[p + "_us"]

            md.append(f"| {r['T']} | {cell('gather')} | {cell('stream')} | {cell('mfma')} | {fast} | {auto} | {ratio} |")
        md += ["", "Table: " + ", ".join(f"{p} for T <= {t}" if t < 2147483647 else f"{p} above" for t, p in iv), ""]
    if n == 0:
        lines.append("    {0, 0, 0, 0, 0, {0}, {0}},  // no measured shape")
    lines.append("};")
    return "\n".join(lines) + "\n", "\n".join(md) + "\n"


def emit():
    inc, md = emit_text()
    with open(TABLE, "w") as f:
        f.write(inc)
    with open(os.path.join(PROFILES, "gate_sweep.md"), "w") as f:
        f.write(md)
    print(inc)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--shape", choices=sorted(SHAPES))
    ap.add_argument("--paths", default=",".join(PATHS))
    ap.add_argument("--max-T", type=int, default=None)
    ap.add_argument("--sets", type=int, default=4)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--emit", action="store_true")
    args = ap.parse_args()
    if args.emit:
        return emit()
    if not args.shape:
        ap.error("--shape or --emit")
    sweep(args)


if __name__ == "__main__":
    main()
