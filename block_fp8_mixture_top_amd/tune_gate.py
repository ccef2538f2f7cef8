"""Measures where each path is fastest, to set the gate's two thresholds on this GPU.

    python -m block_fp8_mixture_top_amd.tune_gate                # decode banks, E=256 H=2048 I=512 k=8
    python -m block_fp8_mixture_top_amd.tune_gate --workload large --max-T 256

For each token count T it times whole forwards with the path forced to GATHER, STREAM and
MFMA (HIP-graph replays over rotating input sets of the synthetic workload). It prints one
JSON line per T and a summary:
- gate_ratio: T*k/E of the largest T at which GATHER is still the fastest path;
- mfma_min_tokens_per_expert: T*k/E of the smallest T from which MFMA stays fastest.

The gate picks GATHER while T*top_k <= gate_ratio*E, otherwise MFMA once T*top_k >=
mfma_min_tokens_per_expert*E, and STREAM in between (gaudi-cookbook "fp8-moe-gather", The
fix: the gathered path for tokens*top_k <= local_experts*ratio).
"""

from __future__ import annotations

import argparse
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

DEFAULT_TS = [1, 2, 4, 8, 12, 16, 24, 32, 48, 64, 96, 128, 192, 256, 384, 512, 768, 1024, 1536, 2048, 3072,
              4096]


def time_path(M, W, torch, cases, banks_k, force, reps):
    """Microseconds per forward, forced to one path, over graph replays of all cases."""
    T, E, H, I = cases[0].T, cases[0].E, cases[0].H, cases[0].I
    dev = cases[0].hidden.device
    outs = [torch.empty((T, H), dtype=torch.bfloat16, device=dev) for _ in cases]
    ws = torch.empty(max(M.workspace_size(T, E, H, I, banks_k, force_path=force), 1), dtype=torch.uint8,
                     device=dev)

    def step(i):
        c = cases[i]
        return M.forward(c.hidden, c.logits, c.w13, c.w2, banks_k, out=outs[i], workspace=ws,
                         force_path=force)[1]

    info = step(0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(len(cases)):
            step(i)
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    assert info["path"] == M.PATH_NAMES[force]
    return a.elapsed_time(b) * 1000.0 / (reps * len(cases))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--workload", default="decode", choices=["decode", "large"])
    ap.add_argument("--max-T", type=int, default=4096)
    ap.add_argument("--sets", type=int, default=4)
    ap.add_argument("--seed", type=int, default=0)
    args = ap.parse_args()

    import torch

    import block_fp8_mixture_top_amd as M
    import workloads as W

    dev = torch.device("cuda:0")
    shp = W.SHAPES[args.workload]
    E, k = shp["E"], shp["top_k"]
    banks = W.make_banks(args.workload, seed=args.seed, device=dev)
    paths = {"gather": M.PATH_GATHER, "stream": M.PATH_STREAM, "mfma": M.PATH_MFMA}
    rows = []
    for T in [t for t in DEFAULT_TS if t <= args.max_T]:
        cases = [W.make_case(args.workload, T=T, seed=args.seed + 1000 + i, device=dev, banks=banks)
                 for i in range(args.sets)]
        reps = max(2, min(200, 2000 // max(1, T // 8)))
        row = {"T": T, "pairs_per_expert": T * k / E}
        for name, pid in paths.items():
            try:
                row[name + "_us"] = round(time_path(M, W, torch, cases, k, pid, reps), 2)
            except M.MoeError:  # a path this shape does not support
                row[name + "_us"] = None
        row["fastest"] = min((n for n in paths if row[n + "_us"] is not None), key=lambda n: row[n + "_us"])
        rows.append(row)
        print(json.dumps(row), flush=True)
        del cases
        torch.cuda.empty_cache()

    # largest T (from the bottom) while GATHER is fastest, smallest T from which MFMA stays fastest
    ratio = None
    for r in rows:
        if r["fastest"] != "gather":
            break
        ratio = r["pairs_per_expert"]
    mfma_min = None
    for r in reversed(rows):
        if r["fastest"] != "mfma":
            break
        mfma_min = r["pairs_per_expert"]
    print(json.dumps({"workload": args.workload, "E": E, "top_k": k, "gate_ratio": ratio,
                      "mfma_min_tokens_per_expert": mfma_min}), flush=True)


if __name__ == "__main__":
    main()
