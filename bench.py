#!/usr/bin/env python3
"""Benchmark of the block-FP8 MoE expert path on one MI355X.

Default workload: single-stream decode, E=256 experts, H=2048, I=512, top_k=8, T=1, bf16
hidden and output, fp8-e4m3 banks with bf16 128x128 block scales (rows padded to 16 B).
The metric is routed-weight GB/s: the bytes of the distinct experts each forward routes
to (codes plus their block scales), divided by the time per forward.

A step is one whole forward (route, sort, GEMM1 + silu*up, GEMM2 + combine) over one
batch of synthetic input already resident in HBM. Steps rotate over up to 64 pre-drawn
routings and 4 replicas of the banks (about 3.2 GB), so the 256 MB Infinity Cache cannot
serve a routed expert from an earlier step. K steps are captured into HIP graphs: one of
S = min(64, K) forwards, replayed K // S times, and one of the K % S remaining forwards;
each is replayed once before the timed region. The timed region is queued behind a spin
kernel, so it measures the GPU running K forwards back to back (HIP events on the stream),
not the host's graph launches.

Also reported on the same JSON line:
  roofline      the dominant kernel's algorithmic bytes per launch over its mean duration,
                timed with HIP events the library attaches to that kernel's dispatch on
                its own stream (moe_fp8_block_forward_timed), against the 8 TB/s HBM peak;
  cpu_baseline  the float64 oracle timed on this host's cores on a bounded sample;
  sweep_T4, sweep_T16, sweep_T64, prefill_T4096, prefill_T16384, prefill_T16384_group_fp8,
  large_T1
                the same measurement (fewer steps) at the decode banks with Zipf(1.1) expert
                popularity at T = 4, 16, 64 (the path the gate picks; routed GB/s), the
                prefill workload (E=256, H=2048, I=512, top_k=8, uniform logits; tokens/s and
                % of fp8 MFMA peak; also with group-fp8 activations) and the large-expert
                decode workload (H=7168, I=2048; routed GB/s), each with its dominant
                kernel's roofline (--no-extra skips them).

  python bench.py [--steps K] [--warmup W] [--workload decode|sweep|large|prefill] [--T T]
                  [--path auto|gather|stream|mfma] [--act path|group_fp8]

Two helpers turn rocprofv3 counters into the HBM traffic the roofline reports:
  python bench.py --copy-calibration
      copies 1 GiB device to device three times: run it under rocprofv3 --pmc FETCH_SIZE
      (then WRITE_SIZE) to learn how those counters scale for a transfer of known size;
  python bench.py --traffic-record --kernel K --workload W --fetch-dir D1 --write-dir D2
                  --copy-fetch-dir D3 --copy-write-dir D4
      reads the four rocprofv3 output folders and writes profiles/traffic_K_W.json: the
      dominant kernel's FETCH_SIZE + WRITE_SIZE per launch, each scaled by what the counter
      read for the known copy, stamped with a digest of the kernel sources (the bench only
      reports it while the sources are unchanged).
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "routed-weight GB/s (% HBM peak) at decode; prefill tokens/s (% fp8 MFMA peak)"
HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0
CPU_REFERENCE_GBS = 53.7  # block-fp8 CPU MoE kernel, 2x Xeon Gold 6526Y (FreeToken PR #662)

WORKLOADS = {
    "decode": dict(T=1, desc="single-stream decode"),
    "sweep": dict(T=12, desc="Zipf(1.1) popularity"),
    "large": dict(T=1, desc="large-expert decode"),
    "prefill": dict(T=4096, desc="prefill grouped GEMM"),
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2048)
    ap.add_argument("--warmup", type=int, default=256)
    ap.add_argument("--workload", default="decode", choices=sorted(WORKLOADS))
    ap.add_argument("--T", type=int, default=None)
    ap.add_argument("--path", default="auto", choices=["auto", "gather", "stream", "mfma"],
                    help="force a path instead of the gate's choice")
    ap.add_argument("--act", default="path", choices=["path", "group_fp8"],
                    help="activation precision (group_fp8: e4m3 per token and 128 columns on GEMM1)")
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--sets", type=int, default=64)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the sweep, prefill and large-expert figures")
    ap.add_argument("--kernel-steps", type=int, default=64, help="steps timed per kernel with events")
    ap.add_argument("--copy-calibration", action="store_true", help="copy 1 GiB three times and exit")
    ap.add_argument("--traffic-record", action="store_true", help="write profiles/traffic_<kernel>_<workload>.json")
    ap.add_argument("--kernel", default="gemm1")
    ap.add_argument("--fetch-dir")
    ap.add_argument("--write-dir")
    ap.add_argument("--copy-fetch-dir")
    ap.add_argument("--copy-write-dir")
    return ap.parse_args()


# kernel kinds of the library -> a substring of their symbol names
KERNEL_SYMBOLS = {"route": "route_", "sort": "sort_", "quant": "quant_rows_bf16", "hquant": "quant_rows_f32",
                  "gemm1": "gemm1_", "gemm2": "gemm2_",
                  "combine": "combine_"}
COPY_BYTES = 1 << 30


def copy_calibration():
    import torch

    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "copies": 3}))


def _counter_per_dispatch(folder: str, counter: str, name_has: str):
    """Mean value of one rocprofv3 counter per dispatch of the kernels whose name contains
    name_has, from the counter_collection CSVs under folder."""
    import csv
    import glob

    vals = []
    for f in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for row in csv.DictReader(fh):
                if row["Counter_Name"] == counter and name_has in row["Kernel_Name"]:
                    vals.append(float(row["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no {counter} records for kernels matching {name_has!r} under {folder}")
    return sum(vals) / len(vals), len(vals)


def traffic_record(args):
    """HBM bytes per launch of one kernel from FETCH_SIZE / WRITE_SIZE (KiB per dispatch),
    each scaled by the same counter's reading for a device copy of known size."""
    copy_sym = "copyBuffer"
    cf, _ = _counter_per_dispatch(args.copy_fetch_dir, "FETCH_SIZE", copy_sym)
    cw, _ = _counter_per_dispatch(args.copy_write_dir, "WRITE_SIZE", copy_sym)
    f_scale = COPY_BYTES / (cf * 1024.0)
    w_scale = COPY_BYTES / (cw * 1024.0)
    sym = KERNEL_SYMBOLS[args.kernel]
    if args.act == "group_fp8" and args.kernel == "quant":
        sym = "quant_groups_bf16"
    if args.act == "path" and args.kernel == "route" and args.workload == "prefill":
        # the MFMA forward's routing kernel, which also quantises x; the plain top-k launches
        # that count each input set's routed experts before timing are left out
        sym = "route_topk_quant"
    kf, nf = _counter_per_dispatch(args.fetch_dir, "FETCH_SIZE", sym)
    kw, nw = _counter_per_dispatch(args.write_dir, "WRITE_SIZE", sym)
    rec = {
        "kernel": args.kernel,
        "workload": args.workload,
        "act": args.act,
        "fetch_kib_per_launch": round(kf, 1),
        "write_kib_per_launch": round(kw, 1),
        "dispatches": [nf, nw],
        "copy_fetch_kib": round(cf, 1),
        "copy_write_kib": round(cw, 1),
        "fetch_scale": round(f_scale, 4),
        "write_scale": round(w_scale, 4),
        "bytes_per_launch": round(kf * 1024.0 * f_scale + kw * 1024.0 * w_scale),
        "source_digest": source_digest(),
    }
    path = os.path.join(ROOT, "profiles", f"traffic_{args.kernel}_{traffic_key(args.workload, args.T, args.act)}.json")
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    print(json.dumps(rec))


class Hip:
    """hipEvent helpers from the HIP runtime (events the library records on its stream)."""

    def __init__(self):
        self.rt = ctypes.CDLL("libamdhip64.so")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def events(self, n):
        out = (ctypes.c_void_p * n)()
        for i in range(n):
            ev = ctypes.c_void_p()
            if self.rt.hipEventCreate(ctypes.byref(ev)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out[i] = ev.value
        return out

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        if self.rt.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def destroy(self, evs):
        for e in evs:
            self.rt.hipEventDestroy(ctypes.c_void_p(e))


def source_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_fp8_mixture_top_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f == "gate_table.inc":  # the gate's table picks paths; it changes no kernel
            continue
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def traffic_key(workload: str, T, act: str = "path") -> str:
    """Name of a workload's traffic record: the workload, plus T when it is not the default,
    plus the activation mode when it is not the path's own."""
    key = workload if T is None or T == WORKLOADS[workload]["T"] else f"{workload}_T{T}"
    return key if act == "path" else f"{key}_{act}"


def committed_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken
    on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_digest") != source_digest():
        return None
    return rec.get("bytes_per_launch")


def _forward_timed_kernels(M, L, hip, cases, outs, ws, fopts, T, E, H, I, k, nk, steps):
    """Per-kernel durations (ms per forward, summed over a kind's kernels) from HIP events the
    library attaches to each kernel's dispatch on the stream the kernels run on. A spin
    kernel first lets the host enqueue every forward before the GPU reaches them."""
    import numpy as np
    import torch

    evs = [hip.events(2 * nk) for _ in range(steps)]
    kinds = (ctypes.c_int32 * nk)()
    torch.cuda.synchronize()
    torch.cuda._sleep(int(2e8))
    for i in range(steps):
        c = cases[i % len(cases)]
        b13 = M.bank_struct(c.w13, E, 2 * I, H, c.hidden.device)
        b2 = M.bank_struct(c.w2, E, H, I, c.hidden.device)
        o = M.make_opts(**fopts)
        ri = L.RunInfo()
        L.check(M.lib().moe_fp8_block_forward_timed(
            ctypes.c_void_p(c.hidden.data_ptr()), ctypes.c_void_p(c.logits.data_ptr()), ctypes.byref(b13),
            ctypes.byref(b2), T, E, H, I, k, ctypes.c_void_p(outs[i % len(outs)].data_ptr()), L.MOE_BF16,
            ctypes.c_void_p(ws.data_ptr()), ws.numel(), None, None, ctypes.byref(o), ctypes.byref(ri),
            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream), evs[i], 2 * nk, kinds))
    torch.cuda.synchronize()
    per_kernel = {}
    for j in range(nk):
        if kinds[j] == 0:  # the forward launched fewer kernels
            break
        name = L.KERNEL_NAMES.get(kinds[j], str(kinds[j]))
        d = [hip.elapsed_ms(evs[i][2 * j], evs[i][2 * j + 1]) for i in range(steps)]
        per_kernel.setdefault(name, []).append(float(np.mean(d)))
    for e_ in evs:
        hip.destroy(e_)
    return {n: sum(v) for n, v in per_kernel.items()}


def _pad128(n: int) -> int:
    return (n + 127) // 128 * 128


def kernel_work(kernel, path, act, T, H, I, k, mean_de, w13_b, w2_b):
    """Algorithmic HBM bytes and flops of one launch of a GEMM kernel (None, None for the
    others): the routed experts' codes and scales (mean_de of them), the activations it
    reads and the results it writes, in the layout the path uses."""
    P = T * k
    if kernel not in ("gemm1", "gemm2"):
        return None, None
    flops = (4.0 if kernel == "gemm1" else 2.0) * P * H * I
    if path != "mfma":  # W8A16: bf16 x, float h; GATHER's GEMM2 writes the output row
        if kernel == "gemm1":
            return mean_de * w13_b + T * H * 2 + P * I * 4, flops
        return mean_de * w2_b + P * I * 4 + T * H * 2, flops
    group = act == "group_fp8"
    parts = -(-_pad128(I) // 512)
    if kernel == "gemm1":
        x = T * H + T * (H // 128) * 4 if group else T * _pad128(H) + T * 4
        h = P * I + P * (I // 128) * 4 if group else P * I * 4
        return mean_de * w13_b + x + h, flops
    h = P * I + P * (I // 128) * 4 if group else P * _pad128(I) + P * 4
    y = parts * P * (H * 2 + -(-H // 32))
    return mean_de * w2_b + h + y, flops


def roofline_of(nbytes, flops, ms):
    """The roofline a kernel sits under: HBM if its bytes at 8 TB/s take longer than its
    flops at the fp8 matrix-core peak, else the matrix cores; achieved = that quantity over
    the measured duration. Both fractions are kept."""
    if nbytes is None:
        return dict(bound=None, achieved=None, peak=None, unit=None, frac=None)
    gbs = nbytes / (ms * 1e-3) / 1e9
    tfl = flops / (ms * 1e-3) / 1e12
    hbm_bound = nbytes / (HBM_PEAK_GBS * 1e9) >= flops / (FP8_PEAK_TFLOPS * 1e12)
    if hbm_bound:
        r = dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s", frac=round(gbs / HBM_PEAK_GBS, 4))
    else:
        r = dict(bound="mfma", achieved=round(tfl, 2), peak=FP8_PEAK_TFLOPS, unit="TFLOP/s",
                 frac=round(tfl / FP8_PEAK_TFLOPS, 4))
    r.update(hbm_frac=round(gbs / HBM_PEAK_GBS, 4), mfma_frac=round(tfl / FP8_PEAK_TFLOPS, 4),
             algorithmic_bytes=round(nbytes), algorithmic_flops=round(flops))
    return r


def measure(wl, T, steps, warmup, sets, replicas, path, act, seed, kernel_steps, quiet=False):
    """Times `steps` whole forwards of one workload and returns its figures.

    The forwards are captured into HIP graphs: one of S = min(sets, steps) forwards over S
    pre-drawn input sets (cycling over `replicas` copies of the banks), replayed steps // S
    times, and one of the remaining steps % S forwards. Every graph the timed region replays
    is replayed once before it. The timed region starts behind a spin kernel, so the host's
    graph launches are queued before the GPU reaches the first forward: what is timed is the
    GPU running `steps` forwards back to back, bracketed by HIP events on the stream.
    """
    import numpy as np
    import torch

    import block_fp8_mixture_top_amd as M
    import workloads as W
    from block_fp8_mixture_top_amd import _lib as L

    dev = torch.device("cuda:0")
    shp = W.SHAPES[wl]
    E, H, I, k = shp["E"], shp["H"], shp["I"], shp["top_k"]
    S = max(1, min(sets, steps))
    R = max(1, min(replicas, S))
    log = (lambda *a: None) if quiet else (lambda *a: print("[bench]", *a, file=sys.stderr, flush=True))
    log(f"workload {wl} T={T} E={E} H={H} I={I} top_k={k}: {R} bank replicas, {S} input sets")
    banks = [W.make_banks(wl, seed=seed + 100 * r, device=dev) for r in range(R)]
    cases = [W.make_case(wl, T=T, seed=seed + 1000 + i, device=dev, banks=banks[i % R]) for i in range(S)]
    outs = [torch.empty((T, H), dtype=torch.bfloat16, device=dev) for _ in range(S)]
    fopts = dict(force_path={"auto": M.PATH_AUTO, "gather": M.PATH_GATHER, "stream": M.PATH_STREAM,
                             "mfma": M.PATH_MFMA}[path],
                 act_mode=M.ACT_GROUP_FP8 if act == "group_fp8" else M.ACT_PATH)
    nbytes = max(M.workspace_size(T, E, H, I, k, **fopts), 1)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    w13_b, w2_b = banks[0][0].expert_bytes, banks[0][1].expert_bytes

    # routed experts of every set (their bytes are the decode metric's numerator)
    d_e = []
    for c in cases:
        r = M.route(c.logits, k, sort=False)
        d_e.append(int(torch.unique(r["ids"]).numel()))
    torch.cuda.synchronize()
    step_bytes = [d * (w13_b + w2_b) for d in d_e]

    def step(i):
        c = cases[i % S]
        return M.forward(c.hidden, c.logits, c.w13, c.w2, k, out=outs[i % S], workspace=ws, **fopts)[1]

    info = step(0)
    torch.cuda.synchronize()
    log(f"path {info['path']}, {info['kernels']} kernels per forward")

    graphs = {}

    def graph_of(n):  # a graph of forwards 0 .. n-1 (input sets cycled)
        if n not in graphs:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(n):
                    step(i)
            graphs[n] = [g, False]
        return graphs[n]

    def run(nsteps):
        plan = [S] * (nsteps // S) + ([nsteps % S] if nsteps % S else [])
        for n in plan:
            g = graph_of(n)
            g[0].replay()
            g[1] = True

    def bytes_of(nsteps):
        full, rem = divmod(nsteps, S)
        return full * sum(step_bytes) + sum(step_bytes[:rem])

    log(f"warmup {warmup} steps")
    run(warmup)
    for n in [S] * (steps // S > 0) + ([steps % S] if steps % S else []):
        g = graph_of(n)
        if not g[1]:  # a graph the timed region uses is replayed once first
            g[0].replay()
            g[1] = True
    torch.cuda.synchronize()

    log(f"timing {steps} steps")
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    torch.cuda._sleep(int(4e6))  # about 2 ms: the launches below are queued behind it
    start.record()
    run(steps)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(end)
    gbs = bytes_of(steps) / (ms * 1e-3) / 1e9
    tok_s = steps * T / (ms * 1e-3)

    hip = Hip()
    nk = info["kernels"]
    per_kernel = _forward_timed_kernels(M, L, hip, cases, outs, ws, fopts, T, E, H, I, k, nk,
                                        min(kernel_steps, max(S, 8)))
    dom = max(per_kernel, key=per_kernel.get)
    dom_ms = per_kernel[dom]
    mean_de = float(np.mean(d_e))
    flops = 6.0 * T * k * H * I
    kb, kf = kernel_work(dom, info["path"], act, T, H, I, k, mean_de, w13_b, w2_b)
    roofline = roofline_of(kb, kf, dom_ms)
    roofline["traffic"] = committed_traffic(dom, traffic_key(wl, T, act))
    roofline["kernel"] = dom
    roofline["kernel_ms"] = round(dom_ms, 5)
    roofline["kernels_ms"] = {n: round(v, 5) for n, v in per_kernel.items()}
    return dict(
        wl=wl, T=T, E=E, H=H, I=I, k=k, info=info, ms=ms, steps=steps, S=S, R=R, wall=wall, gbs=gbs,
        tok_s=tok_s, flops=flops, mean_de=mean_de, total_bytes=bytes_of(steps), roofline=roofline,
        scale_dtype=banks[0][0].scale_dtype, cases=cases, expert_bytes=w13_b + w2_b,
        tflops=flops * steps / (ms * 1e-3) / 1e12,
    )


def summary(m):
    """The compact object a secondary workload contributes to the JSON line."""
    ms_step = m["ms"] / m["steps"]
    d = {
        "workload": f"{m['wl']}: E={m['E']} H={m['H']} I={m['I']} top_k={m['k']} T={m['T']}",
        "path": m["info"]["path"],
        "act_mode": m["info"]["act_mode"],
        "steps": m["steps"],
        "ms_per_step": round(ms_step, 6),
    }
    if m["info"]["path"] == "mfma":
        d.update(tokens_per_s=round(m["tok_s"], 1), tflops=round(m["tflops"], 2),
                 pct_fp8_mfma_peak=round(100.0 * m["tflops"] / FP8_PEAK_TFLOPS, 2),
                 pct_hbm_peak_on_weights=round(100.0 * m["gbs"] / HBM_PEAK_GBS, 2))
    else:
        d.update(routed_gbs=round(m["gbs"], 1), pct_hbm_peak=round(100.0 * m["gbs"] / HBM_PEAK_GBS, 2),
                 tokens_per_s=round(m["tok_s"], 1))
    d["roofline"] = m["roofline"]
    return d


# Secondary workloads reported beside the headline decode line: (name, workload, T, steps,
# warmup, input sets, bank replicas, activations). One replica suffices where a forward
# already touches more than the 256 MB Infinity Cache holds.
EXTRAS = [
    ("sweep_T4", "sweep", 4, 512, 64, 32, 4, "path"),
    ("sweep_T16", "sweep", 16, 256, 32, 16, 4, "path"),
    ("sweep_T64", "sweep", 64, 128, 16, 8, 2, "path"),
    ("prefill_T4096", "prefill", 4096, 40, 4, 4, 1, "path"),
    ("prefill_T16384", "prefill", 16384, 12, 2, 2, 1, "path"),
    ("prefill_T16384_group_fp8", "prefill", 16384, 12, 2, 2, 1, "group_fp8"),
    ("large_T1", "large", 1, 64, 8, 16, 1, "path"),
    ("large_T16", "large", 16, 16, 2, 4, 1, "path"),
]


def main():
    args = parse()
    if args.copy_calibration:
        return copy_calibration()
    if args.traffic_record:
        return traffic_record(args)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures the single-GPU hot path; runs on more than one GPU are not part of this "
              "benchmark (use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    wl = args.workload
    T = args.T or WORKLOADS[wl]["T"]
    R = min(args.replicas, 1) if wl == "large" else args.replicas  # 11.3 GB per replica
    m = measure(wl, T, args.steps, args.warmup, args.sets, R, args.path, args.act, args.seed, args.kernel_steps)
    K = args.steps
    info = m["info"]

    extras = {}
    if wl == "decode" and T == 1 and args.path == "auto" and args.act == "path" and not args.no_extra:
        for name, ewl, eT, esteps, ewarm, esets, erep, eact in EXTRAS:
            torch.cuda.empty_cache()
            em = measure(ewl, eT, esteps, ewarm, esets, erep, "auto", eact, args.seed, 8)
            extras[name] = summary(em)
            print(f"[bench] {name}: {json.dumps(extras[name])}", file=sys.stderr, flush=True)
            del em
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(m["cases"], m["k"], args.cpu_seconds, m["expert_bytes"], prefill=wl == "prefill")

    if info["path"] == "mfma" or wl == "prefill":
        value, unit = m["tok_s"], "tokens/s"
    else:
        value, unit = m["gbs"], "GB/s"
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(m["ms"] / K, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(value / CPU_REFERENCE_GBS, 2) if unit == "GB/s" and wl == "decode" else None,
        "dtype": {0: "fp8e4m3 x bf16 -> fp32", 1: "fp8e4m3 x fp8e4m3 -> fp32",
                  2: "fp8e4m3 x fp8e4m3 -> fp32 (gate/up), fp8e4m3 x fp32 (down)",
                  3: "fp8e4m3 x fp8e4m3 -> fp32, activation scales per 128-column group"}[info["act_mode"]],
        "data": "synthetic",
        "config": {
            "workload": f"{wl}: E={m['E']} H={m['H']} I={m['I']} top_k={m['k']} T={T}, bf16 hidden/out, "
                        f"fp8-e4m3 banks with {m['scale_dtype']} 128x128 block scales",
            "path": info["path"],
            "kernels_per_forward": info["kernels"],
            "routed_experts_mean": m["mean_de"],
            "routed_bytes_per_step": round(m["total_bytes"] / K),
            "bank_replicas": m["R"],
            "input_sets": m["S"],
            "timing": f"{K // m['S']} replays of a {m['S']}-forward graph"
                      + (f" + one {K % m['S']}-forward graph" if K % m["S"] else "")
                      + ", queued behind a spin kernel; HIP events on the stream",
            "pct_hbm_peak": round(100.0 * m["gbs"] / HBM_PEAK_GBS, 2),
            "tokens_per_s": round(m["tok_s"], 1),
            "wall_s": round(m["wall"], 4),
        },
        "roofline": m["roofline"],
        "cpu_baseline": cpu,
    }
    if info["path"] == "mfma":
        rec["config"]["pct_fp8_mfma_peak"] = round(100.0 * m["tflops"] / FP8_PEAK_TFLOPS, 2)
    rec.update(extras)
    print(json.dumps(rec), flush=True)


def cpu_baseline(cases, k, seconds, expert_bytes, prefill=False):
    """The float64 oracle (gathered formulation) on this host, repeated over the first sets
    for about `seconds`; GB/s over the same routed bytes. With `prefill`, the oracle in its
    W8A8 mode (the MFMA path's reading) on successive 16-token slices of the first set,
    reported in tokens/s."""
    import numpy as np
    import torch

    import oracle as O

    try:
        from threadpoolctl import threadpool_info

        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = 1

    def host_bank(bank, experts):
        codes = np.zeros(bank.codes.numel(), dtype=np.uint8)
        st = bank.expert_stride_bytes
        for e in experts:
            codes[e * st:(e + 1) * st] = bank.codes[e * st:(e + 1) * st].cpu().numpy()
        sc = bank.scales.cpu()
        scales = sc.view(torch.int16).numpy().view(np.uint16) if bank.scale_dtype == "bf16" else sc.numpy()
        return dict(codes=codes, scales=scales, scale_dtype=bank.scale_dtype, E=bank.E, N=bank.N, K=bank.K,
                    expert_stride_bytes=st, scale_row_stride=bank.scale_row_stride,
                    scale_expert_stride=bank.scale_expert_stride)

    if prefill:
        c = cases[0]
        hid_all = c.hidden.cpu().view(torch.int16).numpy().view(np.uint16)
        lg_all = c.logits.cpu().numpy()
        spent, tokens, q = 0.0, 0, 0
        while spent < seconds and q * 16 < hid_all.shape[0]:
            rows = slice(q * 16, (q + 1) * 16)
            ids, _, _ = O.route(lg_all[rows], k)
            used = [int(e) for e in O.routed_experts(ids)]
            w13, w2 = host_bank(c.w13, used), host_bank(c.w2, used)
            t0 = time.perf_counter()
            O.forward(hid_all[rows], lg_all[rows], w13, w2, k, act_mode=1)
            spent += time.perf_counter() - t0
            tokens += 16
            q += 1
        return {
            "value": round(tokens / spent, 2),
            "unit": "tokens/s",
            "cores": threads,
            "host_cpus": len(os.sched_getaffinity(0)),
            "kind": "oracle",
            "sample": f"{tokens} tokens of the first input set in 16-token slices (float64 gathered oracle, "
                      f"W8A8 reading, {spent:.1f} s)",
        }

    # host copies of the first few sets (only the routed experts' pages are ever touched),
    # then forwards over them in turn until about `seconds` of oracle time
    prepared = []
    for c in cases[:8]:
        hid = c.hidden.cpu().view(torch.int16).numpy().view(np.uint16)
        lg = c.logits.cpu().numpy()
        ids, _, _ = O.route(lg, k)
        used = [int(e) for e in O.routed_experts(ids)]
        prepared.append((hid, lg, host_bank(c.w13, used), host_bank(c.w2, used), len(used)))
    spent, nbytes, n = 0.0, 0, 0
    while spent < seconds:
        hid, lg, w13, w2, n_used = prepared[n % len(prepared)]
        t0 = time.perf_counter()
        O.forward(hid, lg, w13, w2, k)
        spent += time.perf_counter() - t0
        nbytes += n_used * expert_bytes
        n += 1
    return {
        "value": round(nbytes / spent / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "host_cpus": len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": f"{n} forwards over {len(prepared)} input sets of the same workload "
                  f"(float64 gathered oracle, {spent:.1f} s)",
    }


if __name__ == "__main__":
    main()
