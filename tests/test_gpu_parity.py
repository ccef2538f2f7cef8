"""GPU parity: the HIP library through its C ABI against the float64 oracle.

Routing, sort and every integer result must match bit for bit; float outputs must satisfy
max|out - ref| / max|ref| <= 2e-3 (after the bf16 output rounding for bf16 outputs, and
with the per-output allowance for the e4m3 roundings of h that the oracle's drift bound
leaves undecided on the W8A8 path). The W8A8 path is also checked in halves: GEMM1's h
against the drift bound at every element, and the down GEMM + combine on the oracle's own h
against a per-output accumulation bound. Inputs come from the seeded generators; the oracle
sees host copies of exactly the tensors the library reads.
"""

import numpy as np
import pytest
import torch

import block_fp8_mixture_top_amd as M
import oracle as O
import oracle.oracle as OO
import workloads as W
from helpers import REL_TOL, bank_numpy, bf16_bits, bf16_half_ulp, fp8_ulp_diff, rel_err, rel_err_bf16

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
PATHS = {"gather": M.PATH_GATHER, "stream": M.PATH_STREAM, "mfma": M.PATH_MFMA}


def say(*a):
    print("[case]", *a, flush=True)


def oracle_out(case, rows=None, act_mode=0, experts=None):
    hid = bf16_bits(case.hidden)
    lg = case.logits.detach().cpu().numpy()
    if rows is not None:
        hid, lg = hid[rows], lg[rows]
    w13 = bank_numpy(case.w13, experts)
    w2 = bank_numpy(case.w2, experts)
    return O.forward(hid, lg, w13, w2, case.top_k, act_mode=act_mode)


def check_out(out, res, act_mode, what):
    """The float bar, with bf16 rounding and W8A8 allowance taken out of the error."""
    ref = res["out"]
    o = out.detach().float().cpu().numpy().astype(np.float64)
    den = float(np.max(np.abs(ref)))
    err = np.abs(o - ref)
    if out.dtype == torch.bfloat16:
        err = np.maximum(0.0, err - bf16_half_ulp(np.maximum(np.abs(o), np.abs(ref))))
    extra = ""
    if act_mode in (1, 3):
        err = np.maximum(0.0, err - res["allowance"])
        extra = f"allowance max {float(np.max(res['allowance'])) / den:.3e} flagged {res['n_flagged'] / res['n_h']:.3%}"
    r = float(np.max(err)) / den
    say(what, f"rel={r:.3e}", f"raw={rel_err(o, ref):.3e}", extra)
    assert np.isfinite(o).all(), what
    assert r <= REL_TOL, f"{what}: {r}"
    return r


# ------------------------------------------------------------------- e4m3 conversions

def test_decode_every_code_exactly():
    say("decode 256 codes")
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).to(DEV)
    got = M.decode_e4m3(codes).cpu().numpy().astype(np.float64)
    lut = O.e4m3_lut()
    finite = [c for c in range(256) if (c & 0x7F) != 0x7F]
    assert np.array_equal(got[finite], lut[finite])
    assert np.array_equal(np.signbit(got[finite]), np.signbit(lut[finite]))


def test_every_decode_path_on_every_code_and_position():
    """Every decode the kernels use (word conversion to float, both halves; conversion to
    bf16 with unit scale, both halves; the codes x bf16, e4m3 x e4m3 and codes x float dot
    helpers against one-hot activations) gives every finite code's value exactly, bit for
    bit and with its sign, at every one of the 16 byte positions of a chunk."""
    say("decode paths")
    lut = O.e4m3_lut()
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    n = len(finite)  # 254; chunk i holds finite[(i + 17 j) % 254] at byte j
    idx = (np.arange(n)[:, None] + 17 * np.arange(16)[None, :]) % n
    chunks = finite[idx]
    got = M.decode_e4m3_paths(torch.from_numpy(chunks).to(DEV)).cpu().numpy().astype(np.float64)
    want = lut[chunks]
    for path in range(5):
        g = got[:, :, path]
        # the conversions keep the sign of zero; a dot helper's sum starts at +0, and
        # +0 + (-0) is +0, so for paths 2..4 only the value of 0x80 is compared
        sign = (np.signbit(g) != np.signbit(want)) & ((want != 0) | (path < 2))
        bad = np.nonzero((g != want) | sign)
        assert bad[0].size == 0, (path, [(hex(chunks[i, j]), g[i, j], want[i, j]) for i, j in zip(*bad)][:6])
    # every code reached every position
    for j in range(16):
        assert sorted(chunks[:, j].tolist()) == sorted(finite.tolist())


@pytest.mark.parametrize("path,H", [("gather", 272), ("stream", 272), ("gather", 256), ("stream", 256),
                                    ("mfma", 256)])
def test_subnormal_only_banks(path, H):
    """Banks of subnormal codes only (+-1..7 * 2^-9, unit scales), at the tiny shape and at a
    ragged H (272: a partial last scale block), float output: a flushed or mis-decoded
    subnormal in any kernel moves the output by far more than the bar."""
    c = W.make_case("tiny", T=4, seed=12, H=H, kind="subnormal").to(DEV)
    say("subnormal banks", path, H)
    act = 1 if path == "mfma" else 0
    out, info = M.forward(c.hidden, c.logits, c.w13, c.w2, c.top_k, out_dtype=torch.float32,
                          force_path=PATHS[path])
    assert info["path"] == path
    res = oracle_out(c, act_mode=act)
    assert np.abs(res["out"]).max() > 0
    check_out(out, res, act, f"subnormal {path} H={H}")


def test_encode_matches_oracle():
    say("encode midpoints")
    pos = O.e4m3_lut()[:0x7F]
    mids = 0.5 * (pos[:-1] + pos[1:])
    m32 = mids.astype(np.float32)
    g = np.random.default_rng(11)
    v = np.concatenate([pos, mids, np.nextafter(m32, np.float32(np.inf)), np.nextafter(m32, np.float32(-np.inf)),
                        g.normal(0, 50, 20000), g.uniform(-600, 600, 5000), [0.0, -0.0, 1e30, -1e30, 2.0 ** -11]])
    v = np.concatenate([v, -v]).astype(np.float32)
    got = M.encode_e4m3(torch.from_numpy(v).to(DEV)).cpu().numpy()
    want = O.e4m3_encode(v)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(v[i]), hex(got[i]), hex(want[i])) for i in bad[:8]]


def test_quantize_rows_bit_exact():
    say("quantize rows")
    g = torch.Generator().manual_seed(3)
    x = (torch.randn(37, 2048, generator=g) * torch.rand(37, 1, generator=g) * 5).to(torch.bfloat16)
    x[5] = 0
    x[6, :100] = 300.0
    codes, scales = M.quantize_rows(x.to(DEV))
    q, s = O.quantize_rows(O.bf16_to_f64(bf16_bits(x)).astype(np.float32))
    assert np.array_equal(scales.cpu().numpy(), s)
    assert np.array_equal(codes.cpu().numpy(), q)


# ------------------------------------------------------------------- routing

def _route_check(logits, k, what):
    say("route", what, tuple(logits.shape), k)
    r = M.route(logits.to(DEV), k)
    ids, w, w32 = O.route(logits.cpu().numpy(), k)
    counts, offsets, sp = O.sort_pairs(ids, logits.shape[1])
    assert np.array_equal(r["ids"].cpu().numpy(), ids), what
    gw = r["weights"].cpu().numpy()
    nbad = int((gw != w32).sum())
    assert nbad == 0, f"{what}: {nbad} weights differ (max {np.max(np.abs(gw - w32))})"
    assert np.array_equal(r["counts"].cpu().numpy(), counts), what
    assert np.array_equal(r["offsets"].cpu().numpy(), offsets), what
    assert np.array_equal(r["sorted_pairs"].cpu().numpy(), sp), what


@pytest.mark.parametrize("name,T", [("tiny", 4), ("decode", 1), ("sweep", 1), ("sweep", 12), ("sweep", 64),
                                    ("large", 16), ("prefill", 4096), ("prefill", 16384)])
def test_route_bit_exact(name, T):
    shp = W.SHAPES[name]
    kind = {"tiny": "normal", "decode": "normal", "sweep": "zipf", "large": "normal", "prefill": "uniform"}[name]
    std = 1.5 if name == "decode" else 1.0
    logits = W.make_logits(T, shp["E"], kind, seed=77 + T, std=std)
    _route_check(logits, shp["top_k"], f"{name} T={T}")


def test_route_ties_and_extremes():
    g = torch.Generator().manual_seed(1)
    tied = (torch.randn(300, 64, generator=g) * 2).round() / 2
    tied[0] = 0.25
    _route_check(tied, 6, "ties")
    big = torch.randn(70, 1024, generator=g)
    _route_check(big, 32, "E=1024 k=32")
    _route_check(torch.randn(5000, 1024, generator=g), 1, "E=1024 k=1 multi-block sort")
    _route_check(torch.randn(3, 1, generator=g), 1, "E=1")
    # E=256, k=8: coarse ties that the candidate filter ranks by id (T=40: one wave per
    # token), and rows of one value, where too many logits pass the filter and the
    # round-based selection runs (T=4: routed inside the sort)
    coarse = (torch.randn(40, 256, generator=g) * 2).round() / 2
    _route_check(coarse, 8, "E=256 coarse ties")
    _route_check(coarse[:4], 8, "E=256 coarse ties, T=4")
    flat = torch.full((4, 256), 0.5)
    flat[1, 200] = 1.0
    flat[2, ::3] = -0.0
    _route_check(flat, 8, "E=256 equal rows")
    _route_check(flat.repeat(10, 1), 8, "E=256 equal rows, T=40")


@pytest.mark.parametrize("T,E,k", [(16, 256, 8), (17, 256, 8), (64, 64, 8), (512, 128, 1), (40, 1024, 12),
                                   (512, 256, 8), (513, 256, 8), (4096, 1024, 1), (342, 1024, 12), (100, 3, 3)])
def test_route_plan_boundaries(T, E, k):
    """Around the routing split: up to 16 tokens are routed inside the one-workgroup sort,
    more are routed by one wave per token first; up to 4096 pairs use the one-workgroup sort
    (16 waves, each counting and placing a chunk), more the multi-block one."""
    g = torch.Generator().manual_seed(T * 1000 + E + k)
    _route_check(torch.randn(T, E, generator=g) * 1.5, k, f"T={T} E={E} k={k}")


@pytest.mark.parametrize("T,E,k", [(1, 40, 8), (3, 100, 8), (20, 300, 8), (33, 512, 8), (70, 1024, 8),
                                   (5, 1024, 7), (2, 8, 8)])
def test_route_filtered_top_k_shapes(T, E, k):
    """The candidate-filter top-k (k <= 8) across expert counts: padding lanes (E < 64 and
    E not a multiple of 64), 2 to 16 logits per lane, one wave per token and routing inside
    the sort; plain and coarsely tied logits."""
    g = torch.Generator().manual_seed(T * 7 + E + k)
    plain = torch.randn(T, E, generator=g) * 1.5
    _route_check(plain, k, f"T={T} E={E} k={k}")
    _route_check((plain * 2).round() / 2, k, f"T={T} E={E} k={k} tied")


def test_route_empty():
    r = M.route(torch.empty((0, 16), dtype=torch.float32, device=DEV), 4)
    assert r["ids"].numel() == 0


# ------------------------------------------------------------------- forward parity

@pytest.mark.parametrize("path", ["gather", "stream", "mfma"])
@pytest.mark.parametrize("T", [1, 2, 4, 5])
def test_tiny_forward(path, T):
    c = W.make_case("tiny", T=T, seed=T).to(DEV)
    say("tiny", path, "T", T)
    out, info = M.forward(c.hidden, c.logits, c.w13, c.w2, c.top_k, out_dtype=torch.float32,
                          force_path=PATHS[path], return_routing=True)
    torch.cuda.synchronize()
    assert info["path"] == path
    act = 1 if path == "mfma" else 0
    res = oracle_out(c, act_mode=act)
    assert np.array_equal(info["ids"].cpu().numpy(), res["ids"])
    check_out(out, res, act, f"tiny {path} T={T}")


@pytest.mark.parametrize("path", ["gather", "stream", "mfma"])
@pytest.mark.parametrize("pad", ["row16", "slab16"])
def test_padded_banks(path, pad):
    """Padded scale strides and expert strides with NaN in every padding byte."""
    c = W.make_case("decode", T=3, seed=9, E=16, H=640, I=384, top_k=4, pad=pad, code_pad_bytes=48).to(DEV)
    assert c.w13.scale_row_stride > c.w13.scale_cols or c.w2.scale_row_stride > c.w2.scale_cols
    say("padded", pad, path)
    out, info = M.forward(c.hidden, c.logits, c.w13, c.w2, c.top_k, out_dtype=torch.float32,
                          force_path=PATHS[path])
    act = 1 if path == "mfma" else 0
    check_out(out, oracle_out(c, act_mode=act), act, f"padded {pad} {path}")


def test_decode_workload():
    """E=256, H=2048, I=512, top_k=8, T=1, bf16 out: the gate picks GATHER."""
    say("decode T=1")
    c = W.make_case("decode", T=1, seed=1, device=DEV)
    out, info = M.forward(c.hidden, c.logits, c.w13, c.w2, c.top_k, out_dtype=torch.bfloat16)
    assert info["path"] == "gather" and info["slots"] == 8
    check_out(out, oracle_out(c), 0, "decode T=1 bf16")


@pytest.fixture(scope="module")
def decode_banks():
    return W.make_banks("decode", seed=1, device=DEV)


@pytest.mark.parametrize("T", [1, 4, 12, 16, 32, 64, 96])
def test_sweep_auto(decode_banks, T):
    """Zipf(1.1) popularity over the decode banks, on the path the measured gate picks (GATHER
    for small batches, MFMA from a few dozen tokens at this shape, where the measured table
    puts the boundary); select_path reports the same path."""
    c = W.make_case("sweep", T=T, seed=2, device=DEV, banks=decode_banks)
    say("sweep", T)
    out, info = M.forward(c.hidden, c.logits, c.w13, c.w2, c.top_k, out_dtype=torch.bfloat16)
    assert info["path"] == M.select_path(T, c.E, c.H, c.I, c.top_k)["path"]
    assert info["path"] == ("gather" if T <= 32 else "mfma" if T >= 96 else info["path"])
    assert info["path"] in ("gather", "mfma")
    act = 1 if info["path"] == "mfma" else 0
    check_out(out, oracle_out(c, act_mode=act), act, f"sweep T={T} {info['path']}")


@pytest.mark.parametrize("path", ["gather", "stream"])
def test_sweep_forced(decode_banks, path):
    c = W.make_case("sweep", T=32 if path == "gather" else 4, seed=3, device=DEV, banks=decode_banks)
    say("sweep forced", path)
    out, info = M.forward(c.hidden, c.logits, c.w13, c.w2, c.top_k, out_dtype=torch.float32, force_path=PATHS[path])
    assert info["path"] == path
    check_out(out, oracle_out(c), 0, f"sweep forced {path}")


@pytest.mark.parametrize("path", ["gather", "stream", "mfma"])
@pytest.mark.parametrize("H,I", [(384, 256), (640, 384), (8192, 128)])
def test_odd_shapes_forced(path, H, I):
    """Every path at shapes the decode banks do not reach. H=384: 24 chunks of 16 codes per
    row, so lane groups of 16 with a second chunk that only some lanes have, and a last MFMA
    output chunk of 128 worked by two waves only. I = 256, 384: the down GEMM's other K-block
    counts. H=8192: the largest H the MFMA kernels take."""
    T = 2 if path == "gather" else 48
    c = W.make_case("decode", T=T, seed=21, device=DEV, E=16, H=H, I=I, top_k=4)
    say("odd shape", path, H, I)
    act = 1 if path == "mfma" else 0
    out, info = M.forward(c.hidden, c.logits, c.w13, c.w2, c.top_k, out_dtype=torch.float32,
                          force_path=PATHS[path])
    assert info["path"] == path
    check_out(out, oracle_out(c, act_mode=act), act, f"{path} H={H} I={I}")


@pytest.mark.parametrize("path", ["gather", "stream"])
@pytest.mark.parametrize("H,T", [(4096, 1), (4112, 1), (4112, 6), (7168, 9)])
@pytest.mark.parametrize("bias", [False, True])
def test_long_rows_staged_x(path, H, T, bias):
    """Rows of at least 256 chunks of 16 codes stage x in LDS: once per workgroup with fused
    routing at T=1, and per pair between two barriers with a routing plan (GATHER above four
    tokens, STREAM always), where a workgroup takes one to several pairs of its expert.
    H=4112 leaves a last chunk group that only one lane owns."""
    c = W.make_case("decode", T=T, seed=41, device=DEV, E=16, H=H, I=144, top_k=4,
                   bias_std=0.3 if bias else None)
    say("staged x", path, H, T, bias)
    out, info = M.forward(c.hidden, c.logits, c.w13, c.w2, c.top_k, out_dtype=torch.float32,
                          force_path=PATHS[path])
    assert info["path"] == path
    check_out(out, oracle_out(c), 0, f"{path} H={H} T={T} bias={bias}")


@pytest.mark.parametrize("E,H,T,k", [(40, 16, 17, 4), (100, 528, 40, 6), (300, 1040, 17, 8), (1024, 528, 20, 8),
                                     (200, 4112, 17, 4), (64, 8192, 17, 2), (64, 2064, 600, 8)])
def test_mfma_route_quantises_x(E, H, T, k):
    """On MFMA with per-row activations, the kernel that selects each token's experts also
    quantises the token's row of x whenever the routing starts with a top-k kernel (more
    than 16 tokens, or more than 4096 pairs as at T=600, k=8). Its logit widths (64 to 1024
    experts per wave) and row lengths (one to sixteen 512-column pieces, partial last ones):
    ids and weights bit for bit against the oracle's routing, the output within the bar."""
    c = W.make_case("decode", T=T, seed=61 + E, device=DEV, E=E, H=H, I=144, top_k=k)
    say("route+quant", E, H, T, k)
    out, info = M.forward(c.hidden, c.logits, c.w13, c.w2, c.top_k, out_dtype=torch.float32,
                          force_path=PATHS["mfma"], return_routing=True)
    assert info["path"] == "mfma"
    ids, _, w32 = O.route(c.logits.cpu().numpy(), k)
    assert np.array_equal(info["ids"].cpu().numpy(), ids)
    assert np.array_equal(info["weights"].cpu().numpy(), w32)
    check_out(out, oracle_out(c, act_mode=1), 1, f"E={E} H={H} T={T} k={k}")


@pytest.mark.parametrize("path", [None, "gather", "stream", "mfma"])
@pytest.mark.parametrize("H,I,T", [(144, 80, 1), (144, 80, 3), (2064, 528, 1), (2064, 528, 40), (2064, 528, 300)])
def test_partial_scale_blocks(path, H, I, T):
    """H and I that are multiples of 16 but not of 128: every row ends in a partial scale
    block, and w13's up rows start inside a block (blocks tile the stored rows). On MFMA the
    partial last K blocks multiply zero activation codes, rows past I or H are never stored,
    and the up tiles of a feature block take the scales of the block each lies in."""
    c = W.make_case("decode", T=T, seed=31, device=DEV, E=16, H=H, I=I, top_k=4)
    say("partial blocks", path, H, I, T)
    kw = {} if path is None else {"force_path": PATHS[path]}
    out, info = M.forward(c.hidden, c.logits, c.w13, c.w2, c.top_k, out_dtype=torch.float32, **kw)
    assert info["path"] == (path or info["path"])
    act = 1 if info["path"] == "mfma" else 0
    check_out(out, oracle_out(c, act_mode=act), act, f"{info['path']} H={H} I={I} T={T}")


@pytest.mark.parametrize("path", ["gather", "stream", "mfma"])
@pytest.mark.parametrize("T", [1, 3, 40])
def test_mlp_bias(path, T):
    """Per-expert MLP biases on both banks (gate half then up half for w13, added after the
    down projection for w2), on every path. Undrawn experts hold NaN biases, so a bias read
    from the wrong expert poisons the output."""
    c = W.make_case("decode", T=T, seed=51 + T, device=DEV, E=16, H=640, I=384, top_k=4, bias_std=0.3)
    say("bias", path, T)
    act = 1 if path == "mfma" else 0
    out, info = M.forward(c.hidden, c.logits, c.w13, c.w2, c.top_k, out_dtype=torch.float32,
                          force_path=PATHS[path])
    assert info["path"] == path
    check_out(out, oracle_out(c, act_mode=act), act, f"bias {path} T={T}")


@pytest.mark.parametrize("path", ["gather", "stream"])
def test_mlp_bias_partial_blocks(path):
    """Biases with partial last scale blocks (H, I multiples of 16 only)."""
    c = W.make_case("decode", T=5, seed=57, device=DEV, E=16, H=144, I=80, top_k=4, bias_std=0.3)
    say("bias partial", path)
    out, info = M.forward(c.hidden, c.logits, c.w13, c.w2, c.top_k, out_dtype=torch.float32,
                          force_path=PATHS[path])
    check_out(out, oracle_out(c), 0, f"bias partial {path}")


def test_mlp_bias_decode_and_prefill_sampled():
    """Biases at the decode workload (GATHER, bf16 out) and at T=4096 (MFMA, sampled rows)."""
    banks = W.make_banks("decode", seed=1, device=DEV, bias_std=0.02)
    c = W.make_case("decode", T=1, seed=1, device=DEV, banks=banks)
    say("bias decode")
    out, info = M.forward(c.hidden, c.logits, c.w13, c.w2, c.top_k, out_dtype=torch.bfloat16)
    assert info["path"] == "gather"
    check_out(out, oracle_out(c), 0, "bias decode T=1")
    c = W.make_case("prefill", T=4096, seed=6, device=DEV, banks=banks)
    say("bias prefill")
    out, info = M.forward(c.hidden, c.logits, c.w13, c.w2, c.top_k, out_dtype=torch.bfloat16, return_routing=True)
    torch.cuda.synchronize()
    assert info["path"] == "mfma"
    rows = np.array([0, 1, 777, 4095])
    res = oracle_out(c, rows=rows, act_mode=1)
    assert np.array_equal(info["ids"].cpu().numpy()[rows], res["ids"])
    check_out(out[torch.from_numpy(rows).to(DEV)], res, 1, "bias prefill T=4096 sampled")


@pytest.mark.parametrize("cols", [128, 640, 1024, 2048, 7168])
def test_group_quantisation_bit_exact(cols):
    """Activation codes and scales per (token, 128-column group) match the oracle bit for bit:
    groups of very different magnitudes, an all-zero group (scale 1), a group of bf16
    subnormals (a subnormal float scale) and exact rounding midpoints."""
    say("group quantisation", cols)
    g = torch.Generator().manual_seed(5 + cols)
    ng = cols // 128
    x = torch.randn(9, cols, generator=g) * torch.rand(9, ng, generator=g).repeat_interleave(128, 1) * 9
    x[2, :128] = 0
    x[3, -128:] = torch.randn(128, generator=g) * 1e-39
    x[4, :8] = torch.tensor([448.0, 416.0, 432.0, 3.375, -3.125, 0.0, -0.0, 1.0])
    x = x.to(torch.bfloat16)
    codes, scales = M.quantize_groups(x.to(DEV))
    q, sc = O.quantize_groups(O.bf16_to_f64(bf16_bits(x)).astype(np.float32))
    assert sc[2, 0] == 1.0 and 0 < sc[3, -1] < np.finfo(np.float32).tiny
    assert np.array_equal(scales.cpu().numpy(), sc)
    assert np.array_equal(codes.cpu().numpy(), q)


@pytest.mark.parametrize("path", ["gather", "stream"])
@pytest.mark.parametrize("T", [1, 3, 40])
def test_group_fp8_activations(path, T):
    """GEMM1 on e4m3 activations per (token, 128 columns), GEMM2 on float h, with biases."""
    c = W.make_case("decode", T=T, seed=61 + T, device=DEV, E=16, H=640, I=384, top_k=4, bias_std=0.2)
    say("group fp8", path, T)
    out, info = M.forward(c.hidden, c.logits, c.w13, c.w2, c.top_k, out_dtype=torch.float32,
                          force_path=PATHS[path], act_mode=M.ACT_GROUP_FP8)
    assert (info["path"], info["act_mode"]) == (path, 2)
    check_out(out, oracle_out(c, act_mode=2), 2, f"group fp8 {path} T={T}")


@pytest.mark.parametrize("H", [2048, 640])
def test_group_fp8_in_register_quantisation_matches_row_quantiser(H):
    """At 4 tokens GEMM1 routes and quantises x itself; at 5 the separate row quantiser
    (bit-exact against the oracle) does it. A token's output does not depend on the others,
    so the first 4 rows of the 5-token forward must equal the 4-token forward bit for bit."""
    c = W.make_case("decode", T=5, seed=91 + H, device=DEV, E=32, H=H, I=256, top_k=4)
    say("group fp8 fused vs row quantiser", H)
    kw = dict(out_dtype=torch.float32, force_path=M.PATH_GATHER, act_mode=M.ACT_GROUP_FP8)
    five, i5 = M.forward(c.hidden, c.logits, c.w13, c.w2, c.top_k, **kw)
    four, i4 = M.forward(c.hidden[:4].contiguous(), c.logits[:4].contiguous(), c.w13, c.w2, c.top_k, **kw)
    assert i4["kernels"] < i5["kernels"]  # the fused path ran at 4 tokens
    assert torch.equal(four, five[:4])


def test_group_fp8_decode_and_grouped():
    """The decode workload (GATHER, bf16 out) and T=4096, where the gate takes MFMA with both
    GEMMs on groups (sampled rows; every output equal on a second run)."""
    banks = W.make_banks("decode", seed=1, device=DEV)
    c = W.make_case("decode", T=1, seed=1, device=DEV, banks=banks)
    say("group fp8 decode")
    out, info = M.forward(c.hidden, c.logits, c.w13, c.w2, c.top_k, out_dtype=torch.bfloat16,
                          act_mode=M.ACT_GROUP_FP8)
    assert (info["path"], info["act_mode"]) == ("gather", 2)
    check_out(out, oracle_out(c, act_mode=2), 2, "group fp8 decode T=1")
    c = W.make_case("prefill", T=4096, seed=6, device=DEV, banks=banks)
    say("group fp8 T=4096")
    out, info = M.forward(c.hidden, c.logits, c.w13, c.w2, c.top_k, out_dtype=torch.bfloat16,
                          act_mode=M.ACT_GROUP_FP8)
    again, _ = M.forward(c.hidden, c.logits, c.w13, c.w2, c.top_k, out_dtype=torch.bfloat16,
                         act_mode=M.ACT_GROUP_FP8)
    torch.cuda.synchronize()
    assert (info["path"], info["act_mode"]) == ("mfma", 3)
    assert torch.equal(out, again)
    rows = np.array([0, 5, 2048, 4095])
    res = oracle_out(c, rows=rows, act_mode=3)
    assert res["n_flagged"] <= 0.05 * res["n_h"]
    check_out(out[torch.from_numpy(rows).to(DEV)], res, 3, "group fp8 T=4096 mfma sampled")


@pytest.mark.parametrize("T", [3, 40, 300])
def test_group_fp8_mfma(T):
    """MFMA with both GEMMs on groups (x per (token, 128 columns), h per (pair, 128
    features) quantised inside GEMM1), with biases, against the oracle's act_mode 3 at every
    output; forced, so that few tokens per expert leave partial tiles."""
    c = W.make_case("decode", T=T, seed=71 + T, device=DEV, E=16, H=640, I=384, top_k=4, bias_std=0.2)
    say("group fp8 mfma", T)
    out, info = M.forward(c.hidden, c.logits, c.w13, c.w2, c.top_k, out_dtype=torch.float32,
                          force_path=M.PATH_MFMA, act_mode=M.ACT_GROUP_FP8)
    assert (info["path"], info["act_mode"]) == ("mfma", 3)
    check_out(out, oracle_out(c, act_mode=3), 3, f"group fp8 mfma T={T}")


@pytest.mark.parametrize("T,path", [(1, None), (16, None), (16, "stream")])
def test_large_expert_workload(T, path):
    """E=256, H=7168, I=2048, fp32 scales; only the routed experts are drawn, the rest
    hold NaN codes and NaN scales, so reading an unrouted expert would poison the output."""
    shp = W.SHAPES["large"]
    logits = W.make_logits(T, shp["E"], "normal", seed=40 + T, device="cpu")
    ids, _, _ = O.route(logits.numpy(), shp["top_k"])
    used = O.routed_experts(ids)
    say("large", T, "experts", len(used))
    banks = W.make_banks("large", seed=4, device=DEV, experts=used)
    c = W.make_case("large", T=T, seed=4, device=DEV, banks=banks)
    c.logits = logits.to(DEV)
    kw = {} if path is None else {"force_path": PATHS[path]}
    out, info = M.forward(c.hidden, c.logits, c.w13, c.w2, c.top_k, out_dtype=torch.bfloat16, **kw)
    torch.cuda.synchronize()
    assert info["path"] == (path or "gather")  # the default gate gathers up to 2 pairs per expert
    assert torch.isfinite(out.float()).all()
    rows = np.array([0]) if T == 1 else np.array([0, 7, T - 1])
    need = O.routed_experts(ids[rows])
    check_out(out[torch.from_numpy(rows).to(DEV)], oracle_out(c, rows=rows, experts=need), 0, f"large T={T}")


@pytest.mark.parametrize("T", [4096, 16384])
def test_prefill_sampled(decode_banks, T):
    """MFMA W8A8 at prefill sizes; the oracle computes sampled tokens one by one."""
    c = W.make_case("prefill", T=T, seed=6, device=DEV, banks=decode_banks)
    say("prefill", T)
    out, info = M.forward(c.hidden, c.logits, c.w13, c.w2, c.top_k, out_dtype=torch.bfloat16, return_routing=True)
    again, _ = M.forward(c.hidden, c.logits, c.w13, c.w2, c.top_k, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert info["path"] == "mfma" and info["act_mode"] == 1
    # every output, not only the sampled ones: the path is deterministic
    assert torch.equal(out, again)
    rows = np.unique(np.concatenate([[0, 1, T - 1], np.random.default_rng(T).choice(T, 21, replace=False)]))
    res = oracle_out(c, rows=rows, act_mode=1)
    assert np.array_equal(info["ids"].cpu().numpy()[rows], res["ids"])
    assert res["n_flagged"] <= 0.05 * res["n_h"]
    sub = out[torch.from_numpy(rows).to(DEV)]
    check_out(sub, res, 1, f"prefill T={T} sampled")


def _tiles_of(offsets, tile=128):
    """(expert, tile, half) triples of a routing: each expert's pairs in 128-pair tiles, each
    tile in two halves of 64."""
    out = set()
    for e in range(len(offsets) - 1):
        for p in range(int(offsets[e]), int(offsets[e + 1])):
            q = p - int(offsets[e])
            out.add((e, q // tile, (q % tile) // 64))
    return out


@pytest.mark.parametrize("T", [4096, 16384])
def test_mfma_up_h_within_drift_bound(decode_banks, T):
    """The MFMA path's first half on its own: GEMM1's h for every (token, slot) pair, in
    sorted order, against the oracle's exact h. Every element of every tile must lie within
    the oracle's drift bound (coarse for all pairs; exact for all pairs of two experts), the
    claim the oracle's W8A8 flags rest on."""
    c = W.make_case("prefill", T=T, seed=6, device=DEV, banks=decode_banks)
    say("mfma up", T)
    hg = M.mfma_up(c.hidden, c.logits, c.w13, c.top_k, c.I)
    torch.cuda.synchronize()
    hid = bf16_bits(c.hidden)
    ids, w, _ = O.route(c.logits.cpu().numpy(), c.top_k)
    counts, offsets, sp = O.sort_pairs(ids, c.E)
    w13 = bank_numpy(c.w13)
    hgn = hg.cpu().numpy().astype(np.float64)
    h, d = O.up_w8a8(hid, ids, w13, pairs=sp, coarse=True)
    r = np.abs(hgn - h) / d
    say("mfma up", T, f"max |h_gpu - h| / coarse bound {r.max():.3f}")
    assert np.isfinite(hgn).all() and r.max() <= 1.0
    covered = _tiles_of(offsets)
    assert len(covered) >= c.E and all(cnt > 0 for cnt in counts)
    for e in (0, int(np.argmax(counts))):  # exact bound: the first expert and the busiest one
        pos = np.arange(offsets[e], offsets[e + 1])
        he, de = O.up_w8a8(hid, ids, w13, pairs=sp[pos])
        re = np.abs(hgn[pos] - he) / de
        say("mfma up", T, f"expert {e}: {len(pos)} pairs, max |h_gpu - h| / bound {re.max():.3f}")
        assert re.max() <= 1.0


@pytest.mark.parametrize("T", [4096, 16384])
def test_mfma_down_on_oracle_h_every_output(decode_banks, T):
    """The MFMA path's second half on its own, fed the oracle's h (float32 of the exact h of
    every pair): h quantisation, the down GEMM and the combine against the oracle's
    definition of the same, on every output of every token. The h codes then follow the
    same float32 inputs on both sides, so no rounding is ambiguous; the bound per output is
    the accumulation bound of the down GEMM (coarse), the fp16 storage of y (2^-11 of the
    largest |y| of its 32-output group) and the float32 combine, weighted by |w|."""
    c = W.make_case("prefill", T=T, seed=7, device=DEV, banks=decode_banks)
    say("mfma down", T)
    hid = bf16_bits(c.hidden)
    ids, w, _ = O.route(c.logits.cpu().numpy(), c.top_k)
    counts, offsets, sp = O.sort_pairs(ids, c.E)
    w13, w2 = bank_numpy(c.w13), bank_numpy(c.w2)
    h, _ = O.up_w8a8(hid, ids, w13, coarse=True)
    h32 = h.astype(np.float32)
    out = M.mfma_down(torch.from_numpy(h32[sp]).to(DEV), c.logits, c.w2, c.top_k, c.H)
    torch.cuda.synchronize()
    o = out.cpu().numpy().astype(np.float64)
    ref = O.down_w8a8(h32, ids, w, w2)
    # the bound, pair by pair from the oracle's own y
    q, s = O.quantize_rows(h32)
    hd = O.e4m3_lut()[q] * s.astype(np.float64)[:, None]
    bound = np.zeros_like(ref)
    k = c.top_k
    for e, pairs in OO._pairs_by_expert(ids).items():
        W2 = O.dequant_expert(w2, e)
        y = hd[pairs] @ W2.T
        g32 = np.repeat(np.abs(y).reshape(len(pairs), -1, 32).max(axis=2), 32, axis=1)
        per = O.acc_bound(W2, hd[pairs], coarse=True) + 2.0 ** -11 * 1.01 * g32 + 2.0 ** -21 * np.abs(y)
        bound[pairs // k] += np.abs(w.ravel()[pairs])[:, None] * per
    err = np.abs(o - ref)
    say("mfma down", T, f"max err/max|ref| {err.max() / np.abs(ref).max():.3e}, max err/bound {(err / bound).max():.3f}")
    assert np.isfinite(o).all()
    assert np.all(err <= bound)
    assert len(_tiles_of(offsets)) >= c.E


def _staged_mfma_check(c, what):
    """Both MFMA halves of case c on their own against the oracle, at every pair and output
    (as test_mfma_up_h_within_drift_bound and test_mfma_down_on_oracle_h_every_output)."""
    hid = bf16_bits(c.hidden)
    ids, w, _ = O.route(c.logits.cpu().numpy(), c.top_k)
    counts, offsets, sp = O.sort_pairs(ids, c.E)
    w13, w2 = bank_numpy(c.w13), bank_numpy(c.w2)
    h, d = O.up_w8a8(hid, ids, w13, coarse=True)
    hg = M.mfma_up(c.hidden, c.logits, c.w13, c.top_k, c.I).cpu().numpy().astype(np.float64)
    r = np.abs(hg - h[sp]) / d[sp]
    say(what, f"up: max |h_gpu - h| / coarse bound {r.max():.3f}")
    assert np.isfinite(hg).all() and r.max() <= 1.0
    h32 = h.astype(np.float32)
    out = M.mfma_down(torch.from_numpy(h32[sp]).to(DEV), c.logits, c.w2, c.top_k, c.H)
    o = out.cpu().numpy().astype(np.float64)
    ref = O.down_w8a8(h32, ids, w, w2)
    q, sh = O.quantize_rows(h32)
    hd = O.e4m3_lut()[q] * sh.astype(np.float64)[:, None]
    bound = np.zeros_like(ref)
    nparts = -(-c.I // 512)
    for e, pairs in OO._pairs_by_expert(ids).items():
        W2 = O.dequant_expert(w2, e)
        per = np.zeros((len(pairs), c.H))
        for part in range(nparts):  # each K part is stored in fp16 with its own exponents
            ks = slice(512 * part, min(512 * (part + 1), c.I))
            yp = hd[pairs][:, ks] @ W2[:, ks].T
            eg = -(-c.H // 32)  # exponent groups; a last one may be partial
            ap = np.zeros((len(pairs), eg * 32))
            ap[:, :c.H] = np.abs(yp)
            g32 = np.repeat(ap.reshape(len(pairs), eg, 32).max(axis=2), 32, axis=1)[:, :c.H]
            per += (O.acc_bound(W2[:, ks], hd[pairs][:, ks], coarse=True) + 2.0 ** -11 * 1.01 * g32
                    + 2.0 ** -21 * np.abs(yp))
        bound[pairs // c.top_k] += np.abs(w.ravel()[pairs])[:, None] * per
    err = np.abs(o - ref)
    say(what, f"down: max err/max|ref| {err.max() / np.abs(ref).max():.3e}, max err/bound {(err / bound).max():.3f}")
    assert np.isfinite(o).all() and np.all(err <= bound)
    assert len(_tiles_of(offsets)) >= c.E


def _staged_group_check(c, what):
    """Both halves of the group-scaled MFMA path on their own, at every pair and output.
    Up: the h codes GEMM1 writes decode to the values of the oracle's group quantisation of
    the exact h except where the oracle flags the rounding as ambiguous (coarse drift bound), and each group
    scale lies within the group's largest drift / 448 of the oracle's. Down: fed the oracle's
    codes and scales, the down GEMM and the combine against the oracle's definition, within
    the accumulation, fp16-y and combine bound per output."""
    hid = bf16_bits(c.hidden)
    ids, w, _ = O.route(c.logits.cpu().numpy(), c.top_k)
    counts, offsets, sp = O.sort_pairs(ids, c.E)
    w13, w2 = bank_numpy(c.w13), bank_numpy(c.w2)
    h, d = O.up_w8a8(hid, ids, w13, coarse=True, act_mode=3)
    _, ex = O.requantize_h(h, d, 128)
    codes, scales = M.mfma_up_groups(c.hidden, c.logits, c.w13, c.top_k, c.I)
    cg, sg = codes.cpu().numpy(), scales.cpu().numpy().astype(np.float64)
    lut = O.e4m3_lut()
    diff = lut[cg] != lut[ex["h_codes"][sp]]  # by value: +0 and -0 (an h within its drift of 0) are one
    say(what, f"up: {int(diff.sum())} codes differ, {int(ex['flags'].sum())} flagged of {ex['flags'].size}")
    assert not (diff & ~ex["flags"][sp]).any()
    s_ref = ex["h_scale"][sp].astype(np.float64)
    dmax = d[sp].reshape(len(sp), -1, 128).max(axis=2)
    assert np.all(np.abs(sg - s_ref) <= dmax / 448.0 * 1.001 + 2.0 ** -22 * s_ref)
    q, sh = O.quantize_groups(h.astype(np.float32))
    out = M.mfma_down_groups(torch.from_numpy(q[sp]).to(DEV), torch.from_numpy(sh[sp]).to(DEV), c.logits, c.w2,
                             c.top_k, c.H)
    o = out.cpu().numpy().astype(np.float64)
    ref = O.down_w8a8_groups(q, sh, ids, w, w2)
    hd = O.dequant_groups(q, sh)
    bound = np.zeros_like(ref)
    nparts = -(-c.I // 512)
    for e, pairs in OO._pairs_by_expert(ids).items():
        W2 = O.dequant_expert(w2, e)
        per = np.zeros((len(pairs), c.H))
        for part in range(nparts):
            ks = slice(512 * part, min(512 * (part + 1), c.I))
            yp = hd[pairs][:, ks] @ W2[:, ks].T
            g32 = np.repeat(np.abs(yp).reshape(len(pairs), -1, 32).max(axis=2), 32, axis=1)
            per += (O.acc_bound(W2[:, ks], hd[pairs][:, ks], coarse=True) + 2.0 ** -11 * 1.01 * g32
                    + 2.0 ** -21 * np.abs(yp))
        bound[pairs // c.top_k] += np.abs(w.ravel()[pairs])[:, None] * per
    err = np.abs(o - ref)
    say(what, f"down: max err/max|ref| {err.max() / np.abs(ref).max():.3e}, max err/bound {(err / bound).max():.3f}")
    assert np.isfinite(o).all() and np.all(err <= bound)
    assert len(_tiles_of(offsets)) >= c.E


@pytest.mark.parametrize("E,H,I,k,T", [(256, 2048, 512, 8, 4096), (16, 1024, 640, 4, 256), (16, 512, 1536, 4, 600),
                                       (32, 7168, 2048, 4, 1024)])
def test_mfma_groups_staged(E, H, I, k, T):
    """The group-scaled MFMA halves at the prefill shape (decode banks, T=4096), with I past
    one K part (640, 1536) and at the large-expert shape (H=7168, I=2048, fp32 scales)."""
    name = "large" if H == 7168 else "decode"
    if E == 256:
        c = W.make_case("prefill", T=T, seed=9, device=DEV, banks=W.make_banks("decode", seed=1, device=DEV))
    else:
        c = W.make_case(name, T=T, seed=E + I + 1, device=DEV, E=E, H=H, I=I, top_k=k)
    say("mfma groups staged", E, H, I, k, T)
    _staged_group_check(c, f"groups H={H} I={I} T={T}")


@pytest.mark.parametrize("E,H,I,k,T", [(16, 1024, 640, 4, 256), (16, 512, 1536, 4, 600), (32, 7168, 2048, 4, 1024),
                                       (16, 2064, 528, 4, 300), (8, 144, 80, 2, 60), (16, 1040, 2064, 4, 200)])
def test_mfma_k_parts_staged(E, H, I, k, T):
    """I beyond 512: the down GEMM runs in K parts of up to four 128-wide blocks (640 = 4 + 1,
    1536 = 4 + 4 + 4, and the large-expert shape's 2048 = 4 x 4 with H=7168 and fp32
    scales), each part into its own y plane, summed by the combine; and ragged H and I
    (2064/528, 144/80, 1040/2064: partial last K blocks of both GEMMs, up rows straddling
    scale blocks, a partial last exponent group). Both halves checked at every pair and every
    output."""
    name = "large" if H == 7168 else "decode"
    c = W.make_case(name, T=T, seed=E + I, device=DEV, E=E, H=H, I=I, top_k=k)
    say("mfma k parts", E, H, I, k, T)
    _staged_mfma_check(c, f"k parts H={H} I={I}")


def test_mfma_large_expert_forward():
    """The large-expert workload (E=256, H=7168, I=2048, top_k=8) at T=1024, where the gate
    now picks MFMA; the oracle checks sampled tokens (their experts only)."""
    shp = W.SHAPES["large"]
    T = 1024
    banks = W.make_banks("large", seed=4, device=DEV)
    c = W.make_case("large", T=T, seed=5, device=DEV, banks=banks)
    say("large mfma", T)
    out, info = M.forward(c.hidden, c.logits, c.w13, c.w2, c.top_k, out_dtype=torch.float32, return_routing=True)
    torch.cuda.synchronize()
    assert info["path"] == "mfma"
    rows = np.array([0, 511, 1023])
    ids, _, _ = O.route(c.logits.cpu().numpy()[rows], shp["top_k"])
    res = oracle_out(c, rows=rows, act_mode=1, experts=O.routed_experts(ids))
    assert np.array_equal(info["ids"].cpu().numpy()[rows], res["ids"])
    check_out(out[torch.from_numpy(rows).to(DEV)], res, 1, "large T=1024 mfma")


@pytest.mark.parametrize("T", [40, 100])
def test_mfma_small_sizes_forced(decode_banks, T):
    """Forced MFMA with ragged tiles (few tokens per expert) against all rows; T=40 sorts
    its 320 pairs in one workgroup, T=100 (800 pairs) takes the three-pass sort."""
    c = W.make_case("decode", T=T, seed=8, device=DEV, banks=decode_banks)
    say("mfma forced", T)
    out, info = M.forward(c.hidden, c.logits, c.w13, c.w2, c.top_k, out_dtype=torch.float32,
                          force_path=M.PATH_MFMA)
    res = oracle_out(c, act_mode=1)
    check_out(out, res, 1, f"mfma T={T}")


# ------------------------------------------------------------------- properties

@pytest.mark.parametrize("path", ["gather", "stream", "mfma"])
def test_bf16_is_rounded_fp32_and_deterministic(decode_banks, path):
    c = W.make_case("sweep", T=8, seed=12, device=DEV, banks=decode_banks)
    say("bf16 vs fp32", path)
    f32a, _ = M.forward(c.hidden, c.logits, c.w13, c.w2, c.top_k, out_dtype=torch.float32, force_path=PATHS[path])
    f32b, _ = M.forward(c.hidden, c.logits, c.w13, c.w2, c.top_k, out_dtype=torch.float32, force_path=PATHS[path])
    b16, _ = M.forward(c.hidden, c.logits, c.w13, c.w2, c.top_k, out_dtype=torch.bfloat16, force_path=PATHS[path])
    assert torch.equal(f32a, f32b)
    assert torch.equal(f32a.to(torch.bfloat16), b16)


def test_paths_agree(decode_banks):
    """GATHER and STREAM (both W8A16) agree to fp32 summation-order differences."""
    c = W.make_case("sweep", T=12, seed=13, device=DEV, banks=decode_banks)
    say("gather vs stream")
    a, _ = M.forward(c.hidden, c.logits, c.w13, c.w2, c.top_k, out_dtype=torch.float32, force_path=M.PATH_GATHER)
    b, _ = M.forward(c.hidden, c.logits, c.w13, c.w2, c.top_k, out_dtype=torch.float32, force_path=M.PATH_STREAM)
    d = (a - b).abs().max().item() / a.abs().max().item()
    assert d <= 1e-5


@pytest.mark.parametrize("act", ["path", "group_fp8"])
def test_verify_gather_against_stream_in_fp8_ulps(decode_banks, act):
    """The verify mode of gaudi-cookbook fp8-moe-gather: run the gathered path and the
    grouped one on the same tokens and report outputs that differ by more than 2 fp8 ulps.
    Both compute the same products in float, so none may."""
    c = W.make_case("sweep", T=12, seed=14, device=DEV, banks=decode_banks)
    a_mode = M.ACT_GROUP_FP8 if act == "group_fp8" else M.ACT_PATH
    say("verify", act)
    a, ia = M.forward(c.hidden, c.logits, c.w13, c.w2, c.top_k, out_dtype=torch.float32,
                      force_path=M.PATH_GATHER, act_mode=a_mode)
    b, ib = M.forward(c.hidden, c.logits, c.w13, c.w2, c.top_k, out_dtype=torch.float32,
                      force_path=M.PATH_STREAM, act_mode=a_mode)
    assert ia["act_mode"] == ib["act_mode"]
    d = fp8_ulp_diff(a.cpu().numpy(), b.cpu().numpy())
    say("verify", act, f"max {d.max():.3g} fp8 ulp")
    assert int((d > 2).sum()) == 0


@pytest.mark.parametrize("path,T", [("gather", 1), ("gather", 8), ("stream", 8), ("mfma", 64)])
def test_graph_replays_match_eager(decode_banks, path, T):
    """A forward captured in a HIP graph gives the eager result bit for bit on every replay,
    with other GPU work and host synchronisation between the replays (the benchmark times
    replayed graphs)."""
    c = W.make_case("sweep", T=T, seed=15, device=DEV, banks=decode_banks)
    say("graph", path, T)
    kw = dict(out_dtype=torch.float32, force_path=PATHS[path])
    eager, _ = M.forward(c.hidden, c.logits, c.w13, c.w2, c.top_k, **kw)
    ws = torch.empty(M.workspace_size(T, c.E, c.H, c.I, c.top_k, force_path=PATHS[path]), dtype=torch.uint8,
                     device=DEV)
    out = torch.empty_like(eager)
    M.forward(c.hidden, c.logits, c.w13, c.w2, c.top_k, out=out, workspace=ws, **kw)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        M.forward(c.hidden, c.logits, c.w13, c.w2, c.top_k, out=out, workspace=ws, **kw)
    for rep in range(3):
        out.fill_(float("nan"))
        ws.fill_(0xA5)  # stale workspace contents must not leak into the result
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep}"


@pytest.mark.parametrize("path", ["gather", "stream", "mfma", "mfma_group"])
@pytest.mark.parametrize("E,k,T", [(1, 1, 3), (4, 4, 2), (8, 8, 5)])
def test_degenerate_routings(path, E, k, T):
    """One expert (a plain SwiGLU FFN) and top_k = E (every expert routed, a dense softmax
    mixture), on every path (and MFMA with group-fp8 activations); the last token's hidden
    state is all zero (activation scale 1, h = 0 in every group)."""
    c = W.make_case("decode", T=T, seed=71 + E, device=DEV, E=E, H=256, I=128, top_k=k, bias_std=0.1)
    c.hidden[-1] = 0
    say("degenerate", path, E, k, T)
    act = {"mfma": 1, "mfma_group": 3}.get(path, 0)
    out, info = M.forward(c.hidden, c.logits, c.w13, c.w2, c.top_k, out_dtype=torch.float32,
                          force_path=PATHS[path.split("_")[0]], return_routing=True,
                          act_mode=M.ACT_GROUP_FP8 if path == "mfma_group" else M.ACT_PATH)
    assert info["act_mode"] == act
    res = oracle_out(c, act_mode=act)
    assert np.array_equal(info["ids"].cpu().numpy(), res["ids"])
    check_out(out, res, act, f"degenerate {path} E={E} k={k}")


@pytest.mark.parametrize("T", [1, 3])
def test_fused_routing_with_ties(T):
    """Decode GEMM1 routes inside the kernel; tied logits must select the lower ids, both when
    few logits tie (ranked candidates) and when a whole row ties (round-based selection)."""
    c = W.make_case("decode", T=T, seed=91 + T, device=DEV, H=256, I=128)
    g = torch.Generator().manual_seed(92 + T)
    tied = (torch.randn(T, c.logits.shape[1], generator=g) * 2).round() / 2
    if T > 1:
        tied[1] = 0.25
    c.logits = tied.to(DEV)
    say("fused routing ties", T)
    out, info = M.forward(c.hidden, c.logits, c.w13, c.w2, c.top_k, out_dtype=torch.float32,
                          force_path=PATHS["gather"], return_routing=True)
    res = oracle_out(c, act_mode=0)
    assert np.array_equal(info["ids"].cpu().numpy(), res["ids"])
    assert np.array_equal(info["weights"].cpu().numpy(), res["w32"])
    check_out(out, res, 0, f"fused routing ties T={T}")


@pytest.mark.parametrize("path", ["gather", "stream", "mfma"])
def test_largest_expert_count_and_top_k(path):
    """E = 1024 experts and top_k = 32, the ABI's limits, with small experts; only the routed
    experts are drawn (the others hold NaN codes and scales)."""
    E, k, T = 1024, 32, 3 if path != "mfma" else 70
    logits = W.make_logits(T, E, "normal", seed=81, device="cpu")
    ids, _, _ = O.route(logits.numpy(), k)
    used = O.routed_experts(ids)
    banks = W.make_banks("decode", seed=82, device=DEV, E=E, H=256, I=128, experts=used)
    c = W.make_case("decode", T=T, seed=82, device=DEV, banks=banks, E=E, H=256, I=128, top_k=k)
    c.logits = logits.to(DEV)
    say("E=1024 k=32", path, T)
    act = 1 if path == "mfma" else 0
    out, info = M.forward(c.hidden, c.logits, c.w13, c.w2, c.top_k, out_dtype=torch.float32,
                          force_path=PATHS[path], return_routing=True)
    torch.cuda.synchronize()
    assert info["path"] == path
    rows = np.arange(T) if T <= 3 else np.array([0, 33, T - 1])
    res = oracle_out(c, rows=rows, act_mode=act, experts=O.routed_experts(ids[rows]))
    assert np.array_equal(info["ids"].cpu().numpy()[rows], res["ids"])
    check_out(out[torch.from_numpy(rows).to(DEV)], res, act, f"E=1024 k=32 {path}")


def _random_configs(n, seed):
    """n configurations drawn from a fixed seed: workload style (bank kind and logit
    distribution), E, top_k (up to 12: past 8 the round-based selection runs), H and I
    (multiples of 16, or of 128 for group-fp8 activations), T (every fourth 64-160 tokens,
    where more than 512 pairs take the multi-block sort), the path (or the gate),
    activations, biases, scale dtype and scale padding."""
    import random

    rng = random.Random(seed)
    out = []
    for i in range(n):
        E = rng.choice([1, 3, 8, 16, 40, 64, 130])
        group = rng.random() < 0.3
        path = rng.choice([None, "gather", "stream", "mfma"])
        I = 128 * rng.randint(1, 4) if group and (path == "mfma" or rng.random() < 0.5) else 16 * rng.randint(1, 40)
        out.append(dict(
            i=i, name=rng.choice(["tiny", "decode", "sweep", "large"]), E=E, k=rng.randint(1, min(E, 12)),
            H=128 * rng.randint(1, 8) if group else 16 * rng.randint(1, 64), I=I,
            T=rng.randint(64, 160) if i % 4 == 3 else rng.randint(1, 48),
            path=path, group=group, bias=rng.random() < 0.3,
            sdt=rng.choice([torch.float32, torch.bfloat16]), pad=rng.choice(["none", "row16", "slab16"])))
    return out


def _random_large_configs(n, seed):
    """As _random_configs at larger sizes: E from 64 to 1000, T from 17 to 1200 (routing by a
    top-k kernel; more than 4096 pairs take the multi-block sort), H and I up to 1024 and
    768."""
    import random

    rng = random.Random(seed)
    out = []
    for i in range(n):
        E = rng.choice([64, 200, 256, 512, 1000])
        group = rng.random() < 0.3
        path = rng.choice([None, "gather", "stream", "mfma"])
        I = 128 * rng.randint(1, 4) if group and (path == "mfma" or rng.random() < 0.5) else 16 * rng.randint(1, 48)
        out.append(dict(
            i=i, big=True, name=rng.choice(["decode", "sweep", "large"]), E=E, k=rng.randint(1, min(E, 12)),
            H=128 * rng.randint(1, 8) if group else 16 * rng.randint(1, 64), I=I, T=rng.randint(17, 1200),
            path=path, group=group, bias=rng.random() < 0.3,
            sdt=rng.choice([torch.float32, torch.bfloat16]), pad=rng.choice(["none", "row16", "slab16"])))
    return out


@pytest.mark.parametrize("cfg", _random_configs(200, 2027) + _random_large_configs(16, 2029),
                         ids=lambda c: f"{'big' if c.get('big') else 'cfg'}{c['i']}")
def test_random_configurations(cfg):
    """Seeded random configurations across every option the forward takes, each against the
    oracle: ids and weights bit for bit, outputs to the float bar in the precision the
    reported act_mode fixes."""
    c = W.make_case(cfg["name"], T=cfg["T"], seed=300 + cfg["i"], device=DEV, E=cfg["E"], H=cfg["H"],
                    I=cfg["I"], top_k=cfg["k"], scale_dtype=cfg["sdt"], pad=cfg["pad"],
                    bias_std=0.2 if cfg["bias"] else None)
    say("random", {k: v for k, v in cfg.items() if k != "sdt"}, cfg["sdt"])
    kw = {} if cfg["path"] is None else {"force_path": PATHS[cfg["path"]]}
    if cfg["group"]:
        kw["act_mode"] = M.ACT_GROUP_FP8
    out, info = M.forward(c.hidden, c.logits, c.w13, c.w2, c.top_k, out_dtype=torch.float32,
                          return_routing=True, **kw)
    if cfg["path"] is not None:
        assert info["path"] == cfg["path"]
    res = oracle_out(c, act_mode=info["act_mode"])
    assert np.array_equal(info["ids"].cpu().numpy(), res["ids"])
    assert np.array_equal(info["weights"].cpu().numpy(), res["w32"])
    check_out(out, res, info["act_mode"], f"random cfg{cfg['i']} {info['path']} act {info['act_mode']}")


def test_zero_tokens():
    c = W.make_case("tiny", T=1, seed=1).to(DEV)
    out, info = M.forward(c.hidden[:0], c.logits[:0], c.w13, c.w2, c.top_k, out_dtype=torch.float32)
    assert out.shape == (0, c.H) and info["kernels"] == 0
