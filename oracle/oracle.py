"""Float64 CPU oracle for the block-FP8 mixture-of-experts expert computation.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU-baseline
leg may use this module. The HIP library never calls it, it imports nothing from the
library, and the two share no code: the only thing both sides see is the seeded inputs.

It is deliberately plain numpy: a 256-entry e4m3 table built from the closed form,
whole-expert dequantisation, float64 matrix products, an explicit loop over (token, slot)
pairs, and a second, dense all-experts loop. Nothing is blocked, fused or reordered.

Sources (the three pages; each function names the passage it follows):
  [gather] gaudi-cookbook, fixes page "fp8-moe-gather": sections Problem, The fix.
  [tpu]    tpu-inference PR #3040 "Add another fused EP MoE kernels": review of the w1
           weight/scale DMA (gate half first, up half second) and of the w1 bias DMA (the
           gate and up halves of the MLP bias come from their own offsets; the w2 bias is
           added after the down projection).
  [cpu]    FreeToken PR #662 "serve block-fp8 experts on the cpu and hybrid backends": the
           PR body (bank format, e4m3 exactness), commit "honor padded fp8 scale strides",
           commit "add float64 parity reference", the final description (Kernels).

Pins (tests/test_oracle_*.py, run without a GPU):
  e4m3_lut          closed form vs the fp16-bit identity of [cpu] Kernels, vs torch's
                    float8_e4m3fn, bf16 carries every finite code, range 2^-9..448.
  e4m3_encode       vs torch's float8_e4m3fn cast on every midpoint +-1 ulp and at random;
                    saturation and signed zero by definition.
  quantize_rows     hand-checked rows (power-of-two amax, zero row).
  quantize_groups   scalar loops with a brute-force nearest-code search per 128-column
                    group; one group per row reduces to quantize_rows.
  dequant_expert    padded-stride invariance with NaN in the padding; power-of-two codes
                    with unit scales give exact small integers; a pure-Python scalar loop.
  route             brute-force sort by (-logit, id); k=E gives the full softmax.
  sort_pairs        brute-force stable counting sort.
  forward           pure-Python scalar loops on tiny shapes (also with partial scale blocks
                    and with MLP biases); dense == gathered; unrouted experts contribute
                    exactly zero; E=1,k=1 is a textbook SwiGLU FFN (torch), with and
                    without biases; expert permutation and token independence invariants;
                    act_mode 2 against scalar loops over group-dequantised activations;
                    act_modes 1 and 3 against torch's e4m3 cast with fp32 scales, every
                    x and h code and scale compared.
  e4m3_midpoint_distance
                    a linear walk over every finite value at every value, midpoint and
                    its float32 neighbours, and at random magnitudes.
  h_drift / flags   GEMM1 evaluated on the CPU with float32 sums in several orders and
                    with a truncating aligned accumulator: every h stays within the bound
                    and every code that changes is flagged, for h scaled per row and per
                    128-feature group; on the GPU, the MFMA path's h lies within the bound
                    at every element. The allowance equals the output moved by rounding
                    each flagged element the other way. The constants are a reading
                    (the pages fix no accumulation precision), documented at ACC_MMA.
"""

from __future__ import annotations

import math

import numpy as np

BLOCK = 128
E4M3_MAX = 448.0


# ----------------------------------------------------------------------------- e4m3

def e4m3_value(code: int) -> float:
    """Value of one OCP e4m3fn byte: sign bit, 4 exponent bits (bias 7), 3 mantissa bits.

    Exponent field 0 is subnormal, m * 2^-9; 0x7F and 0xFF are NaN; everything else is
    2^(e-7) * (1 + m/8). The range 2^-9..448 is the one [cpu] PR body gives for e4m3.
    """
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        mag = m * 2.0 ** -9
    else:
        mag = 2.0 ** (e - 7) * (1.0 + m / 8.0)
    return -mag if s else mag


_LUT = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
_POS = _LUT[:0x7F].copy()  # codes 0x00..0x7E: the non-negative finite values, increasing


def e4m3_lut() -> np.ndarray:
    """The 256-entry decode table ([cpu] PR body: the scalar tier decodes through one)."""
    return _LUT.copy()


def e4m3_encode(v) -> np.ndarray:
    """Round float32 values to the nearest finite e4m3 value; return the codes.

    Ties go to the even mantissa, magnitudes past 448 saturate to 448, and the sign of
    zero is kept. The step between neighbours is 2^(e-3) in the binade [2^e, 2^(e+1)) for
    e >= -6 and 2^-9 below 2^-6 (the subnormals), so rounding is an integer rounding of
    |v| / step. Pinned against torch's float8_e4m3fn cast.
    """
    v32 = np.asarray(v, dtype=np.float32)
    a = np.abs(v32.astype(np.float64))
    a = np.minimum(a, E4M3_MAX)
    _, ex = np.frexp(a)
    e = np.maximum(ex - 1, -6)
    step = np.ldexp(1.0, e - 3)
    r = np.rint(a / step) * step  # np.rint rounds half to even
    idx = np.searchsorted(_POS, r)
    if not np.array_equal(_POS[np.minimum(idx, 0x7E)], r):
        raise AssertionError("rounded value is not an e4m3 value")
    codes = idx.astype(np.uint8) | (np.signbit(v32).astype(np.uint8) << 7)
    return codes


def e4m3_midpoint_distance(v32: np.ndarray):
    """Distance from |v| to the midpoint of its bracketing e4m3 pair, and that pair's step.

    Used for the W8A8 ambiguity flags: a value within the drift bound of a midpoint
    may round either way. Values at or past 448 have no midpoint above them.
    """
    a = np.abs(np.asarray(v32, dtype=np.float64))
    hi_idx = np.clip(np.searchsorted(_POS, a, side="right"), 1, 0x7E)
    lo, hi = _POS[hi_idx - 1], _POS[hi_idx]
    dist = np.abs(a - 0.5 * (lo + hi))
    dist = np.where(a >= E4M3_MAX, np.inf, dist)
    return dist, hi - lo


# ----------------------------------------------------------------------------- banks

def bf16_to_f64(bits) -> np.ndarray:
    """bf16 is the upper half of an fp32 word."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def _scales_f64(bank: dict) -> np.ndarray:
    if bank["scale_dtype"] == "bf16":
        return bf16_to_f64(bank["scales"])
    return np.asarray(bank["scales"], dtype=np.float32).astype(np.float64)


def block_scales(bank: dict, e: int) -> np.ndarray:
    """Scale grid [ceil(N/128), ceil(K/128)] of expert e, read through the explicit strides.

    The scale of block (n//128, k//128) sits at e*expert_stride + (n//128)*row_stride +
    k//128; the row stride may exceed ceil(K/128) ([cpu] commit "honor padded fp8 scale
    strides": the stride is read off the bank, never recomputed).
    """
    s = _scales_f64(bank)
    rows, cols = -(-bank["N"] // BLOCK), -(-bank["K"] // BLOCK)
    base = e * bank["scale_expert_stride"]
    r = np.arange(rows)[:, None] * bank["scale_row_stride"]
    c = np.arange(cols)[None, :]
    return s[base + r + c]


def dequant_expert(bank: dict, e: int) -> np.ndarray:
    """Expert e of a bank as float64 [N, K]: LUT[code] times its 128x128 block's scale.

    [cpu] PR body: fp8-e4m3 row-major [rows, K], K contiguous per output row, one scale
    per 128x128 block; the scale multiplies the decoded value.
    """
    N, K = bank["N"], bank["K"]
    start = e * bank["expert_stride_bytes"]
    codes = np.asarray(bank["codes"][start:start + N * K], dtype=np.uint8).reshape(N, K)
    S = block_scales(bank, e)
    S_full = np.repeat(np.repeat(S, BLOCK, axis=0)[:N], BLOCK, axis=1)[:, :K]
    return _LUT[codes] * S_full


# ----------------------------------------------------------------------------- routing

def route(logits, top_k: int):
    """Top-k experts per token and their renormalised softmax weights.

    Experts are ordered by the key (-logit, expert id) on the fp32 logits, so ties go to
    the lower id and slot 0 holds the largest logit. The weights are the softmax over the
    selected logits, which equals the full softmax renormalised over the top-k, computed
    in float64 as exp(l_j - l_0) / sum_i exp(l_i - l_0) with the sum taken in slot order.
    Returns ids int32 [T, k], float64 weights [T, k] and the same rounded to fp32.
    """
    lg = np.asarray(logits, dtype=np.float32)
    T, E = lg.shape
    ids = np.empty((T, top_k), dtype=np.int32)
    w = np.empty((T, top_k), dtype=np.float64)
    expert = np.arange(E)
    for t in range(T):
        order = np.lexsort((expert, -lg[t].astype(np.float64)))[:top_k]
        ids[t] = order
        sel = lg[t, order].astype(np.float64)
        ex = np.exp(sel - sel[0])
        tot = 0.0
        for j in range(top_k):
            tot += ex[j]
        w[t] = ex / tot
    return ids, w, w.astype(np.float32)


def sort_pairs(ids, E: int):
    """Pair p = t*k + j grouped by expert, stable within an expert.

    Returns counts [E], offsets [E+1] (exclusive prefix sums) and sorted_pairs [T*k].
    """
    flat = np.asarray(ids, dtype=np.int64).ravel()
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    order = np.argsort(flat, kind="stable").astype(np.int32)
    return counts, offsets, order


def gathered_count(T: int, E: int, top_k: int) -> int:
    """g = min(E, T*top_k): the static number of expert slots on the gather path ([gather] The fix)."""
    return min(E, T * top_k)


# ----------------------------------------------------------------------------- activations

def quantize_rows(x32):
    """Dynamic per-row e4m3 quantisation, emulated exactly in fp32.

    One scale per row: s = amax / 448 (fp32 division, correctly rounded), s = 1 for an
    all-zero row, codes = e4m3_encode(x / s) with the division in fp32. The dequantised
    row is LUT[code] * s. Rows are tokens for the gate/up GEMM and (token, slot) pairs
    for the down GEMM ([gather] Who is affected: dynamic activation scales).
    """
    x = np.asarray(x32, dtype=np.float32)
    amax = np.max(np.abs(x), axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    s = np.where(amax == 0, np.float32(1.0), s).astype(np.float32)
    v = (x / s[:, None]).astype(np.float32)
    return e4m3_encode(v), s


def quantize_groups(x32, group: int = BLOCK):
    """Dynamic e4m3 per (row, group of `group` consecutive columns), emulated exactly in fp32.

    Each group is quantised as its own row by quantize_rows: scale amax/448 over the
    group's columns, codes e4m3_encode(x / scale). With the default group of 128 the
    activation groups line up with the 128-wide K blocks of the weight scales, so one
    activation scale and one weight scale apply to each 128-long piece of a dot product
    ([gather] Who is affected: block-quantized FP8 checkpoints with dynamic activation
    scales; The fix: up/gate as one native FP8 GEMM). Returns codes [R, C] and scales
    [R, C // group].
    """
    x = np.asarray(x32, dtype=np.float32)
    R, C = x.shape
    assert C % group == 0, "columns must be a whole number of groups"
    q, s = quantize_rows(x.reshape(R * (C // group), group))
    return q.reshape(R, C), s.reshape(R, C // group)


def dequant_groups(q, s, group: int = BLOCK) -> np.ndarray:
    """LUT[code] * the scale of the code's group, float64."""
    return _LUT[np.asarray(q)] * np.repeat(np.asarray(s, dtype=np.float64), group, axis=1)


def silu(g):
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def _silu_grad(g):
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-g))
    return sig * (1.0 + g * (1.0 - sig))


# ----------------------------------------------------------------------------- forward

def expert_bias(bank: dict, e: int) -> np.ndarray:
    """Bias row of expert e as float64 [N], zeros if the bank has none. Rows follow the
    codes' rows, so w13's bias holds the gate half 0..I-1 then the up half I..2I-1
    ([tpu] review of the w1 bias DMA: each half must come from its own offset)."""
    b = bank.get("bias")
    if b is None:
        return np.zeros(bank["N"], dtype=np.float64)
    return np.asarray(b, dtype=np.float64).reshape(bank["E"], bank["N"])[e]


def _expert_cache(w13: dict, w2: dict):
    cache = {}

    def get(e):
        if e not in cache:
            cache.clear()  # one expert at a time: the large banks hold hundreds of MB each
            cache[e] = (dequant_expert(w13, e), dequant_expert(w2, e), expert_bias(w13, e), expert_bias(w2, e))
        return cache[e]
    return get


# Drift bound for the W8A8 re-quantisation of h. The pages fix no accumulation order and
# no accumulation precision for the fp8 matrix products ([cpu] PR body: results differ
# only in summation order; [cpu] commit "add float64 parity reference": a loose tolerance
# cannot see accumulator precision loss), so an h element whose scaled value lies close to
# an e4m3 rounding midpoint may legitimately round either way. h_drift bounds how far an
# implementation's h may sit from the exact h:
#   * fp32 evaluation: 2^-24 * sqrt(K) * (root sum of squares of the K terms), F32_RW
#     times. Summing exact code products in float32 in any order (sequential, pairwise,
#     128-blocked, with float32 block-scale multiplies) stays within 0.15 of it.
#   * fp8 matrix-core accumulation: the matrix cores sum a block of 128 code products in a
#     fixed-width aligned adder, which drops low bits of the products relative to the
#     block's largest one (measured on gfx950: at most 2^-11 of that product's binade per
#     block, about 2^-15 typically). The bound per row is ACC_MMA times the root sum of
#     squares over the K blocks of each block's largest |product|.
#   * the elementwise SiLU and product: H_REL * |h|.
# A test evaluates GEMM1 on the CPU with a truncating aligned accumulator and with float32
# sums in several orders; a GPU test checks that the MFMA path's h lies within the bound
# for every element. These constants are a reading (the pages are silent), not page values.
F32_RW = 1.0
ACC_MMA = 3.0e-4
H_REL = 2.0 ** -22
U32 = 2.0 ** -24


def acc_bound(W, X, coarse: bool = False):
    """Accumulation bound of W @ x for every row x of X: [n, N].

    F32_RW * 2^-24 * sqrt(K) * (root sum of squares of the K terms W[i,k] x[k]) plus
    ACC_MMA * sqrt(sum over 128-wide K blocks of the block's largest |W[i,k] x[k]|^2).
    coarse: each block's largest term replaced by the product of the block's largest |W|
    and largest |x| (never smaller, and cheap for many rows).
    """
    X = np.atleast_2d(X)
    n, K = X.shape
    N = W.shape[0]
    rss = np.sqrt((W * W) @ (X * X).T).T  # [n, N]
    nkb = -(-K // BLOCK)
    aw = np.zeros((N, nkb * BLOCK))
    aw[:, :K] = np.abs(W)
    aw = aw.reshape(N, nkb, BLOCK)
    ax = np.zeros((n, nkb * BLOCK))
    ax[:, :K] = np.abs(X)
    ax = ax.reshape(n, nkb, BLOCK)
    if coarse:
        wm, xm = aw.max(axis=2), ax.max(axis=2)  # [N, nkb], [n, nkb]
        mb = np.sqrt((xm * xm) @ (wm * wm).T)
    else:
        mb = np.empty((n, N))
        for i in range(n):
            m = (aw * ax[i][None]).max(axis=2)  # [N, nkb]
            mb[i] = np.sqrt((m * m).sum(axis=1))
    return F32_RW * U32 * math.sqrt(K) * rss + ACC_MMA * mb


def h_drift(W13, X, g, u, h, coarse: bool = False):
    """Bound on |h_impl - h| for each h = silu(g) * u, rows of X the tokens ([n, I]; first
    order in the gate and up errors; see ACC_MMA; coarse as in acc_bound)."""
    I = np.atleast_2d(g).shape[1]
    b = acc_bound(W13, X, coarse)
    return np.abs(_silu_grad(g) * u) * b[:, :I] + np.abs(silu(g)) * b[:, I:] + H_REL * np.abs(h)


def _expert_up(W13, X, b13=None):
    """a = W13 x (+ b13) for each row x of X; gate rows 0..I-1 and up rows I..2I-1 ([tpu]
    review of the w1 DMA: gate half first, up half second; the bias follows the rows, [tpu]
    review of the w1 bias DMA). Returns g, u and h = silu(g) * u, each [n, I]."""
    I = W13.shape[0] // 2
    A = np.atleast_2d(X) @ W13.T
    if b13 is not None:
        A = A + b13[None, :]
    g, u = A[:, :I], A[:, I:]
    return g, u, silu(g) * u


def _h_group(act_mode: int, I: int) -> int:
    """Columns of h that share one re-quantisation scale: the whole row (I) for act_mode 1,
    128 for act_mode 3 (one scale per (pair, 128-feature group), the granularity of the
    weight blocks along the down GEMM's K)."""
    return BLOCK if act_mode == 3 else I


def _requantize_h(W13, X, g, u, h, group=None):
    """act_modes 1 and 3: requantize_h with the drift bound h_drift of these tokens."""
    return requantize_h(h, h_drift(W13, X, g, u, h), group)


def requantize_h(h, d, group=None):
    """h [n, I] (float64) re-quantised to e4m3 before the down GEMM, one scale per group of
    `group` consecutive columns of a (token, slot) row (the whole row by default; scale
    group amax/448 in float32 emulation, quantize_groups), and the elements whose rounding
    an implementation may decide either way flagged, d being the drift bound of each h:
    |v - midpoint| <= d_i/s + |v| * d_r/amax, with r the argmax of the element's group and
    s, amax that group's scale and maximum (the second term is the scale moving with amax).
    Returns the dequantised h and a dict of codes, scales (per row, or [n, I/group]), flags,
    the distance between each element's two neighbouring codes (step) and d."""
    h32 = h.astype(np.float32)
    n, I = h32.shape
    group = I if group is None else group
    q, s = quantize_groups(h32, group)
    s_el = np.repeat(s.astype(np.float64), group, axis=1)  # each element's scale
    h_deq = _LUT[q] * s_el
    a = np.abs(h32).reshape(n, I // group, group)
    amax = a.max(axis=2).astype(np.float64)  # [n, groups]
    r = a.argmax(axis=2)
    dr = np.take_along_axis(d.reshape(n, I // group, group), r[:, :, None], axis=2)[:, :, 0]
    v = (h32 / s_el.astype(np.float32)).astype(np.float32).astype(np.float64)
    dist, step = e4m3_midpoint_distance(v)
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(amax > 0, dr / amax, 0.0)
    flags = dist <= d / s_el + np.abs(v) * np.repeat(rel, group, axis=1)
    return h_deq, dict(h_codes=q, h_scale=s if group != I else s[:, 0], flags=flags, step=step, drift=d,
                       h_scale_el=s_el)


def _expert_mlp(W13, W2, X, act_mode: int, b13=None, b2=None):
    """The tokens X [n, H] routed to one expert: a = W13 x + b13, h = silu(a[:I]) * a[I:],
    y = W2 h + b2, for each row. act_modes 1 and 3 re-quantise h first (_requantize_h, per
    row or per 128-feature group). Returns Y [n, H] and, for those modes, the h codes,
    scales, flags and steps."""
    g, u, h = _expert_up(W13, X, b13)
    extra = None
    if act_mode in (1, 3):
        h, extra = _requantize_h(W13, np.atleast_2d(X), g, u, h, _h_group(act_mode, h.shape[1]))
    Y = h @ W2.T
    if b2 is not None:
        Y = Y + b2[None, :]
    return Y, extra


def _x_used(x, act_mode: int, res: dict):
    """The activations the up/gate GEMM multiplies: x itself (act_mode 0), x quantised per
    token (1) or per (token, 128-column group) (2 and 3), dequantised in float64."""
    if act_mode == 0:
        return x
    if act_mode == 1:
        xq, xs = quantize_rows(x.astype(np.float32))
        res.update(x_codes=xq, x_scales=xs)
        return _LUT[xq] * xs.astype(np.float64)[:, None]
    if act_mode in (2, 3):
        xq, xs = quantize_groups(x.astype(np.float32))
        res.update(x_codes=xq, x_scales=xs)
        return dequant_groups(xq, xs)
    raise ValueError(f"act_mode {act_mode}")


def _pairs_by_expert(ids):
    """{expert: array of pairs p = t*k + j routed to it}, experts ascending."""
    flat = np.asarray(ids).ravel()
    return {int(e): np.nonzero(flat == e)[0] for e in np.unique(flat)}


def forward(hidden_bf16, logits, w13: dict, w2: dict, top_k: int, act_mode: int = 0):
    """Gathered formulation: out[t] = sum_j w_tj * expert_{ids[t,j]}(x_t).

    hidden_bf16: uint16 bf16 bits [T, H]; logits: fp32 [T, E]; w13: bank with N = 2I,
    K = H; w2: bank with N = H, K = I (dicts as produced by the generators' numpy()).
    act_mode 0 is W8A16 (x exact, h float64); act_mode 1 is W8A8: x quantised per token
    and h per pair, both in fp32 emulation ([gather] The fix: the routed experts are
    gathered, up/gate run as one GEMM and the down projection follows); act_mode 2 is
    the gather variant of [gather] The fix: the up/gate GEMM on e4m3 activations quantised
    per (token, 128-column group) and the down projection on h in full precision;
    act_mode 3 is W8A8 with both GEMMs on groups: x per (token, 128-column group) as in
    act_mode 2 and h per (pair, 128-feature group).
    Only the routed experts are read; each is evaluated once on all the tokens routed to
    it (one matrix product per expert), and its contribution w_tj * y is added to each of
    those tokens. Returns a dict with out (float64 [T, H]), routing, the x quantisation for
    act_modes 1 to 3, and for act_modes 1 and 3 the h quantisation (per pair p = t*k + j:
    codes and the row's scale, or its [I/128] group scales) and the per-output allowance
    for ambiguous h roundings.
    """
    x = bf16_to_f64(hidden_bf16)
    T, H = x.shape
    E = np.asarray(logits).shape[1]
    ids, w, w32 = route(logits, top_k)
    counts, offsets, sorted_pairs = sort_pairs(ids, E)
    res = dict(ids=ids, w=w, w32=w32, counts=counts, offsets=offsets, sorted_pairs=sorted_pairs)
    x_used = _x_used(x, act_mode, res)
    h_mode = act_mode if act_mode in (1, 3) else 0  # act_modes 1 and 3 re-quantise h
    get = _expert_cache(w13, w2)
    out = np.zeros((T, H), dtype=np.float64)
    allowance = np.zeros((T, H), dtype=np.float64)
    n_flag = 0
    h_codes, h_scales = {}, {}
    wf = w.ravel()
    for e, pairs in _pairs_by_expert(ids).items():
        W13, W2, b13, b2 = get(e)
        toks = pairs // top_k
        for c0 in range(0, len(pairs), 64):
            sl = slice(c0, c0 + 64)
            Y, extra = _expert_mlp(W13, W2, x_used[toks[sl]], h_mode, b13, b2)
            out[toks[sl]] += wf[pairs[sl], None] * Y  # a token holds each expert once
            if extra is not None:
                f = extra["flags"]
                n_flag += int(f.sum())
                amt = np.where(f, extra["step"] * extra["h_scale_el"], 0.0)
                allowance[toks[sl]] += np.abs(wf[pairs[sl], None]) * (amt @ np.abs(W2).T)
                for r, p in enumerate(pairs[sl]):
                    h_codes[int(p)] = extra["h_codes"][r]
                    h_scales[int(p)] = extra["h_scale"][r]
    res["out"] = out
    if act_mode in (1, 3):
        res.update(allowance=allowance, n_flagged=n_flag, n_h=T * top_k * (w13["N"] // 2),
                   h_codes=h_codes, h_scales=h_scales)
    return res


def up_w8a8(hidden_bf16, ids, w13: dict, pairs=None, coarse: bool = False, act_mode: int = 1):
    """The first half of act_mode 1 (or 3) on its own: h = silu(gate) * up for every pair
    p = t*k + j (or the listed pairs), float64 [len(pairs), I] in the order given, from x
    quantised per token (per (token, 128-column group)). Also returns the drift bound of
    each h (h_drift, coarse or not)."""
    assert act_mode in (1, 3)
    x = bf16_to_f64(hidden_bf16)
    xu = _x_used(x, act_mode, {})
    ids = np.asarray(ids)
    k = ids.shape[1]
    pairs = np.arange(ids.size) if pairs is None else np.asarray(pairs)
    I = w13["N"] // 2
    h = np.empty((len(pairs), I))
    d = np.empty((len(pairs), I))
    flat = ids.ravel()[pairs]
    for e in np.unique(flat):
        W13 = dequant_expert(w13, int(e))
        b13 = expert_bias(w13, int(e))
        rows = np.nonzero(flat == e)[0]
        X = xu[pairs[rows] // k]
        g, u, hh = _expert_up(W13, X, b13)
        h[rows] = hh
        d[rows] = h_drift(W13, X, g, u, hh, coarse)
    return h, d


def down_w8a8(h32_pairs, ids, w, w2: dict):
    """The second half of act_mode 1 on its own: each pair's float32 h row [T*k, I] (pair
    p = t*k + j) is quantised per row (quantize_rows), multiplied by its expert's w2 and
    added to out[t] with the router weight w[t, j]. Returns out float64 [T, H]."""
    ids = np.asarray(ids)
    T, k = ids.shape
    q, s = quantize_rows(np.asarray(h32_pairs, dtype=np.float32))
    hd = _LUT[q] * s.astype(np.float64)[:, None]
    out = np.zeros((T, w2["N"]))
    wf = np.asarray(w, dtype=np.float64).ravel()
    for e, pairs in _pairs_by_expert(ids).items():
        W2 = dequant_expert(w2, e)
        b2 = expert_bias(w2, e)
        out[pairs // k] += wf[pairs, None] * (hd[pairs] @ W2.T + b2[None, :])
    return out


def down_w8a8_groups(h_codes, h_scales, ids, w, w2: dict):
    """The second half of act_mode 3 on given h codes: each pair's e4m3 codes [T*k, I] with
    one scale per (pair, 128-feature group) [T*k, I/128] (pair p = t*k + j) are dequantised,
    multiplied by the expert's w2 and added to out[t] with the router weight w[t, j].
    Returns out float64 [T, H]."""
    ids = np.asarray(ids)
    T, k = ids.shape
    hd = dequant_groups(h_codes, h_scales)
    out = np.zeros((T, w2["N"]))
    wf = np.asarray(w, dtype=np.float64).ravel()
    for e, pairs in _pairs_by_expert(ids).items():
        W2 = dequant_expert(w2, e)
        b2 = expert_bias(w2, e)
        out[pairs // k] += wf[pairs, None] * (hd[pairs] @ W2.T + b2[None, :])
    return out


def forward_dense(hidden_bf16, logits, w13: dict, w2: dict, top_k: int, act_mode: int = 0):
    """Dense all-experts formulation: out[t] = sum_e C[t, e] * expert_e(x_t).

    C is the [T, E] combine matrix, zero off the routes. Every expert is evaluated on
    every token, as the stock op reads every local expert ([gather] Problem). Returns the
    float64 output [T, H].
    """
    x = bf16_to_f64(hidden_bf16)
    T, H = x.shape
    E = np.asarray(logits).shape[1]
    ids, w, _ = route(logits, top_k)
    C = np.zeros((T, E), dtype=np.float64)
    for t in range(T):
        for j in range(top_k):
            C[t, ids[t, j]] = w[t, j]
    x_used = _x_used(x, act_mode, {})
    out = np.zeros((T, H), dtype=np.float64)
    for e in range(E):
        W13, W2 = dequant_expert(w13, e), dequant_expert(w2, e)
        b13, b2 = expert_bias(w13, e), expert_bias(w2, e)
        Y, _ = _expert_mlp(W13, W2, x_used, act_mode if act_mode in (1, 3) else 0, b13, b2)
        out += C[:, e:e + 1] * Y
    return out


def routed_experts(ids) -> np.ndarray:
    """Distinct experts a routing touches (their bytes are what the gather path reads)."""
    return np.unique(np.asarray(ids).ravel())
