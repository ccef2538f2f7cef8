"""Pins for the oracle's e4m3 decode, encode and per-row quantisation (CPU only)."""

import math

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from helpers import read_golden, torch_e4m3_table

FINITE = [c for c in range(256) if (c & 0x7F) != 0x7F]


def test_lut_matches_page_facts():
    lut = O.e4m3_lut()
    for name, code, value in read_golden("e4m3_facts.txt"):
        if name.startswith("fp16_trick"):
            continue
        assert lut[int(code, 16)] == float(value), name
    pos = lut[1:0x7F]
    assert np.all(np.diff(pos) > 0), "positive codes must increase"
    assert lut[0] == 0.0 and not np.signbit(lut[0])
    assert lut[0x80] == 0.0 and np.signbit(lut[0x80])
    assert math.isnan(lut[0x7F]) and math.isnan(lut[0xFF])
    # sign symmetry
    for c in FINITE:
        assert lut[c ^ 0x80] == -lut[c]
    # smallest normal, one
    assert lut[0x08] == 2.0 ** -6
    assert lut[0x38] == 1.0


def test_lut_matches_fp16_bit_identity():
    """(b & 0x80) << 8 | (b & 0x7F) << 7 read as fp16 is the e4m3 value times 2^-8."""
    lut = O.e4m3_lut()
    b = np.arange(256, dtype=np.uint16)
    h = (((b & 0x80) << 8) | ((b & 0x7F) << 7)).astype(np.uint16).view(np.float16).astype(np.float64) * 256.0
    for c in FINITE:
        assert h[c] == lut[c], hex(c)
    facts = {name: (int(code, 16), float(v)) for name, code, v in read_golden("e4m3_facts.txt")}
    for key in ("fp16_trick_nan_pos", "fp16_trick_nan_neg"):
        code, v = facts[key]
        assert h[code] == v


def test_lut_matches_torch_float8():
    lut = O.e4m3_lut()
    ref = torch_e4m3_table()
    same = (lut == ref) | (np.isnan(lut) & np.isnan(ref))
    assert same.all()
    assert np.array_equal(np.signbit(lut[FINITE]), np.signbit(ref[FINITE]))


def test_bf16_carries_every_finite_code():
    lut = O.e4m3_lut()[FINITE]
    rt = torch.from_numpy(lut).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(rt, lut)


def _midpoint_probes():
    pos = O.e4m3_lut()[: 0x7F]
    mids = 0.5 * (pos[:-1] + pos[1:])
    vals = [pos, mids]
    m32 = mids.astype(np.float32)
    vals.append(np.nextafter(m32, np.float32(np.inf)).astype(np.float64))
    vals.append(np.nextafter(m32, np.float32(-np.inf)).astype(np.float64))
    v = np.concatenate(vals).astype(np.float32)
    return np.concatenate([v, -v])


def test_encode_matches_torch_at_midpoints():
    v = _midpoint_probes()
    ours = O.e4m3_encode(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = np.nonzero(ours != ref)[0]
    assert bad.size == 0, [(float(v[i]), int(ours[i]), int(ref[i])) for i in bad[:10]]


def test_encode_matches_torch_random():
    g = np.random.default_rng(5)
    parts = [g.normal(0, s, 20000) for s in (1e-3, 1e-2, 1.0, 30.0, 200.0)]
    parts.append(g.uniform(-448, 448, 20000))
    v = np.concatenate(parts).astype(np.float32)
    # torch's cast does not saturate (it gives NaN from 464 on), so compare inside the
    # finite range; saturation is checked by definition below
    v = v[np.abs(v) <= 448.0]
    ours = O.e4m3_encode(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_encode_saturates_and_keeps_zero_sign():
    v = np.array([448.0, 449.0, 463.9, 464.0, 470.0, 1e6, np.inf, -500.0], dtype=np.float32)
    assert list(O.e4m3_encode(v)) == [0x7E] * 7 + [0xFE]
    z = np.array([0.0, -0.0, 2.0 ** -11, -(2.0 ** -11), 2.0 ** -10, 3 * 2.0 ** -11], dtype=np.float32)
    # 2^-11 rounds to +-0; 2^-10 is the midpoint of 0 and 2^-9 and ties to the even
    # code 0; 3*2^-11 is nearer to 2^-9 than to 0
    assert list(O.e4m3_encode(z)) == [0x00, 0x80, 0x00, 0x80, 0x00, 0x01]


def test_quantize_rows_definition():
    x = np.array([
        [448.0, -224.0, 1.0, 0.0],      # amax 448 -> s = 1, codes are the encodes
        [0.0, 0.0, 0.0, 0.0],           # zero row -> s = 1, all codes zero
        [7.0, -3.5, 1.75, 0.4375],      # s = 7/448 = 1/64 exactly
    ], dtype=np.float32)
    q, s = O.quantize_rows(x)
    assert s[0] == 1.0 and s[1] == 1.0 and s[2] == np.float32(1.0 / 64.0)
    lut = O.e4m3_lut()
    assert np.array_equal(lut[q[0]], x[0].astype(np.float64))
    assert np.all(q[1] == 0)
    assert np.array_equal(lut[q[2]] * s[2], x[2].astype(np.float64))


def test_quantize_rows_vs_torch():
    g = np.random.default_rng(9)
    x = (g.normal(0, 1, (64, 512)) * g.uniform(0.01, 10, (64, 1))).astype(np.float32)
    q, s = O.quantize_rows(x)
    xt = torch.from_numpy(x)
    st = xt.abs().amax(dim=1) / torch.tensor(448.0, dtype=torch.float32)
    qt = (xt / st[:, None]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(s, st.numpy())
    assert np.array_equal(q, qt)


def test_scale_padding_rule_matches_page():
    for rule, rows, cols, esz, want in read_golden("scale_padding.txt"):
        assert W.scale_cols_padded(int(rows), int(cols), int(esz), rule) == int(want)
    # the per-row rule the workloads use: 4 bf16 columns (8 B) grow to 8 (16 B)
    assert W.scale_cols_padded(16, 4, 2, "row16") == 8
    assert W.scale_cols_padded(56, 16, 4, "row16") == 16


@pytest.mark.parametrize("rule", ["row16", "slab16"])
def test_dequant_ignores_padding(rule):
    """Padded scale strides with NaN in the padding give the same expert as no padding."""
    kw = dict(kind="uniform", scale_dtype=torch.bfloat16, seed=3, tensor_id=1)
    plain = W.make_bank(3, 256, 640, pad="none", **kw).numpy()
    padded = W.make_bank(3, 256, 640, pad=rule, code_pad_bytes=32, **kw).numpy()
    assert padded["scale_row_stride"] > plain["scale_row_stride"]
    for e in range(3):
        a = O.dequant_expert(plain, e)
        b = O.dequant_expert(padded, e)
        assert np.array_equal(a, b)
        assert np.isfinite(b).all()


def test_dequant_power_of_two_codes_unit_scales():
    """Codes for 2^j with unit scales dequantise to exact powers of two."""
    N, K = 256, 384
    codes = np.zeros((N, K), dtype=np.uint8)
    pw = {0x38: 1.0, 0x40: 2.0, 0x48: 4.0, 0x30: 0.5, 0xB8: -1.0}
    keys = np.array(list(pw))
    g = np.random.default_rng(1)
    codes[:] = keys[g.integers(0, len(keys), (N, K))]
    bank = dict(codes=codes.ravel(), scales=np.ones(6, dtype=np.float32), scale_dtype="f32", E=1,
                N=N, K=K, expert_stride_bytes=N * K, scale_row_stride=3, scale_expert_stride=6)
    W_ = O.dequant_expert(bank, 0)
    want = np.vectorize(pw.get)(codes).astype(np.float64)
    assert np.array_equal(W_, want)


def test_fp8_ulp_diff_counts_e4m3_steps():
    """The verify unit: neighbouring e4m3 values are one ulp apart everywhere, normal and
    subnormal, and the distance between any two codes of one binade is their code distance."""
    from helpers import fp8_ulp_diff
    lut = O.e4m3_lut()
    pos = lut[:0x7F]  # 0 .. 448, ascending
    d = fp8_ulp_diff(pos[1:], pos[:-1])
    # steps inside a binade are one ulp; crossing up into the next binade the step below
    # is measured in the larger value's ulp, i.e. half an ulp
    upper = np.frexp(pos[1:])[1] != np.frexp(pos[:-1])[1]
    assert np.all(d[~upper | (pos[1:] <= 2.0 ** -6)] == 1.0)
    assert np.all(d[upper & (pos[1:] > 2.0 ** -6)] == 0.5)
    assert fp8_ulp_diff(np.array([1.0]), np.array([1.25]))[0] == 2.0
    assert fp8_ulp_diff(np.array([-3.0]), np.array([3.0]))[0] == 24.0  # spacing 0.25 in [2, 4)
    assert fp8_ulp_diff(np.array([0.0]), np.array([0.0]))[0] == 0.0


def _brute_midpoint(a: float):
    """Distance from a >= 0 to the midpoint of the two neighbouring finite e4m3 values
    that bracket it, found by walking the list of all finite values, and that pair's
    spacing; infinite distance at or past the largest value."""
    vals = sorted({abs(float(x)) for x in O.e4m3_lut()[FINITE]})
    if a >= vals[-1]:
        return math.inf, None
    for lo, hi in zip(vals, vals[1:]):
        if lo <= a < hi:
            return abs(a - (lo + hi) / 2.0), hi - lo
    raise AssertionError("unreachable")


def test_midpoint_distance_matches_brute_force():
    """e4m3_midpoint_distance (used by the W8A8 ambiguity flags) against a linear walk over
    every finite value: at every value, every midpoint and its float32 neighbours, between
    every pair of neighbours, at random magnitudes and signs, and past the largest value."""
    pos = sorted({abs(float(x)) for x in O.e4m3_lut()[FINITE]})
    mids = [(a + b) / 2 for a, b in zip(pos, pos[1:])]
    g = np.random.default_rng(5)
    probes = list(pos) + mids
    probes += [float(np.nextafter(np.float32(m), np.float32(np.inf))) for m in mids]
    probes += [float(np.nextafter(np.float32(m), np.float32(-np.inf))) for m in mids]
    probes += [a + (b - a) * f for a, b in zip(pos, pos[1:]) for f in (0.1, 0.3, 0.7, 0.9)]
    probes += list(np.exp(g.uniform(np.log(2.0 ** -12), np.log(460.0), 3000)))
    probes += [448.0, 449.0, 1e6]
    v = np.array(probes, dtype=np.float64)
    v = np.concatenate([v, -v])
    dist, step = O.e4m3_midpoint_distance(v)
    for x, d, s in zip(v, dist, step):
        bd, bs = _brute_midpoint(abs(float(x)))
        if math.isinf(bd):
            assert math.isinf(d), x
            continue
        assert d == bd and s == bs, (x, d, bd, s, bs)
