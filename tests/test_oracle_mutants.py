"""The oracle's pins must catch plausible mistakes.

Each mutant plants one mistake in the oracle (swapped gate/up halves, a transposed or
recomputed scale index, a wrong tie-break, a dropped router weight, ...) and the test
asserts that at least one pin then fails. Everything runs on the CPU.
"""

import numpy as np
import pytest
import torch

import oracle
import oracle.oracle as OO
import test_oracle_e4m3 as PE
import test_oracle_forward as PF

PINS = [
    PE.test_lut_matches_page_facts,
    PE.test_lut_matches_fp16_bit_identity,
    PE.test_encode_matches_torch_at_midpoints,
    PE.test_quantize_rows_vs_torch,
    lambda: PE.test_dequant_ignores_padding("slab16"),
    PE.test_dequant_power_of_two_codes_unit_scales,
    PF.test_route_matches_bruteforce_with_ties,
    PF.test_route_is_renormalised_full_softmax,
    PF.test_sort_pairs_bruteforce,
    lambda: PF.test_forward_matches_scalar_loops(torch.float32),
    PF.test_forward_matches_scalar_loops_with_biases,
    lambda: PF.test_single_expert_is_swiglu(None),
    lambda: PF.test_single_expert_is_swiglu(0.5),
    PF.test_w8a8_matches_torch_quantised_reference,
    PF.test_group_quantisation_matches_scalar_search,
    PF.test_group_w8a8_matches_torch_quantised_reference,
]


def _failures():
    n = 0
    for pin in PINS:
        try:
            pin()
        except Exception:
            n += 1
    return n


def _mlp_swapped(W13, W2, X, act_mode, b13=None, b2=None):
    I = W13.shape[0] // 2
    A = np.atleast_2d(X) @ W13.T + (0.0 if b13 is None else b13[None, :])
    g, u = A[:, I:], A[:, :I]
    return (OO.silu(g) * u) @ W2.T + (0.0 if b2 is None else b2[None, :]), None


def _mlp_no_silu(W13, W2, X, act_mode, b13=None, b2=None):
    I = W13.shape[0] // 2
    A = np.atleast_2d(X) @ W13.T + (0.0 if b13 is None else b13[None, :])
    return (A[:, :I] * A[:, I:]) @ W2.T + (0.0 if b2 is None else b2[None, :]), None


def _bias_halves_swapped(bank, e):
    """The bias analogue of loading the next gate slice where the up bias belongs."""
    b = OO.__dict__["_orig_expert_bias"](bank, e)
    n = b.shape[0] // 2
    return np.concatenate([b[n:], b[:n]])


def _bias_dropped(bank, e):
    return np.zeros(bank["N"], dtype=np.float64)


def _scales_transposed(bank, e):
    s = OO._scales_f64(bank)
    rows, cols = -(-bank["N"] // 128), -(-bank["K"] // 128)
    base = e * bank["scale_expert_stride"]
    r = np.arange(rows)[:, None]
    c = np.arange(cols)[None, :] * bank["scale_row_stride"]
    idx = np.minimum(base + r + c, s.size - 1)
    return s[idx]


def _scales_recomputed_stride(bank, e):
    s = OO._scales_f64(bank)
    rows, cols = -(-bank["N"] // 128), -(-bank["K"] // 128)
    base = e * bank["scale_expert_stride"]
    r = np.arange(rows)[:, None] * cols
    return s[base + r + np.arange(cols)[None, :]]


def _route_high_id_wins(logits, top_k):
    lg = np.asarray(logits, dtype=np.float32)
    T, E = lg.shape
    ids = np.empty((T, top_k), dtype=np.int32)
    w = np.empty((T, top_k))
    for t in range(T):
        order = np.lexsort((-np.arange(E), -lg[t].astype(np.float64)))[:top_k]
        ids[t] = order
        ex = np.exp(lg[t, order].astype(np.float64) - lg[t, order[0]])
        w[t] = ex / ex.sum()
    return ids, w, w.astype(np.float32)


def _route_not_renormalised(logits, top_k):
    ids, _, _ = OO.__dict__["_orig_route"](logits, top_k)
    lg = np.asarray(logits, dtype=np.float64)
    p = np.exp(lg - lg.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    w = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    return ids, w, w.astype(np.float32)


def _encode_ties_away(v):
    v32 = np.asarray(v, dtype=np.float32)
    a = np.minimum(np.abs(v32.astype(np.float64)), 448.0)
    _, ex = np.frexp(a)
    step = np.ldexp(1.0, np.maximum(ex - 1, -6) - 3)
    r = np.floor(a / step + 0.5) * step
    idx = np.minimum(np.searchsorted(OO._POS, r), 0x7E)
    return idx.astype(np.uint8) | (np.signbit(v32).astype(np.uint8) << 7)


def _bf16_wrong_shift(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 15
    return b.view(np.float32).astype(np.float64)


def _groups_tiled(q, s, group=128):
    """Group scales laid out group-major instead of each one over its own columns."""
    return OO._LUT[np.asarray(q)] * np.tile(np.asarray(s, dtype=np.float64), group)


def _groups_of_64(x32, group=128):
    """Activation groups half as wide as the weight blocks."""
    q, s = OO.quantize_rows(np.asarray(x32, np.float32).reshape(-1, 64))
    R, C = np.asarray(x32).shape
    return q.reshape(R, C), np.repeat(s.reshape(R, C // 64)[:, ::2], 1, axis=1)


def _h_group_whole_row(act_mode, I):
    """act_mode 3 re-quantising h with one scale per row instead of per 128-feature group."""
    return I


def _h_group_of_64(act_mode, I):
    """h groups half as wide as the weight blocks along the down GEMM's K."""
    return 64 if act_mode == 3 else I


MUTANTS = {
    "gate_up_swapped": ("_expert_mlp", _mlp_swapped),
    "silu_dropped": ("_expert_mlp", _mlp_no_silu),
    "scale_index_transposed": ("block_scales", _scales_transposed),
    "scale_stride_recomputed": ("block_scales", _scales_recomputed_stride),
    "tie_break_high_id": ("route", _route_high_id_wins),
    "weights_not_renormalised": ("route", _route_not_renormalised),
    "encode_ties_away": ("e4m3_encode", _encode_ties_away),
    "bf16_decode_shift": ("bf16_to_f64", _bf16_wrong_shift),
    "bias_halves_swapped": ("expert_bias", _bias_halves_swapped),
    "bias_dropped": ("expert_bias", _bias_dropped),
    "group_scales_tiled": ("dequant_groups", _groups_tiled),
    "groups_of_64": ("quantize_groups", _groups_of_64),
    "h_group_whole_row": ("_h_group", _h_group_whole_row),
    "h_group_of_64": ("_h_group", _h_group_of_64),
}


def test_unmutated_oracle_passes_every_pin():
    assert _failures() == 0


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(OO, "_orig_route", OO.route, raising=False)
    monkeypatch.setattr(OO, "_orig_expert_bias", OO.expert_bias, raising=False)
    monkeypatch.setattr(OO, attr, fn)
    if hasattr(oracle, attr):
        monkeypatch.setattr(oracle, attr, fn)
    assert _failures() >= 1, f"no pin catches the mutant {name}"
