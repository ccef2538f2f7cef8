"""The C ABI without a GPU: exports, version, the gate, and every argument check.

Every call here is rejected before the library makes any HIP call (the header promises
that), so fake non-NULL device pointers are safe: nothing dereferences them.
"""

import ctypes
import os
import re

import pytest

from block_fp8_mixture_top_amd import _lib as L

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moe_fp8_block.h")
FAKE = ctypes.c_void_p(0x10000)  # 16-byte aligned, never dereferenced


@pytest.fixture(scope="module")
def lib():
    return L.load()


def header_text():
    with open(HEADER) as f:
        return f.read()


def test_exports_every_declared_symbol(lib):
    names = sorted(set(re.findall(r"\b(moe_fp8_block_\w+)\s*\(", header_text())))
    assert names, "no declarations found"
    assert sorted(L.EXPORTS) == names
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_matches_header(lib):
    ver = int(re.search(r"#define MOE_FP8_BLOCK_ABI_VERSION (\d+)", header_text()).group(1))
    assert lib.moe_fp8_block_abi_version() == ver == L.ABI_VERSION


def test_default_opts(lib):
    o = L.Opts()
    assert lib.moe_fp8_block_default_opts(ctypes.byref(o)) == 0
    assert o.gate_ratio == pytest.approx(2.0)
    assert (o.force_path, o.mfma_min_tokens_per_expert, o.act_mode, o.use_measured_gate) == (0, 2, 0, 1)
    assert lib.moe_fp8_block_default_opts(None) == -1
    assert b"NULL" in lib.moe_fp8_block_last_error()


def _path(lib, T, E, k, H=2048, I=512, **kw):
    o = L.Opts()
    lib.moe_fp8_block_default_opts(ctypes.byref(o))
    o.use_measured_gate = 0  # the two thresholds (the measured table is tested on its own)
    for a, v in kw.items():
        setattr(o, a, v)
    info = L.RunInfo()
    st = lib.moe_fp8_block_select_path(T, E, H, I, k, ctypes.byref(o), ctypes.byref(info))
    return st, info


@pytest.mark.parametrize("T,path", [(1, 1), (4, 1), (12, 1), (64, 1), (65, 3), (96, 3), (1024, 3), (4096, 3)])
def test_gate_on_the_decode_shape(lib, T, path):
    """Defaults: gather iff T*k <= 2*E (E=256, k=8: T <= 64); MFMA from 2 pairs per expert."""
    st, info = _path(lib, T, 256, 8)
    assert st == 0
    assert info.path == path
    assert info.act_mode == (1 if path == 3 else 0)
    assert info.slots == min(256, T * 8)


def test_gate_ratio_and_forced_paths(lib):
    assert _path(lib, 16, 256, 8, gate_ratio=1.0)[1].path == 1
    assert _path(lib, 1, 256, 8, gate_ratio=0.0)[1].path == 2
    # the page's ratio and a high MFMA threshold leave STREAM in between
    assert _path(lib, 13, 256, 8, gate_ratio=0.4, mfma_min_tokens_per_expert=32)[1].path == 2
    assert _path(lib, 1024, 256, 8, gate_ratio=0.4, mfma_min_tokens_per_expert=32)[1].path == 3
    for forced in (1, 2, 3):
        assert _path(lib, 4096, 256, 8, force_path=forced)[1].path == forced
    assert _path(lib, 1, 256, 8, force_path=7)[0] == -1
    assert _path(lib, 1, 256, 8, act_mode=1)[0] == -1  # reported only, never asked for
    assert _path(lib, 1, 256, 8, act_mode=3)[0] == -1
    assert _path(lib, 1, 256, 8, mfma_min_tokens_per_expert=0)[0] == -1


def test_size_checks(lib):
    assert _path(lib, 1, 0, 1)[0] == -1
    assert _path(lib, 1, 1025, 8)[0] == -1
    assert _path(lib, 1, 8, 9)[0] == -1
    assert _path(lib, 1, 64, 33)[0] == -1
    assert _path(lib, -1, 8, 2)[0] == -1
    assert _path(lib, 0, 8, 2)[0] == 0


def test_workspace_size(lib):
    o = L.Opts()
    lib.moe_fp8_block_default_opts(ctypes.byref(o))
    a = lib.moe_fp8_block_workspace_size(1, 256, 2048, 512, 8, ctypes.byref(o))
    b = lib.moe_fp8_block_workspace_size(4096, 256, 2048, 512, 8, ctypes.byref(o))
    assert 0 < a < b
    assert lib.moe_fp8_block_workspace_size(1, 256, 2048, 512, 300, ctypes.byref(o)) == 0
    assert lib.moe_fp8_block_route_workspace_size(1, 0, 1) == 0
    assert lib.moe_fp8_block_route_workspace_size(4096, 256, 8) > 0


def _bank(N, K, **kw):
    b = L.Bank()
    b.codes = 0x10000
    b.scales = 0x20000
    b.scale_dtype = L.MOE_BF16
    b.reserved = 0
    b.expert_stride_bytes = N * K
    b.scale_row_stride = -(-K // 128)
    b.scale_expert_stride = -(-N // 128) * b.scale_row_stride
    for a, v in kw.items():
        setattr(b, a, v)
    return b


def _forward(lib, T=1, E=8, H=256, I=128, k=2, w13=None, w2=None, out_dtype=0, ws_bytes=1 << 30, opts=None,
             hidden=FAKE, workspace=FAKE):
    w13 = w13 or _bank(2 * I, H)
    w2 = w2 or _bank(H, I)
    info = L.RunInfo()
    st = lib.moe_fp8_block_forward(hidden, FAKE, ctypes.byref(w13), ctypes.byref(w2), T, E, H, I, k, FAKE,
                                   out_dtype, workspace, ws_bytes, None, None,
                                   ctypes.byref(opts) if opts else None, ctypes.byref(info), None)
    return st, lib.moe_fp8_block_last_error().decode(), info


def test_forward_rejects_bad_arguments(lib):
    assert _forward(lib, k=9)[0] == -1
    assert _forward(lib, E=2000)[0] == -1
    assert _forward(lib, H=200)[0] == -2
    assert _forward(lib, I=200)[0] == -2
    assert _forward(lib, out_dtype=5)[0] == -1
    assert _forward(lib, hidden=None)[0] == -1
    assert _forward(lib, w13=_bank(256, 256, codes=None))[0] == -1
    assert _forward(lib, w2=_bank(256, 128, scale_dtype=9))[0] == -1
    assert _forward(lib, w2=_bank(256, 128, reserved=3))[0] == -1


def test_forward_rejects_bad_strides(lib):
    """The unpadded extent must fit (FreeToken PR #662, commit honor padded fp8 scale strides)."""
    st, msg, _ = _forward(lib, w13=_bank(256, 256, scale_row_stride=1))
    assert st == -3 and "scale_row_stride" in msg
    st, msg, _ = _forward(lib, w2=_bank(256, 128, scale_expert_stride=1))
    assert st == -3 and "scale_expert_stride" in msg
    st, msg, _ = _forward(lib, w13=_bank(256, 256, expert_stride_bytes=256 * 256 - 16))
    assert st == -3
    # padded strides are accepted up to the workspace check
    st, msg, _ = _forward(lib, w13=_bank(256, 256, scale_row_stride=8, scale_expert_stride=16), ws_bytes=16)
    assert st == -5


def test_forward_rejects_misalignment(lib):
    assert _forward(lib, w13=_bank(256, 256, codes=0x10008))[0] == -4
    assert _forward(lib, w13=_bank(256, 256, expert_stride_bytes=256 * 256 + 8))[0] == -4
    assert _forward(lib, hidden=ctypes.c_void_p(0x10002))[0] == -4
    assert _forward(lib, workspace=ctypes.c_void_p(0x10010))[0] == -4
    st, msg, _ = _forward(lib, w2=_bank(256, 128, bias=0x30004))
    assert st == -4 and "bias" in msg
    # an aligned bias gets as far as the workspace check
    assert _forward(lib, w13=_bank(256, 256, bias=0x30000), w2=_bank(256, 128, bias=0x40000), ws_bytes=16)[0] == -5


def test_partial_scale_blocks_are_accepted(lib):
    """H and I need only be multiples of 16 (a last 128-wide scale block may be partial) on
    every path, MFMA included; the call then gets as far as the workspace check. The MFMA
    workspace holds the x and h code rows padded to whole 128-wide blocks."""
    st, msg, _ = _forward(lib, H=144, I=80, w13=_bank(160, 144), w2=_bank(144, 80), ws_bytes=16)
    assert st == -5 and "workspace" in msg
    o = L.Opts()
    lib.moe_fp8_block_default_opts(ctypes.byref(o))
    o.force_path = 3
    st, msg, info = _forward(lib, H=144, I=80, w13=_bank(160, 144), w2=_bank(144, 80), opts=o, ws_bytes=16)
    assert st == -5 and "workspace" in msg and info.path == 3
    ragged = lib.moe_fp8_block_workspace_size(64, 256, 2064, 528, 8, ctypes.byref(o))
    whole = lib.moe_fp8_block_workspace_size(64, 256, 2048, 512, 8, ctypes.byref(o))
    assert ragged > whole > 0
    # the gate keeps MFMA for ragged grouped work
    st, info = _path(lib, 4096, 256, 8, H=2064, I=528)
    assert st == 0 and info.path == 3
    # sizes past the kernels' limits are refused on a forced MFMA
    st, msg, _ = _forward(lib, H=8208, I=80, w13=_bank(160, 8208), w2=_bank(8208, 80), opts=o)
    assert st == -2 and "MFMA" in msg


def test_forward_rejects_small_workspace(lib):
    st, msg, info = _forward(lib, ws_bytes=64)
    assert st == -5 and "workspace" in msg
    assert _forward(lib, workspace=None)[0] == -5


def test_forward_forced_path_is_never_downgraded(lib):
    o = L.Opts()
    lib.moe_fp8_block_default_opts(ctypes.byref(o))
    o.force_path = 3
    st, msg, _ = _forward(lib, T=4, H=256, I=4224, opts=o)
    assert st == -2 and "MFMA" in msg
    o.force_path = 0
    # the gate alone may move off an unsupported MFMA shape, and reports it
    st, _, info = _forward(lib, T=4096, E=8, H=256, I=4224, ws_bytes=16, opts=o)
    assert st == -5 and info.path == 2


def test_forward_T0_is_a_noop(lib):
    st, _, info = _forward(lib, T=0, workspace=None, ws_bytes=0)
    assert st == 0 and info.kernels == 0


def test_route_argument_checks(lib):
    f = lib.moe_fp8_block_route
    assert f(FAKE, 4, 8, 2, FAKE, FAKE, FAKE, None, None, FAKE, 1 << 20, None) == -1
    assert f(FAKE, 4, 8, 9, FAKE, FAKE, None, None, None, None, 0, None) == -1
    assert f(None, 4, 8, 2, FAKE, FAKE, None, None, None, None, 0, None) == -1
    assert f(FAKE, 4, 8, 2, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == -5
    assert f(FAKE, 0, 8, 2, None, None, None, None, None, None, 0, None) == 0


def test_small_entry_checks(lib):
    assert lib.moe_fp8_block_quantize_rows(FAKE, 4, 24, FAKE, FAKE, None) == -2
    assert lib.moe_fp8_block_quantize_rows(FAKE, 4, 8208, FAKE, FAKE, None) == -2
    assert lib.moe_fp8_block_quantize_rows(None, 4, 32, FAKE, FAKE, None) == -1
    assert lib.moe_fp8_block_quantize_rows(ctypes.c_void_p(0x10004), 4, 32, FAKE, FAKE, None) == -4
    assert lib.moe_fp8_block_quantize_groups(FAKE, 4, 144, FAKE, FAKE, None) == -2  # not whole groups
    assert lib.moe_fp8_block_quantize_groups(FAKE, 4, 8320, FAKE, FAKE, None) == -2
    assert lib.moe_fp8_block_quantize_groups(FAKE, -1, 128, FAKE, FAKE, None) == -1
    assert lib.moe_fp8_block_quantize_groups(None, 4, 128, FAKE, FAKE, None) == -1
    assert lib.moe_fp8_block_quantize_groups(ctypes.c_void_p(0x10004), 4, 128, FAKE, FAKE, None) == -4
    assert lib.moe_fp8_block_quantize_groups(None, 0, 128, None, None, None) == 0
    assert lib.moe_fp8_block_decode_e4m3(FAKE, FAKE, -1, None) == -1
    assert lib.moe_fp8_block_decode_e4m3(None, None, 0, None) == 0
    assert lib.moe_fp8_block_encode_e4m3(None, FAKE, 3, None) == -1


def test_group_mfma_half_checks(lib):
    """The MFMA halves (group-scaled and per-row) refuse shapes without whole 128-wide
    groups, NULL buffers and a short workspace before any HIP call (the routing they enqueue
    first comes after every check)."""
    w13, w2 = _bank(2 * 80, 256), _bank(256, 80)
    up, down = lib.moe_fp8_block_mfma_up_groups, lib.moe_fp8_block_mfma_down_groups
    assert up(FAKE, FAKE, ctypes.byref(w13), 4, 8, 256, 80, 2, FAKE, FAKE, FAKE, 1 << 30, None) == -2
    assert down(FAKE, FAKE, FAKE, ctypes.byref(w2), 4, 8, 256, 80, 2, FAKE, 0, FAKE, 1 << 30, None) == -2
    w13, w2 = _bank(256, 256), _bank(256, 128)
    assert up(FAKE, FAKE, ctypes.byref(w13), 4, 8, 256, 128, 2, None, FAKE, FAKE, 1 << 30, None) == -1
    assert down(None, FAKE, FAKE, ctypes.byref(w2), 4, 8, 256, 128, 2, FAKE, 0, FAKE, 1 << 30, None) == -1
    assert lib.moe_fp8_block_mfma_up(FAKE, FAKE, ctypes.byref(w13), 4, 8, 256, 128, 2, None, FAKE, 1 << 30,
                                     None) == -1
    assert lib.moe_fp8_block_mfma_down(FAKE, FAKE, ctypes.byref(w2), 4, 8, 256, 128, 2, None, 0, FAKE, 1 << 30,
                                       None) == -1
    assert up(FAKE, FAKE, ctypes.byref(w13), 4, 8, 256, 128, 2, FAKE, FAKE, FAKE, 16, None) == -5
    assert down(FAKE, FAKE, FAKE, ctypes.byref(w2), 4, 8, 256, 128, 2, FAKE, 7, FAKE, 1 << 30, None) == -1
    assert down(FAKE, FAKE, FAKE, ctypes.byref(w2), 4, 8, 256, 128, 2, FAKE, 0, FAKE, 16, None) == -5
    assert up(None, None, ctypes.byref(w13), 0, 8, 256, 128, 2, None, None, None, 0, None) == 0


def test_binding_refuses_a_missing_library(tmp_path):
    saved = L._lib
    try:
        L._lib = None
        with pytest.raises(ImportError, match="missing"):
            L.load(str(tmp_path / "nope.so"))
    finally:
        L._lib = saved


def test_group_fp8_activations_gate_and_checks(lib):
    """MOE_ACT_GROUP_FP8 takes the thresholds: GATHER at T=1, MFMA (reported as act_mode 3,
    both GEMMs on groups) at T=4096. H must be a multiple of 128 on every path and I on
    MFMA too: the gate's MFMA choice then moves to STREAM, a forced MFMA is refused."""
    st, info = _path(lib, 1, 256, 8, act_mode=2)
    assert st == 0 and (info.path, info.act_mode) == (1, 2)
    st, info = _path(lib, 4096, 256, 8, act_mode=2)
    assert st == 0 and (info.path, info.act_mode) == (3, 3)
    st, info = _path(lib, 4096, 256, 8, act_mode=2, I=528)
    assert st == 0 and (info.path, info.act_mode) == (2, 2)
    st, info = _path(lib, 4096, 256, 8, act_mode=2, force_path=3, I=528)
    assert st == -2
    st, info = _path(lib, 4096, 256, 8)
    assert st == 0 and (info.path, info.act_mode) == (3, 1)

    def ws(act, path):
        o = L.Opts()
        lib.moe_fp8_block_default_opts(ctypes.byref(o))
        o.act_mode, o.force_path = act, path
        return lib.moe_fp8_block_workspace_size(4096, 256, 2048, 512, 8, ctypes.byref(o))
    # group codes and scales on top of STREAM's buffers; on MFMA no float h
    assert ws(2, 2) > ws(0, 2) > 0
    assert 0 < ws(2, 3) < ws(0, 3)
    o = L.Opts()
    lib.moe_fp8_block_default_opts(ctypes.byref(o))
    o.act_mode = 2
    o.force_path = 3
    st, msg, _ = _forward(lib, T=64, opts=o, ws_bytes=16)
    assert st == -5  # accepted on MFMA; only the workspace is short
    st, msg, _ = _forward(lib, T=64, I=80, w13=_bank(160, 256), w2=_bank(256, 80), opts=o)
    assert st == -2 and "I % 128" in msg
    o.force_path = 0
    st, msg, _ = _forward(lib, H=144, I=80, w13=_bank(160, 144), w2=_bank(144, 80), opts=o)
    assert st == -2 and "128" in msg
    st, msg, _ = _forward(lib, opts=o, ws_bytes=16)
    assert st == -5


def test_measured_gate_table_is_generated_from_the_profiles():
    """csrc/gate_table.inc is exactly what tune_gate.py --emit makes from the committed sweeps
    (nobody edited it by hand, and no sweep was left out)."""
    from block_fp8_mixture_top_amd import tune_gate as TG

    inc, _ = TG.emit_text()
    with open(TG.TABLE) as f:
        assert f.read() == inc


def test_measured_gate_follows_its_table(lib):
    """For every measured shape, select_path with use_measured_gate picks, at each swept T,
    the path the table gives there, and at the geometric-mean boundaries the right side."""
    import glob
    import json

    from block_fp8_mixture_top_amd import tune_gate as TG

    for path in glob.glob(os.path.join(TG.PROFILES, "gate_sweep_E*_H*_I*_k*.json")):
        with open(path) as f:
            prof = json.load(f)
        s = prof["shape"]
        iv = TG.intervals(TG.best_paths(list(prof["rows"].values())))
        for r in prof["rows"].values():
            T = r["T"]
            want = next(p for t, p in iv if T <= t)
            st, info = _path(lib, T, s["E"], s["top_k"], H=s["H"], I=s["I"], use_measured_gate=1)
            assert st == 0 and info.path == TG.PATH_IDS[want], (path, T, info.path, want)
        for (t, p), (_, q) in zip(iv, iv[1:]):
            assert _path(lib, t, s["E"], s["top_k"], H=s["H"], I=s["I"], use_measured_gate=1)[1].path == TG.PATH_IDS[p]
            assert _path(lib, t + 1, s["E"], s["top_k"], H=s["H"], I=s["I"], use_measured_gate=1)[1].path == TG.PATH_IDS[q]


def test_use_measured_gate_must_be_a_flag(lib):
    st, _ = _path(lib, 4, 256, 8, use_measured_gate=2)
    assert st == -1 and b"use_measured_gate" in lib.moe_fp8_block_last_error()
