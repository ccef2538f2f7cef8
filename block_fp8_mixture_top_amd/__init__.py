"""Block-FP8 mixture-of-experts expert computation on MI355X (gfx950).

A thin binding of the C ABI in include/moe_fp8_block.h: it checks tensor dtypes and
devices, passes raw device pointers and torch's current HIP stream, and raises MoeError
on a non-zero status. Every step of the computation runs in the library's HIP kernels;
this module only marshals arguments. PyTorch supplies device memory and streams.
"""

from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib as L
from ._lib import (  # noqa: F401
    ACT_GROUP_FP8,
    ACT_GROUP_FP8_W8A8,
    ACT_PATH,
    ACT_ROW_FP8,
    MOE_BF16,
    MOE_F32,
    PATH_AUTO,
    PATH_GATHER,
    PATH_MFMA,
    PATH_NAMES,
    PATH_STREAM,
    MoeError,
)

__all__ = [
    "abi_version", "lib", "make_opts", "bank_struct", "check_bank_extents", "select_path", "route_workspace_size", "route", "workspace_size",
    "forward", "forward_static", "mfma_up", "mfma_down", "mfma_up_groups", "mfma_down_groups", "quantize_rows", "quantize_groups", "decode_e4m3", "decode_e4m3_paths", "encode_e4m3", "MoeError", "PATH_AUTO", "PATH_GATHER",
    "PATH_STREAM", "PATH_MFMA", "PATH_NAMES", "ACT_PATH", "ACT_ROW_FP8", "ACT_GROUP_FP8",
    "ACT_GROUP_FP8_W8A8",
]


def lib() -> ctypes.CDLL:
    return L.load()


def abi_version() -> int:
    return lib().moe_fp8_block_abi_version()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def make_opts(force_path: Optional[int] = None, gate_ratio: Optional[float] = None,
              mfma_min_tokens_per_expert: Optional[int] = None, act_mode: Optional[int] = None,
              use_measured_gate: Optional[bool] = None) -> L.Opts:
    o = L.Opts()
    L.check(lib().moe_fp8_block_default_opts(ctypes.byref(o)))
    if use_measured_gate is not None:
        o.use_measured_gate = int(bool(use_measured_gate))
    if act_mode is not None:
        o.act_mode = int(act_mode)
    if force_path is not None:
        o.force_path = int(force_path)
    if gate_ratio is not None:
        o.gate_ratio = float(gate_ratio)
    if mfma_min_tokens_per_expert is not None:
        o.mfma_min_tokens_per_expert = int(mfma_min_tokens_per_expert)
    return o


def _info_dict(info: L.RunInfo) -> dict:
    return dict(path=PATH_NAMES[info.path], path_id=info.path, act_mode=info.act_mode, slots=info.slots,
                kernels=info.kernels)


def select_path(T: int, E: int, H: int, I: int, top_k: int, **opts) -> dict:
    """The path forward would take for these sizes (host only)."""
    info = L.RunInfo()
    o = make_opts(**opts)
    L.check(lib().moe_fp8_block_select_path(T, E, H, I, top_k, ctypes.byref(o), ctypes.byref(info)))
    return _info_dict(info)


def check_bank_extents(bank, E: int, N: int, K: int) -> None:
    """Raise ValueError unless the bank's tensors hold every element a call reading E
    experts of [N, K] codes may touch (see bank_struct). Host-only; reads shapes, not data."""
    for name, want in (("E", E), ("N", N), ("K", K)):
        have = getattr(bank, name, None)
        if have is not None and int(have) != int(want):
            raise ValueError(f"bank has {name}={have}, the call needs {name}={want}")
    es, srow, sexp = int(bank.expert_stride_bytes), int(bank.scale_row_stride), int(bank.scale_expert_stride)
    if es < N * K or srow < -(-K // 128) or sexp < 0:
        raise ValueError(f"bank strides too small for [{N}, {K}] experts (the library reports which)")
    need_codes = (E - 1) * es + N * K
    if bank.codes.numel() < need_codes:
        raise ValueError(f"bank.codes holds {bank.codes.numel()} bytes, {E} experts of [{N}, {K}] with "
                         f"expert stride {es} need {need_codes}")
    need_scales = (E - 1) * sexp + (-(-N // 128) - 1) * srow + -(-K // 128)
    if bank.scales.numel() < need_scales:
        raise ValueError(f"bank.scales holds {bank.scales.numel()} elements, the strides need {need_scales}")
    bias = getattr(bank, "bias", None)
    if bias is not None and bias.numel() < E * N:
        raise ValueError(f"bank.bias holds {bias.numel()} floats, [{E}, {N}] needs {E * N}")


def bank_struct(bank, E: Optional[int] = None, N: Optional[int] = None, K: Optional[int] = None,
                device=None) -> L.Bank:
    """A moe_fp8_bank from an object with codes/scales tensors, the stride fields and an
    optional float32 [E, N] MLP bias (``bias``, None for none).

    With E, N and K (what the call will read: E experts of [N, K] codes), the tensors are
    checked to hold every byte the kernels may read before anything is launched, since the
    C ABI only sees raw pointers: codes at least (E-1)*expert_stride_bytes + N*K bytes,
    scales at least (E-1)*scale_expert_stride + (ceil(N/128)-1)*scale_row_stride +
    ceil(K/128) elements (FreeToken PR #662, commit "honor padded fp8 scale strides": the
    shape check asserts that the unpadded extent is present), a bias at least E*N floats.
    A bank that states its own E, N or K must agree with them.
    """
    _need(bank.codes, "bank.codes", torch.uint8, device)
    if bank.scales.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("bank.scales must be bfloat16 or float32")
    if bank.scales.device != bank.codes.device or not bank.scales.is_contiguous():
        raise ValueError("bank.scales must be contiguous and on the codes' device")
    bias = getattr(bank, "bias", None)
    if bias is not None:
        _need(bias, "bank.bias", torch.float32, bank.codes.device)
    if E is not None:
        check_bank_extents(bank, E, N, K)
    b = L.Bank()
    b.codes = bank.codes.data_ptr()
    b.expert_stride_bytes = int(bank.expert_stride_bytes)
    b.scales = bank.scales.data_ptr()
    b.scale_dtype = L.MOE_BF16 if bank.scales.dtype == torch.bfloat16 else L.MOE_F32
    b.reserved = 0
    b.scale_row_stride = int(bank.scale_row_stride)
    b.scale_expert_stride = int(bank.scale_expert_stride)
    if bias is not None:
        b.bias = bias.data_ptr()
    return b


def route_workspace_size(T: int, E: int, top_k: int) -> int:
    return int(lib().moe_fp8_block_route_workspace_size(T, E, top_k))


def route(logits: torch.Tensor, top_k: int, sort: bool = True, workspace: Optional[torch.Tensor] = None) -> dict:
    """Top-k routing (and the token-to-expert sort) on the GPU."""
    _need(logits, "logits", torch.float32)
    T, E = logits.shape
    dev = logits.device
    ids = torch.empty((T, top_k), dtype=torch.int32, device=dev)
    w = torch.empty((T, top_k), dtype=torch.float32, device=dev)
    res = dict(ids=ids, weights=w)
    counts = offsets = sorted_pairs = None
    nbytes = 0
    if sort:
        counts = torch.empty(E, dtype=torch.int32, device=dev)
        offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
        sorted_pairs = torch.empty(T * top_k, dtype=torch.int32, device=dev)
        nbytes = route_workspace_size(T, E, top_k)
        if workspace is None:
            workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
        res.update(counts=counts, offsets=offsets, sorted_pairs=sorted_pairs)
    L.check(lib().moe_fp8_block_route(
        _ptr(logits), T, E, top_k, _ptr(ids), _ptr(w), _ptr(counts), _ptr(offsets), _ptr(sorted_pairs),
        _ptr(workspace), workspace.numel() if workspace is not None else 0, _stream(logits)))
    return res


def workspace_size(T: int, E: int, H: int, I: int, top_k: int, **opts) -> int:
    o = make_opts(**opts)
    return int(lib().moe_fp8_block_workspace_size(T, E, H, I, top_k, ctypes.byref(o)))


def forward(hidden: torch.Tensor, logits: torch.Tensor, w13, w2, top_k: int, out_dtype=torch.bfloat16,
            out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
            return_routing: bool = False, **opts):
    """The expert computation for T tokens. Returns (out [T, H], info dict).

    w13 / w2 are banks (objects with codes, scales, expert_stride_bytes, scale_row_stride,
    scale_expert_stride, optional bias); opts are force_path, gate_ratio,
    mfma_min_tokens_per_expert and act_mode (ACT_PATH or ACT_GROUP_FP8).
    With return_routing the info dict also holds the ids and weights tensors.
    """
    _need(hidden, "hidden", torch.bfloat16)
    dev = hidden.device
    _need(logits, "logits", torch.float32, dev)
    if hidden.dim() != 2 or logits.dim() != 2:
        raise ValueError("hidden must be [T, H] and logits [T, E]")
    T, H = hidden.shape
    E = logits.shape[1]
    if logits.shape[0] != T:
        raise ValueError("hidden and logits disagree on T")
    I = int(w2.K)
    if out is None:
        out = torch.empty((T, H), dtype=out_dtype, device=dev)
    if out.dtype not in (torch.float32, torch.bfloat16) or tuple(out.shape) != (T, H):
        raise ValueError("out must be [T, H] float32 or bfloat16")
    _need(out, "out", out.dtype, dev)
    o = make_opts(**opts)
    nbytes = int(lib().moe_fp8_block_workspace_size(T, E, H, I, top_k, ctypes.byref(o)))
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, dev)
    b13 = bank_struct(w13, E, 2 * I, H, dev)
    b2 = bank_struct(w2, E, H, I, dev)
    ids = w = None
    if return_routing:
        ids = torch.empty((T, top_k), dtype=torch.int32, device=dev)
        w = torch.empty((T, top_k), dtype=torch.float32, device=dev)
    info = L.RunInfo()
    L.check(lib().moe_fp8_block_forward(
        _ptr(hidden), _ptr(logits), ctypes.byref(b13), ctypes.byref(b2), T, E, H, I, top_k, _ptr(out),
        L.MOE_BF16 if out.dtype == torch.bfloat16 else L.MOE_F32, _ptr(workspace), workspace.numel(),
        _ptr(ids), _ptr(w), ctypes.byref(o), ctypes.byref(info), _stream(hidden)))
    d = _info_dict(info)
    if return_routing:
        d.update(ids=ids, weights=w)
    return out, d


def forward_static(hidden: torch.Tensor, logits: torch.Tensor, w13, w2, top_k: int, out: torch.Tensor,
                   ids: Optional[torch.Tensor] = None, weights: Optional[torch.Tensor] = None, **opts) -> dict:
    """moe_fp8_block_forward_static: the forward with the library's static device workspace
    (no workspace argument, nothing allocated by the call). `out` [T, H] float32 or
    bfloat16 must be given; ids / weights [T, top_k] optional. Returns the info dict."""
    _need(hidden, "hidden", torch.bfloat16)
    dev = hidden.device
    _need(logits, "logits", torch.float32, dev)
    T, H = hidden.shape
    E = logits.shape[1]
    if logits.shape[0] != T:
        raise ValueError("hidden and logits disagree on T")
    I = int(w2.K)
    if out.dtype not in (torch.float32, torch.bfloat16) or tuple(out.shape) != (T, H):
        raise ValueError("out must be [T, H] float32 or bfloat16")
    _need(out, "out", out.dtype, dev)
    for t, name, dt in ((ids, "ids", torch.int32), (weights, "weights", torch.float32)):
        if t is not None:
            _need(t, name, dt, dev)
            if tuple(t.shape) != (T, top_k):
                raise ValueError(f"{name} must be [T, top_k]")
    o = make_opts(**opts)
    b13 = bank_struct(w13, E, 2 * I, H, dev)
    b2 = bank_struct(w2, E, H, I, dev)
    info = L.RunInfo()
    L.check(lib().moe_fp8_block_forward_static(
        _ptr(hidden), _ptr(logits), ctypes.byref(b13), ctypes.byref(b2), T, E, H, I, top_k, _ptr(out),
        L.MOE_BF16 if out.dtype == torch.bfloat16 else L.MOE_F32, _ptr(ids), _ptr(weights), ctypes.byref(o),
        ctypes.byref(info), _stream(hidden)))
    return _info_dict(info)


def mfma_up(hidden: torch.Tensor, logits: torch.Tensor, w13, top_k: int, I: int) -> torch.Tensor:
    """Test export: the MFMA path's first half. Returns h [T*top_k, I] float32, row p for the
    pair at sorted position p."""
    _need(hidden, "hidden", torch.bfloat16)
    dev = hidden.device
    _need(logits, "logits", torch.float32, dev)
    T, H = hidden.shape
    E = logits.shape[1]
    b13 = bank_struct(w13, E, 2 * I, H, dev)
    ws = torch.empty(max(workspace_size(T, E, H, I, top_k, force_path=PATH_MFMA), 1), dtype=torch.uint8, device=dev)
    h = torch.empty((T * top_k, I), dtype=torch.float32, device=dev)
    L.check(lib().moe_fp8_block_mfma_up(_ptr(hidden), _ptr(logits), ctypes.byref(b13), T, E, H, I, top_k, _ptr(h),
                                        _ptr(ws), ws.numel(), _stream(hidden)))
    return h


def mfma_down(h: torch.Tensor, logits: torch.Tensor, w2, top_k: int, H: int, out_dtype=torch.float32) -> torch.Tensor:
    """Test export: the MFMA path's second half on h [T*top_k, I] float32 in sorted-position
    order. Returns out [T, H]."""
    _need(h, "h", torch.float32)
    dev = h.device
    _need(logits, "logits", torch.float32, dev)
    T, E = logits.shape
    I = h.shape[1]
    if h.shape[0] != T * top_k:
        raise ValueError("h must have T*top_k rows")
    b2 = bank_struct(w2, E, H, I, dev)
    ws = torch.empty(max(workspace_size(T, E, H, I, top_k, force_path=PATH_MFMA), 1), dtype=torch.uint8, device=dev)
    out = torch.empty((T, H), dtype=out_dtype, device=dev)
    L.check(lib().moe_fp8_block_mfma_down(_ptr(h), _ptr(logits), ctypes.byref(b2), T, E, H, I, top_k, _ptr(out),
                                          L.MOE_BF16 if out_dtype == torch.bfloat16 else L.MOE_F32, _ptr(ws),
                                          ws.numel(), _stream(h)))
    return out


def mfma_up_groups(hidden: torch.Tensor, logits: torch.Tensor, w13, top_k: int, I: int):
    """Test export: the first half of the group-scaled MFMA path. Returns (h codes [T*top_k,
    I] uint8, h scales [T*top_k, I/128] float32), row p for the pair at sorted position p."""
    _need(hidden, "hidden", torch.bfloat16)
    dev = hidden.device
    _need(logits, "logits", torch.float32, dev)
    T, H = hidden.shape
    E = logits.shape[1]
    b13 = bank_struct(w13, E, 2 * I, H, dev)
    ws = torch.empty(max(workspace_size(T, E, H, I, top_k, force_path=PATH_MFMA, act_mode=ACT_GROUP_FP8), 1),
                     dtype=torch.uint8, device=dev)
    codes = torch.empty((T * top_k, I), dtype=torch.uint8, device=dev)
    scales = torch.empty((T * top_k, max(I // 128, 1)), dtype=torch.float32, device=dev)
    L.check(lib().moe_fp8_block_mfma_up_groups(_ptr(hidden), _ptr(logits), ctypes.byref(b13), T, E, H, I, top_k,
                                               _ptr(codes), _ptr(scales), _ptr(ws), ws.numel(), _stream(hidden)))
    return codes, scales


def mfma_down_groups(codes: torch.Tensor, scales: torch.Tensor, logits: torch.Tensor, w2, top_k: int, H: int,
                     out_dtype=torch.float32) -> torch.Tensor:
    """Test export: the second half of the group-scaled MFMA path on h codes [T*top_k, I]
    uint8 and scales [T*top_k, I/128] float32 in sorted-position order. Returns out [T, H]."""
    _need(codes, "codes", torch.uint8)
    dev = codes.device
    _need(scales, "scales", torch.float32, dev)
    _need(logits, "logits", torch.float32, dev)
    T, E = logits.shape
    I = codes.shape[1]
    if codes.shape[0] != T * top_k or tuple(scales.shape) != (T * top_k, I // 128) or I % 128 != 0:
        raise ValueError("codes must be [T*top_k, I] with I % 128 == 0 and scales [T*top_k, I/128]")
    b2 = bank_struct(w2, E, H, I, dev)
    ws = torch.empty(max(workspace_size(T, E, H, I, top_k, force_path=PATH_MFMA, act_mode=ACT_GROUP_FP8), 1),
                     dtype=torch.uint8, device=dev)
    out = torch.empty((T, H), dtype=out_dtype, device=dev)
    L.check(lib().moe_fp8_block_mfma_down_groups(_ptr(codes), _ptr(scales), _ptr(logits), ctypes.byref(b2), T, E, H,
                                                 I, top_k, _ptr(out),
                                                 L.MOE_BF16 if out_dtype == torch.bfloat16 else L.MOE_F32, _ptr(ws),
                                                 ws.numel(), _stream(codes)))
    return out


def quantize_rows(x: torch.Tensor):
    """Per-row dynamic e4m3 of a bf16 [rows, cols] tensor -> (codes uint8, scales float32)."""
    _need(x, "x", torch.bfloat16)
    rows, cols = x.shape
    codes = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    scales = torch.empty(rows, dtype=torch.float32, device=x.device)
    L.check(lib().moe_fp8_block_quantize_rows(_ptr(x), rows, cols, _ptr(codes), _ptr(scales), _stream(x)))
    return codes, scales


def quantize_groups(x: torch.Tensor):
    """Dynamic e4m3 per (row, 128-column group) of a bf16 [rows, cols] tensor -> (codes
    uint8 [rows, cols], scales float32 [rows, cols/128])."""
    _need(x, "x", torch.bfloat16)
    rows, cols = x.shape
    codes = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    scales = torch.empty((rows, max(cols // 128, 1)), dtype=torch.float32, device=x.device)
    L.check(lib().moe_fp8_block_quantize_groups(_ptr(x), rows, cols, _ptr(codes), _ptr(scales), _stream(x)))
    return codes, scales


def decode_e4m3(codes: torch.Tensor) -> torch.Tensor:
    _need(codes, "codes", torch.uint8)
    out = torch.empty(codes.shape, dtype=torch.float32, device=codes.device)
    L.check(lib().moe_fp8_block_decode_e4m3(_ptr(codes), _ptr(out), codes.numel(), _stream(codes)))
    return out


def decode_e4m3_paths(chunks: torch.Tensor) -> torch.Tensor:
    """Every decode path of the kernels on [n, 16] uint8 chunks of finite codes -> [n, 16, 5]
    float32 (see moe_fp8_block_decode_e4m3_paths)."""
    _need(chunks, "chunks", torch.uint8)
    if chunks.dim() != 2 or chunks.shape[1] != 16:
        raise ValueError("chunks must be [n, 16]")
    out = torch.empty((chunks.shape[0], 16, 5), dtype=torch.float32, device=chunks.device)
    L.check(lib().moe_fp8_block_decode_e4m3_paths(_ptr(chunks), _ptr(out), chunks.shape[0], _stream(chunks)))
    return out


def encode_e4m3(x: torch.Tensor) -> torch.Tensor:
    _need(x, "x", torch.float32)
    out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    L.check(lib().moe_fp8_block_encode_e4m3(_ptr(x), _ptr(out), x.numel(), _stream(x)))
    return out
