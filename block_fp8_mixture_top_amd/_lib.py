"""ctypes view of libmoe_fp8_block.so: the structs and signatures of include/moe_fp8_block.h."""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_fp8_block.so")

STATIC_WORKSPACE_BYTES = 64 << 20  # MOE_FP8_BLOCK_STATIC_WORKSPACE_BYTES
ABI_VERSION = 5  # MOE_FP8_BLOCK_ABI_VERSION of the header this binding mirrors

MOE_OK = 0
STATUS_NAMES = {
    0: "MOE_OK",
    -1: "MOE_ERR_ARG",
    -2: "MOE_ERR_UNSUPPORTED",
    -3: "MOE_ERR_STRIDE",
    -4: "MOE_ERR_ALIGN",
    -5: "MOE_ERR_WORKSPACE",
    -6: "MOE_ERR_HIP",
}
MOE_F32, MOE_BF16 = 0, 1
PATH_AUTO, PATH_GATHER, PATH_STREAM, PATH_MFMA = 0, 1, 2, 3
PATH_NAMES = {PATH_AUTO: "auto", PATH_GATHER: "gather", PATH_STREAM: "stream", PATH_MFMA: "mfma"}
ACT_PATH, ACT_ROW_FP8, ACT_GROUP_FP8, ACT_GROUP_FP8_W8A8 = 0, 1, 2, 3
KERNEL_NAMES = {1: "route", 2: "sort", 3: "quant", 4: "hquant", 5: "gemm1", 6: "gemm2", 7: "combine"}
EXPORTS = [
    "moe_fp8_block_abi_version",
    "moe_fp8_block_last_error",
    "moe_fp8_block_default_opts",
    "moe_fp8_block_select_path",
    "moe_fp8_block_route_workspace_size",
    "moe_fp8_block_route",
    "moe_fp8_block_workspace_size",
    "moe_fp8_block_forward",
    "moe_fp8_block_forward_timed",
    "moe_fp8_block_forward_static",
    "moe_fp8_block_mfma_up",
    "moe_fp8_block_mfma_down",
    "moe_fp8_block_mfma_up_groups",
    "moe_fp8_block_mfma_down_groups",
    "moe_fp8_block_quantize_rows",
    "moe_fp8_block_quantize_groups",
    "moe_fp8_block_decode_e4m3",
    "moe_fp8_block_decode_e4m3_paths",
    "moe_fp8_block_encode_e4m3",
]


class Bank(ctypes.Structure):
    _fields_ = [
        ("codes", ctypes.c_void_p),
        ("expert_stride_bytes", ctypes.c_int64),
        ("scales", ctypes.c_void_p),
        ("scale_dtype", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("scale_row_stride", ctypes.c_int64),
        ("scale_expert_stride", ctypes.c_int64),
        ("bias", ctypes.c_void_p),
    ]


class Opts(ctypes.Structure):
    _fields_ = [
        ("gate_ratio", ctypes.c_float),
        ("force_path", ctypes.c_int32),
        ("mfma_min_tokens_per_expert", ctypes.c_int32),
        ("act_mode", ctypes.c_int32),
        ("use_measured_gate", ctypes.c_int32),
    ]


class RunInfo(ctypes.Structure):
    _fields_ = [
        ("path", ctypes.c_int32),
        ("act_mode", ctypes.c_int32),
        ("slots", ctypes.c_int32),
        ("kernels", ctypes.c_int32),
    ]


class MoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t

_SIGS = {
    "moe_fp8_block_abi_version": (_I, []),
    "moe_fp8_block_last_error": (ctypes.c_char_p, []),
    "moe_fp8_block_default_opts": (_I, [ctypes.POINTER(Opts)]),
    "moe_fp8_block_select_path": (_I, [_I, _I, _I, _I, _I, ctypes.POINTER(Opts), ctypes.POINTER(RunInfo)]),
    "moe_fp8_block_route_workspace_size": (_SZ, [_I, _I, _I]),
    "moe_fp8_block_route": (_I, [_P, _I, _I, _I, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_fp8_block_workspace_size": (_SZ, [_I, _I, _I, _I, _I, ctypes.POINTER(Opts)]),
    "moe_fp8_block_forward": (
        _I,
        [_P, _P, ctypes.POINTER(Bank), ctypes.POINTER(Bank), _I, _I, _I, _I, _I, _P, _I, _P, _SZ, _P, _P,
         ctypes.POINTER(Opts), ctypes.POINTER(RunInfo), _P],
    ),
    "moe_fp8_block_forward_timed": (
        _I,
        [_P, _P, ctypes.POINTER(Bank), ctypes.POINTER(Bank), _I, _I, _I, _I, _I, _P, _I, _P, _SZ, _P, _P,
         ctypes.POINTER(Opts), ctypes.POINTER(RunInfo), _P, ctypes.POINTER(ctypes.c_void_p), _I,
         ctypes.POINTER(ctypes.c_int32)],
    ),
    "moe_fp8_block_forward_static": (
        _I,
        [_P, _P, ctypes.POINTER(Bank), ctypes.POINTER(Bank), _I, _I, _I, _I, _I, _P, _I, _P, _P,
         ctypes.POINTER(Opts), ctypes.POINTER(RunInfo), _P],
    ),
    "moe_fp8_block_mfma_up": (_I, [_P, _P, ctypes.POINTER(Bank), _I, _I, _I, _I, _I, _P, _P, _SZ, _P]),
    "moe_fp8_block_mfma_down": (_I, [_P, _P, ctypes.POINTER(Bank), _I, _I, _I, _I, _I, _P, _I, _P, _SZ, _P]),
    "moe_fp8_block_mfma_up_groups": (_I, [_P, _P, ctypes.POINTER(Bank), _I, _I, _I, _I, _I, _P, _P, _P, _SZ, _P]),
    "moe_fp8_block_mfma_down_groups": (
        _I, [_P, _P, _P, ctypes.POINTER(Bank), _I, _I, _I, _I, _I, _P, _I, _P, _SZ, _P]),
    "moe_fp8_block_quantize_rows": (_I, [_P, _I, _I, _P, _P, _P]),
    "moe_fp8_block_quantize_groups": (_I, [_P, _I, _I, _P, _P, _P]),
    "moe_fp8_block_decode_e4m3": (_I, [_P, _P, ctypes.c_int64, _P]),
    "moe_fp8_block_decode_e4m3_paths": (_I, [_P, _P, ctypes.c_int64, _P]),
    "moe_fp8_block_encode_e4m3": (_I, [_P, _P, ctypes.c_int64, _P]),
}

_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the library once; refuse a missing or stale build loudly."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python -m block_fp8_mixture_top_amd.build`; "
            "there is no fallback implementation"
        )
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    got = lib.moe_fp8_block_abi_version()
    if got != ABI_VERSION:
        raise ImportError(f"{path} has ABI version {got}, this binding expects {ABI_VERSION}; rebuild it")
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != MOE_OK:
        msg = _lib.moe_fp8_block_last_error().decode() if _lib is not None else ""
        raise MoeError(status, msg)
