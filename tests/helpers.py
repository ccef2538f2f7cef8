"""Helpers shared by the tests: host views of generated cases and tolerance checks.

Nothing here computes any part of the method; it converts tensors and measures errors.
"""

from __future__ import annotations

import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# max|err| / max|ref| bar for floating-point outputs against the float64 oracle
REL_TOL = 2e-3


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def case_numpy(case) -> dict:
    return dict(
        hidden=bf16_bits(case.hidden),
        logits=case.logits.detach().cpu().numpy(),
        w13=case.w13.numpy(),
        w2=case.w2.numpy(),
        top_k=case.top_k,
    )


def read_golden(name: str):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def torch_e4m3_table() -> np.ndarray:
    """Decode of all 256 bytes by torch's float8_e4m3fn dtype (a library routine)."""
    c = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return c.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    """Half a bf16 ulp at |x| (8 significant bits)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    return np.where(a > 0, np.ldexp(1.0, ex - 1 - 8), 0.0)


def rel_err(out, ref) -> float:
    ref = np.asarray(ref, dtype=np.float64)
    out = np.asarray(out, dtype=np.float64)
    den = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(out - ref))) / (den if den > 0 else 1.0)


def rel_err_bf16(out, ref) -> float:
    """Error beyond the bf16 output rounding, relative to max|ref|.

    Rounding an exact result to bf16 alone moves it by up to half a bf16 ulp, which is
    up to 2^-8 of the value and so more than the 2e-3 bar; that rounding is subtracted
    before the comparison.
    """
    ref = np.asarray(ref, dtype=np.float64)
    out = np.asarray(out, dtype=np.float64)
    slack = bf16_half_ulp(np.maximum(np.abs(out), np.abs(ref)))
    excess = np.maximum(0.0, np.abs(out - ref) - slack)
    den = float(np.max(np.abs(ref)))
    return float(np.max(excess)) / (den if den > 0 else 1.0)


def bank_numpy(bank, experts=None) -> dict:
    """Host arrays of a bank for the oracle; with ``experts`` only those experts' codes are
    copied (the rest of the host buffer stays zero and is never read by the oracle)."""
    if experts is None:
        return bank.numpy()
    codes = np.zeros(bank.codes.numel(), dtype=np.uint8)
    st = bank.expert_stride_bytes
    for e in sorted(set(int(x) for x in experts)):
        codes[e * st:(e + 1) * st] = bank.codes[e * st:(e + 1) * st].cpu().numpy()
    if bank.scale_dtype == "bf16":
        scales = bank.scales.cpu().view(torch.int16).numpy().view(np.uint16)
    else:
        scales = bank.scales.cpu().numpy()
    d = dict(codes=codes, scales=scales, scale_dtype=bank.scale_dtype, E=bank.E, N=bank.N, K=bank.K,
             expert_stride_bytes=st, scale_row_stride=bank.scale_row_stride,
             scale_expert_stride=bank.scale_expert_stride,
             bias=None if getattr(bank, "bias", None) is None else bank.bias.cpu().numpy())
    return d


def fp8_ulp_diff(a, b) -> np.ndarray:
    """|a - b| in units of the e4m3 spacing at max(|a|, |b|), elementwise.

    The e4m3 spacing at a magnitude v is 2^(floor(log2 v) - 3) for normal values and the
    subnormal step 2^-9 below 2^-6 (OCP e4m3fn: 3 mantissa bits, bias 7). This is the
    unit of the gaudi-cookbook fp8-moe-gather verify mode, which runs two paths and reports
    differences above 2 fp8 ulps.
    """
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    m = np.maximum(np.abs(a), np.abs(b))
    _, ex = np.frexp(np.where(m > 0, m, 1.0))  # m = f * 2^ex with f in [0.5, 1)
    step = np.where(m >= 2.0 ** -6, np.ldexp(1.0, ex - 1 - 3), 2.0 ** -9)
    return np.abs(a - b) / step
