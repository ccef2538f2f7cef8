"""Seeded generators for the synthetic block-FP8 MoE workloads.

Every tensor is drawn from a ``torch.Generator`` seeded from (workload seed, tensor id,
expert), so a bank can be rebuilt expert by expert and the same call on the same device
always returns the same bytes. Values depend on the device the generator runs on (the
CPU and GPU random streams differ); callers hand the oracle host copies of exactly the
tensors they give the library.

What is drawn follows the workloads the pages describe (FreeToken PR #662, "serve
block-fp8 experts on the cpu and hybrid backends": row-major fp8-e4m3 banks, one scale
per 128x128 block, scale rows padded to 16 bytes) at the sizes of the five workloads:

* ``tiny``    E=8,   H=256,  I=128,  top_k=2: codes uniform over the 254 finite e4m3
  codes (both signs, subnormals included), fp32 block scales log-uniform in
  [2^-10, 2^-6], logits N(0,1), fp32 output.
* ``decode``  E=256, H=2048, I=512,  top_k=8: weights N(0, 0.02) quantised per 128x128
  block with bf16 scales, scale rows padded to 16 bytes, logits N(0, 1.5), bf16 output.
* ``sweep``   the ``decode`` banks with Zipf(1.1) expert popularity (Gumbel top-k).
* ``large``   E=256, H=7168, I=2048, top_k=8: fp32 block scales, explicit row stride.
* ``prefill`` the ``decode`` banks with uniform logits (about T*k/E tokens per expert).

Quantising the drawn weights to e4m3 codes uses torch's own ``float8_e4m3fn`` cast: it
only makes inputs and shares nothing with the code under test.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

BLOCK = 128
E4M3_FINITE_MAX = 448.0

SHAPES = {
    "tiny": dict(E=8, H=256, I=128, top_k=2),
    "decode": dict(E=256, H=2048, I=512, top_k=8),
    "sweep": dict(E=256, H=2048, I=512, top_k=8),
    "large": dict(E=256, H=7168, I=2048, top_k=8),
    "prefill": dict(E=256, H=2048, I=512, top_k=8),
}

DEFAULT_T = {"tiny": 4, "decode": 1, "sweep": 12, "large": 1, "prefill": 4096}

# workloads with the same family number share their banks
_BANK_FAMILY = {"tiny": 1, "decode": 2, "sweep": 2, "prefill": 2, "large": 3}

# tensor ids mixed into the seeds
_TID_W13, _TID_W2, _TID_HIDDEN, _TID_LOGITS, _TID_PERM = 1, 2, 3, 4, 5
_TID_BIAS = 6  # added to a bank's tensor id for its MLP bias


def _seed(*parts: int) -> int:
    h = 0x9E3779B1
    for p in parts:
        h = (h * 1_000_003 + int(p) + 0x7F4A7C15) % (1 << 61)
    return h % (1 << 62)


def _gen(device, *parts: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*parts))
    return g


def finite_e4m3_codes() -> torch.Tensor:
    """The 254 byte values that are finite in OCP e4m3fn (all but 0x7F and 0xFF)."""
    c = torch.arange(256, dtype=torch.int32)
    return c[(c & 0x7F) != 0x7F].to(torch.uint8)


def scale_cols_padded(rows: int, cols: int, elem_bytes: int, rule: str) -> int:
    """Trailing dimension of a padded scale bank.

    ``row16``: each scale row is padded to a 16-byte multiple.
    ``slab16``: the trailing dimension grows until one expert's rows*cols*elem_bytes is a
    16-byte multiple (FreeToken PR #662, commit "honor padded fp8 scale strides": 20x5
    bf16 = 200 B grows to 20x6).
    ``none``: no padding.
    """
    if rule == "none":
        return cols
    if rule == "row16":
        per = 16 // elem_bytes
        return -(-cols // per) * per
    if rule == "slab16":
        c = cols
        while (rows * c * elem_bytes) % 16:
            c += 1
        return c
    raise ValueError(f"unknown padding rule {rule!r}")


@dataclasses.dataclass
class FP8Bank:
    """One fp8-e4m3 weight bank: E experts of [N, K] codes, K contiguous per row.

    ``codes`` is flat uint8 with expert e at ``e*expert_stride_bytes``; ``scales`` is flat
    (bfloat16 or float32) with the scale of block (n//128, k//128) of expert e at
    ``e*scale_expert_stride + (n//128)*scale_row_stride + k//128``.
    """

    codes: torch.Tensor
    scales: torch.Tensor
    E: int
    N: int
    K: int
    expert_stride_bytes: int
    scale_row_stride: int
    scale_expert_stride: int
    bias: Optional[torch.Tensor] = None  # float32 [E, N] MLP bias (rows as the codes' rows), or None

    @property
    def scale_dtype(self) -> str:
        return "bf16" if self.scales.dtype == torch.bfloat16 else "f32"

    @property
    def scale_rows(self) -> int:
        return -(-self.N // BLOCK)

    @property
    def scale_cols(self) -> int:
        return -(-self.K // BLOCK)

    @property
    def expert_bytes(self) -> int:
        """Algorithmic bytes of one expert: its codes plus its unpadded scales."""
        esz = 2 if self.scale_dtype == "bf16" else 4
        return self.N * self.K + self.scale_rows * self.scale_cols * esz

    def to(self, device) -> "FP8Bank":
        return dataclasses.replace(self, codes=self.codes.to(device), scales=self.scales.to(device),
                                   bias=None if self.bias is None else self.bias.to(device))

    def numpy(self) -> dict:
        """Host arrays for the oracle: codes uint8, scales as uint16 bf16 bits or float32."""
        codes = self.codes.cpu().numpy()
        if self.scale_dtype == "bf16":
            scales = self.scales.cpu().view(torch.int16).numpy().view(np.uint16)
        else:
            scales = self.scales.cpu().numpy()
        return dict(
            codes=codes,
            scales=scales,
            scale_dtype=self.scale_dtype,
            E=self.E,
            N=self.N,
            K=self.K,
            expert_stride_bytes=self.expert_stride_bytes,
            scale_row_stride=self.scale_row_stride,
            scale_expert_stride=self.scale_expert_stride,
            bias=None if self.bias is None else self.bias.cpu().numpy(),
        )


def make_bank(
    E: int,
    N: int,
    K: int,
    *,
    kind: str,
    scale_dtype: torch.dtype,
    pad: str,
    seed: int,
    tensor_id: int,
    device="cpu",
    code_pad_bytes: int = 0,
    pad_fill: float = float("nan"),
    std: float = 0.02,
    experts=None,
    bias_std: Optional[float] = None,
) -> FP8Bank:
    """Draw an fp8 block bank expert by expert.

    kind ``uniform``: codes uniform over the finite e4m3 codes, scales 2^U(-10,-6).
    kind ``subnormal``: codes uniform over the 14 nonzero subnormal codes (+-1..7 * 2^-9),
    every scale 1.
    kind ``normal``: weights N(0, std) quantised per 128x128 block with scale
    amax/448 (stored in ``scale_dtype``) and torch's e4m3fn cast of weight/scale.
    Scale padding holds ``pad_fill`` (NaN by default, so a reader of padding sees it);
    ``code_pad_bytes`` of 0x7F (NaN codes) follow each expert's codes. With ``experts``
    only those experts are drawn; the others keep NaN codes and NaN scales, so any read
    of an expert that should not be read poisons the result. With ``bias_std`` each expert
    also gets a float32 MLP bias row drawn from N(0, bias_std) (NaN for undrawn experts).
    """
    esz = 2 if scale_dtype == torch.bfloat16 else 4
    rows, cols = -(-N // BLOCK), -(-K // BLOCK)
    rstride = scale_cols_padded(rows, cols, esz, pad)
    sstride = rows * rstride
    estride = N * K + code_pad_bytes
    assert estride % 16 == 0, "expert stride must keep 16-byte alignment"
    codes = torch.full((E, estride), 0x7F, dtype=torch.uint8, device=device)
    scales = torch.full((E, rows, rstride), pad_fill, dtype=scale_dtype, device=device)
    finite = finite_e4m3_codes().to(device)
    for e in range(E) if experts is None else sorted(set(int(x) for x in experts)):
        g = _gen(device, seed, tensor_id, e)
        if kind == "uniform":
            idx = torch.randint(0, finite.numel(), (N * K,), generator=g, device=device)
            codes[e, : N * K] = finite[idx]
            u = torch.rand((rows, cols), generator=g, device=device, dtype=torch.float64)
            scales[e, :, :cols] = torch.exp2(-10.0 + 4.0 * u).to(scale_dtype)
        elif kind == "subnormal":
            sub = torch.tensor([m | sgn for sgn in (0x00, 0x80) for m in range(1, 8)], dtype=torch.uint8,
                               device=device)
            idx = torch.randint(0, sub.numel(), (N * K,), generator=g, device=device)
            codes[e, : N * K] = sub[idx]
            scales[e, :, :cols] = 1.0
        elif kind == "normal":
            w = torch.randn((N, K), generator=g, device=device, dtype=torch.float32) * std
            wp = torch.zeros((rows * BLOCK, cols * BLOCK), dtype=torch.float32, device=device)
            wp[:N, :K] = w
            blk = wp.view(rows, BLOCK, cols, BLOCK)
            amax = blk.abs().amax(dim=(1, 3))
            s = (amax / E4M3_FINITE_MAX).to(scale_dtype)
            sf = s.to(torch.float32)
            sf = torch.where(sf > 0, sf, torch.ones_like(sf))
            q = (blk / sf[:, None, :, None]).clamp(-E4M3_FINITE_MAX, E4M3_FINITE_MAX)
            q8 = q.to(torch.float8_e4m3fn).view(torch.uint8).view(rows * BLOCK, cols * BLOCK)
            codes[e, : N * K] = q8[:N, :K].reshape(-1)
            scales[e, :, :cols] = s
        else:
            raise ValueError(f"unknown bank kind {kind!r}")
    bias = None
    if bias_std is not None:
        bias = torch.full((E, N), float("nan"), dtype=torch.float32, device=device)
        for e in range(E) if experts is None else sorted(set(int(x) for x in experts)):
            g = _gen(device, seed, tensor_id + _TID_BIAS, e)
            bias[e] = torch.randn((N,), generator=g, device=device, dtype=torch.float32) * bias_std
    return FP8Bank(
        codes=codes.reshape(-1),
        scales=scales.reshape(-1),
        E=E,
        N=N,
        K=K,
        expert_stride_bytes=estride,
        scale_row_stride=rstride,
        scale_expert_stride=sstride,
        bias=bias,
    )


def make_hidden(T: int, H: int, seed: int, device="cpu") -> torch.Tensor:
    """Hidden states, bf16 drawn from N(0, 1)."""
    g = _gen(device, seed, _TID_HIDDEN)
    return torch.randn((T, H), generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


def make_logits(T: int, E: int, kind: str, seed: int, device="cpu", std: float = 1.0, alpha: float = 1.1) -> torch.Tensor:
    """Router logits, fp32.

    ``normal``: N(0, std^2). ``uniform``: U(0, 1). ``zipf``: log p_e + Gumbel(0,1) with
    p over a seeded permutation of experts proportional to rank^-alpha, so that each
    token's top-k set is a draw without replacement from that skewed popularity.
    """
    g = _gen(device, seed, _TID_LOGITS)
    if kind == "normal":
        return torch.randn((T, E), generator=g, device=device, dtype=torch.float32) * std
    if kind == "uniform":
        return torch.rand((T, E), generator=g, device=device, dtype=torch.float32)
    if kind == "zipf":
        gp = _gen("cpu", seed, _TID_PERM)
        rank = torch.randperm(E, generator=gp)
        p = torch.arange(1, E + 1, dtype=torch.float64).pow(-alpha)
        p = p / p.sum()
        logp = torch.log(p[rank]).to(torch.float32).to(device)
        u = torch.rand((T, E), generator=g, device=device, dtype=torch.float32)
        u = u.clamp(1e-12, 1.0 - 1e-7)
        gumbel = -torch.log(-torch.log(u))
        return logp[None, :] + gumbel
    raise ValueError(f"unknown logits kind {kind!r}")


@dataclasses.dataclass
class MoECase:
    name: str
    T: int
    E: int
    H: int
    I: int
    top_k: int
    hidden: torch.Tensor  # [T, H] bfloat16
    logits: torch.Tensor  # [T, E] float32
    w13: FP8Bank  # N = 2I (gate rows 0..I-1, up rows I..2I-1), K = H
    w2: FP8Bank  # N = H, K = I
    out_dtype: torch.dtype

    def to(self, device) -> "MoECase":
        return dataclasses.replace(
            self,
            hidden=self.hidden.to(device),
            logits=self.logits.to(device),
            w13=self.w13.to(device),
            w2=self.w2.to(device),
        )


def make_banks(name: str, seed: int, device="cpu", *, E: Optional[int] = None, H: Optional[int] = None,
               I: Optional[int] = None, pad: Optional[str] = None, code_pad_bytes: int = 0,
               scale_dtype: Optional[torch.dtype] = None, experts=None, bias_std: Optional[float] = None,
               kind: Optional[str] = None) -> tuple:
    """The (w13, w2) banks of a workload; shapes (and the bank kind) may be overridden for tests."""
    shp = dict(SHAPES[name])
    E = E or shp["E"]
    H = H or shp["H"]
    I = I or shp["I"]
    if name == "tiny":
        kind_, sdt, rule = "uniform", torch.float32, "none"
    elif name == "large":
        kind_, sdt, rule = "normal", torch.float32, "row16"
    else:
        kind_, sdt, rule = "normal", torch.bfloat16, "row16"
    if kind is not None:
        kind_ = kind
    if scale_dtype is not None:
        sdt = scale_dtype
    if pad is not None:
        rule = pad
    # the decode, sweep and prefill workloads share one set of banks
    bank_seed = _seed(seed, _BANK_FAMILY[name])
    w13 = make_bank(E, 2 * I, H, kind=kind_, scale_dtype=sdt, pad=rule, seed=bank_seed,
                    tensor_id=_TID_W13, device=device, code_pad_bytes=code_pad_bytes, experts=experts,
                    bias_std=bias_std)
    w2 = make_bank(E, H, I, kind=kind_, scale_dtype=sdt, pad=rule, seed=bank_seed,
                   tensor_id=_TID_W2, device=device, code_pad_bytes=code_pad_bytes, experts=experts,
                   bias_std=bias_std)
    return w13, w2


def make_case(name: str, T: Optional[int] = None, seed: int = 0, device="cpu", banks=None, **bank_kw) -> MoECase:
    """A whole workload: hidden, logits and both banks, all from ``seed``."""
    shp = dict(SHAPES[name])
    for k in ("E", "H", "I"):
        if bank_kw.get(k):
            shp[k] = bank_kw[k]
    if "top_k" in bank_kw:
        shp["top_k"] = bank_kw.pop("top_k")
    T = DEFAULT_T[name] if T is None else T
    E, H, I, k = shp["E"], shp["H"], shp["I"], shp["top_k"]
    if banks is None:
        banks = make_banks(name, seed, device, **bank_kw)
    w13, w2 = banks
    hidden = make_hidden(T, H, _seed(seed, T, 11), device)
    if name == "tiny":
        logits = make_logits(T, E, "normal", _seed(seed, T, 12), device, std=1.0)
    elif name == "decode":
        logits = make_logits(T, E, "normal", _seed(seed, T, 12), device, std=1.5)
    elif name == "sweep":
        logits = make_logits(T, E, "zipf", _seed(seed, T, 12), device, alpha=1.1)
    elif name == "large":
        logits = make_logits(T, E, "normal", _seed(seed, T, 12), device, std=1.0)
    elif name == "prefill":
        logits = make_logits(T, E, "uniform", _seed(seed, T, 12), device)
    else:
        raise ValueError(name)
    out_dtype = torch.float32 if name == "tiny" else torch.bfloat16
    return MoECase(name=name, T=T, E=E, H=H, I=I, top_k=k, hidden=hidden, logits=logits,
                   w13=w13, w2=w2, out_dtype=out_dtype)


def bank_bytes_touched(bank: FP8Bank, experts) -> int:
    """Algorithmic bytes of the listed distinct experts."""
    return len(set(int(e) for e in experts)) * bank.expert_bytes


__all__ = [
    "SHAPES", "DEFAULT_T", "FP8Bank", "MoECase", "make_bank", "make_banks", "make_case",
    "make_hidden", "make_logits", "scale_cols_padded", "finite_e4m3_codes", "bank_bytes_touched",
]
