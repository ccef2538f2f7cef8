"""The Python binding's host-side checks of bank extents: a bank whose tensors are too
small for the shapes a call reads is refused before anything is launched (the C ABI sees
raw pointers and cannot check extents itself)."""

import dataclasses

import pytest
import torch

import block_fp8_mixture_top_amd as M
import workloads as W


def _bank():
    # E=4 experts of [N=256, K=384] codes, bf16 scales with padded rows (3 -> 8 columns)
    return W.make_bank(4, 256, 384, kind="uniform", scale_dtype=torch.bfloat16, pad="row16", seed=1,
                       tensor_id=1, bias_std=0.1)


def test_extents_accept_a_whole_bank():
    M.check_bank_extents(_bank(), 4, 256, 384)


def test_extents_accept_a_bank_trimmed_to_its_unpadded_extent():
    b = _bank()
    last_codes = 3 * b.expert_stride_bytes + 256 * 384
    last_scales = 3 * b.scale_expert_stride + (2 - 1) * b.scale_row_stride + 3
    b = dataclasses.replace(b, codes=b.codes[:last_codes], scales=b.scales[:last_scales])
    M.check_bank_extents(b, 4, 256, 384)


@pytest.mark.parametrize("what", ["codes", "scales", "bias"])
def test_extents_refuse_one_element_short(what):
    b = _bank()
    need = {"codes": 3 * b.expert_stride_bytes + 256 * 384,
            "scales": 3 * b.scale_expert_stride + b.scale_row_stride + 3,
            "bias": 4 * 256}[what]
    short = dataclasses.replace(b, **{what: getattr(b, what).reshape(-1)[:need - 1]})
    with pytest.raises(ValueError, match=what):
        M.check_bank_extents(short, 4, 256, 384)


@pytest.mark.parametrize("E,N,K", [(5, 256, 384), (4, 512, 384), (4, 256, 256)])
def test_extents_refuse_shapes_the_bank_does_not_have(E, N, K):
    with pytest.raises(ValueError):
        M.check_bank_extents(_bank(), E, N, K)


def test_extents_refuse_small_strides():
    b = dataclasses.replace(_bank(), expert_stride_bytes=256 * 384 - 16)
    with pytest.raises(ValueError, match="strides"):
        M.check_bank_extents(b, 4, 256, 384)
    b = dataclasses.replace(_bank(), scale_row_stride=2)
    with pytest.raises(ValueError, match="strides"):
        M.check_bank_extents(b, 4, 256, 384)


@pytest.mark.gpu
def test_forward_refuses_mismatched_banks_before_launch():
    """forward() raises for banks that do not fit the call, and nothing reaches the GPU."""
    dev = torch.device("cuda:0")
    c = W.make_case("tiny", T=2, seed=3).to(dev)
    torch.cuda.synchronize()
    bad = [
        (dataclasses.replace(c.w13, codes=c.w13.codes[:-1]), c.w2),  # last expert short
        (c.w13, dataclasses.replace(c.w2, scales=c.w2.scales[:-1])),  # last scale missing
        (dataclasses.replace(c.w13, K=c.H // 2), c.w2),  # a bank of another shape
        (c.w13, dataclasses.replace(c.w2, codes=c.w2.codes.cpu())),  # bank on the host
    ]
    for w13, w2 in bad:
        with pytest.raises((ValueError, TypeError)):
            M.forward(c.hidden, c.logits, w13, w2, c.top_k, out_dtype=torch.float32)
    with pytest.raises(ValueError):  # logits for more experts than the banks hold
        M.forward(c.hidden, torch.zeros((2, c.E + 1), device=dev), c.w13, c.w2, c.top_k)
    torch.cuda.synchronize()
