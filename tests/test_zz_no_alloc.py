"""moe_fp8_block_forward_static, the entry point that allocates nothing (its workspace is a
static device array of the library): through the C ABI, against moe_fp8_block_forward on
the same inputs, bit for bit (every path is deterministic), on calls in a row whose second
input is smaller; and the rejection of a call too large for the static workspace."""

import numpy as np
import pytest
import torch

import block_fp8_mixture_top_amd as M
import workloads as W
from block_fp8_mixture_top_amd import _lib as L

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _both(c, **opts):
    ref, info_ref = M.forward(c.hidden, c.logits, c.w13, c.w2, c.top_k, out_dtype=torch.float32,
                              return_routing=True, **opts)
    out = torch.full_like(ref, float("nan"))
    ids = torch.full((c.T, c.top_k), -1, dtype=torch.int32, device=DEV)
    w = torch.full((c.T, c.top_k), float("nan"), dtype=torch.float32, device=DEV)
    info = M.forward_static(c.hidden, c.logits, c.w13, c.w2, c.top_k, out, ids=ids, weights=w, **opts)
    torch.cuda.synchronize()
    return ref, info_ref, out, info, ids, w


@pytest.mark.parametrize("path", ["gather", "stream", "mfma"])
def test_static_forward_equals_forward_on_two_calls(path):
    banks = W.make_banks("decode", seed=1, device=DEV)
    fp = {"gather": M.PATH_GATHER, "stream": M.PATH_STREAM, "mfma": M.PATH_MFMA}[path]
    for T in (96, 5):  # the second call is smaller and reuses the array the first one wrote
        c = W.make_case("sweep", T=T, seed=30 + T, device=DEV, banks=banks)
        print(f"[case] static forward {path} T={T}", flush=True)
        assert M.workspace_size(T, c.E, c.H, c.I, c.top_k, force_path=fp) <= L.STATIC_WORKSPACE_BYTES
        ref, info_ref, out, info, ids, w = _both(c, force_path=fp)
        assert info["path"] == info_ref["path"] == path and info["kernels"] == info_ref["kernels"]
        assert torch.equal(out, ref)
        assert torch.equal(ids, info_ref["ids"]) and torch.equal(w, info_ref["weights"])


def test_static_forward_decode_and_tiny():
    """The auto path at the decode workload (bf16 out) and the tiny workload, in a row."""
    c = W.make_case("decode", T=1, seed=1, device=DEV)
    print("[case] static forward decode T=1", flush=True)
    ref, _ = M.forward(c.hidden, c.logits, c.w13, c.w2, c.top_k, out_dtype=torch.bfloat16)
    out = torch.empty_like(ref)
    info = M.forward_static(c.hidden, c.logits, c.w13, c.w2, c.top_k, out)
    torch.cuda.synchronize()
    assert info["path"] == "gather" and torch.equal(out, ref)
    c = W.make_case("tiny", T=4, seed=2).to(DEV)
    print("[case] static forward tiny T=4", flush=True)
    ref, _ = M.forward(c.hidden, c.logits, c.w13, c.w2, c.top_k, out_dtype=torch.float32)
    out = torch.empty_like(ref)
    M.forward_static(c.hidden, c.logits, c.w13, c.w2, c.top_k, out)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


def test_static_forward_refuses_a_call_larger_than_its_array():
    banks = W.make_banks("decode", seed=1, device=DEV)
    c = W.make_case("prefill", T=4096, seed=3, device=DEV, banks=banks)
    need = M.workspace_size(c.T, c.E, c.H, c.I, c.top_k)
    assert need > L.STATIC_WORKSPACE_BYTES
    out = torch.full((c.T, c.H), 7.0, dtype=torch.float32, device=DEV)
    print("[case] static forward too large", flush=True)
    with pytest.raises(M.MoeError) as ex:
        M.forward_static(c.hidden, c.logits, c.w13, c.w2, c.top_k, out)
    assert ex.value.status == -5 and "static workspace" in str(ex.value)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())  # nothing ran
