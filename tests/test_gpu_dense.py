"""GPU parity of dense coded projections (the one-expert case of the routed
kernels) with the dense export's additive biases: the gate/up bias before
the SwiGLU, the down bias on the output."""
import numpy as np
import pytest
import torch

import oracle
from bit_trellis_quantized_amd import synth
from tests._gpu_util import announce, assert_close, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def escha():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from bit_trellis_quantized_amd import escha as mod
    return mod


@pytest.fixture(scope="module")
def mlp():
    return synth.dense_mlp_tensors(80)


def _dev(escha, M, bias=True):
    gu = escha.Proj(to_dev(M["gu_code"]), to_dev(M["gu_rin"]), to_dev(M["gu_rout"]))
    dn = escha.Proj(to_dev(M["dn_code"]), to_dev(M["dn_rin"]), to_dev(M["dn_rout"]))
    if not bias:
        return escha.DenseMLP(gu, dn)
    return escha.DenseMLP(gu, dn, to_dev(M["gu_bias"]), to_dev(M["dn_bias"]))


@pytest.mark.parametrize("proj,T", [("gu", 1), ("gu", 3), ("dn", 2)])
def test_dense_gemv_with_bias(escha, mlp, proj, T):
    announce(f"dense_gemv {proj} T={T}")
    in_f, out_f, K = (2048, 1024, 2) if proj == "gu" else (512, 2048, 3)
    w = escha.Proj(to_dev(mlp[f"{proj}_code"]), to_dev(mlp[f"{proj}_rin"]), to_dev(mlp[f"{proj}_rout"]))
    bias = mlp[f"{proj}_bias"]
    x = synth.activations(81, T, in_f)
    y = escha.escha_dense_gemv(w, to_dev(x), bias=to_dev(bias)).cpu().numpy()
    ref = oracle.dense_gemv(mlp[f"{proj}_code"][0], mlp[f"{proj}_rin"][0], mlp[f"{proj}_rout"][0], bias,
                            in_f, out_f, K, x)
    assert_close(y, ref, f"dense_gemv {proj} T={T}")


# 1, 7: streaming kernels; 16: small tiles; 40: 128-token tiles (decode entry)
@pytest.mark.parametrize("T", [1, 7, 16, 40])
def test_dense_mlp_decode(escha, mlp, T):
    announce(f"dense_mlp_decode T={T}")
    Md = _dev(escha, mlp)
    x = synth.activations(82, T, synth.HIDDEN)
    h = torch.empty(T, synth.INTER, dtype=torch.float32, device="cuda")
    y = escha.escha_dense_mlp_decode(Md, to_dev(x), inter_out=h)
    ref_y, ref_h = oracle.dense_mlp(mlp, x, want_inter=True)
    assert_close(y.cpu().numpy(), ref_y, f"dense decode T={T} y")
    assert_close(h.cpu().numpy(), ref_h, f"dense decode T={T} h")


def test_dense_mlp_prefill(escha, mlp):
    """300 tokens: one expert, expert_offsets = [0, 300], three 128-token tiles."""
    T = 300
    announce(f"dense_mlp_prefill T={T}")
    Md = _dev(escha, mlp)
    x = synth.activations(83, T, synth.HIDDEN)
    h = torch.empty(T, synth.INTER, dtype=torch.float32, device="cuda")
    y = escha.escha_dense_mlp_prefill(Md, to_dev(x), inter_out=h)
    ref_y, ref_h = oracle.dense_mlp(mlp, x, want_inter=True)
    assert_close(y.cpu().numpy(), ref_y, "dense prefill y")
    assert_close(h.cpu().numpy(), ref_h, "dense prefill h")


@pytest.mark.parametrize("T", [3, 20])
def test_dense_without_bias_is_the_one_expert_layer(escha, mlp, T):
    """Without biases the dense call runs the routed layer's kernels with
    one expert, id 0, weight 1: the same bits."""
    announce(f"dense without bias vs one-expert layer T={T}")
    Md = _dev(escha, mlp, bias=False)
    x = to_dev(synth.activations(84, T, synth.HIDDEN))
    y = escha.escha_dense_mlp_decode(Md, x)
    layer = escha.MoeLayer(Md.gate_up, Md.down, 1)
    ids = torch.zeros(T, 1, dtype=torch.int32, device="cuda")
    w = torch.ones(T, 1, dtype=torch.float32, device="cuda")
    ref = escha.escha_moe_layer_decode(layer, x, ids, w)
    assert torch.equal(y, ref)
