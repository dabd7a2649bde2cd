"""GPU parity of the shared expert (w8a16 int8 weights, f32 group-128
scales, fp16 sigmoid gate) against the fp64 oracle, alone and summed into
the routed experts' output of the same layer (the MoE block's output)."""
import numpy as np
import pytest
import torch

import oracle
from bit_trellis_quantized_amd import synth
from tests._gpu_util import announce, assert_close, layer_to_dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def escha():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from bit_trellis_quantized_amd import escha as mod
    return mod


def _dev_shared(escha, S):
    return escha.SharedExpert(torch.from_numpy(S["gu_w"]).cuda(), torch.from_numpy(S["gu_s"]).cuda(),
                              torch.from_numpy(S["dn_w"]).cuda(), torch.from_numpy(S["dn_s"]).cuda(),
                              to_dev(S["gate"]))


@pytest.mark.parametrize("hidden,inter,T", [(2048, 512, 1), (2048, 512, 9), (2048, 512, 64),
                                            (1024, 1024, 5), (4096, 2048, 3)])
def test_shared_expert_vs_oracle(escha, hidden, inter, T):
    announce(f"shared expert hidden={hidden} inter={inter} T={T}")
    S = synth.shared_expert_tensors(60, hidden=hidden, inter=inter)
    Sd = _dev_shared(escha, S)
    x = synth.activations(61, T, hidden)
    y = escha.escha_shared_expert(Sd, to_dev(x)).cpu().numpy()
    ref = oracle.shared_expert(S, x)
    assert_close(y, ref, f"shared expert {hidden}/{inter} T={T}")


def test_shared_expert_gate_extremes(escha):
    """A gate row that drives the sigmoid of one token's logit to ~1 (the
    other token's logit is large in magnitude too; the dot product is not
    rounded)."""
    announce("shared expert gate extremes")
    S = synth.shared_expert_tensors(62)
    x = synth.activations(63, 2, synth.HIDDEN)
    xd = np.array([[oracle.bf16_to_double(int(v)) for v in row] for row in x])
    gate = np.zeros(synth.HIDDEN)
    gate[:64] = 3.0 * np.sign(xd[0, :64])  # token 0: large positive logit
    S["gate"] = gate.astype(np.float16).view(np.uint16)
    Sd = _dev_shared(escha, S)
    y = escha.escha_shared_expert(Sd, to_dev(x)).cpu().numpy()
    ref, g = oracle.shared_expert(S, x, want_gate=True)
    assert g[0] > 0.999
    assert_close(y, ref, "shared expert gate extremes")


@pytest.mark.parametrize("T", [1, 32])
def test_moe_block_routed_plus_shared(escha, T):
    """The MoE block's output: the routed layer (decode entry) and the shared
    expert added into it on the same stream."""
    announce(f"routed + shared, T={T}")
    E = 64
    L = synth.layer_tensors(64, 0, n_experts=E)
    Ldev = layer_to_dev(L)
    S = synth.shared_expert_tensors(64)
    Sd = _dev_shared(escha, S)
    x = synth.activations(65, T, synth.HIDDEN)
    ids, w = oracle.route_topk(synth.normal_logits(65, T, E), 8)
    y = escha.escha_moe_layer_decode(Ldev, to_dev(x), to_dev(ids), to_dev(w.astype(np.float32)))
    escha.escha_shared_expert(Sd, to_dev(x), out=y, accumulate=True)
    ref = oracle.moe_layer(L, x, ids, w.astype(np.float32)) + oracle.shared_expert(S, x)
    assert_close(y.cpu().numpy(), ref, f"routed + shared T={T}")
