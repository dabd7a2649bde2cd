"""The entry point that allocates nothing (escha_moe_layer_decode_static):
the library's own device scratch instead of a caller workspace. Its output
must equal escha_moe_layer_decode's bit for bit (the same kernels in the
same order) on two calls in a row, the second with fewer tokens, and for a
streaming-path and a grouped-path token count; a request larger than the
scratch is refused before any launch."""
import numpy as np
import pytest
import torch

from bit_trellis_quantized_amd import synth
from tests._gpu_util import announce, layer_to_dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def escha():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from bit_trellis_quantized_amd import escha as mod
    return mod


@pytest.fixture(scope="module")
def layer(escha):
    return layer_to_dev(synth.layer_tensors(2, 0))


def _inputs(T, seed):
    x = synth.activations(seed, T, synth.HIDDEN)
    logits = synth.normal_logits(seed, T)
    return to_dev(x), to_dev(logits)


@pytest.mark.parametrize("sizes", [(8, 3), (64, 20)])
def test_static_decode_equals_workspace_decode(escha, layer, sizes):
    for i, T in enumerate(sizes):
        announce(f"decode_static T={T} (call {i + 1} of {len(sizes)})")
        x, logits = _inputs(T, 50 + T)
        ids, w = escha.escha_route_topk(logits, synth.TOP_K)
        ref = escha.escha_moe_layer_decode(layer, x, ids, w)
        inter_ref = torch.empty(T * synth.TOP_K, synth.INTER, dtype=torch.float32, device="cuda")
        escha.escha_moe_layer_decode(layer, x, ids, w, inter_out=inter_ref)
        out = torch.full((T, synth.HIDDEN), float("nan"), dtype=torch.float32, device="cuda")
        inter = torch.full_like(inter_ref, float("nan"))
        escha.escha_moe_layer_decode_static(layer, x, ids, w, out=out, inter_out=inter)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"T={T}: output differs from the workspace entry point"
        assert torch.equal(inter, inter_ref), f"T={T}: intermediate differs"


def test_static_decode_refuses_oversize(escha, layer):
    announce("decode_static refuses 11 tokens")
    x, logits = _inputs(11, 7)
    ids, w = escha.escha_route_topk(logits, synth.TOP_K)
    with pytest.raises(escha.EschaError, match="ESCHA_E_WORKSPACE"):
        escha.escha_moe_layer_decode_static(layer, x, ids, w)
