"""GPU parity away from unit-scale activations, and the prune skips.

Activations enter the matrix cores as fp16. The grouped and small-tile
kernels scale each row (or 128-input block) by a power of two before that
rounding and undo it in fp32; the one-launch stack scales a block whose
values are all large or all small. Inputs scaled by 2^14 (rotated values
past fp16's 65504 without the scaling) and by 2^-14 (the intermediate h near
1e-9, below fp16's smallest subnormal) must still meet the tolerance
against the fp64 oracle, through every decode path and the prefill path.

A 128-channel block of h that is exactly zero contributes exactly zero to
down_proj, and the kernels skip its codes: the streaming kernel per pair,
the grouped kernels per tile (every token of the tile zero on the block).
These cases are forced here with an expert whose gate rout is zero on a
whole block.
"""
import numpy as np
import pytest
import torch

import oracle
from bit_trellis_quantized_amd import synth
from tests._gpu_util import announce, assert_close, layer_to_dev, to_dev, u16

pytestmark = pytest.mark.gpu

E = 64  # experts of the test layers (the oracle rebuilds every routed one)


@pytest.fixture(scope="module")
def escha():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from bit_trellis_quantized_amd import escha as mod
    return mod


@pytest.fixture(scope="module")
def layer():
    return synth.layer_tensors(40, 0, n_experts=E)


@pytest.fixture(scope="module")
def layer_dev(escha, layer):
    return layer_to_dev(layer)


def _scaled_x(seed, T, scale):
    x = np.random.default_rng(seed).standard_normal((T, synth.HIDDEN)).astype(np.float32)
    return synth.to_bf16_bits(x * np.float32(scale))


def _route(seed, T):
    return oracle.route_topk(synth.normal_logits(seed, T, E), 8)


def _check(escha, L, Ldev, x, ids, w, entry, what):
    inter = torch.empty(ids.size, synth.INTER, dtype=torch.float32, device="cuda")
    y = entry(Ldev, to_dev(x), to_dev(ids), to_dev(w.astype(np.float32)), inter_out=inter)
    ref_y, ref_h = oracle.moe_layer(L, x, ids, w.astype(np.float32), want_inter=True)
    assert_close(y.cpu().numpy(), ref_y, f"{what} y")
    assert_close(inter.cpu().numpy(), ref_h, f"{what} h")
    hh = inter.cpu().numpy()
    for p, e in enumerate(ids.ravel()):
        assert np.all(hh[p][L["mask"][e]] == 0.0), f"{what}: pair {p} pruned channel not zero"


# T = 3: streaming kernels (fp32 activations); 32: small tiles; 200: the
# 128-token tiles through the decode entry (more than 16 pairs per expert)
@pytest.mark.parametrize("T", [3, 32, 200])
@pytest.mark.parametrize("scale", [2.0 ** -14, 2.0 ** 14])
def test_decode_scaled_activations(escha, layer, layer_dev, T, scale):
    announce(f"decode, x scaled by {scale:g}, T={T}")
    x = _scaled_x(T, T, scale)
    ids, w = _route(100 + T, T)
    _check(escha, layer, layer_dev, x, ids, w, escha.escha_moe_layer_decode, f"decode x{scale:g} T={T}")


@pytest.mark.parametrize("scale", [2.0 ** -14, 2.0 ** 14])
def test_prefill_scaled_activations(escha, layer, layer_dev, scale):
    announce(f"prefill, x scaled by {scale:g}, T=160")
    x = _scaled_x(7, 160, scale)
    ids, w = _route(207, 160)
    _check(escha, layer, layer_dev, x, ids, w, escha.escha_moe_layer_prefill, f"prefill x{scale:g}")


@pytest.mark.parametrize("scale", [2.0 ** -14, 2.0 ** 14])
def test_one_launch_stack_scaled_input(escha, scale):
    """The first layer of the one-launch stack on a scaled input (later
    layers see normalised inputs): its recorded next input against the
    oracle's RMSNorm of the oracle's layer output."""
    announce(f"one-launch stack, x0 scaled by {scale:g}")
    NLs, T, Es = 2, 2, 16
    host = [synth.layer_tensors(41, l, n_experts=Es) for l in range(NLs)]
    st = escha.Stack([layer_to_dev(L) for L in host])
    rs = np.random.default_rng(5)
    ids = np.stack([np.stack([rs.permutation(Es)[:8] for _ in range(T)]) for _ in range(NLs)]).astype(np.int32)
    w = rs.random((NLs, T, 8)).astype(np.float32)
    x0 = _scaled_x(8, T, scale)
    ws = torch.zeros(st.workspace_bytes(T), dtype=torch.uint8, device="cuda")
    chain = torch.empty(NLs, T, synth.HIDDEN, dtype=torch.int16, device="cuda")
    y = escha.escha_moe_stack_decode_persistent(st, to_dev(x0), to_dev(ids), to_dev(w), x_chain=chain,
                                                workspace=ws)
    ch = u16(chain)
    assert np.array_equal(ch[0], x0)
    ref0 = oracle.moe_layer(host[0], ch[0], ids[0], w[0])
    nxt = oracle.rmsnorm_bf16(ref0)
    steps = np.abs(ch[1].astype(np.int32) - nxt.astype(np.int32))
    assert steps.max() <= 1 and np.mean(steps > 0) < 0.02, f"next input off: {steps.max()} steps"
    assert_close(y.cpu().numpy(), oracle.moe_layer(host[1], ch[1], ids[1], w[1]), "stack last layer")


# ------------------------------------------------------------------ prune skips

PRUNED_EXPERT = 5
PRUNED_BLOCK = 1  # intermediate channels 128..255


@pytest.fixture(scope="module")
def pruned_layer():
    """The test layer with expert 5's gate rout zero on a whole 128-channel
    block: h of that block is exactly zero for every token routed there."""
    L = {k: v.copy() for k, v in synth.layer_tensors(40, 0, n_experts=E).items()}
    c0 = 128 * PRUNED_BLOCK
    L["gu_rout"][PRUNED_EXPERT, c0:c0 + 128] = 0
    L["mask"][PRUNED_EXPERT, c0:c0 + 128] = True
    return L


def _with_expert(ids, T, every=1):
    """Route slot 2 of every `every`-th token to the pruned expert."""
    ids = ids.copy()
    for t in range(0, T, every):
        if PRUNED_EXPERT not in ids[t]:
            ids[t, 2] = PRUNED_EXPERT
    return ids


# T = 2: streaming down kernel; 24: small-tile down kernel; 160: the
# 128-token tile down kernel through the decode entry
@pytest.mark.parametrize("T", [2, 24, 160])
def test_decode_pruned_block_skip(escha, pruned_layer, T):
    announce(f"decode with a fully pruned 128-channel block, T={T}")
    Ldev = layer_to_dev(pruned_layer)
    x = _scaled_x(300 + T, T, 1.0)
    ids, w = _route(300 + T, T)
    ids = _with_expert(ids, T)
    _check(escha, pruned_layer, Ldev, x, ids, w, escha.escha_moe_layer_decode, f"pruned block T={T}")


def test_prefill_pruned_block_skip(escha, pruned_layer):
    announce("prefill with a fully pruned 128-channel block, T=96")
    Ldev = layer_to_dev(pruned_layer)
    x = _scaled_x(400, 96, 1.0)
    ids, w = _route(400, 96)
    ids = _with_expert(ids, 96)
    _check(escha, pruned_layer, Ldev, x, ids, w, escha.escha_moe_layer_prefill, "pruned block prefill")


# ------------------------------------------------------- blocks far below their row

# expert 5's (gate, up) rout on three 128-channel blocks, as fp16 bits
# (None: unchanged): h there ends near 2^-38, 2^-20 and 2^-12 of the row's
# largest value
FAR_BLOCKS = {1: (0x0001, 0x0001), 2: (0x0001, None), 3: (0x0100, None)}


@pytest.fixture(scope="module")
def far_layer():
    """The test layer with expert 5's gate (and on one block up) rout at fp16
    subnormals: the down kernels see block exponents 8 to 40 above the row
    exponent, so the rescale to the row exponent lands in fp16 subnormals
    (2^-12, 2^-20) or below them (2^-38, where the block gives zeros)."""
    L = {k: v.copy() for k, v in synth.layer_tensors(40, 0, n_experts=E).items()}
    rs = np.random.default_rng(9)
    inter = L["mask"].shape[1]
    for blk, (g_bits, u_bits) in FAR_BLOCKS.items():
        for off, bits in ((0, g_bits), (inter, u_bits)):
            if bits is not None:
                sign = rs.integers(0, 2, 128).astype(np.uint16) << 15
                pruned = L["mask"][PRUNED_EXPERT, 128 * blk:128 * blk + 128]  # rout stays zero there
                L["gu_rout"][PRUNED_EXPERT, off + 128 * blk:off + 128 * blk + 128] = np.where(
                    pruned, np.uint16(0), sign | np.uint16(bits))
    return L


@pytest.mark.parametrize("T", [2, 24, 160])
def test_decode_far_blocks(escha, far_layer, T):
    announce(f"decode with blocks far below their row, T={T}")
    Ldev = layer_to_dev(far_layer)
    x = _scaled_x(500 + T, T, 1.0)
    ids, w = _route(500 + T, T)
    ids = _with_expert(ids, T)
    _check(escha, far_layer, Ldev, x, ids, w, escha.escha_moe_layer_decode, f"far blocks T={T}")


def test_prefill_far_blocks(escha, far_layer):
    announce("prefill with blocks far below their row, T=96")
    Ldev = layer_to_dev(far_layer)
    x = _scaled_x(600, 96, 1.0)
    ids, w = _route(600, 96)
    ids = _with_expert(ids, 96)
    _check(escha, far_layer, Ldev, x, ids, w, escha.escha_moe_layer_prefill, "far blocks prefill")
