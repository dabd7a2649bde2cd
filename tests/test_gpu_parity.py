"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Inputs come from the seeded generator; routings fed to the layer tests are
the oracle's (the GPU router is tested on its own). Decoded weights and every
integer result must match exactly; fp32 outputs must meet the relative-L2 and
max-abs bounds in ``_gpu_util``.
"""
import numpy as np
import pytest
import torch

import oracle
from bit_trellis_quantized_amd import synth
from tests._gpu_util import announce, assert_close, errors, layer_to_dev, to_dev, u16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def escha():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from bit_trellis_quantized_amd import escha as mod
    return mod


@pytest.fixture(scope="module")
def layer2():
    """Config 2's layer: 256 experts, gate_up K=2, down K=3, prune masks."""
    return synth.layer_tensors(2, 0)


@pytest.fixture(scope="module")
def layer2_dev(escha, layer2):
    return layer_to_dev(layer2)


# ------------------------------------------------------------------ decode

def test_decode_tiles_config1_bit_exact(escha):
    announce("decode_tiles config1 256x256 K=2")
    code, rin, rout = synth.single_proj(1, 256, 256, 2)
    w = escha.Proj(to_dev(code), to_dev(rin), to_dev(rout))
    got = u16(escha.escha_decode_tiles(w, 0))
    ref = oracle.reconstruct(code, 256, 256, 2)
    assert np.count_nonzero(got != ref) == 0


@pytest.mark.parametrize("expert", [0, 1, 137, 255])
def test_decode_tiles_layer_experts_bit_exact(escha, layer2, layer2_dev, expert):
    announce(f"decode_tiles layer2 expert {expert}")
    got_gu = u16(escha.escha_decode_tiles(layer2_dev.gate_up, expert))
    got_dn = u16(escha.escha_decode_tiles(layer2_dev.down, expert))
    ref_gu = oracle.reconstruct(layer2["gu_code"][expert], 2048, 1024, 2)
    ref_dn = oracle.reconstruct(layer2["dn_code"][expert], 512, 2048, 3)
    assert np.count_nonzero(got_gu != ref_gu) == 0
    assert np.count_nonzero(got_dn != ref_dn) == 0


@pytest.mark.parametrize("K", [2, 3])
def test_decode_tiles_special_words(escha, K):
    """All-zero, all-one and alternating words (wrap windows included)."""
    announce(f"decode_tiles special words K={K}")
    in_f, out_f = 128, 256
    shape = (in_f // 16, out_f // 16, 16 * K)
    for fill in (0x0000, 0xFFFF, 0xAAAA, 0x8001):
        code = np.full(shape, fill, dtype=np.uint16)
        _, rin, rout = synth.single_proj(3, in_f, out_f, K)
        w = escha.Proj(to_dev(code), to_dev(rin), to_dev(rout))
        got = u16(escha.escha_decode_tiles(w, 0))
        assert np.array_equal(got, oracle.reconstruct(code, in_f, out_f, K)), hex(fill)


# The decoders of the fused kernels, written back in [out][in] order: the
# matrix-operand decoder (one-launch stack, small tiles), the LDS-tile
# decoder (128-token grouped kernels) and the K=2 column-pair decoder (the
# one-launch stack's gate_up tasks) must give the format's bits exactly.
FUSED_LAYOUTS = [1, 2]  # LAYOUT_MFMA_OPERAND, LAYOUT_LDS_TILE
PAIR_LAYOUTS = [3, 4]   # LAYOUT_MFMA_PAIRS, LAYOUT_MFMA_TILE_PAIRS (K=2 only)


@pytest.mark.parametrize("layout", FUSED_LAYOUTS)
@pytest.mark.parametrize("K", [2, 3])
def test_decode_layouts_single_matrix_bit_exact(escha, layout, K):
    announce(f"decode layout {layout} 256x256 K={K}")
    code, rin, rout = synth.single_proj(1, 256, 256, K)
    w = escha.Proj(to_dev(code), to_dev(rin), to_dev(rout))
    got = u16(escha.escha_decode_tiles_layout(w, 0, layout))
    ref = oracle.reconstruct(code, 256, 256, K)
    assert np.count_nonzero(got != ref) == 0


@pytest.mark.parametrize("layout", FUSED_LAYOUTS)
@pytest.mark.parametrize("expert", [0, 1, 137, 255])
def test_decode_layouts_layer_experts_bit_exact(escha, layer2, layer2_dev, layout, expert):
    announce(f"decode layout {layout} layer2 expert {expert}")
    got_gu = u16(escha.escha_decode_tiles_layout(layer2_dev.gate_up, expert, layout))
    got_dn = u16(escha.escha_decode_tiles_layout(layer2_dev.down, expert, layout))
    ref_gu = oracle.reconstruct(layer2["gu_code"][expert], 2048, 1024, 2)
    ref_dn = oracle.reconstruct(layer2["dn_code"][expert], 512, 2048, 3)
    assert np.count_nonzero(got_gu != ref_gu) == 0
    assert np.count_nonzero(got_dn != ref_dn) == 0


@pytest.mark.parametrize("layout", [0] + FUSED_LAYOUTS)
@pytest.mark.parametrize("K", [2, 3])
def test_decode_layouts_special_words(escha, layout, K):
    """Constant words (all-zero, all-one, alternating, end bits) and a
    mixture with one constant word per tile position, so that every window,
    the wrapping ones included, sees distinct neighbours."""
    announce(f"decode layout {layout} special words K={K}")
    in_f, out_f = 128, 256
    shape = (in_f // 16, out_f // 16, 16 * K)
    _, rin, rout = synth.single_proj(3, in_f, out_f, K)
    cases = [np.full(shape, f, dtype=np.uint16) for f in (0x0000, 0xFFFF, 0xAAAA, 0x8001)]
    mixed = np.random.default_rng(K).integers(0, 65536, size=shape, dtype=np.uint16)
    mixed[..., 0] = 0xFFFF   # first word of every tile (the wrap target)
    mixed[..., -1] = 0x8001  # last word of every tile (the wrap source)
    cases.append(mixed)
    for code in cases:
        w = escha.Proj(to_dev(code), to_dev(rin), to_dev(rout))
        got = u16(escha.escha_decode_tiles_layout(w, 0, layout))
        assert np.array_equal(got, oracle.reconstruct(code, in_f, out_f, K)), hex(int(code.flat[1]))


@pytest.mark.parametrize("layout", PAIR_LAYOUTS)
@pytest.mark.parametrize("expert", [0, 137])
def test_decode_pairs_layout_bit_exact(escha, layer2, layer2_dev, layout, expert):
    announce(f"decode layout {layout} layer2 gate_up expert {expert}")
    got = u16(escha.escha_decode_tiles_layout(layer2_dev.gate_up, expert, layout))
    assert np.count_nonzero(got != oracle.reconstruct(layer2["gu_code"][expert], 2048, 1024, 2)) == 0


@pytest.mark.parametrize("layout", PAIR_LAYOUTS)
def test_decode_pairs_layout_matrix_and_special_words(escha, layout):
    announce(f"decode layout {layout} 256x256 and special words")
    code, rin, rout = synth.single_proj(1, 256, 256, 2)
    w = escha.Proj(to_dev(code), to_dev(rin), to_dev(rout))
    assert np.count_nonzero(u16(escha.escha_decode_tiles_layout(w, 0, layout))
                            != oracle.reconstruct(code, 256, 256, 2)) == 0
    in_f, out_f = 128, 256
    shape = (in_f // 16, out_f // 16, 32)
    _, rin, rout = synth.single_proj(3, in_f, out_f, 2)
    mixed = np.random.default_rng(2).integers(0, 65536, size=shape, dtype=np.uint16)
    mixed[..., 0] = 0xFFFF   # the wrap target
    mixed[..., -1] = 0x8001  # the wrap source
    for code in [np.full(shape, f, dtype=np.uint16) for f in (0x0000, 0xFFFF, 0xAAAA, 0x8001)] + [mixed]:
        w = escha.Proj(to_dev(code), to_dev(rin), to_dev(rout))
        got = u16(escha.escha_decode_tiles_layout(w, 0, layout))
        assert np.array_equal(got, oracle.reconstruct(code, in_f, out_f, 2)), hex(int(code.flat[1]))


# ------------------------------------------------------------------ Hadamard

def test_hadamard128(escha):
    announce("hadamard128")
    eye = torch.eye(256, dtype=torch.float32, device="cuda")
    Hn = escha.escha_hadamard128(eye).cpu().numpy().astype(np.float64)
    assert np.allclose(Hn @ Hn.T, np.eye(256), atol=1e-6)
    x = np.random.default_rng(0).standard_normal((37, 384)).astype(np.float32)
    got = escha.escha_hadamard128(to_dev(x)).cpu().numpy()
    ref = oracle.hadamard128(x.astype(np.float64))
    assert np.max(np.abs(got - ref)) <= 1e-5 * np.max(np.abs(ref))


# ------------------------------------------------------------------ routing

@pytest.mark.parametrize("cfg,T", [(2, 1), (3, 64), (5, 4096), (3, 7)])
def test_route_topk_vs_oracle(escha, cfg, T):
    announce(f"route_topk cfg{cfg} T={T}")
    logits = synth.zipf_logits(cfg, T) if cfg == 3 else synth.normal_logits(cfg, T)
    ids, w = escha.escha_route_topk(to_dev(logits), 8)
    ref_ids, ref_w = oracle.route_topk(logits, 8)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    assert np.allclose(w.cpu().numpy(), ref_w, rtol=2e-6, atol=0)


def test_route_topk_ties(escha):
    announce("route_topk ties")
    logits = np.zeros((2, 256), dtype=np.float32)
    logits[0, [200, 17, 90, 3, 250, 11, 40, 8, 9]] = 1.0
    logits[1, :] = 0.5  # all tied
    ids, _ = escha.escha_route_topk(to_dev(logits), 8)
    ref_ids, _ = oracle.route_topk(logits, 8)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)


@pytest.mark.parametrize("cfg,T", [(2, 1), (3, 64), (5, 4096), (3, 3)])
def test_group_vs_oracle(escha, cfg, T):
    announce(f"moe_group cfg{cfg} T={T}")
    logits = synth.zipf_logits(cfg, T) if cfg == 3 else synth.normal_logits(cfg, T)
    ids, _ = oracle.route_topk(logits, 8)
    counts, offsets, perm = escha.escha_moe_group(to_dev(ids), 256)
    rc, ro, rp = oracle.group(ids, 256)
    assert np.array_equal(counts.cpu().numpy(), rc)
    assert np.array_equal(offsets.cpu().numpy(), ro)
    assert np.array_equal(perm.cpu().numpy(), rp)


def _group_check(escha, ids, E, what):
    """Grouping of ``ids`` over E experts against the oracle; ids outside
    [0, E) are left out of the grouping, which is the oracle's grouping over
    one more expert (index E, taking every bad id) with that expert dropped."""
    announce(f"moe_group {what}")
    bad = (ids < 0) | (ids >= E)
    ids_o = np.where(bad, E, ids).astype(np.int32)
    rc, ro, rp = oracle.group(ids_o, E + 1)
    counts, offsets, perm = escha.escha_moe_group(to_dev(ids.astype(np.int32)), E)
    n = int(ro[E])
    assert np.array_equal(counts.cpu().numpy(), rc[:E]), what
    assert np.array_equal(offsets.cpu().numpy(), ro[:E + 1]), what
    assert np.array_equal(perm.cpu().numpy()[:n], rp[:n]), what


@pytest.mark.parametrize("T", [1024, 1025, 8192])
def test_group_one_expert_for_all(escha, T):
    """Every pair on one expert: 8192 pairs (the most one work-group groups),
    8200 and 65536 (the multi-pass path); ranks in pair order across all
    waves and chunks."""
    _group_check(escha, np.full((T, 8), 77, dtype=np.int32), 256, f"one expert T={T}")


@pytest.mark.parametrize("E", [1, 2, 255, 256, 257, 300])
def test_group_expert_counts(escha, E):
    """Expert counts around the one-work-group limit (256) and the smallest
    (one expert: no index bits)."""
    rng = np.random.default_rng(900 + E)
    T = 700
    ids = rng.integers(0, E, size=(T, 8)).astype(np.int32)
    _group_check(escha, ids, E, f"E={E} T={T}")


@pytest.mark.parametrize("T", [37, 1100])
def test_group_bad_ids(escha, T):
    """Ids below 0 or at/above E are left out (counts, offsets and the sorted
    part of perm over the valid pairs only), on both grouping paths."""
    rng = np.random.default_rng(40 + T)
    ids = rng.integers(0, 256, size=(T, 8)).astype(np.int32)
    flat = ids.reshape(-1)
    pick = rng.choice(flat.size, size=flat.size // 10, replace=False)
    flat[pick] = rng.choice(np.array([-1, -7, 256, 1000], dtype=np.int32), size=pick.size)
    _group_check(escha, ids, 256, f"bad ids T={T}")


@pytest.mark.parametrize("T,zipf", [(1, False), (3, False), (15, True), (16, False), (64, True)])
def test_layer_decode_logits(escha, layer2, layer2_dev, T, zipf):
    """The layer with its router step inside (top-k in the streaming gate_up
    kernel below 16 tokens, a router kernel of its own from 16 on): the
    selections are the router step's bits, and y is the bits of the router
    step followed by the layer call; y also against the oracle."""
    announce(f"layer decode with routing, T={T} zipf={zipf}")
    x = synth.activations(70 + T, T, 2048)
    logits = synth.zipf_logits(3, T) if zipf else synth.normal_logits(70 + T, T)
    xd, ld = to_dev(x), to_dev(logits.astype(np.float32))
    y, ids, w = escha.escha_moe_layer_decode_logits(layer2_dev, xd, ld)
    ids2, w2 = escha.escha_route_topk(ld, 8)
    assert torch.equal(ids, ids2)
    assert torch.equal(w.view(torch.int32), w2.view(torch.int32))
    y2 = escha.escha_moe_layer_decode(layer2_dev, xd, ids2, w2)
    assert torch.equal(y.view(torch.int32), y2.view(torch.int32))
    ref_ids, ref_w = oracle.route_topk(logits, 8)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    ref = oracle.moe_layer(layer2, x, ref_ids, w.cpu().numpy())
    assert_close(y.cpu().numpy(), ref, f"decode with routing T={T}")


def test_layer_decode_logits_ties(escha, layer2, layer2_dev):
    """Tied logits inside the fused router step: ties go to the lower expert
    index, as in the router step of its own."""
    announce("layer decode with routing, tied logits")
    T = 20
    logits = np.zeros((T, 256), dtype=np.float32)
    logits[0, [200, 17, 90, 3, 250, 11, 40, 8, 9]] = 1.0
    logits[1:, :] = 0.5
    x = synth.activations(7, T, 2048)
    for n in (2, T):  # router step in the streaming kernel; a router kernel of its own
        ld = to_dev(logits[:n])
        _, ids, w = escha.escha_moe_layer_decode_logits(layer2_dev, to_dev(x[:n]), ld)
        ref_ids, _ = oracle.route_topk(logits[:n], 8)
        assert np.array_equal(ids.cpu().numpy(), ref_ids)


# ------------------------------------------------------------------ projections

@pytest.mark.parametrize("T", [1, 3])
def test_expert_gemv_config1(escha, T):
    announce(f"expert_gemv config1 T={T}")
    code, rin, rout = synth.single_proj(1, 256, 256, 2)
    x = synth.activations(1, T, 256)
    w = escha.Proj(to_dev(code), to_dev(rin), to_dev(rout))
    y = escha.escha_expert_gemv(w, 0, to_dev(x)).cpu().numpy()
    ref = oracle.expert_gemv(code, rin, rout, 256, 256, 2, x)
    assert_close(y, ref, f"expert_gemv T={T}")


def test_expert_gemv_layer_shapes(escha, layer2, layer2_dev):
    """gate_up (K=2) and down (K=3) of one expert through the single-projection call."""
    e = 77
    x_gu = synth.activations(11, 2, 2048)
    y = escha.escha_expert_gemv(layer2_dev.gate_up, e, to_dev(x_gu)).cpu().numpy()
    ref = oracle.expert_gemv(layer2["gu_code"][e], layer2["gu_rin"][e], layer2["gu_rout"][e],
                             2048, 1024, 2, x_gu)
    assert_close(y, ref, "expert_gemv gate_up")
    assert np.all(y[:, np.concatenate([layer2["mask"][e]] * 2)] == 0.0)
    x_dn = synth.activations(12, 2, 512)
    y = escha.escha_expert_gemv(layer2_dev.down, e, to_dev(x_dn)).cpu().numpy()
    ref = oracle.expert_gemv(layer2["dn_code"][e], layer2["dn_rin"][e], layer2["dn_rout"][e],
                             512, 2048, 3, x_dn)
    assert_close(y, ref, "expert_gemv down")


# ------------------------------------------------------------------ MoE layer

def _check_layer(escha, L, Ldev, x, ids, w, entry, what):
    inter = torch.empty(ids.size, 512, dtype=torch.float32, device="cuda")
    y = entry(Ldev, to_dev(x), to_dev(ids), to_dev(w.astype(np.float32)), inter_out=inter)
    y = y.cpu().numpy()
    inter = inter.cpu().numpy()
    ref_y, ref_inter = oracle.moe_layer(L, x, ids, w.astype(np.float32), want_inter=True)
    assert_close(y, ref_y, f"{what} y")
    assert_close(inter, ref_inter, f"{what} h")
    for p, e in enumerate(ids.ravel()):
        assert np.all(inter[p][L["mask"][e]] == 0.0), f"pair {p}: pruned channel not zero"
    return y


def test_layer_decode_config2(escha, layer2, layer2_dev):
    announce("moe_layer_decode config2 T=1")
    x = synth.activations(2, 1, 2048)
    ids, w = oracle.route_topk(synth.normal_logits(2, 1), 8)
    y1 = _check_layer(escha, layer2, layer2_dev, x, ids, w, escha.escha_moe_layer_decode, "cfg2")
    y2 = escha.escha_moe_layer_decode(layer2_dev, to_dev(x), to_dev(ids),
                                      to_dev(w.astype(np.float32))).cpu().numpy()
    assert np.array_equal(y1, y2), "decode is not bit-reproducible"


def test_layer_decode_config3_zipf(escha):
    announce("moe_layer_decode config3 T=64 zipf")
    L = synth.layer_tensors(3, 0)
    Ldev = layer_to_dev(L)
    x = synth.activations(3, 64, 2048)
    ids, w = oracle.route_topk(synth.zipf_logits(3, 64), 8)
    _check_layer(escha, L, Ldev, x, ids, w, escha.escha_moe_layer_decode, "cfg3")


def test_layer_ragged_and_bad_ids(escha, layer2, layer2_dev):
    """T=5 (ragged), and out-of-range ids contribute exactly nothing."""
    announce("moe_layer_decode ragged T=5 with bad ids")
    x = synth.activations(21, 5, 2048)
    ids, w = oracle.route_topk(synth.normal_logits(21, 5), 8)
    bad = ids.copy()
    bad[1, 3] = -1
    bad[4, 0] = 256
    y = escha.escha_moe_layer_decode(layer2_dev, to_dev(x), to_dev(bad),
                                     to_dev(w.astype(np.float32))).cpu().numpy()
    w0 = w.astype(np.float32).copy()
    w0[1, 3] = 0.0
    w0[4, 0] = 0.0
    ref = oracle.moe_layer(layer2, x, ids, w0)
    assert_close(y, ref, "bad ids")


def test_layer_prefill_matches_oracle_on_subset(escha):
    """Config 5: 4096 tokens; oracle on tokens 0..255; pruned h == 0 for all pairs."""
    announce("moe_layer_prefill config5 T=4096")
    L = synth.layer_tensors(5, 0)
    Ldev = layer_to_dev(L)
    T, n_check = 4096, 256
    x = synth.activations(5, T, 2048)
    ids, w = oracle.route_topk(synth.normal_logits(5, T), 8)
    inter = torch.empty(T * 8, 512, dtype=torch.float32, device="cuda")
    y = escha.escha_moe_layer_prefill(Ldev, to_dev(x), to_dev(ids), to_dev(w.astype(np.float32)),
                                      inter_out=inter).cpu().numpy()
    inter = inter.cpu().numpy()
    ref_y, ref_inter = oracle.moe_layer(L, x[:n_check], ids[:n_check], w[:n_check].astype(np.float32),
                                        want_inter=True)
    assert_close(y[:n_check], ref_y, "prefill y[0:256]")
    assert_close(inter[:n_check * 8], ref_inter, "prefill h[0:256]")
    masks = L["mask"][ids.ravel()]
    assert np.all(inter[masks] == 0.0)
    assert np.all(np.isfinite(y))


def test_prefill_equals_decode_path(escha, layer2, layer2_dev):
    """Both entry points compute the same function (T=31: the decode entry
    streams every pair, the prefill entry runs the grouped kernels)."""
    announce("prefill vs decode T=31")
    x = synth.activations(31, 31, 2048)
    ids, w = oracle.route_topk(synth.normal_logits(31, 31), 8)
    a = escha.escha_moe_layer_decode(layer2_dev, to_dev(x), to_dev(ids), to_dev(w.astype(np.float32)))
    b = escha.escha_moe_layer_prefill(layer2_dev, to_dev(x), to_dev(ids), to_dev(w.astype(np.float32)))
    rel, mx = errors(b.cpu().numpy(), a.cpu().numpy())
    assert rel <= 1e-3 and mx <= 2e-3


def test_zero_tokens_is_a_no_op(escha, layer2_dev):
    x = torch.empty(0, 2048, dtype=torch.int16, device="cuda")
    ids = torch.empty(0, 8, dtype=torch.int32, device="cuda")
    w = torch.empty(0, 8, dtype=torch.float32, device="cuda")
    y = escha.escha_moe_layer_decode(layer2_dev, x, ids, w)
    assert y.shape == (0, 2048)


def test_rmsnorm_bf16(escha):
    announce("rmsnorm_bf16")
    y = np.random.default_rng(4).standard_normal((8, 2048)) * 3
    got = u16(escha.escha_rmsnorm_bf16(to_dev(y.astype(np.float32))))
    ref = oracle.rmsnorm_bf16(y.astype(np.float32).astype(np.float64))
    # the same decision in different precision may differ by one bf16 step
    diff = np.abs(got.astype(np.int32) - ref.astype(np.int32))
    assert diff.max() <= 1 and np.mean(diff) < 1e-2


# ------------------------------------------------------------------ grouped path

def test_grouped_config3_zipf(escha):
    """Config 3 (64 tokens, Zipf routing) through the grouped kernels: each
    expert's tiles decoded once per 64-token tile, MFMA contraction."""
    announce("grouped (prefill entry) config3 T=64 zipf")
    L = synth.layer_tensors(3, 0)
    Ldev = layer_to_dev(L)
    x = synth.activations(3, 64, 2048)
    ids, w = oracle.route_topk(synth.zipf_logits(3, 64), 8)
    _check_layer(escha, L, Ldev, x, ids, w, escha.escha_moe_layer_prefill, "grouped cfg3")


@pytest.mark.parametrize("T", [1, 2, 65])
def test_grouped_small_batches_and_bad_ids(escha, layer2, layer2_dev, T):
    announce(f"grouped T={T} with a bad id")
    x = synth.activations(40 + T, T, 2048)
    ids, w = oracle.route_topk(synth.normal_logits(40 + T, T), 8)
    bad = ids.copy()
    bad[0, 5] = 1000
    y = escha.escha_moe_layer_prefill(layer2_dev, to_dev(x), to_dev(bad),
                                      to_dev(w.astype(np.float32))).cpu().numpy()
    w0 = w.astype(np.float32).copy()
    w0[0, 5] = 0.0
    ref = oracle.moe_layer(layer2, x, ids, w0)
    assert_close(y, ref, f"grouped T={T}")


@pytest.mark.parametrize("T", [20, 48])
def test_small_tile_decode_bad_ids(escha, layer2, layer2_dev, T):
    """The decode entry from 16 tokens (the one-launch small-tile layer):
    ids below 0 or at/above the expert count contribute nothing, the other
    pairs are exact to tolerance, pruned channels stay exactly zero."""
    announce(f"small-tile decode, T={T}, bad ids")
    x = synth.activations(60 + T, T, 2048)
    ids, w = oracle.route_topk(synth.normal_logits(60 + T, T), 8)
    bad = ids.copy()
    bad[0, 5] = 256
    bad[T - 1, 0] = -1
    bad[T // 2, 7] = 1 << 20
    inter = torch.empty(T * 8, 512, dtype=torch.float32, device="cuda")
    y = escha.escha_moe_layer_decode(layer2_dev, to_dev(x), to_dev(bad), to_dev(w.astype(np.float32)),
                                     inter_out=inter).cpu().numpy()
    w0 = w.astype(np.float32).copy()
    w0[bad != ids] = 0.0
    ref, ref_inter = oracle.moe_layer(layer2, x, ids, w0, want_inter=True)
    assert_close(y, ref, f"small-tile decode T={T} with bad ids")
    got = inter.cpu().numpy()
    ok = (bad == ids).reshape(-1)
    assert_close(got[ok], ref_inter[ok], f"small-tile decode T={T} h")
    assert np.all(got[ok][ref_inter[ok] == 0] == 0)


def test_grouped_one_hot_expert(escha, layer2, layer2_dev):
    """Every token routed to the same 8 experts: 130 tokens per expert = 3 tiles."""
    announce("grouped, all tokens on the same experts")
    T = 130
    x = synth.activations(50, T, 2048)
    ids = np.tile(np.array([[3, 9, 27, 81, 100, 200, 250, 7]], dtype=np.int32), (T, 1))
    w = np.full((T, 8), 0.125, dtype=np.float32)
    _check_layer(escha, layer2, layer2_dev, x, ids, w, escha.escha_moe_layer_prefill, "hot experts")


def test_prefill_partial_tiles(escha, layer2, layer2_dev):
    """128-token tiles whose token counts end inside every 32-token sub-tile
    of both token halves (1, 20, 29, 32, 33, 40, 59, 64, 65, 69, 70, 96, 97,
    100, 128 and 129 = a full tile plus one): every matrix wave meets no,
    one or two live sub-tiles, and the padded columns are never stored."""
    announce("prefill partial tiles T=129")
    T = 129
    # slot j: expert experts[i] for tokens bounds[i - 1] .. bounds[i] - 1 of plan[j]
    plan = [((20, 60, 129), (10, 11, 12)), ((70, 129), (13, 14)), ((100, 129), (15, 16)),
            ((128, 129), (17, 18)), ((129,), (19,)), ((64, 129), (20, 21)),
            ((96, 129), (22, 23)), ((97, 129), (24, 25))]
    ids = np.empty((T, 8), dtype=np.int32)
    for j, (bounds, experts) in enumerate(plan):
        lo = 0
        for hi, e in zip(bounds, experts):
            ids[lo:hi, j] = e
            lo = hi
    counts = sorted(np.bincount(ids.ravel())[10:26].tolist())
    assert counts == [1, 20, 29, 32, 33, 40, 59, 64, 65, 69, 70, 96, 97, 100, 128, 129]
    x = synth.activations(51, T, 2048)
    rng = np.random.default_rng(51)
    w = rng.random((T, 8)).astype(np.float32)
    w /= w.sum(axis=1, keepdims=True)
    _check_layer(escha, layer2, layer2_dev, x, ids, w, escha.escha_moe_layer_prefill, "partial tiles")
