"""Pins of the CPU oracle against what the pages and the mathematics fix.

No GPU. Each test ties one oracle function to something other than itself:
values the pages print (``tests/golden/cba_printed.txt``), an independent
exact-rational computation, a library routine (numpy float16, torch
bfloat16, scipy's Sylvester Hadamard, stable argsort), a closed form, or brute
force on a literal bit string.
"""
from fractions import Fraction
from pathlib import Path

import numpy as np
import pytest
import scipy.linalg

import oracle
from bit_trellis_quantized_amd import synth

GOLDEN = Path(__file__).parent / "golden" / "cba_printed.txt"


def _golden():
    d = {}
    for line in GOLDEN.read_text().splitlines():
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, *vals = line.split()
        d[key] = [int(v, 0) for v in vals]
    return d


# ------------------------------------------------------------ independent paths

def _hash_halves_numpy(states):
    """The pages' hash, in numpy uint64 arithmetic: (lo16, hi16) bit patterns."""
    g = _golden()
    s = np.asarray(states, dtype=np.uint64)
    r = (s * np.uint64(g["hash_mul"][0])) & np.uint64(0xFFFFFFFF)
    r = (r & np.uint64(g["hash_mask"][0])) ^ np.uint64(g["hash_xor"][0])
    return (r & np.uint64(0xFFFF)).astype(np.uint16), (r >> np.uint64(16)).astype(np.uint16)


def _codebook_numpy(states):
    """Sum the halves in float64 (exact) and round once with numpy's float16 cast."""
    lo, hi = _hash_halves_numpy(states)
    s = lo.view(np.float16).astype(np.float64) + hi.view(np.float16).astype(np.float64)
    return s.astype(np.float16).view(np.uint16)


def _f16_fraction(bits):
    """Exact rational value of an fp16 bit pattern (finite only)."""
    sign = -1 if bits >> 15 else 1
    e = (bits >> 10) & 31
    m = bits & 1023
    assert e != 31
    if e == 0:
        return sign * Fraction(m, 2 ** 24)
    return sign * Fraction(1024 + m, 1024) * (Fraction(2) ** (e - 15))


def _fraction_to_f16(q: Fraction, mode: str):
    """Encode an exact rational as fp16 bits; mode 'rne' or 'trunc' (toward zero)."""
    if q == 0:
        return 0
    sign = 0x8000 if q < 0 else 0
    a = abs(q)
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    assert -14 <= e <= 15, "test values stay in the normal range"
    scaled = a * 1024  # in [1024, 2048)
    fl = scaled.numerator // scaled.denominator
    rem = scaled - fl
    if mode == "rne" and (rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1)):
        fl += 1
    if fl == 2048:
        fl = 1024
        e += 1
    return sign | ((e + 15) << 10) | (fl - 1024)


def _codebook_fraction(s, mode="rne"):
    lo, hi = _hash_halves_numpy([s])
    return _fraction_to_f16(_f16_fraction(int(lo[0])) + _f16_fraction(int(hi[0])), mode)


@pytest.fixture(scope="module")
def codebook(oracle_lib):
    return oracle.codebook()


# ------------------------------------------------------------ printed values

def test_state3_printed_rne_value(oracle_lib):
    g = _golden()
    s, v = g["state_rne"]
    assert oracle.cba_decode_state(s) == v


def test_truncation_misses_exactly_the_printed_states(oracle_lib):
    """A planted mistake (truncating instead of RNE) must miss exactly 3, 6, 7."""
    g = _golden()
    s3, trunc3 = g["state_trunc"]
    assert _codebook_fraction(s3, "trunc") == trunc3
    differs = [s for s in range(8) if _codebook_fraction(s, "trunc") != oracle.cba_decode_state(s)]
    assert differs == g["trunc_differs"]


def test_distinct_values_printed(codebook):
    g = _golden()
    assert codebook.size == g["alphabet"][0]
    assert len(np.unique(codebook)) == g["distinct_values"][0]


# ------------------------------------------------------------ codebook, independently

def test_codebook_matches_numpy_float16_path(codebook):
    assert np.array_equal(codebook, _codebook_numpy(np.arange(65536)))


def test_codebook_matches_exact_rationals(codebook):
    gen = np.random.default_rng(7)
    lo, hi = _hash_halves_numpy(np.arange(65536))
    zero_states = np.nonzero(lo.view(np.float16).astype(np.float64)
                             + hi.view(np.float16).astype(np.float64) == 0)[0]
    sample = np.unique(np.concatenate([np.arange(64), zero_states, gen.integers(0, 65536, 1500)]))
    for s in sample:
        assert codebook[s] == _codebook_fraction(int(s)), s


def test_codebook_derived_properties(codebook):
    lo, hi = _hash_halves_numpy(np.arange(65536))
    for half in (lo, hi):
        a = np.abs(half.view(np.float16).astype(np.float64))
        assert a.min() >= 0.125 and a.max() < 2.0
    w = codebook.view(np.float16).astype(np.float64)
    zeros = np.nonzero(w == 0)[0]
    assert len(zeros) == 12
    assert np.all(codebook[zeros] == 0x0000)  # +0, never -0
    nz = np.abs(w[w != 0])
    assert nz.min() == 2.0 ** -13  # no fp16 subnormal can appear
    assert np.abs(w).max() < 4.0
    assert abs(np.mean(w * w) - synth.CODEBOOK_SECOND_MOMENT) < 1e-4


# ------------------------------------------------------------ number formats

def test_f16_decode_matches_numpy(oracle_lib):
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_double(b) for b in bits])
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    assert np.array_equal(np.signbit(got[finite]), np.signbit(ref[finite]))
    assert np.all(np.isnan(got[np.isnan(ref)]))


def test_f16_rne_matches_numpy(oracle_lib):
    gen = np.random.default_rng(3)
    mags = np.exp(gen.uniform(np.log(1e-9), np.log(7e4), 4000))
    vals = mags * np.where(gen.integers(0, 2, mags.size) == 1, -1, 1)
    # exact ties between neighbouring fp16 values, normal and subnormal
    h = gen.integers(1, 0x7BFF, 1000).astype(np.uint16)
    a = h.view(np.float16).astype(np.float64)
    b = (h + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    ties = (a + b) / 2
    vals = np.concatenate([vals, ties, -ties, [65504.0, 65519.99, 65520.0, 2.0 ** -25, 3 * 2.0 ** -26]])
    with np.errstate(over="ignore"):
        ref = vals.astype(np.float16).view(np.uint16)
    got = np.array([oracle.double_to_f16_rne(v) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, ref)


def test_bf16_conversions_match_torch(oracle_lib):
    import torch
    bits = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.bf16_to_double(b) for b in bits])
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    gen = np.random.default_rng(5)
    v32 = (gen.standard_normal(4000) * np.exp(gen.uniform(-20, 20, 4000))).astype(np.float32)
    ref_b = torch.from_numpy(v32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got_b = np.array([oracle.double_to_bf16_rne(float(v)) for v in v32], dtype=np.uint16)
    assert np.array_equal(got_b, ref_b)


# ------------------------------------------------------------ tiles, brute force

def _bitstring_states(words, K):
    """States from a literal '0'/'1' string: word bits LSB first (reading A1),
    the stream repeated once for the wrap (A2), first bit = LSB (A3)."""
    stream = "".join(format(int(w), "016b")[::-1] for w in words)
    assert len(stream) == 256 * K
    stream2 = stream + stream
    return [int(stream2[K * i:K * i + 16][::-1], 2) for i in range(256)]


@pytest.mark.parametrize("K", [2, 3])
@pytest.mark.parametrize("kind", ["random", "zeros", "ones", "alternating"])
def test_tile_decode_brute_force(oracle_lib, K, kind):
    gen = np.random.default_rng(11 + K)
    words = {"random": gen.integers(0, 65536, 16 * K),
             "zeros": np.zeros(16 * K, dtype=np.int64),
             "ones": np.full(16 * K, 0xFFFF),
             "alternating": np.full(16 * K, 0xAAAA)}[kind].astype(np.uint16)
    states = _bitstring_states(words, K)
    for i in (0, 1, 7, 8, 100, 250, 255):
        assert oracle.tile_state(words, K, i) == states[i]
    assert np.array_equal(oracle.decode_tile(words, K), _codebook_numpy(states))


@pytest.mark.parametrize("K", [2, 3])
def test_reconstruct_placement(oracle_lib, K):
    """Reading A4: weight i of tile (kt, nt) lands at W[16nt + i%16][16kt + i//16]."""
    gen = np.random.default_rng(21)
    in_f, out_f = 48, 32
    code = gen.integers(0, 65536, (in_f // 16, out_f // 16, 16 * K)).astype(np.uint16)
    W = oracle.reconstruct(code, in_f, out_f, K)
    for kt in range(in_f // 16):
        for nt in range(out_f // 16):
            tile = _codebook_numpy(_bitstring_states(code[kt, nt], K))
            for i in range(256):
                assert W[16 * nt + i % 16, 16 * kt + i // 16] == tile[i]


# ------------------------------------------------------------ Hadamard

def test_hadamard_is_sylvester_and_orthogonal(oracle_lib):
    H = np.array([[oracle.hadamard_entry(i, j) for j in range(128)] for i in range(128)])
    assert np.array_equal(H, scipy.linalg.hadamard(128))
    assert np.array_equal(H.astype(np.int64) @ H.T.astype(np.int64), 128 * np.eye(128, dtype=np.int64))


def test_hadamard128_transform(oracle_lib):
    Hn = oracle.hadamard128(np.eye(256))  # rows: H_n applied to unit vectors
    ref = np.kron(np.eye(2), scipy.linalg.hadamard(128) / np.sqrt(128))
    assert np.allclose(Hn, ref, atol=1e-15, rtol=0)
    assert np.allclose(Hn @ Hn.T, np.eye(256), atol=1e-13)
    e0 = np.zeros(128)
    e0[0] = 1
    assert np.allclose(oracle.hadamard128(e0), np.full(128, 1 / np.sqrt(128)), atol=1e-16)
    x = np.random.default_rng(2).standard_normal((3, 384))
    y = oracle.hadamard128(x)
    assert np.allclose(oracle.hadamard128(y), x, atol=1e-13)  # involutory
    assert np.allclose(np.sum(y * y, axis=1), np.sum(x * x, axis=1), rtol=1e-13)  # Parseval


# ------------------------------------------------------------ projection

def _small_proj(seed=4, in_f=256, out_f=384, K=2):
    code, rin, rout = synth.single_proj(seed, in_f, out_f, K)
    W = oracle.reconstruct(code, in_f, out_f, K)
    x = np.random.default_rng(seed).standard_normal(in_f)
    return W, rin, rout, x


def _blockdiag_h(n):
    return np.kron(np.eye(n // 128), scipy.linalg.hadamard(128) / np.sqrt(128))


def test_staged_equals_weff(oracle_lib):
    W, rin, rout, x = _small_proj()
    y = oracle.proj(W, rin, rout, x)
    We = oracle.proj_weff(W, rin, rout)
    assert np.allclose(y, We @ x, rtol=0, atol=1e-11 * np.abs(y).max())


def test_transform_order_against_library_matrices(oracle_lib):
    """rin before H on the input, H before rout on the output (reading A8);
    the alternative orders give visibly different outputs on these inputs."""
    W, rin, rout, x = _small_proj()
    Wd = W.view(np.float16).astype(np.float64)
    ri = rin.view(np.float16).astype(np.float64)
    ro = rout.view(np.float16).astype(np.float64)
    Hi, Ho = _blockdiag_h(W.shape[1]), _blockdiag_h(W.shape[0])
    y = oracle.proj(W, rin, rout, x)
    ref = ro * (Ho @ (Wd @ (Hi @ (ri * x))))
    assert np.allclose(y, ref, rtol=0, atol=1e-11 * np.abs(ref).max())
    alt_in = ro * (Ho @ (Wd @ (ri * (Hi @ x))))
    alt_out = Ho @ (ro * (Wd @ (Hi @ (ri * x))))
    for alt in (alt_in, alt_out):
        assert np.linalg.norm(alt - ref) > 0.5 * np.linalg.norm(ref)


def test_all_zero_code_closed_form(oracle_lib):
    """All-zero words: every state is 0, every weight 0x3f60 = 1.84375, so
    W = 1.84375 * J and z is constant; H_n maps a constant block c to
    c*sqrt(128) at index 0 of the block and zeros elsewhere."""
    in_f, out_f, K = 256, 256, 3
    code = np.zeros((in_f // 16, out_f // 16, 16 * K), dtype=np.uint16)
    W = oracle.reconstruct(code, in_f, out_f, K)
    assert np.all(W == 0x3F60) and np.float16(1.84375).view(np.uint16) == 0x3F60
    _, rin, rout = synth.single_proj(9, in_f, out_f, K)
    x = np.random.default_rng(9).standard_normal(in_f)
    ri = rin.view(np.float16).astype(np.float64)
    ro = rout.view(np.float16).astype(np.float64)
    xt = _blockdiag_h(in_f) @ (ri * x)
    c = 1.84375 * xt.sum()
    expect = np.zeros(out_f)
    expect[0::128] = c * np.sqrt(128)
    expect *= ro
    y = oracle.proj(W, rin, rout, x)
    assert np.allclose(y, expect, rtol=0, atol=1e-11 * abs(c) * 12)


def test_nan_weight_is_not_skipped(oracle_lib):
    """0 * NaN must stay NaN: a NaN weight behind a zero rotated activation."""
    W, rin, rout, _ = _small_proj()
    W = W.copy()
    W[5, 3] = 0x7E00
    ri = rin.view(np.float16).astype(np.float64)
    e = np.zeros(W.shape[1])
    e[10] = 1.0
    x = ri * (_blockdiag_h(W.shape[1]) @ e)  # rotated activation = e_10, zero at 3
    y = oracle.proj(W, rin, rout, x)
    assert np.all(np.isnan(y[0:128]))  # the NaN spreads over output block 0
    assert np.all(np.isfinite(y[128:]))


def test_gate_is_first_half(oracle_lib):
    g = np.full(4, -30.0)
    u = np.full(4, 5.0)
    h = oracle.swiglu(np.concatenate([g, u]))
    assert np.all(np.abs(h) < 1e-9)  # a swap would give SiLU(5) * -30 ~ -149
    h2 = oracle.swiglu(np.concatenate([u, g]))
    assert np.all(h2 < -140)


# ------------------------------------------------------------ routing

def test_route_topk_vs_sort_and_softmax(oracle_lib):
    import scipy.special
    logits = synth.normal_logits(1, 16)
    ids, w = oracle.route_topk(logits, 8)
    ref = np.argsort(-logits.astype(np.float64), axis=1, kind="stable")[:, :8]
    assert np.array_equal(ids, ref)
    p = scipy.special.softmax(logits.astype(np.float64), axis=1)
    assert np.allclose(w, np.take_along_axis(p, ref, axis=1), rtol=1e-13, atol=0)


def test_route_tie_goes_to_lower_index(oracle_lib):
    logits = np.zeros((1, 256), dtype=np.float32)
    logits[0, [200, 17, 90, 3, 250, 11, 40, 8, 9]] = 1.0  # nine tied leaders
    ids, w = oracle.route_topk(logits, 8)
    assert list(ids[0]) == [3, 8, 9, 11, 17, 40, 90, 200]
    assert np.allclose(w[0], w[0, 0])


def test_group_vs_stable_argsort(oracle_lib):
    ids, _ = oracle.route_topk(synth.zipf_logits(3, 64), 8)
    counts, offsets, perm = oracle.group(ids, 256)
    flat = ids.ravel()
    assert np.array_equal(counts, np.bincount(flat, minlength=256))
    assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
    assert np.array_equal(perm, np.argsort(flat, kind="stable"))


# ------------------------------------------------------------ MoE layer

def _tiny_layer(seed=5, E=6, H=256, I=128):
    t = synth.layer_tensors(seed, 0, n_experts=E, hidden=H, inter=I)
    return t


def test_layer_matches_composed_projections(oracle_lib):
    L = _tiny_layer()
    H, I = 256, 128
    x = synth.activations(5, 3, H)
    ids = np.array([[0, 3], [5, 0], [2, 2]], dtype=np.int32)
    w = np.array([[0.7, 0.2], [0.5, 0.25], [0.1, 0.3]], dtype=np.float32)
    y, inter, pairs = oracle.moe_layer(L, x, ids, w, want_inter=True, want_pairs=True, n_threads=3)
    for p in range(6):
        t, e = p // 2, ids.ravel()[p]
        xd = np.array([oracle.bf16_to_double(b) for b in x[t]])
        Wgu = oracle.reconstruct(L["gu_code"][e], H, 2 * I, 2)
        Wdn = oracle.reconstruct(L["dn_code"][e], I, H, 3)
        h = oracle.swiglu(oracle.proj(Wgu, L["gu_rin"][e], L["gu_rout"][e], xd))
        assert np.array_equal(inter[p], h)
        assert np.array_equal(pairs[p], oracle.proj(Wdn, L["dn_rin"][e], L["dn_rout"][e], h))
    for t in range(3):
        ref = w[t, 0].astype(np.float64) * pairs[2 * t] + w[t, 1].astype(np.float64) * pairs[2 * t + 1]
        assert np.array_equal(y[t], ref)


def test_pruned_channels_exactly_zero(oracle_lib):
    L = _tiny_layer()
    x = synth.activations(6, 2, 256)
    ids = np.array([[1, 4], [3, 0]], dtype=np.int32)
    w = np.full((2, 2), 0.5, dtype=np.float32)
    _, inter = oracle.moe_layer(L, x, ids, w, want_inter=True)
    for p, e in enumerate(ids.ravel()):
        m = L["mask"][e]
        assert m.any() and np.all(inter[p][m] == 0.0)
        assert np.all(inter[p][~m] != 0.0)


def test_combine_single_slot_and_slot_permutation(oracle_lib):
    L = _tiny_layer()
    x = synth.activations(8, 1, 256)
    ids = np.array([[2, 5, 1]], dtype=np.int32)
    y, pairs = oracle.moe_layer(L, x, ids, np.array([[1, 0, 0]], dtype=np.float32), want_pairs=True)
    assert np.array_equal(y[0], pairs[0])
    w = np.array([[0.5, 0.3, 0.2]], dtype=np.float32)
    y1 = oracle.moe_layer(L, x, ids, w)
    y2 = oracle.moe_layer(L, x, ids[:, [2, 0, 1]], w[:, [2, 0, 1]])
    assert np.allclose(y1, y2, rtol=0, atol=1e-14 * np.abs(y1).max())


def test_expert_gemv_matches_weff(oracle_lib):
    in_f, out_f, K = 256, 256, 2
    code, rin, rout = synth.single_proj(1, in_f, out_f, K)
    x = synth.activations(1, 2, in_f)
    y = oracle.expert_gemv(code, rin, rout, in_f, out_f, K, x)
    We = oracle.proj_weff(oracle.reconstruct(code, in_f, out_f, K), rin, rout)
    xd = np.array([[oracle.bf16_to_double(b) for b in row] for row in x])
    assert np.allclose(y, xd @ We.T, rtol=0, atol=1e-11 * np.abs(y).max())


def test_rmsnorm_closed_forms(oracle_lib):
    y = np.vstack([np.full(2048, 3.0), np.tile([1.0, -2.0], 1024)])
    x = oracle.rmsnorm_bf16(y, 1e-6)
    c0 = 3.0 / np.sqrt(9.0 + 1e-6)
    c1 = 1.0 / np.sqrt(2.5 + 1e-6)
    assert np.all(x[0] == oracle.double_to_bf16_rne(c0))
    assert np.all(x[1, 0::2] == oracle.double_to_bf16_rne(c1))
    assert np.all(x[1, 1::2] == oracle.double_to_bf16_rne(-2 * c1))


# ------------------------------------------------------------ router logits

def _bf16_as_f32(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32)


def test_router_logits_one_hot_rows(oracle_lib):
    """Gate row e = 2^-3 at input e, zero elsewhere: the logit is the fp16
    rounding of x_e / 8 (numpy's float16 cast rounds to nearest even)."""
    T, H, E = 5, 64, 16
    x = synth.activations(61, T, H)
    gate = np.zeros((E, H), dtype=np.uint16)
    gate[np.arange(E), np.arange(E)] = np.float16(0.125).view(np.uint16)
    got = oracle.router_logits(x, gate)
    want = (_bf16_as_f32(x)[:, :E].astype(np.float64) / 8).astype(np.float16).astype(np.float32)
    assert np.array_equal(got, want)


def test_router_logits_vs_numpy_matmul(oracle_lib):
    """Random gate and states against numpy's fp64 matmul and float16 cast."""
    T, H, E = 6, 256, 40
    x = synth.activations(62, T, H)
    gate = synth.router_gate(62, E, H)
    got, raw = oracle.router_logits(x, gate, want_raw=True)
    ref = _bf16_as_f32(x).astype(np.float64) @ gate.view(np.float16).astype(np.float64).T
    assert np.allclose(raw, ref, rtol=0, atol=1e-12)
    assert np.array_equal(got, ref.astype(np.float16).astype(np.float32))
    assert np.abs(got).max() > 0.5  # logits of order one, not all rounded to zero


def test_router_f16_rounding_makes_ties(oracle_lib):
    """Exact sums 1 + 2^-12 (expert 5) and 1 (expert 2) both round to the
    fp16 value 1 (half an ulp at 1 is 2^-11): the logits tie and the top-1
    goes to the lower index, although the exact sums order them the other
    way."""
    H, E = 16, 8
    x = np.zeros((1, H), dtype=np.uint16)
    x[0, 0] = 0x3F80  # 1.0
    x[0, 1] = 0x3980  # 2^-12
    gate = np.zeros((E, H), dtype=np.uint16)
    gate[:, 0] = np.float16(0.25).view(np.uint16)
    gate[5, 0] = gate[2, 0] = np.float16(1.0).view(np.uint16)
    gate[5, 1] = np.float16(1.0).view(np.uint16)
    logits, raw = oracle.router_logits(x, gate, want_raw=True)
    assert raw[0, 5] == 1.0 + 2.0 ** -12 and raw[0, 2] == 1.0
    assert logits[0, 5] == logits[0, 2] == 1.0
    ids, _ = oracle.route_topk(logits, 2)
    assert list(ids[0]) == [2, 5]
    ids_exact, _ = oracle.route_topk(raw.astype(np.float32), 2)
    assert list(ids_exact[0]) == [5, 2]


# ------------------------------------------------------------ shared expert (w8a16)

def test_q8_dequant_is_one_binary32_product(oracle_lib):
    """The exactness table's dequantisation, scale * w8 in f32: numpy's
    float32 multiply (IEEE, round to nearest even) gives the same values,
    over the whole int8 range and random scales."""
    rs = np.random.default_rng(3)
    q = np.arange(-128, 128, dtype=np.int8)
    for scale in rs.uniform(1e-4, 1.0, size=6).astype(np.float32):
        ref = (np.float32(scale) * q.astype(np.float32)).astype(np.float64)
        got = np.array([oracle.q8_weight(int(v), float(scale)) for v in q])
        assert np.array_equal(got, ref)
    # a product that is not exact in binary32 is rounded, not kept in fp64
    s = np.float32(1.0 + 2.0 ** -23)
    assert oracle.q8_weight(3, float(s)) == float(np.float32(s * np.float32(3.0)))
    assert oracle.q8_weight(3, float(s)) != 3.0 * float(s)


def test_q8_linear_vs_numpy_matmul(oracle_lib):
    """Against a numpy fp64 matmul of the numpy-dequantised matrix."""
    S = synth.shared_expert_tensors(5, hidden=256, inter=128)
    W, sc = S["gu_w"], S["gu_s"]
    x = np.random.default_rng(1).standard_normal(W.shape[1])
    deq = (np.repeat(sc, 128, axis=1) * W.astype(np.float32)).astype(np.float64)
    ref = deq @ x
    got = oracle.q8_linear(W, sc, x)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_q8_group_index_is_input_over_128(oracle_lib):
    """Scales 2^g on group g, unit weights: a one-hot input at i returns
    2^(i // 128) on every row (a per-row or i % 128 indexing would not)."""
    out_f, in_f = 4, 512
    W = np.ones((out_f, in_f), dtype=np.int8)
    sc = np.tile(2.0 ** np.arange(in_f // 128), (out_f, 1)).astype(np.float32)
    for i in (0, 127, 128, 300, 511):
        x = np.zeros(in_f)
        x[i] = 1.0
        assert np.all(oracle.q8_linear(W, sc, x) == 2.0 ** (i // 128))


def _tiny_shared(H=128, I=128, q=1, scale=1.0, gate=0.0):
    return dict(gu_w=np.full((2 * I, H), q, np.int8), gu_s=np.full((2 * I, H // 128), scale, np.float32),
                dn_w=np.full((H, I), q, np.int8), dn_s=np.full((H, I // 128), scale, np.float32),
                gate=np.full(H, gate, np.float16).view(np.uint16))


def test_shared_expert_closed_form(oracle_lib):
    """Unit weights and scales s, a constant input a, a zero gate: gate and
    up are s H a, h = SiLU(s H a) s H a, the down output is s I h, and the
    sigmoid of a zero logit is exactly 1/2."""
    H, I, s, a = 128, 128, 0.001, 0.5
    S = _tiny_shared(H, I, 1, s, 0.0)
    x = np.full((1, H), 0x3F00, np.uint16)  # bf16 0.5
    out, g = oracle.shared_expert(S, x, want_gate=True)
    gu = np.float64(np.float32(s)) * H * a
    h = gu / (1.0 + np.exp(-gu)) * gu
    assert g[0] == 0.5
    assert np.allclose(out, 0.5 * np.float64(np.float32(s)) * I * h, rtol=1e-13, atol=0)


def test_shared_expert_gate_is_sigmoid_of_fp16_dot(oracle_lib):
    """Gate row fp16, input one-hot: the logit is that fp16 entry times the
    bf16 input, and the output scales by its logistic function (scipy)."""
    import scipy.special
    H, I = 128, 128
    S = _tiny_shared(H, I, 1, 0.001, 0.0)
    gate = np.zeros(H, np.float16)
    gate[17] = np.float16(-1.375)
    S["gate"] = gate.view(np.uint16)
    x = np.zeros((1, H), np.uint16)
    x[0, 17] = 0x4000  # bf16 2.0
    out, g = oracle.shared_expert(S, x, want_gate=True)
    assert np.isclose(g[0], scipy.special.expit(-2.75), rtol=1e-15)
    S0 = dict(S, gate=np.zeros(H, np.uint16))
    out0 = oracle.shared_expert(S0, x)
    assert np.allclose(out, out0 / 0.5 * g[0], rtol=1e-14, atol=0)


def test_shared_expert_gate_rows_first(oracle_lib):
    """h is SiLU of the first half of gate_up times the second half (the
    halves taken from the int8 product), and swapping the halves changes h."""
    H, I = 128, 128
    S = synth.shared_expert_tensors(9, hidden=H, inter=I)
    x = synth.activations(9, 1, H)
    _, h = oracle.shared_expert(S, x, want_inter=True)
    Sw = dict(S, gu_w=np.concatenate([S["gu_w"][I:], S["gu_w"][:I]]),
              gu_s=np.concatenate([S["gu_s"][I:], S["gu_s"][:I]]))
    _, hw = oracle.shared_expert(Sw, x, want_inter=True)
    xd = np.array([oracle.bf16_to_double(int(v)) for v in x[0]])
    gu = oracle.q8_linear(S["gu_w"], S["gu_s"], xd)
    g, u = gu[:I], gu[I:]
    assert np.allclose(h[0], g / (1 + np.exp(-g)) * u, rtol=1e-12, atol=1e-15)
    assert not np.allclose(h, hw)


# ------------------------------------------------------------ dense projections with bias

def _dense_unbatched(M):
    return {k: (v[0] if k in ("gu_code", "gu_rin", "gu_rout", "dn_code", "dn_rin", "dn_rout") else v)
            for k, v in M.items()}


def test_dense_gemv_bias_vs_weff_matmul(oracle_lib):
    """One coded projection plus its bias against numpy: W_eff @ x + b."""
    M = synth.dense_mlp_tensors(3, hidden=256, inter=128)
    D = _dense_unbatched(M)
    x = synth.activations(3, 2, 256)
    xd = np.array([[oracle.bf16_to_double(int(v)) for v in row] for row in x])
    W = oracle.reconstruct(D["gu_code"], 256, 256, 2)
    Weff = oracle.proj_weff(W, D["gu_rin"], D["gu_rout"])
    ref = xd @ Weff.T + M["gu_bias"].astype(np.float64)
    got = oracle.dense_gemv(D["gu_code"], D["gu_rin"], D["gu_rout"], M["gu_bias"], 256, 256, 2, x)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_dense_mlp_zero_input_isolates_the_biases(oracle_lib):
    """x = 0 makes gate_up's coded output exactly zero, so the MLP reduces to
    h = SiLU(b_gate) * b_up (the gate/up bias before the SwiGLU) and
    y = down(h) + b_down; a bias added after the SwiGLU would give another h."""
    H, I = 256, 128
    M = synth.dense_mlp_tensors(4, hidden=H, inter=I)
    D = _dense_unbatched(M)
    x = np.zeros((1, H), np.uint16)
    y, h = oracle.dense_mlp(M, x, want_inter=True)
    bg, bu = M["gu_bias"][:I].astype(np.float64), M["gu_bias"][I:].astype(np.float64)
    h_ref = bg / (1.0 + np.exp(-bg)) * bu
    assert np.allclose(h[0], h_ref, rtol=1e-14, atol=0)
    Wd = oracle.reconstruct(D["dn_code"], I, H, 3)
    y_ref = oracle.proj_weff(Wd, D["dn_rin"], D["dn_rout"]) @ h_ref + M["dn_bias"].astype(np.float64)
    assert np.allclose(y[0], y_ref, rtol=1e-12, atol=1e-12 * np.abs(y_ref).max())
    h_after = np.zeros(I) + M["gu_bias"][:I]  # SiLU(0) * 0 + bias: the wrong placement
    assert not np.allclose(h[0], h_after)


def test_dense_mlp_without_bias_is_the_one_expert_layer(oracle_lib):
    """A dense MLP is the routed layer with one expert, id 0, weight 1."""
    H, I = 256, 128
    M = synth.dense_mlp_tensors(5, hidden=H, inter=I)
    M0 = dict(M, gu_bias=None, dn_bias=None)
    x = synth.activations(5, 3, H)
    y = oracle.dense_mlp(M0, x)
    ids = np.zeros((3, 1), np.int32)
    w = np.ones((3, 1), np.float32)
    ref = oracle.moe_layer(M, x, ids, w)
    assert np.array_equal(y, ref)
