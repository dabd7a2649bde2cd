"""Seeded synthetic inputs for the trellis-coded MoE expert path.

This module holds no arithmetic of the method: it draws code bytes, sign and
scale vectors, prune masks, activations and router logits from seeded numpy
streams. Both the GPU tests and the CPU oracle's tests take their inputs from
here, so the two sides always see identical bytes. Every tensor has its own
stream ``default_rng([seed, layer, expert, tensor_id])`` and can therefore be
regenerated alone (the oracle only rebuilds the experts it needs).

Workload shapes follow the Qwen3.6-35B-A3B-class expert layer: hidden 2048,
256 experts, top-8, expert width 512; gate_up (2048 -> 1024, K=2) and down
(512 -> 2048, K=3). Code words are uniform random, so trellis states are
uniform over the 65,536-state alphabet, as in a real projection.
"""
from __future__ import annotations

import numpy as np

HIDDEN = 2048
INTER = 512
N_EXPERTS = 256
TOP_K = 8
K_GU = 2
K_DN = 3

# Second moment of the decoded codebook over uniform states (a fixed number
# of the format, used here only to size the synthetic output scales so that
# activations stay O(1) through the layer).
CODEBOOK_SECOND_MOMENT = 1.5478

# tensor ids inside one (layer, expert) stream family
_T_CODE, _T_RIN, _T_ROUT, _T_MASK = 0, 1, 2, 3
_GU, _DN = 0, 10
_T_X, _T_LOGITS, _T_POP, _T_GATE = 100, 101, 102, 103

F16_ONE = 0x3C00
F16_MINUS_ONE = 0xBC00


def rng(seed: int, *ids: int) -> np.random.Generator:
    return np.random.default_rng([int(seed)] + [int(i) for i in ids])


def code_words(seed: int, layer: int, expert: int, proj: int, in_f: int, out_f: int,
               K: int) -> np.ndarray:
    """uint16 [in/16][out/16][16K], uniform random words."""
    n_words = (in_f // 16) * (out_f // 16) * 16 * K
    raw = rng(seed, layer, expert, proj + _T_CODE).bytes(2 * n_words)
    return np.frombuffer(raw, dtype=np.uint16).reshape(in_f // 16, out_f // 16, 16 * K)


def sign_vector(seed: int, layer: int, expert: int, proj: int, n: int) -> np.ndarray:
    """fp16 bits of +-1 with random signs."""
    s = rng(seed, layer, expert, proj + _T_RIN).integers(0, 2, size=n)
    return np.where(s == 1, F16_MINUS_ONE, F16_ONE).astype(np.uint16)


def prune_mask(seed: int, layer: int, expert: int, inter: int,
               lo: float = 0.14, hi: float = 0.58) -> np.ndarray:
    """bool [inter], True = pruned. The pruned fraction is U(lo, hi) per expert."""
    g = rng(seed, layer, expert, _T_MASK)
    frac = g.uniform(lo, hi)
    n_pruned = int(round(frac * inter))
    mask = np.zeros(inter, dtype=bool)
    mask[g.permutation(inter)[:n_pruned]] = True
    return mask


def scale_vector(seed: int, layer: int, expert: int, proj: int, n: int, scale: float,
                 zero: np.ndarray | None = None) -> np.ndarray:
    """fp16 bits of +-U(0.5, 2) * scale; entries where ``zero`` is True are +0."""
    g = rng(seed, layer, expert, proj + _T_ROUT)
    mag = g.uniform(0.5, 2.0, size=n) * scale
    sgn = np.where(g.integers(0, 2, size=n) == 1, -1.0, 1.0)
    v = (sgn * mag).astype(np.float16)
    if zero is not None:
        v[zero] = np.float16(0.0)
    return v.view(np.uint16).copy()


def fanin_scale(in_f: int) -> float:
    return 1.0 / (np.sqrt(CODEBOOK_SECOND_MOMENT) * np.sqrt(in_f))


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits (round to nearest even, via torch's conversion)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def activations(seed: int, T: int, n: int, layer: int = 0) -> np.ndarray:
    """bf16 bits [T][n] of N(0, 1)."""
    x = rng(seed, layer, 0, _T_X).standard_normal((T, n)).astype(np.float32)
    return to_bf16_bits(x)


def router_gate(seed: int, E: int = N_EXPERTS, n: int = HIDDEN, layer: int = 0) -> np.ndarray:
    """fp16 bits [E][n] of N(0, 1/n): a router gate whose logits on N(0, 1)
    hidden states are about N(0, 1), like the routing workloads' logits."""
    g = rng(seed, layer, 0, _T_GATE).standard_normal((E, n)) / np.sqrt(n)
    return g.astype(np.float16).view(np.uint16).copy()


def normal_logits(seed: int, T: int, E: int = N_EXPERTS, layer: int = 0) -> np.ndarray:
    return rng(seed, layer, 0, _T_LOGITS).standard_normal((T, E)).astype(np.float32)


def zipf_logits(seed: int, T: int, E: int = N_EXPERTS, s: float = 1.1, layer: int = 0) -> np.ndarray:
    """Skewed popularity: logit = -s*ln(rank) + Gumbel noise.

    Taking the top-k of Gumbel-perturbed log-weights draws k experts without
    replacement with probabilities proportional to rank^-s (Zipf). The
    popularity ranking itself is a seeded permutation of the experts.
    """
    g = rng(seed, layer, 0, _T_POP)
    rank = np.empty(E, dtype=np.float64)
    rank[g.permutation(E)] = np.arange(1, E + 1)
    gumbel = rng(seed, layer, 0, _T_LOGITS).gumbel(size=(T, E))
    return (-s * np.log(rank)[None, :] + gumbel).astype(np.float32)


# ---------------------------------------------------------------- projections

def single_proj(seed: int, in_f: int, out_f: int, K: int, *, unit_scale: bool = True,
                layer: int = 0, expert: int = 0, proj: int = _GU):
    """One coded matrix: (code, rin, rout). unit_scale: rout = +-U(0.5, 2)."""
    code = code_words(seed, layer, expert, proj, in_f, out_f, K)
    rin = sign_vector(seed, layer, expert, proj, in_f)
    rout = scale_vector(seed, layer, expert, proj, out_f,
                        1.0 if unit_scale else fanin_scale(in_f))
    return code, rin, rout


def expert_tensors(seed: int, layer: int, expert: int, hidden: int = HIDDEN, inter: int = INTER,
                   k_gu: int = K_GU, k_dn: int = K_DN, masks: bool = True):
    """All leaves of one expert: gate_up and down (code, rin, rout) + its mask."""
    mask = prune_mask(seed, layer, expert, inter) if masks else np.zeros(inter, dtype=bool)
    gu_code = code_words(seed, layer, expert, _GU, hidden, 2 * inter, k_gu)
    gu_rin = sign_vector(seed, layer, expert, _GU, hidden)
    gu_rout = scale_vector(seed, layer, expert, _GU, 2 * inter, fanin_scale(hidden),
                           zero=np.concatenate([mask, mask]))
    dn_code = code_words(seed, layer, expert, _DN, inter, hidden, k_dn)
    dn_rin = sign_vector(seed, layer, expert, _DN, inter)
    dn_rout = scale_vector(seed, layer, expert, _DN, hidden, fanin_scale(inter))
    return dict(gu_code=gu_code, gu_rin=gu_rin, gu_rout=gu_rout, dn_code=dn_code,
                dn_rin=dn_rin, dn_rout=dn_rout, mask=mask)


def layer_tensors(seed: int, layer: int, n_experts: int = N_EXPERTS, experts=None, **kw):
    """Stacked leaves of a layer, [E][...] each. ``experts`` limits which
    experts carry generated data (the others are left zero), which the
    oracle uses to rebuild only what a routing touches."""
    todo = list(range(n_experts)) if experts is None else sorted(set(int(e) for e in experts))
    out = None
    for e in todo:
        t = expert_tensors(seed, layer, e, **kw)
        if out is None:
            alloc = np.empty if experts is None else np.zeros
            out = {k: alloc((n_experts,) + v.shape, dtype=v.dtype) for k, v in t.items()}
        for k, v in t.items():
            out[k][e] = v
    if out is None:  # no expert requested: shapes from expert 0, all zero
        t = expert_tensors(seed, layer, 0, **kw)
        out = {k: np.zeros((n_experts,) + v.shape, dtype=v.dtype) for k, v in t.items()}
    return out


# ---------------------------------------------------------------- dense projections

_BIAS = 30  # tensor ids of dense biases: _BIAS + 0 (gate_up), + 1 (down)


def dense_mlp_tensors(seed: int, layer: int = 0, hidden: int = HIDDEN, inter: int = INTER,
                      k_gu: int = K_GU, k_dn: int = K_DN, bias_scale: float = 0.25):
    """A dense MLP of coded projections (the one-expert case, no prune mask):
    the leaves of expert 0 at [1][...] plus f32 output biases of
    N(0, bias_scale^2) on gate_up [2*inter] and down [hidden]."""
    t = expert_tensors(seed, layer, 0, hidden=hidden, inter=inter, k_gu=k_gu, k_dn=k_dn, masks=False)
    out = {k: v[None] for k, v in t.items() if k != "mask"}
    out["gu_bias"] = (rng(seed, layer, 0, _BIAS).standard_normal(2 * inter) * bias_scale).astype(np.float32)
    out["dn_bias"] = (rng(seed, layer, 0, _BIAS + 1).standard_normal(hidden) * bias_scale).astype(np.float32)
    return out


# ---------------------------------------------------------------- shared expert

SHARED_INTER = 512
_SH = 20  # tensor ids of the shared expert: _SH + 0..4
# second moment of a uniform int8 value over [-128, 127]
INT8_SECOND_MOMENT = (sum(q * q for q in range(-128, 128)) / 256.0)


def shared_expert_tensors(seed: int, layer: int = 0, hidden: int = HIDDEN, inter: int = SHARED_INTER):
    """The shared expert of a layer in the w8a16 form: int8 weights uniform
    over [-128, 127] (gate_up [2*inter][hidden], gate rows first; down
    [hidden][inter]), f32 scales per group of 128 inputs of
    U(0.5, 2) / (sqrt(E[q^2]) sqrt(in)) (outputs stay O(1)), and the fp16
    shared_expert_gate row [hidden] of N(0, 1/hidden)."""
    def q8(tid, out_f, in_f):
        g = rng(seed, layer, 0, _SH + tid)
        w = g.integers(-128, 128, size=(out_f, in_f), dtype=np.int16).astype(np.int8)
        sc = (g.uniform(0.5, 2.0, size=(out_f, in_f // 128)) /
              (np.sqrt(INT8_SECOND_MOMENT) * np.sqrt(in_f))).astype(np.float32)
        return w, sc
    gu_w, gu_s = q8(0, 2 * inter, hidden)
    dn_w, dn_s = q8(1, hidden, inter)
    gate = (rng(seed, layer, 0, _SH + 2).standard_normal(hidden) / np.sqrt(hidden)).astype(np.float16)
    return dict(gu_w=gu_w, gu_s=gu_s, dn_w=dn_w, dn_s=dn_s, gate=gate.view(np.uint16).copy())


# ---------------------------------------------------------------- workloads

def stack_token_inputs(seed: int, n_layers: int, T: int, entry: int, E: int = N_EXPERTS,
                       hidden: int = HIDDEN):
    """Inputs of one decode step of the layer stack: x0 bf16 bits [T][hidden]
    and router logits fp32 [n_layers][T][E], N(0, 1). ``entry`` selects one
    of several independent steps (a pool the benchmark cycles through)."""
    x0 = activations(seed, T, hidden, layer=100000 + entry)
    logits = np.stack([normal_logits(seed, T, E, layer=1000 * (entry + 1) + l)
                       for l in range(n_layers)])
    return x0, logits


CONFIGS = {
    1: dict(name="gemv-256x256-k2", in_f=256, out_f=256, K=2, T=1),
    2: dict(name="layer-decode-b1", T=1, logits="normal"),
    3: dict(name="layer-decode-b64-zipf1.1", T=64, logits="zipf"),
    4: dict(name="stack-40x256-decode", layers=40, T=(1, 8), logits="normal"),
    5: dict(name="layer-prefill-4096", T=4096, logits="normal", oracle_tokens=256),
}
