"""CPU oracle for the trellis-coded ("eschamoe") routed-expert path.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. It shares no
code with the GPU library and never imports it.

The arithmetic lives in ``escha_oracle.c`` (plain loops, fp64), compiled with
gcc into ``liboracle.so`` next to this file. This module is argument
marshalling over ctypes plus numpy views; see the C file's header for the
pages it follows and the readings it takes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "escha_oracle.c"
_LIB_PATH = _HERE / "liboracle.so"

_u16p = ctypes.POINTER(ctypes.c_uint16)
_i32p = ctypes.POINTER(ctypes.c_int32)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i8p = ctypes.POINTER(ctypes.c_int8)


def build(force: bool = True) -> Path:
    """Compile liboracle.so with gcc (IEEE fp64, no contraction, no fast-math)."""
    if force or not _LIB_PATH.exists():
        tmp = _LIB_PATH.with_suffix(".so.tmp%d" % os.getpid())
        cmd = [
            "gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
            "-ffp-contract=off", "-fno-fast-math", "-fvisibility=hidden",
            "-Wall", "-Wextra", "-Wno-unused-parameter",
            str(_SRC), "-o", str(tmp), "-lm",
        ]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Layer(ctypes.Structure):
    _fields_ = [
        ("gu_code", _u16p), ("gu_rin", _u16p), ("gu_rout", _u16p),
        ("dn_code", _u16p), ("dn_rin", _u16p), ("dn_rout", _u16p),
        ("n_experts", ctypes.c_int32), ("hidden", ctypes.c_int32),
        ("inter", ctypes.c_int32), ("k_gu", ctypes.c_int32),
        ("k_dn", ctypes.c_int32), ("top_k", ctypes.c_int32),
    ]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not _LIB_PATH.exists() or _LIB_PATH.stat().st_mtime < _SRC.stat().st_mtime:
            build()
        L = ctypes.CDLL(str(_LIB_PATH))
        L.eo_f16_to_double.argtypes = [ctypes.c_uint16]
        L.eo_f16_to_double.restype = ctypes.c_double
        L.eo_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.eo_bf16_to_double.restype = ctypes.c_double
        L.eo_double_to_f16_rne.argtypes = [ctypes.c_double]
        L.eo_double_to_f16_rne.restype = ctypes.c_uint16
        L.eo_double_to_bf16_rne.argtypes = [ctypes.c_double]
        L.eo_double_to_bf16_rne.restype = ctypes.c_uint16
        L.eo_cba_decode_state.argtypes = [ctypes.c_uint32]
        L.eo_cba_decode_state.restype = ctypes.c_uint16
        L.eo_tile_state.argtypes = [_u16p, ctypes.c_int, ctypes.c_int]
        L.eo_tile_state.restype = ctypes.c_uint32
        L.eo_decode_tile.argtypes = [_u16p, ctypes.c_int, _u16p]
        L.eo_decode_tile.restype = None
        L.eo_reconstruct.argtypes = [_u16p, ctypes.c_int, ctypes.c_int, ctypes.c_int, _u16p]
        L.eo_reconstruct.restype = ctypes.c_int
        L.eo_hadamard_entry.argtypes = [ctypes.c_int, ctypes.c_int]
        L.eo_hadamard_entry.restype = ctypes.c_double
        L.eo_hadamard128.argtypes = [_f64p, ctypes.c_int64, ctypes.c_int, _f64p]
        L.eo_hadamard128.restype = None
        L.eo_proj.argtypes = [_u16p, _u16p, _u16p, ctypes.c_int, ctypes.c_int, _f64p, _f64p]
        L.eo_proj.restype = None
        L.eo_proj_weff.argtypes = [_u16p, _u16p, _u16p, ctypes.c_int, ctypes.c_int, _f64p]
        L.eo_proj_weff.restype = None
        L.eo_swiglu.argtypes = [_f64p, ctypes.c_int, _f64p]
        L.eo_swiglu.restype = None
        L.eo_route_topk.argtypes = [_f32p, ctypes.c_int, ctypes.c_int, ctypes.c_int, _i32p, _f64p]
        L.eo_route_topk.restype = None
        L.eo_router_logits.argtypes = [_u16p, ctypes.c_int, ctypes.c_int, _u16p, ctypes.c_int, _f32p,
                                       _f64p]
        L.eo_router_logits.restype = None
        L.eo_group.argtypes = [_i32p, ctypes.c_int, ctypes.c_int, ctypes.c_int, _i32p, _i32p, _i32p]
        L.eo_group.restype = None
        L.eo_moe_layer.argtypes = [ctypes.POINTER(_Layer), _u16p, ctypes.c_int, _i32p, _f32p,
                                   _f64p, _f64p, _f64p, ctypes.c_int]
        L.eo_moe_layer.restype = ctypes.c_int
        L.eo_expert_gemv.argtypes = [_u16p, _u16p, _u16p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     _u16p, ctypes.c_int, _f64p]
        L.eo_expert_gemv.restype = ctypes.c_int
        L.eo_dense_gemv.argtypes = [_u16p, _u16p, _u16p, _f32p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                    _u16p, ctypes.c_int, _f64p]
        L.eo_dense_gemv.restype = ctypes.c_int
        L.eo_dense_mlp.argtypes = [_u16p, _u16p, _u16p, _f32p, _u16p, _u16p, _u16p, _f32p, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_int, _u16p, ctypes.c_int, _f64p,
                                   _f64p]
        L.eo_dense_mlp.restype = ctypes.c_int
        L.eo_q8_weight.argtypes = [ctypes.c_int8, ctypes.c_float]
        L.eo_q8_weight.restype = ctypes.c_double
        L.eo_q8_linear.argtypes = [_i8p, _f32p, ctypes.c_int, ctypes.c_int, _f64p, _f64p]
        L.eo_q8_linear.restype = None
        L.eo_shared_expert.argtypes = [_i8p, _f32p, _i8p, _f32p, _u16p, ctypes.c_int, ctypes.c_int,
                                       _u16p, ctypes.c_int, _f64p, _f64p, _f64p]
        L.eo_shared_expert.restype = ctypes.c_int
        L.eo_rmsnorm_bf16.argtypes = [_f64p, ctypes.c_int, ctypes.c_int, ctypes.c_double, _u16p]
        L.eo_rmsnorm_bf16.restype = None
        _lib = L
    return _lib


def _p(a: np.ndarray, ct):
    return a.ctypes.data_as(ct)


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a), dtype=dtype)


# ---------------------------------------------------------------- scalars

def f16_to_double(h: int) -> float:
    return lib().eo_f16_to_double(int(h))


def bf16_to_double(b: int) -> float:
    return lib().eo_bf16_to_double(int(b))


def double_to_f16_rne(v: float) -> int:
    return int(lib().eo_double_to_f16_rne(float(v)))


def double_to_bf16_rne(v: float) -> int:
    return int(lib().eo_double_to_bf16_rne(float(v)))


def cba_decode_state(s: int) -> int:
    """fp16 bits of the weight that 16-bit state ``s`` decodes to."""
    return int(lib().eo_cba_decode_state(int(s)))


def codebook() -> np.ndarray:
    """All 65,536 states decoded, as uint16 fp16 bits (state order)."""
    return np.array([cba_decode_state(s) for s in range(65536)], dtype=np.uint16)


# ---------------------------------------------------------------- tiles

def tile_state(words, K: int, i: int) -> int:
    w = _c(words, np.uint16)
    assert w.size == 16 * K
    return int(lib().eo_tile_state(_p(w, _u16p), K, i))


def decode_tile(words, K: int) -> np.ndarray:
    """256 fp16 bit patterns of one tile, in weight order i."""
    w = _c(words, np.uint16)
    assert w.size == 16 * K
    out = np.zeros(256, dtype=np.uint16)
    lib().eo_decode_tile(_p(w, _u16p), K, _p(out, _u16p))
    return out


def reconstruct(code, in_f: int, out_f: int, K: int) -> np.ndarray:
    """code uint16 [in/16][out/16][16K] -> W fp16 bits [out][in]."""
    c = _c(code, np.uint16)
    assert c.size == (in_f // 16) * (out_f // 16) * 16 * K
    W = np.zeros((out_f, in_f), dtype=np.uint16)
    rc = lib().eo_reconstruct(_p(c, _u16p), in_f, out_f, K, _p(W, _u16p))
    if rc:
        raise ValueError("reconstruct: bad shape")
    return W


# ---------------------------------------------------------------- transforms

def hadamard_entry(i: int, j: int) -> float:
    return lib().eo_hadamard_entry(i, j)


def hadamard128(x) -> np.ndarray:
    a = _c(x, np.float64)
    n = a.shape[-1]
    assert n % 128 == 0
    rows = a.size // n
    y = np.zeros_like(a)
    lib().eo_hadamard128(_p(a, _f64p), rows, n, _p(y, _f64p))
    return y


def proj(W, rin, rout, x) -> np.ndarray:
    """Staged projection of one activation vector (double) -> double [out]."""
    Wc = _c(W, np.uint16)
    out_f, in_f = Wc.shape
    rin_c, rout_c, xc = _c(rin, np.uint16), _c(rout, np.uint16), _c(x, np.float64)
    assert rin_c.size == in_f and rout_c.size == out_f and xc.size == in_f
    y = np.zeros(out_f, dtype=np.float64)
    lib().eo_proj(_p(Wc, _u16p), _p(rin_c, _u16p), _p(rout_c, _u16p), in_f, out_f,
                  _p(xc, _f64p), _p(y, _f64p))
    return y


def proj_weff(W, rin, rout) -> np.ndarray:
    Wc = _c(W, np.uint16)
    out_f, in_f = Wc.shape
    rin_c, rout_c = _c(rin, np.uint16), _c(rout, np.uint16)
    We = np.zeros((out_f, in_f), dtype=np.float64)
    lib().eo_proj_weff(_p(Wc, _u16p), _p(rin_c, _u16p), _p(rout_c, _u16p), in_f, out_f,
                       _p(We, _f64p))
    return We


def swiglu(y_gu) -> np.ndarray:
    y = _c(y_gu, np.float64)
    inter = y.size // 2
    h = np.zeros(inter, dtype=np.float64)
    lib().eo_swiglu(_p(y, _f64p), inter, _p(h, _f64p))
    return h


# ---------------------------------------------------------------- routing

def route_topk(logits, top_k: int):
    """logits fp32 [T][E] -> (ids int32 [T][k], w double [T][k])."""
    l = _c(logits, np.float32)
    T, E = l.shape
    ids = np.zeros((T, top_k), dtype=np.int32)
    w = np.zeros((T, top_k), dtype=np.float64)
    lib().eo_route_topk(_p(l, _f32p), T, E, top_k, _p(ids, _i32p), _p(w, _f64p))
    return ids, w


def router_logits(x_bf16, gate_f16, *, want_raw=False):
    """x bf16 bits [T][H], gate fp16 bits [E][H] -> logits fp32 [T][E] (each
    an fp16 value: the rounded exact dot product), and the fp64 sums."""
    x = _c(x_bf16, np.uint16)
    g = _c(gate_f16, np.uint16)
    T, H = x.shape
    E = g.shape[0]
    assert g.shape[1] == H
    logits = np.zeros((T, E), dtype=np.float32)
    raw = np.zeros((T, E), dtype=np.float64)
    lib().eo_router_logits(_p(x, _u16p), T, H, _p(g, _u16p), E, _p(logits, _f32p), _p(raw, _f64p))
    return (logits, raw) if want_raw else logits


def group(ids, n_experts: int):
    """ids [T][k] -> (counts [E], offsets [E+1], perm [T*k])."""
    i = _c(ids, np.int32)
    T, k = i.shape
    counts = np.zeros(n_experts, dtype=np.int32)
    offsets = np.zeros(n_experts + 1, dtype=np.int32)
    perm = np.zeros(T * k, dtype=np.int32)
    lib().eo_group(_p(i, _i32p), T, k, n_experts, _p(counts, _i32p), _p(offsets, _i32p),
                   _p(perm, _i32p))
    return counts, offsets, perm


# ---------------------------------------------------------------- layer

def moe_layer(layer: dict, x_bf16, ids, w, *, want_inter=False, want_pairs=False,
              n_threads: int = 0):
    """One MoE layer on the CPU.

    ``layer`` holds uint16 numpy arrays ``gu_code [E][H/16][2I/16][16Kgu]``,
    ``gu_rin [E][H]``, ``gu_rout [E][2I]``, ``dn_code [E][I/16][H/16][16Kdn]``,
    ``dn_rin [E][I]``, ``dn_rout [E][H]`` (fp16 bits). ``x_bf16`` uint16
    [T][H]; ``ids`` int32 [T][k]; ``w`` fp32 [T][k]. Returns ``y`` double
    [T][H] and, on request, ``inter`` [T*k][I] and per-pair outputs.
    """
    arrs = {n: _c(layer[n], np.uint16) for n in
            ("gu_code", "gu_rin", "gu_rout", "dn_code", "dn_rin", "dn_rout")}
    E = arrs["gu_code"].shape[0]
    H = arrs["gu_rin"].shape[1]
    I = arrs["dn_rin"].shape[1]
    k_gu = arrs["gu_code"].shape[-1] // 16
    k_dn = arrs["dn_code"].shape[-1] // 16
    x = _c(x_bf16, np.uint16).reshape(-1, H)
    T = x.shape[0]
    ids_c = _c(ids, np.int32).reshape(T, -1)
    top_k = ids_c.shape[1]
    w_c = _c(w, np.float32).reshape(T, top_k)
    L = _Layer(_p(arrs["gu_code"], _u16p), _p(arrs["gu_rin"], _u16p), _p(arrs["gu_rout"], _u16p),
               _p(arrs["dn_code"], _u16p), _p(arrs["dn_rin"], _u16p), _p(arrs["dn_rout"], _u16p),
               E, H, I, k_gu, k_dn, top_k)
    y = np.zeros((T, H), dtype=np.float64)
    inter = np.zeros((T * top_k, I), dtype=np.float64) if want_inter else None
    pairs = np.zeros((T * top_k, H), dtype=np.float64) if want_pairs else None
    rc = lib().eo_moe_layer(ctypes.byref(L), _p(x, _u16p), T, _p(ids_c, _i32p), _p(w_c, _f32p),
                            _p(y, _f64p), _p(inter, _f64p) if inter is not None else None,
                            _p(pairs, _f64p) if pairs is not None else None, int(n_threads))
    if rc:
        raise ValueError("moe_layer failed with code %d" % rc)
    out = [y]
    if want_inter:
        out.append(inter)
    if want_pairs:
        out.append(pairs)
    return out[0] if len(out) == 1 else tuple(out)


def expert_gemv(code, rin, rout, in_f: int, out_f: int, K: int, x_bf16) -> np.ndarray:
    c, ri, ro = _c(code, np.uint16), _c(rin, np.uint16), _c(rout, np.uint16)
    x = _c(x_bf16, np.uint16).reshape(-1, in_f)
    T = x.shape[0]
    y = np.zeros((T, out_f), dtype=np.float64)
    rc = lib().eo_expert_gemv(_p(c, _u16p), _p(ri, _u16p), _p(ro, _u16p), in_f, out_f, K,
                              _p(x, _u16p), T, _p(y, _f64p))
    if rc:
        raise ValueError("expert_gemv: bad shape")
    return y


def rmsnorm_bf16(y, eps: float = 1e-6) -> np.ndarray:
    yc = _c(y, np.float64)
    T, n = yc.shape
    x = np.zeros((T, n), dtype=np.uint16)
    lib().eo_rmsnorm_bf16(_p(yc, _f64p), T, n, float(eps), _p(x, _u16p))
    return x


# ---------------------------------------------------------------- shared expert

def q8_weight(q: int, scale: float) -> float:
    """The f32 dequantised int8 weight scale * q."""
    return float(lib().eo_q8_weight(int(q), float(scale)))


def q8_linear(W, scales, x) -> np.ndarray:
    """y = dequant(W) x in fp64: W int8 [out][in], scales f32 [out][in/128], x [in]."""
    Wc = _c(W, np.int8)
    out_f, in_f = Wc.shape
    sc = _c(scales, np.float32)
    xc = _c(x, np.float64)
    y = np.zeros(out_f, dtype=np.float64)
    lib().eo_q8_linear(_p(Wc, _i8p), _p(sc, _f32p), in_f, out_f, _p(xc, _f64p), _p(y, _f64p))
    return y


def shared_expert(S: dict, x_bf16, *, want_gate=False, want_inter=False):
    """Shared expert + sigmoid gate of every token: S holds ``gu_w`` int8
    [2I][H], ``gu_s`` f32 [2I][H/128], ``dn_w`` int8 [H][I], ``dn_s`` f32
    [H][I/128], ``gate`` fp16 bits [H]. Returns out double [T][H] (and the
    gates [T], the intermediate h [T][I] on request)."""
    gu_w, gu_s = _c(S["gu_w"], np.int8), _c(S["gu_s"], np.float32)
    dn_w, dn_s = _c(S["dn_w"], np.int8), _c(S["dn_s"], np.float32)
    gate = _c(S["gate"], np.uint16)
    H = gu_w.shape[1]
    I = dn_w.shape[1]
    x = _c(x_bf16, np.uint16).reshape(-1, H)
    T = x.shape[0]
    out = np.zeros((T, H), dtype=np.float64)
    g = np.zeros(T, dtype=np.float64)
    h = np.zeros((T, I), dtype=np.float64)
    rc = lib().eo_shared_expert(_p(gu_w, _i8p), _p(gu_s, _f32p), _p(dn_w, _i8p), _p(dn_s, _f32p),
                                _p(gate, _u16p), H, I, _p(x, _u16p), T, _p(out, _f64p), _p(g, _f64p),
                                _p(h, _f64p))
    if rc:
        raise ValueError("shared_expert: bad shape")
    res = [out]
    if want_gate:
        res.append(g)
    if want_inter:
        res.append(h)
    return res[0] if len(res) == 1 else tuple(res)


# ---------------------------------------------------------------- dense projections with bias

def dense_gemv(code, rin, rout, bias, in_f: int, out_f: int, K: int, x_bf16) -> np.ndarray:
    """One coded projection (the one-expert case) plus an f32 output bias (or None)."""
    c, ri, ro = _c(code, np.uint16), _c(rin, np.uint16), _c(rout, np.uint16)
    b = None if bias is None else _c(bias, np.float32)
    x = _c(x_bf16, np.uint16).reshape(-1, in_f)
    T = x.shape[0]
    y = np.zeros((T, out_f), dtype=np.float64)
    rc = lib().eo_dense_gemv(_p(c, _u16p), _p(ri, _u16p), _p(ro, _u16p), _p(b, _f32p) if b is not None else None,
                             in_f, out_f, K, _p(x, _u16p), T, _p(y, _f64p))
    if rc:
        raise ValueError("dense_gemv: bad shape")
    return y


def dense_mlp(M: dict, x_bf16, *, want_inter=False):
    """A dense MLP of coded projections with f32 biases: M holds ``gu_code``
    [H/16][2I/16][16Kgu], ``gu_rin``, ``gu_rout``, ``gu_bias`` (f32 [2I] or
    None), ``dn_code``, ``dn_rin``, ``dn_rout``, ``dn_bias`` (f32 [H] or None).
    Returns y double [T][H] (and h [T][I])."""
    a = {n: _c(M[n], np.uint16) for n in ("gu_code", "gu_rin", "gu_rout", "dn_code", "dn_rin", "dn_rout")}
    gb = None if M.get("gu_bias") is None else _c(M["gu_bias"], np.float32)
    db = None if M.get("dn_bias") is None else _c(M["dn_bias"], np.float32)
    H = a["gu_rin"].shape[-1]
    I = a["dn_rin"].shape[-1]
    k_gu = a["gu_code"].shape[-1] // 16
    k_dn = a["dn_code"].shape[-1] // 16
    x = _c(x_bf16, np.uint16).reshape(-1, H)
    T = x.shape[0]
    y = np.zeros((T, H), dtype=np.float64)
    h = np.zeros((T, I), dtype=np.float64)
    rc = lib().eo_dense_mlp(_p(a["gu_code"], _u16p), _p(a["gu_rin"], _u16p), _p(a["gu_rout"], _u16p),
                            _p(gb, _f32p) if gb is not None else None, _p(a["dn_code"], _u16p),
                            _p(a["dn_rin"], _u16p), _p(a["dn_rout"], _u16p),
                            _p(db, _f32p) if db is not None else None, H, I, k_gu, k_dn, _p(x, _u16p), T,
                            _p(y, _f64p), _p(h, _f64p))
    if rc:
        raise ValueError("dense_mlp: bad shape")
    return (y, h) if want_inter else y
