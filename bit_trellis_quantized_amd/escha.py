"""Python binding of libescha.so (the C ABI in include/escha.h).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, their pointers and the current HIP stream are handed to the C
entry point of the same name, and a non-zero status becomes ``EschaError``.
Every step of the path runs in the library's HIP kernels; if the library is
missing, importing this module raises.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from pathlib import Path

import torch

_LIB_PATH = Path(__file__).resolve().parent / "libescha.so"

if not _LIB_PATH.exists():
    raise ImportError(
        f"{_LIB_PATH} is not built; run `python -m bit_trellis_quantized_amd.build` "
        "(the trellis path has no fallback)")

_lib = ctypes.CDLL(str(_LIB_PATH))

ESCHA_OK = 0
STATUS_INCOMPLETE = 1  # escha_moe_stack_status: a dependency wait gave up
STATUS = {
    -1: "ESCHA_E_NULL", -2: "ESCHA_E_SHAPE", -3: "ESCHA_E_KBITS", -4: "ESCHA_E_WORKSPACE",
    -5: "ESCHA_E_HIP", -6: "ESCHA_E_UNSUPPORTED", -7: "ESCHA_E_ARG",
}


class EschaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


class escha_proj_t(ctypes.Structure):
    _fields_ = [("code", ctypes.c_void_p), ("rin", ctypes.c_void_p), ("rout", ctypes.c_void_p),
                ("n_experts", ctypes.c_int32), ("in_features", ctypes.c_int32),
                ("out_features", ctypes.c_int32), ("k_bits", ctypes.c_int32)]


class escha_shared_expert_t(ctypes.Structure):
    _fields_ = [("gate_up", ctypes.c_void_p), ("gate_up_scale", ctypes.c_void_p), ("down", ctypes.c_void_p),
                ("down_scale", ctypes.c_void_p), ("gate", ctypes.c_void_p), ("hidden", ctypes.c_int32),
                ("inter", ctypes.c_int32)]


class escha_moe_layer_t(ctypes.Structure):
    _fields_ = [("gate_up", escha_proj_t), ("down", escha_proj_t), ("hidden", ctypes.c_int32),
                ("inter", ctypes.c_int32), ("top_k", ctypes.c_int32)]


class escha_dense_mlp_t(ctypes.Structure):
    _fields_ = [("gate_up", escha_proj_t), ("down", escha_proj_t), ("gate_up_bias", ctypes.c_void_p),
                ("down_bias", ctypes.c_void_p), ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32)]


_vp, _i32, _i64, _sz, _f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
_P = ctypes.POINTER

_SIGS = {
    "escha_decode_tiles": ([_P(escha_proj_t), _i32, _vp, _vp], ctypes.c_int),
    "escha_decode_tiles_layout": ([_P(escha_proj_t), _i32, _i32, _vp, _vp], ctypes.c_int),
    "escha_hadamard128": ([_vp, _i64, _i32, _vp, _vp], ctypes.c_int),
    "escha_route_topk": ([_vp, _i32, _i32, _i32, _vp, _vp, _vp], ctypes.c_int),
    "escha_router_workspace_bytes": ([_i32, _i32, _i32], _sz),
    "escha_router_logits": ([_vp, _i32, _i32, _vp, _i32, _vp, _vp, _sz, _vp], ctypes.c_int),
    "escha_moe_group_workspace_bytes": ([_i32, _i32, _i32], _sz),
    "escha_moe_group": ([_vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _sz, _vp], ctypes.c_int),
    "escha_expert_gemv_workspace_bytes": ([_P(escha_proj_t), _i32], _sz),
    "escha_expert_gemv": ([_P(escha_proj_t), _i32, _vp, _i32, _vp, _vp, _sz, _vp], ctypes.c_int),
    "escha_moe_workspace_bytes": ([_P(escha_moe_layer_t), _i32, _i32], _sz),
    "escha_moe_layer_decode": ([_P(escha_moe_layer_t), _vp, _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
                               ctypes.c_int),
    "escha_moe_layer_prefill": ([_P(escha_moe_layer_t), _vp, _i32, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
                                ctypes.c_int),
    "escha_moe_layer_decode_static": ([_P(escha_moe_layer_t), _vp, _i32, _vp, _vp, _vp, _vp, _vp],
                                      ctypes.c_int),
    "escha_moe_layer_decode_logits": ([_P(escha_moe_layer_t), _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                                       _vp], ctypes.c_int),
    "escha_dense_mlp_workspace_bytes": ([_P(escha_dense_mlp_t), _i32, _i32], _sz),
    "escha_dense_mlp_decode": ([_P(escha_dense_mlp_t), _vp, _i32, _vp, _vp, _vp, _sz, _vp], ctypes.c_int),
    "escha_dense_mlp_prefill": ([_P(escha_dense_mlp_t), _vp, _i32, _vp, _vp, _vp, _sz, _vp], ctypes.c_int),
    "escha_dense_gemv": ([_P(escha_proj_t), _vp, _vp, _i32, _vp, _vp, _sz, _vp], ctypes.c_int),
    "escha_shared_expert_workspace_bytes": ([_P(escha_shared_expert_t), _i32], _sz),
    "escha_shared_expert": ([_P(escha_shared_expert_t), _vp, _i32, _vp, _i32, _vp, _sz, _vp], ctypes.c_int),
    "escha_rmsnorm_bf16": ([_vp, _i32, _i32, _f32, _vp, _vp], ctypes.c_int),
    "escha_moe_stack_workspace_bytes": ([_P(escha_moe_layer_t), _i32, _i32], _sz),
    "escha_moe_stack_decode": ([_P(escha_moe_layer_t), _i32, _vp, _i32, _vp, _vp, _f32, _vp, _vp,
                                _vp, _sz, _vp, _vp], ctypes.c_int),
    "escha_moe_stack_decode_persistent": ([_P(escha_moe_layer_t), _i32, _vp, _i32, _vp, _vp, _f32,
                                           _vp, _vp, _vp, _sz, _vp, _vp], ctypes.c_int),
    "escha_moe_stack_status": ([_vp, _P(_i32), _vp], ctypes.c_int),
    "escha_probe_events_set": ([_vp, _i32], ctypes.c_int),
    "escha_last_error": ([], ctypes.c_char_p),
}
for _name, (_args, _res) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res

EXPORTS = tuple(_SIGS)


def _check(rc: int):
    if rc != ESCHA_OK:
        raise EschaError(rc, _lib.escha_last_error().decode())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _ptr(t: torch.Tensor | None, dtype=None, name="tensor"):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    return ctypes.c_void_p(t.data_ptr())


# 16-bit tensors are passed as their bit patterns: a raw int16/uint16 view,
# or the matching float type (bf16 for activations, fp16 for scales and
# gates); the other float type is rejected rather than reinterpreted.
_U16_BITS = (torch.int16, torch.uint16)
_BF16 = _U16_BITS + (torch.bfloat16,)
_F16 = _U16_BITS + (torch.float16,)


def _check_out(t: torch.Tensor, shape, dtypes, name: str):
    """A caller-provided tensor must have exactly the shape the call reads or writes."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype not in (dtypes if isinstance(dtypes, tuple) else (dtypes,)):
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtypes}")


# ------------------------------------------------------------------ descriptors

ESCHA_LEAVES = ("escha_code", "escha_rin", "escha_rout")
# optional leaves a checkpoint may carry; they change nothing in the path
# (s_in/s_out ship as ones, config/layer_meta are informational)
ESCHA_OPTIONAL = ("escha_s_in", "escha_s_out", "escha_config")


@dataclass
class Proj:
    """One coded projection for all experts of a layer (device tensors)."""
    code: torch.Tensor  # int16 [E][in/16][out/16][16K]
    rin: torch.Tensor   # fp16 bits [E][in]
    rout: torch.Tensor  # fp16 bits [E][out]

    def __post_init__(self):
        if self.code.dim() == 3:
            self.code = self.code.unsqueeze(0)
        if self.rin.dim() == 1:
            self.rin = self.rin.unsqueeze(0)
        if self.rout.dim() == 1:
            self.rout = self.rout.unsqueeze(0)
        if self.code.dim() != 4 or self.code.shape[-1] % 16:
            raise ValueError(f"code shape {tuple(self.code.shape)} is not [E][in/16][out/16][16K]")

    @property
    def k_bits(self) -> int:
        # K comes from the code tensor's own last dimension
        return self.code.shape[-1] // 16

    @property
    def in_features(self) -> int:
        return self.code.shape[1] * 16

    @property
    def out_features(self) -> int:
        return self.code.shape[2] * 16

    @property
    def n_experts(self) -> int:
        return self.code.shape[0]

    def c(self) -> escha_proj_t:
        E = self.n_experts
        if tuple(self.rin.shape) != (E, self.in_features) or tuple(self.rout.shape) != (E, self.out_features):
            raise ValueError("rin/rout shapes do not match the code tensor")
        return escha_proj_t(_ptr(self.code, _U16_BITS, "code").value, _ptr(self.rin, _F16, "rin").value,
                            _ptr(self.rout, _F16, "rout").value, E, self.in_features,
                            self.out_features, self.k_bits)

    @classmethod
    def from_leaves(cls, leaves: dict, prefix: str = ""):
        """Build from checkpoint-style leaves ``{prefix}escha_code`` etc.

        The three required leaves must all be present; an unknown ``escha_*``
        leaf (a rotation variant this path does not implement) is an error.
        """
        names = {k[len(prefix):]: v for k, v in leaves.items() if k.startswith(prefix)}
        missing = [n for n in ESCHA_LEAVES if n not in names]
        if missing:
            raise ValueError(f"missing required leaves: {missing}")
        unknown = [n for n in names if n.startswith("escha_") and n not in ESCHA_LEAVES + ESCHA_OPTIONAL]
        if unknown:
            raise ValueError(f"unknown escha leaves (unsupported variant): {unknown}")
        return cls(names["escha_code"], names["escha_rin"], names["escha_rout"])


@dataclass
class MoeLayer:
    gate_up: Proj
    down: Proj
    top_k: int = 8

    @property
    def hidden(self) -> int:
        return self.gate_up.in_features

    @property
    def inter(self) -> int:
        return self.down.in_features

    def c(self) -> escha_moe_layer_t:
        return escha_moe_layer_t(self.gate_up.c(), self.down.c(), self.hidden, self.inter, self.top_k)


def _ws(nbytes: int, device) -> torch.Tensor:
    # zero-filled: the one-launch stack path requires it on first use
    return torch.zeros(max(int(nbytes), 1), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------ entry points

def escha_decode_tiles(w: Proj, expert: int, out: torch.Tensor | None = None, stream=None):
    if out is None:
        out = torch.empty(w.out_features, w.in_features, dtype=torch.int16, device=w.code.device)
    _check_out(out, (w.out_features, w.in_features), _U16_BITS, "out")
    wc = w.c()
    _check(_lib.escha_decode_tiles(ctypes.byref(wc), expert, _ptr(out, _U16_BITS, "out"), _stream(stream)))
    return out


LAYOUT_QUARTER, LAYOUT_MFMA_OPERAND, LAYOUT_LDS_TILE, LAYOUT_MFMA_PAIRS, LAYOUT_MFMA_TILE_PAIRS = 0, 1, 2, 3, 4


def escha_decode_tiles_layout(w: Proj, expert: int, layout: int, out: torch.Tensor | None = None,
                              stream=None):
    """Decode through one fused kernel's decoder (LAYOUT_*); fp16 bits [out][in]."""
    if out is None:
        out = torch.empty(w.out_features, w.in_features, dtype=torch.int16, device=w.code.device)
    _check_out(out, (w.out_features, w.in_features), _U16_BITS, "out")
    wc = w.c()
    _check(_lib.escha_decode_tiles_layout(ctypes.byref(wc), expert, layout, _ptr(out, _U16_BITS, "out"),
                                          _stream(stream)))
    return out


def escha_hadamard128(x: torch.Tensor, out: torch.Tensor | None = None, stream=None):
    n = x.shape[-1]
    rows = x.numel() // n if n else 0
    if out is None:
        out = torch.empty_like(x)
    _check_out(out, tuple(x.shape), torch.float32, "out")
    _check(_lib.escha_hadamard128(_ptr(x, torch.float32, "x"), rows, n, _ptr(out, torch.float32, "y"),
                                  _stream(stream)))
    return out


def escha_route_topk(logits: torch.Tensor, top_k: int, stream=None, ids=None, w=None):
    T, E = logits.shape
    if ids is None:
        ids = torch.empty(T, top_k, dtype=torch.int32, device=logits.device)
    if w is None:
        w = torch.empty(T, top_k, dtype=torch.float32, device=logits.device)
    _check_out(ids, (T, top_k), torch.int32, "ids")
    _check_out(w, (T, top_k), torch.float32, "w")
    _check(_lib.escha_route_topk(_ptr(logits, torch.float32, "logits"), T, E, top_k,
                                 _ptr(ids), _ptr(w), _stream(stream)))
    return ids, w


def escha_router_workspace_bytes(n_tokens: int, hidden: int, n_experts: int) -> int:
    return int(_lib.escha_router_workspace_bytes(n_tokens, hidden, n_experts))


def escha_router_logits(x_bf16: torch.Tensor, gate_f16: torch.Tensor, out: torch.Tensor | None = None,
                        workspace: torch.Tensor | None = None, stream=None):
    """x bf16 [T][H] (bf16 or 16-bit integer view), gate fp16 [E][H] -> fp32
    logits [T][E], each an fp16 value."""
    T, H = x_bf16.shape
    E, H2 = gate_f16.shape
    if H2 != H:
        raise ValueError(f"gate has {H2} inputs, x has {H}")
    if out is None:
        out = torch.empty(T, E, dtype=torch.float32, device=x_bf16.device)
    _check_out(out, (T, E), torch.float32, "out")
    nbytes = escha_router_workspace_bytes(T, H, E)
    if workspace is None and nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=x_bf16.device)
    _check(_lib.escha_router_logits(_ptr(x_bf16, _BF16, "x_bf16"), T, H, _ptr(gate_f16, _F16, "gate_f16"),
                                    E, _ptr(out, torch.float32, "logits"), _ptr(workspace),
                                    workspace.numel() if workspace is not None else 0, _stream(stream)))
    return out


def escha_moe_group(topk_ids: torch.Tensor, n_experts: int, stream=None):
    T, k = topk_ids.shape
    dev = topk_ids.device
    counts = torch.empty(n_experts, dtype=torch.int32, device=dev)
    offsets = torch.empty(n_experts + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(max(T * k, 1), dtype=torch.int32, device=dev)
    nbytes = _lib.escha_moe_group_workspace_bytes(T, k, n_experts)
    ws = _ws(nbytes, dev)
    _check(_lib.escha_moe_group(_ptr(topk_ids, torch.int32, "topk_ids"), T, k, n_experts,
                                _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(ws), nbytes,
                                _stream(stream)))
    return counts, offsets, perm[:T * k]


def escha_expert_gemv(w: Proj, expert: int, x_bf16: torch.Tensor, out: torch.Tensor | None = None,
                      workspace: torch.Tensor | None = None, stream=None):
    x2 = x_bf16.reshape(-1, w.in_features)
    T = x2.shape[0]
    if out is None:
        out = torch.empty(T, w.out_features, dtype=torch.float32, device=x_bf16.device)
    _check_out(out, (T, w.out_features), torch.float32, "out")
    wc = w.c()
    nbytes = _lib.escha_expert_gemv_workspace_bytes(ctypes.byref(wc), T)
    if workspace is None:
        workspace = _ws(nbytes, x_bf16.device)
    _check(_lib.escha_expert_gemv(ctypes.byref(wc), expert, _ptr(x2, _BF16, "x"), T,
                                  _ptr(out, torch.float32, "y"), _ptr(workspace),
                                  workspace.numel(), _stream(stream)))
    return out


def escha_moe_workspace_bytes(layer: MoeLayer, n_tokens: int, prefill: bool = False) -> int:
    lc = layer.c()
    return int(_lib.escha_moe_workspace_bytes(ctypes.byref(lc), n_tokens, int(prefill)))


def _moe_call(fn, layer, x_bf16, topk_ids, topk_w, out, inter_out, workspace, stream, prefill):
    T = x_bf16.shape[0]
    lc = layer.c()
    if out is None:
        out = torch.empty(T, layer.hidden, dtype=torch.float32, device=x_bf16.device)
    _check_out(x_bf16, (T, layer.hidden), _BF16, "x_bf16")
    _check_out(out, (T, layer.hidden), torch.float32, "out")
    _check_out(topk_ids, (T, layer.top_k), torch.int32, "topk_ids")
    _check_out(topk_w, (T, layer.top_k), torch.float32, "topk_w")
    if inter_out is not None:
        _check_out(inter_out, (T * layer.top_k, layer.inter), torch.float32, "inter_out")
    nbytes = _lib.escha_moe_workspace_bytes(ctypes.byref(lc), T, int(prefill))
    if workspace is None:
        workspace = _ws(nbytes, x_bf16.device)
    _check(fn(ctypes.byref(lc), _ptr(x_bf16, _BF16, "x"), T, _ptr(topk_ids, torch.int32, "topk_ids"),
              _ptr(topk_w, torch.float32, "topk_w"), _ptr(out, torch.float32, "y"),
              _ptr(inter_out, torch.float32, "inter_out"), _ptr(workspace), workspace.numel(),
              _stream(stream)))
    return out


def escha_moe_layer_decode(layer: MoeLayer, x_bf16, topk_ids, topk_w, out=None, inter_out=None,
                           workspace=None, stream=None):
    return _moe_call(_lib.escha_moe_layer_decode, layer, x_bf16, topk_ids, topk_w, out, inter_out,
                     workspace, stream, False)


def escha_moe_layer_decode_logits(layer: MoeLayer, x_bf16, logits, out=None, topk_ids=None, topk_w=None,
                                  inter_out=None, workspace=None, stream=None):
    """The layer with its router step: returns (y, topk_ids, topk_w)."""
    T = x_bf16.shape[0]
    dev = x_bf16.device
    lc = layer.c()
    if out is None:
        out = torch.empty(T, layer.hidden, dtype=torch.float32, device=dev)
    if topk_ids is None:
        topk_ids = torch.empty(T, layer.top_k, dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty(T, layer.top_k, dtype=torch.float32, device=dev)
    _check_out(x_bf16, (T, layer.hidden), _BF16, "x_bf16")
    _check_out(logits, (T, layer.gate_up.n_experts), torch.float32, "logits")
    _check_out(out, (T, layer.hidden), torch.float32, "out")
    _check_out(topk_ids, (T, layer.top_k), torch.int32, "topk_ids")
    _check_out(topk_w, (T, layer.top_k), torch.float32, "topk_w")
    if inter_out is not None:
        _check_out(inter_out, (T * layer.top_k, layer.inter), torch.float32, "inter_out")
    nbytes = _lib.escha_moe_workspace_bytes(ctypes.byref(lc), T, 0)
    if workspace is None:
        workspace = _ws(nbytes, dev)
    _check(_lib.escha_moe_layer_decode_logits(
        ctypes.byref(lc), _ptr(x_bf16, _BF16, "x"), T, _ptr(logits, torch.float32, "logits"),
        _ptr(topk_ids, torch.int32, "topk_ids"), _ptr(topk_w, torch.float32, "topk_w"),
        _ptr(out, torch.float32, "y"), _ptr(inter_out, torch.float32, "inter_out"), _ptr(workspace),
        workspace.numel(), _stream(stream)))
    return out, topk_ids, topk_w


def escha_moe_layer_prefill(layer: MoeLayer, x_bf16, topk_ids, topk_w, out=None, inter_out=None,
                            workspace=None, stream=None):
    return _moe_call(_lib.escha_moe_layer_prefill, layer, x_bf16, topk_ids, topk_w, out, inter_out,
                     workspace, stream, True)


def escha_moe_layer_decode_static(layer: MoeLayer, x_bf16, topk_ids, topk_w, out=None, inter_out=None,
                                  stream=None):
    """escha_moe_layer_decode with the library's own device scratch (no
    workspace, no allocation in the library; ``out`` may be passed so that
    the call allocates nothing at all)."""
    T = x_bf16.shape[0]
    lc = layer.c()
    if out is None:
        out = torch.empty(T, layer.hidden, dtype=torch.float32, device=x_bf16.device)
    _check_out(x_bf16, (T, layer.hidden), _BF16, "x_bf16")
    _check_out(out, (T, layer.hidden), torch.float32, "out")
    _check_out(topk_ids, (T, layer.top_k), torch.int32, "topk_ids")
    _check_out(topk_w, (T, layer.top_k), torch.float32, "topk_w")
    if inter_out is not None:
        _check_out(inter_out, (T * layer.top_k, layer.inter), torch.float32, "inter_out")
    _check(_lib.escha_moe_layer_decode_static(
        ctypes.byref(lc), _ptr(x_bf16, _BF16, "x"), T, _ptr(topk_ids, torch.int32, "topk_ids"),
        _ptr(topk_w, torch.float32, "topk_w"), _ptr(out, torch.float32, "y"),
        _ptr(inter_out, torch.float32, "inter_out"), _stream(stream)))
    return out


@dataclass
class DenseMLP:
    """A dense MLP of coded projections (one expert each) with fp32 biases."""
    gate_up: Proj
    down: Proj
    gate_up_bias: torch.Tensor | None = None  # fp32 [2*inter]
    down_bias: torch.Tensor | None = None     # fp32 [hidden]

    @property
    def hidden(self) -> int:
        return self.gate_up.in_features

    @property
    def inter(self) -> int:
        return self.down.in_features

    def c(self) -> escha_dense_mlp_t:
        if self.gate_up_bias is not None:
            _check_out(self.gate_up_bias, (2 * self.inter,), torch.float32, "gate_up_bias")
        if self.down_bias is not None:
            _check_out(self.down_bias, (self.hidden,), torch.float32, "down_bias")
        gb = _ptr(self.gate_up_bias, torch.float32, "gate_up_bias")
        db = _ptr(self.down_bias, torch.float32, "down_bias")
        return escha_dense_mlp_t(self.gate_up.c(), self.down.c(), gb.value if gb else None,
                                 db.value if db else None, self.hidden, self.inter)


def _dense_call(fn, M: DenseMLP, x_bf16, out, inter_out, workspace, stream, prefill):
    T = x_bf16.shape[0]
    mc = M.c()
    if out is None:
        out = torch.empty(T, M.hidden, dtype=torch.float32, device=x_bf16.device)
    _check_out(x_bf16, (T, M.hidden), _BF16, "x_bf16")
    _check_out(out, (T, M.hidden), torch.float32, "out")
    if inter_out is not None:
        _check_out(inter_out, (T, M.inter), torch.float32, "inter_out")
    nbytes = _lib.escha_dense_mlp_workspace_bytes(ctypes.byref(mc), T, int(prefill))
    if workspace is None:
        workspace = _ws(nbytes, x_bf16.device)
    _check(fn(ctypes.byref(mc), _ptr(x_bf16, _BF16, "x"), T, _ptr(out, torch.float32, "y"),
              _ptr(inter_out, torch.float32, "inter_out"), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


def escha_dense_mlp_decode(M: DenseMLP, x_bf16, out=None, inter_out=None, workspace=None, stream=None):
    return _dense_call(_lib.escha_dense_mlp_decode, M, x_bf16, out, inter_out, workspace, stream, False)


def escha_dense_mlp_prefill(M: DenseMLP, x_bf16, out=None, inter_out=None, workspace=None, stream=None):
    return _dense_call(_lib.escha_dense_mlp_prefill, M, x_bf16, out, inter_out, workspace, stream, True)


def escha_dense_gemv(w: Proj, x_bf16: torch.Tensor, bias: torch.Tensor | None = None,
                     out: torch.Tensor | None = None, workspace: torch.Tensor | None = None, stream=None):
    x2 = x_bf16.reshape(-1, w.in_features)
    T = x2.shape[0]
    if out is None:
        out = torch.empty(T, w.out_features, dtype=torch.float32, device=x_bf16.device)
    _check_out(out, (T, w.out_features), torch.float32, "out")
    if bias is not None:
        _check_out(bias, (w.out_features,), torch.float32, "bias")
    wc = w.c()
    nbytes = _lib.escha_expert_gemv_workspace_bytes(ctypes.byref(wc), T)
    if workspace is None:
        workspace = _ws(nbytes, x_bf16.device)
    _check(_lib.escha_dense_gemv(ctypes.byref(wc), _ptr(bias, torch.float32, "bias"), _ptr(x2, _BF16, "x"), T,
                                 _ptr(out, torch.float32, "y"), _ptr(workspace), workspace.numel(),
                                 _stream(stream)))
    return out


@dataclass
class SharedExpert:
    """The shared expert in its w8a16 form (device tensors): int8 weights,
    f32 group-128 scales, the fp16 shared_expert_gate row."""
    gate_up: torch.Tensor        # int8 [2*inter][hidden]
    gate_up_scale: torch.Tensor  # f32 [2*inter][hidden/128]
    down: torch.Tensor           # int8 [hidden][inter]
    down_scale: torch.Tensor     # f32 [hidden][inter/128]
    gate: torch.Tensor           # fp16 bits [hidden]

    @property
    def hidden(self) -> int:
        return self.gate_up.shape[1]

    @property
    def inter(self) -> int:
        return self.down.shape[1]

    def c(self) -> escha_shared_expert_t:
        H, I = self.hidden, self.inter
        _check_out(self.gate_up, (2 * I, H), torch.int8, "gate_up")
        _check_out(self.gate_up_scale, (2 * I, H // 128), torch.float32, "gate_up_scale")
        _check_out(self.down, (H, I), torch.int8, "down")
        _check_out(self.down_scale, (H, I // 128), torch.float32, "down_scale")
        _check_out(self.gate, (H,), _F16, "gate")
        return escha_shared_expert_t(_ptr(self.gate_up).value, _ptr(self.gate_up_scale).value,
                                     _ptr(self.down).value, _ptr(self.down_scale).value,
                                     _ptr(self.gate).value, H, I)


def escha_shared_expert(S: SharedExpert, x_bf16: torch.Tensor, out: torch.Tensor | None = None,
                        accumulate: bool = False, workspace: torch.Tensor | None = None, stream=None):
    """out (+)= sigmoid(gate . x) * shared_expert(x) per token (fp32 [T][hidden])."""
    T = x_bf16.shape[0]
    sc = S.c()
    if out is None:
        if accumulate:
            raise ValueError("accumulate needs the output to add into")
        out = torch.empty(T, S.hidden, dtype=torch.float32, device=x_bf16.device)
    _check_out(x_bf16, (T, S.hidden), _BF16, "x_bf16")
    _check_out(out, (T, S.hidden), torch.float32, "out")
    nbytes = _lib.escha_shared_expert_workspace_bytes(ctypes.byref(sc), T)
    if workspace is None:
        workspace = torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=x_bf16.device)
    _check(_lib.escha_shared_expert(ctypes.byref(sc), _ptr(x_bf16, _BF16, "x"), T, _ptr(out, torch.float32, "y"),
                                    int(bool(accumulate)), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


def escha_rmsnorm_bf16(y: torch.Tensor, eps: float = 1e-6, out: torch.Tensor | None = None, stream=None):
    T, n = y.shape
    if out is None:
        out = torch.empty(T, n, dtype=torch.int16, device=y.device)
    _check_out(out, (T, n), _BF16, "out")
    _check(_lib.escha_rmsnorm_bf16(_ptr(y, torch.float32, "y"), T, n, eps, _ptr(out, _BF16, "x"),
                                   _stream(stream)))
    return out


class Stack:
    """A host array of layer descriptors for escha_moe_stack_decode."""

    def __init__(self, layers):
        self.layers = list(layers)
        self.arr = (escha_moe_layer_t * len(self.layers))(*[l.c() for l in self.layers])

    def workspace_bytes(self, n_tokens: int) -> int:
        return int(_lib.escha_moe_stack_workspace_bytes(self.arr, len(self.layers), n_tokens))


def _stack_call(fn, n_events, stack, x0_bf16, topk_ids, topk_w, eps, out, x_chain, workspace,
                probe_events, stream):
    T = x0_bf16.shape[0]
    NL = len(stack.layers)
    hidden = stack.layers[0].hidden
    k = stack.layers[0].top_k
    if out is None:
        out = torch.empty(T, hidden, dtype=torch.float32, device=x0_bf16.device)
    _check_out(x0_bf16, (T, hidden), _BF16, "x0_bf16")
    _check_out(out, (T, hidden), torch.float32, "out")
    _check_out(topk_ids, (NL, T, k), torch.int32, "topk_ids")
    _check_out(topk_w, (NL, T, k), torch.float32, "topk_w")
    if x_chain is not None:
        _check_out(x_chain, (NL, T, hidden), _BF16, "x_chain")
    nbytes = stack.workspace_bytes(T)
    if workspace is None:
        workspace = _ws(nbytes, x0_bf16.device)
    _check(fn(stack.arr, NL, _ptr(x0_bf16, _BF16, "x0"), T,
              _ptr(topk_ids, torch.int32, "topk_ids"), _ptr(topk_w, torch.float32, "topk_w"), eps,
              _ptr(out, torch.float32, "y"), _ptr(x_chain, _BF16, "x_chain"), _ptr(workspace),
              workspace.numel(), _events(probe_events, n_events), _stream(stream)))
    return out, workspace


def escha_moe_stack_decode(stack: Stack, x0_bf16, topk_ids, topk_w, eps: float = 1e-6, out=None,
                           x_chain=None, workspace=None, probe_events=None, stream=None):
    """probe_events: optional sequence of 2*n_layers raw hipEvent_t handles (ints)."""
    return _stack_call(_lib.escha_moe_stack_decode, 2 * len(stack.layers), stack, x0_bf16, topk_ids,
                       topk_w, eps, out, x_chain, workspace, probe_events, stream)[0]


def escha_moe_stack_decode_persistent(stack: Stack, x0_bf16, topk_ids, topk_w, eps: float = 1e-6,
                                      out=None, x_chain=None, workspace=None, probe_events=None,
                                      stream=None, check_status: bool = True):
    """One persistent launch for the whole stack; probe_events: 2 raw hipEvent_t handles.

    The C call returns before the kernel has run, so a dependency wait that
    gave up (its outputs then incomplete) shows only in the status word. With
    ``check_status`` (the default) this waits for the stream, reads the word
    and raises ``EschaError`` when it is set; pass False to keep the call
    asynchronous (inside graph capture it must be False) and check
    ``escha_moe_stack_status`` later.
    """
    if check_status and torch.cuda.is_current_stream_capturing():
        raise ValueError("check_status=True needs a synchronising read; pass False under graph capture")
    out, ws = _stack_call(_lib.escha_moe_stack_decode_persistent, 2, stack, x0_bf16, topk_ids, topk_w,
                          eps, out, x_chain, workspace, probe_events, stream)
    if check_status and escha_moe_stack_status(ws, stream) != 0:
        raise EschaError(STATUS_INCOMPLETE, "a dependency wait of the one-launch stack gave up; "
                                            "the outputs are incomplete")
    return out


def escha_moe_stack_status(workspace: torch.Tensor, stream=None) -> int:
    """Status word of the last persistent stack call on this workspace (waits for the stream)."""
    v = ctypes.c_int32(-1)
    _check(_lib.escha_moe_stack_status(_ptr(workspace), ctypes.byref(v), _stream(stream)))
    return int(v.value)


def escha_probe_events_set(handles=None):
    """Install (two raw hipEvent_t handles) or remove (None) this thread's
    projection probes: later layer calls record them around their gate_up
    and down projection kernels."""
    if handles is None:
        _check(_lib.escha_probe_events_set(None, 0))
    else:
        _check(_lib.escha_probe_events_set(_events(handles, 2), 2))


def _events(handles, n):
    if handles is None:
        return None
    if len(handles) != n:
        raise ValueError(f"need {n} probe events, got {len(handles)}")
    return ctypes.cast((ctypes.c_void_p * n)(*[int(h) for h in handles]), ctypes.c_void_p)
