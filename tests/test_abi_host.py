"""Host-side checks of the C ABI: the library loads, exports every entry
point declared in include/escha.h, and rejects bad arguments before any
launch (no GPU needed: validation returns before touching the device)."""
import ctypes
import re
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "escha.h"
LIB = ROOT / "bit_trellis_quantized_amd" / "libescha.so"


def _declared():
    src = HEADER.read_text()
    return sorted(set(re.findall(r"ESCHA_API\s+[\w\s\*]+?\b(escha_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    import torch  # noqa: F401  (load torch's HIP runtime first, as the binding does)
    if not LIB.exists():
        from bit_trellis_quantized_amd import build
        build.build()
    return ctypes.CDLL(str(LIB))


def test_header_declares_the_path(lib):
    names = _declared()
    for required in ("escha_expert_gemv", "escha_moe_layer_decode", "escha_moe_layer_prefill",
                     "escha_decode_tiles", "escha_hadamard128", "escha_route_topk",
                     "escha_moe_group", "escha_moe_stack_decode", "escha_last_error"):
        assert required in names


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def test_binding_covers_every_declared_symbol():
    src = (ROOT / "bit_trellis_quantized_amd" / "escha.py").read_text()
    for name in _declared():
        assert f'"{name}"' in src, name


class Proj(ctypes.Structure):
    _fields_ = [("code", ctypes.c_void_p), ("rin", ctypes.c_void_p), ("rout", ctypes.c_void_p),
                ("n_experts", ctypes.c_int32), ("in_features", ctypes.c_int32),
                ("out_features", ctypes.c_int32), ("k_bits", ctypes.c_int32)]


class Layer(ctypes.Structure):
    _fields_ = [("gate_up", Proj), ("down", Proj), ("hidden", ctypes.c_int32),
                ("inter", ctypes.c_int32), ("top_k", ctypes.c_int32)]


FAKE = 0x10000  # never dereferenced: every case below fails validation first


def _proj(**kw):
    d = dict(code=FAKE, rin=FAKE, rout=FAKE, n_experts=256, in_features=2048, out_features=1024,
             k_bits=2)
    d.update(kw)
    return Proj(**d)


def _layer(**kw):
    L = Layer(_proj(), _proj(in_features=512, out_features=2048, k_bits=3), 2048, 512, 8)
    for k, v in kw.items():
        setattr(L, k, v)
    return L


def _err(lib):
    lib.escha_last_error.restype = ctypes.c_char_p
    return lib.escha_last_error().decode()


def test_decode_tiles_validation(lib):
    f = lib.escha_decode_tiles
    f.argtypes = [ctypes.POINTER(Proj), ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    assert f(None, 0, FAKE, None) == -1
    assert f(ctypes.byref(_proj(k_bits=4)), 0, FAKE, None) == -3
    assert "k_bits" in _err(lib)
    assert f(ctypes.byref(_proj(in_features=100)), 0, FAKE, None) == -2
    assert f(ctypes.byref(_proj(out_features=128)), 0, FAKE, None) == -2
    assert f(ctypes.byref(_proj()), 256, FAKE, None) == -7
    assert f(ctypes.byref(_proj()), -1, FAKE, None) == -7
    assert f(ctypes.byref(_proj(code=FAKE + 2)), 0, FAKE, None) == -7  # misaligned code
    assert f(ctypes.byref(_proj(rout=None)), 0, FAKE, None) == -1
    assert f(ctypes.byref(_proj()), 0, None, None) == -1


def test_layer_validation(lib):
    f = lib.escha_moe_layer_decode
    f.argtypes = [ctypes.POINTER(Layer), ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_size_t, ctypes.c_void_p]
    ok = _layer()
    assert f(None, FAKE, 1, FAKE, FAKE, FAKE, None, FAKE, 1 << 40, None) == -1
    assert f(ctypes.byref(_layer(hidden=4096)), FAKE, 1, FAKE, FAKE, FAKE, None, FAKE, 1 << 40, None) == -2
    assert f(ctypes.byref(_layer(top_k=0)), FAKE, 1, FAKE, FAKE, FAKE, None, FAKE, 1 << 40, None) == -7
    assert f(ctypes.byref(_layer(top_k=300)), FAKE, 1, FAKE, FAKE, FAKE, None, FAKE, 1 << 40, None) == -7
    assert f(ctypes.byref(ok), FAKE, -1, FAKE, FAKE, FAKE, None, FAKE, 1 << 40, None) == -7
    assert f(ctypes.byref(ok), None, 1, FAKE, FAKE, FAKE, None, FAKE, 1 << 40, None) == -1
    # workspace too small: rejected before launch (>= check, not ==)
    ws = lib.escha_moe_workspace_bytes
    ws.argtypes = [ctypes.POINTER(Layer), ctypes.c_int32, ctypes.c_int32]
    ws.restype = ctypes.c_size_t
    need = ws(ctypes.byref(ok), 1, 0)
    assert need > 0
    assert f(ctypes.byref(ok), FAKE, 1, FAKE, FAKE, FAKE, None, FAKE, need - 1, None) == -4
    assert "workspace" in _err(lib)
    # mismatched expert counts
    bad = _layer()
    bad.down.n_experts = 128
    assert f(ctypes.byref(bad), FAKE, 1, FAKE, FAKE, FAKE, None, FAKE, 1 << 40, None) == -2
    # zero tokens is a valid no-op (nothing launched, nothing dereferenced)
    assert f(ctypes.byref(ok), None, 0, None, None, None, None, None, 0, None) == 0


def test_layer_decode_logits_validation(lib):
    f = lib.escha_moe_layer_decode_logits
    f.argtypes = [ctypes.POINTER(Layer), ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_size_t, ctypes.c_void_p]
    ok = _layer()
    big = 1 << 40
    assert f(None, FAKE, 1, FAKE, FAKE, FAKE, FAKE, None, FAKE, big, None) == -1
    assert f(ctypes.byref(_layer(top_k=0)), FAKE, 1, FAKE, FAKE, FAKE, FAKE, None, FAKE, big, None) == -7
    assert f(ctypes.byref(ok), FAKE, -1, FAKE, FAKE, FAKE, FAKE, None, FAKE, big, None) == -7
    # logits, topk_ids (an output here), topk_w and y are required
    for i in range(4):
        args = [FAKE, FAKE, FAKE, FAKE]
        args[i] = None
        assert f(ctypes.byref(ok), FAKE, 1, *args, None, FAKE, big, None) == -1
        assert "NULL" in _err(lib)
    ws = lib.escha_moe_workspace_bytes
    ws.argtypes = [ctypes.POINTER(Layer), ctypes.c_int32, ctypes.c_int32]
    ws.restype = ctypes.c_size_t
    need = ws(ctypes.byref(ok), 3, 0)
    assert f(ctypes.byref(ok), FAKE, 3, FAKE, FAKE, FAKE, FAKE, None, FAKE, need - 1, None) == -4
    # zero tokens: a no-op
    assert f(ctypes.byref(ok), None, 0, None, None, None, None, None, None, 0, None) == 0


def test_route_and_group_validation(lib):
    r = lib.escha_route_topk
    r.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_void_p]
    assert r(FAKE, 1, 256, 0, FAKE, FAKE, None) == -7
    assert r(FAKE, 1, 256, 33, FAKE, FAKE, None) == -7
    assert r(FAKE, 1, 2048, 8, FAKE, FAKE, None) == -7
    assert r(None, 1, 256, 8, FAKE, FAKE, None) == -1
    assert r(None, 0, 256, 8, None, None, None) == 0
    g = lib.escha_moe_group
    g.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    assert g(FAKE, 4, 8, 256, FAKE, FAKE, FAKE, FAKE, 0, None) == -4


def test_router_logits_validation(lib):
    f = lib.escha_router_logits
    f.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    wsb = lib.escha_router_workspace_bytes
    wsb.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
    wsb.restype = ctypes.c_size_t
    assert f(FAKE, 1, 48, FAKE, 256, FAKE, None, 0, None) == -2     # hidden not a multiple of 32
    assert f(FAKE, 1, 2048, FAKE, 0, FAKE, None, 0, None) == -7     # no experts
    assert f(FAKE, 1, 2048, FAKE, 1025, FAKE, None, 0, None) == -7
    assert f(FAKE, -1, 2048, FAKE, 256, FAKE, None, 0, None) == -7
    assert f(None, 1, 2048, FAKE, 256, FAKE, None, 0, None) == -1
    assert f(FAKE + 2, 1, 2048, FAKE, 256, FAKE, None, 0, None) == -7  # misaligned x
    assert f(None, 0, 2048, None, 256, None, None, 0, None) == 0     # zero tokens: no-op
    # 64 tokens split the inputs: partial sums need the workspace
    need = wsb(64, 2048, 256)
    assert need >= 32 * 64 * 256 * 4
    assert f(FAKE, 64, 2048, FAKE, 256, FAKE, FAKE, need - 1, None) == -4
    assert wsb(8, 2048, 256) == 0  # up to 8 tokens: one wave per expert, no partial sums
    assert wsb(4096, 2048, 256) >= 2 * 4096 * 256 * 4
    assert wsb(1, 48, 256) == 0


def test_stack_validation(lib):
    f = lib.escha_moe_stack_decode
    f.argtypes = [ctypes.POINTER(Layer), ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    arr = (Layer * 2)(_layer(), _layer(inter=256))
    arr[1].gate_up.out_features = 512
    arr[1].down.in_features = 256
    assert f(arr, 2, FAKE, 1, FAKE, FAKE, 1e-6, FAKE, None, FAKE, 1 << 40, None, None) == -2
    assert f(arr, 0, FAKE, 1, FAKE, FAKE, 1e-6, FAKE, None, FAKE, 1 << 40, None, None) == -7
    arr2 = (Layer * 1)(_layer())
    assert f(arr2, 1, FAKE, 1, FAKE, FAKE, -1.0, FAKE, None, FAKE, 1 << 40, None, None) == -7


def test_persistent_stack_validation(lib):
    f = lib.escha_moe_stack_decode_persistent
    f.argtypes = [ctypes.POINTER(Layer), ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    big = 1 << 44
    # shared checks with the layer-by-layer stack
    assert f(None, 1, FAKE, 1, FAKE, FAKE, 1e-6, FAKE, None, FAKE, big, None, None) == -1
    arr1 = (Layer * 1)(_layer())
    assert f(arr1, 1, FAKE, 1, FAKE, FAKE, -1.0, FAKE, None, FAKE, big, None, None) == -7
    assert f(arr1, 1, FAKE, 1, FAKE, FAKE, 1e-6, FAKE, None, FAKE, 16, None, None) == -4
    # limits of the persistent path
    arr65 = (Layer * 65)(*[_layer() for _ in range(65)])
    assert f(arr65, 65, FAKE, 1, FAKE, FAKE, 1e-6, FAKE, None, FAKE, big, None, None) == -6
    assert "n_layers" in _err(lib)
    assert f(arr1, 1, FAKE, 65, FAKE, FAKE, 1e-6, FAKE, None, FAKE, big, None, None) == -6
    mixed = (Layer * 2)(_layer(), _layer())
    mixed[1].down.k_bits = 2
    assert f(mixed, 2, FAKE, 1, FAKE, FAKE, 1e-6, FAKE, None, FAKE, big, None, None) == -6
    assert "k_bits" in _err(lib)
    mixed = (Layer * 2)(_layer(), _layer())
    mixed[1].gate_up.n_experts = mixed[1].down.n_experts = 128
    assert f(mixed, 2, FAKE, 1, FAKE, FAKE, 1e-6, FAKE, None, FAKE, big, None, None) == -6
    # zero tokens: a no-op that launches nothing
    assert f(arr1, 1, None, 0, None, None, 1e-6, None, None, None, 0, None, None) == 0
    s = lib.escha_moe_stack_status
    s.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32), ctypes.c_void_p]
    assert s(None, None, None) == -1


def test_stack_workspace_holds_the_counters(lib):
    """The stack workspace grows with the layers' dependency counters."""
    ws = lib.escha_moe_stack_workspace_bytes
    ws.argtypes = [ctypes.POINTER(Layer), ctypes.c_int32, ctypes.c_int32]
    ws.restype = ctypes.c_size_t
    arr = (Layer * 40)(*[_layer() for _ in range(40)])
    one, two = ws(arr, 1, 1), ws(arr, 2, 1)
    # one more layer: 8 pair counters + 8 group counters + 1 token counter, 64 B each
    assert two - one >= (8 + 8 + 1) * 64 - 255
    lay1 = ws(arr, 40, 1)
    assert lay1 >= 40 * (8 + 8 + 1) * 64


def test_leaf_contract():
    """Required leaves must be present; unknown escha_* leaves are rejected by name."""
    import importlib.util
    src = (ROOT / "bit_trellis_quantized_amd" / "escha.py").read_text()
    assert 'ESCHA_LEAVES = ("escha_code", "escha_rin", "escha_rout")' in src
    if importlib.util.find_spec("torch") is None:
        pytest.skip("torch missing")
    from bit_trellis_quantized_amd import escha  # loads the library (no GPU needed)
    import torch
    t = torch.zeros(1, 8, 16, 32, dtype=torch.int16)
    leaves = {"x.escha_code": t, "x.escha_rin": torch.zeros(1, 128, dtype=torch.int16),
              "x.escha_rout": torch.zeros(1, 256, dtype=torch.int16)}
    p = escha.Proj.from_leaves(leaves, "x.")
    assert p.k_bits == 2 and p.in_features == 128 and p.out_features == 256
    with pytest.raises(ValueError, match="missing"):
        escha.Proj.from_leaves({k: v for k, v in leaves.items() if "rout" not in k}, "x.")
    with pytest.raises(ValueError, match="escha_rotation_theta"):
        escha.Proj.from_leaves(dict(leaves, **{"x.escha_rotation_theta": t}), "x.")


def test_decode_tiles_layout_rejects_unknown_layout(lib):
    f = lib.escha_decode_tiles_layout
    f.argtypes = [ctypes.POINTER(Proj), ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    p = _proj()
    assert f(ctypes.byref(p), 0, 5, ctypes.c_void_p(FAKE), None) == -7
    assert "layout" in _err(lib)
    p3 = _proj(in_features=512, out_features=2048, k_bits=3)
    for layout in (3, 4):  # the column-pair layouts are K=2 only
        assert f(ctypes.byref(p3), 0, layout, ctypes.c_void_p(FAKE), None) == -7
        assert "K=2" in _err(lib)
    assert f(ctypes.byref(p), 256, 1, ctypes.c_void_p(FAKE), None) == -7  # expert out of range
    assert f(ctypes.byref(p), 0, 2, None, None) == -1
    assert f(ctypes.byref(p), 0, 1, ctypes.c_void_p(FAKE + 8), None) == -7  # not 16-byte aligned


def test_probe_events_set_validates(lib):
    f = lib.escha_probe_events_set
    f.argtypes = [ctypes.c_void_p, ctypes.c_int32]
    arr = (ctypes.c_void_p * 2)(FAKE, None)
    assert f(ctypes.cast(arr, ctypes.c_void_p), 2) == -1
    assert f(ctypes.cast(arr, ctypes.c_void_p), 3) == -7
    assert f(None, 0) == 0


class Shared(ctypes.Structure):
    _fields_ = [("gate_up", ctypes.c_void_p), ("gate_up_scale", ctypes.c_void_p), ("down", ctypes.c_void_p),
                ("down_scale", ctypes.c_void_p), ("gate", ctypes.c_void_p), ("hidden", ctypes.c_int32),
                ("inter", ctypes.c_int32)]


def test_shared_expert_validates(lib):
    f = lib.escha_shared_expert
    f.argtypes = [ctypes.POINTER(Shared), ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
                  ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    ok = dict(gate_up=FAKE, gate_up_scale=FAKE, down=FAKE, down_scale=FAKE, gate=FAKE, hidden=2048, inter=512)
    x, y = ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE)
    assert f(ctypes.byref(Shared(**dict(ok, down=None))), x, 1, y, 0, x, 1 << 20, None) == -1
    assert f(ctypes.byref(Shared(**dict(ok, hidden=2000))), x, 1, y, 0, x, 1 << 20, None) == -2
    assert f(ctypes.byref(Shared(**dict(ok, hidden=8192))), x, 1, y, 0, x, 1 << 20, None) == -2
    assert f(ctypes.byref(Shared(**dict(ok, inter=384))), x, 1, y, 0, x, 1 << 20, None) == -2
    assert f(ctypes.byref(Shared(**dict(ok, gate_up=FAKE + 8))), x, 1, y, 0, x, 1 << 20, None) == -7
    assert f(ctypes.byref(Shared(**ok)), x, 1, y, 0, x, 16, None) == -4
    assert f(ctypes.byref(Shared(**ok)), x, 0, y, 0, None, 0, None) == 0


class DenseMLP(ctypes.Structure):
    _fields_ = [("gate_up", Proj), ("down", Proj), ("gate_up_bias", ctypes.c_void_p),
                ("down_bias", ctypes.c_void_p), ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32)]


def test_dense_entry_points_validate(lib):
    f = lib.escha_dense_mlp_decode
    f.argtypes = [ctypes.POINTER(DenseMLP), ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    M = DenseMLP(_proj(n_experts=1), _proj(n_experts=1, in_features=512, out_features=2048, k_bits=3),
                 None, None, 2048, 512)
    x = ctypes.c_void_p(FAKE)
    assert f(ctypes.byref(M), x, 4, x, None, x, 16, None) == -4  # workspace too small
    M2 = DenseMLP(_proj(n_experts=2), M.down, None, None, 2048, 512)
    assert f(ctypes.byref(M2), x, 4, x, None, x, 1 << 30, None) == -2  # not the one-expert case
    M3 = DenseMLP(M.gate_up, M.down, None, None, 2048, 256)
    assert f(ctypes.byref(M3), x, 4, x, None, x, 1 << 30, None) == -2  # inter disagrees
    g = lib.escha_dense_gemv
    g.argtypes = [ctypes.POINTER(Proj), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    p = _proj(n_experts=3)
    assert g(ctypes.byref(p), None, x, 1, x, x, 1 << 30, None) == -2
