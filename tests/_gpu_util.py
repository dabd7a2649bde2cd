"""Helpers shared by the GPU parity tests (not collected by pytest)."""
from __future__ import annotations

import sys

import numpy as np
import torch

from bit_trellis_quantized_amd import synth

# Tolerance for floating-point outputs, relative to the fp64 oracle over the
# whole output tensor: relative L2 error and max-abs error as a fraction of
# the reference's max magnitude.
REL_L2 = 1e-3
MAX_ABS = 2e-3


def announce(msg: str):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray) -> torch.Tensor:
    """uint16 / int32 / float32 numpy -> device tensor (uint16 as int16 bits)."""
    a = np.array(a, copy=True, order="C")
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def u16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def layer_to_dev(L: dict, top_k: int = synth.TOP_K):
    from bit_trellis_quantized_amd import escha
    gu = escha.Proj(to_dev(L["gu_code"]), to_dev(L["gu_rin"]), to_dev(L["gu_rout"]))
    dn = escha.Proj(to_dev(L["dn_code"]), to_dev(L["dn_rin"]), to_dev(L["dn_rout"]))
    return escha.MoeLayer(gu, dn, top_k)


def errors(y: np.ndarray, ref: np.ndarray):
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rel = np.linalg.norm(y - ref) / max(np.linalg.norm(ref), 1e-300)
    mx = np.max(np.abs(y - ref)) / max(np.max(np.abs(ref)), 1e-300)
    return rel, mx


def assert_close(y, ref, what=""):
    rel, mx = errors(y, ref)
    announce(f"{what}: rel_l2={rel:.3e} max_abs/max|ref|={mx:.3e}")
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    assert rel <= REL_L2, f"{what}: rel_l2 {rel:.3e} > {REL_L2}"
    assert mx <= MAX_ABS, f"{what}: max-abs {mx:.3e} > {MAX_ABS}"
