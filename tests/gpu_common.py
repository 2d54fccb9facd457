"""Helpers shared by the GPU parity tests: device placement of synthetic
inputs and the output-tolerance check.

Tolerance for layer outputs (fp32 accumulation over bf16 activations):
relative L2 error <= 2e-3 and max |err| <= 1e-2 * max |ref|.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from expert_offload_serving_amd import layer as dl
from expert_offload_serving_amd import synth

REL_L2 = 2e-3
MAX_REL = 1e-2


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def close_enough(y: np.ndarray, ref: np.ndarray, rel_l2: float = REL_L2, max_rel: float = MAX_REL):
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = y - ref
    nref = np.linalg.norm(ref)
    rel = np.linalg.norm(err) / nref if nref > 0 else np.linalg.norm(err)
    mx = np.abs(err).max() if err.size else 0.0
    mref = np.abs(ref).max() if ref.size else 0.0
    ok = rel <= rel_l2 and mx <= max_rel * mref
    return ok, rel, mx, mref


def assert_close(y, ref, what=""):
    ok, rel, mx, mref = close_enough(y, ref)
    assert ok, f"{what}: rel L2 {rel:.3e} (bar {REL_L2}), max|err| {mx:.3e} vs max|ref| {mref:.3e}"
    return rel


def device_layer(L: synth.LayerInputs, fmt: str = "nvfp4") -> dl.DeviceLayer:
    return dl.DeviceLayer(L.H, L.I, L.E, L.k, dl.to_device_u8(L.bank), torch.from_numpy(L.slot_of_expert).cuda(),
                          L.shared_slot, dl.to_device_bf16(L.wg), fmt)


def device_x(L: synth.LayerInputs) -> torch.Tensor:
    return dl.to_device_bf16(L.x)


def device_logits(L: synth.LayerInputs) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(L.logits)).cuda()
