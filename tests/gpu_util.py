"""Helpers for the GPU parity tests: moving seeded inputs to the device
bit-exactly and the error metric.

Error metric: for each (sequence, v-head) slice, max|x - ref| / max|ref|;
the test reports the max over slices.  Tolerances come from the layer's
stated bars: fp32 inputs <= 2e-3, bf16 inputs <= 2e-2; conv and indexing
bit-exact.
"""
from __future__ import annotations

import sys

import numpy as np

TOL = {"f32": 2e-3, "bf16": 2e-2}


def note(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def torch_dtype(dtype: str):
    import torch
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def to_dev(a: np.ndarray, dtype: str = "f32"):
    """fp32 numpy (dtype-representable) -> device tensor, exactly."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch_dtype(dtype)).cuda()


def bits_to_dev(bits: np.ndarray):
    """bf16 bit patterns (uint16) -> device bf16 tensor."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.cuda()


def to_np(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float32).cpu().numpy()


def rel_err_slices(x: np.ndarray, ref: np.ndarray, cu_seqlens=None) -> float:
    """x, ref: o [N_tok][H][d] (slices by sequence and head) or S
    [N][H][dk][dv] (slices by leading two axes)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    worst = 0.0
    if x.ndim == 4:
        for s in range(x.shape[0]):
            for h in range(x.shape[1]):
                den = np.max(np.abs(ref[s, h]))
                num = np.max(np.abs(x[s, h] - ref[s, h]))
                worst = max(worst, num / den if den > 0 else num)
        return worst
    cu = [0, x.shape[0]] if cu_seqlens is None else list(cu_seqlens)
    for i in range(len(cu) - 1):
        a, b = int(cu[i]), int(cu[i + 1])
        if a == b:
            continue
        for h in range(x.shape[1]):
            den = np.max(np.abs(ref[a:b, h]))
            num = np.max(np.abs(x[a:b, h] - ref[a:b, h]))
            worst = max(worst, num / den if den > 0 else num)
    return worst


def conv_inputs(orc, inp, *, gpu_dtype=None):
    """Run the oracle's fp32 conv (+SiLU) on a workload's raw inputs, returning
    y as fp32 numpy holding exactly the dtype's values (bf16-rounded for bf16)."""
    if inp.dtype == "bf16":
        bits = orc.conv1d_f32(inp.x, inp.conv_w, inp.cu_seqlens, window=inp.conv_state0, out_bf16=True)
        return (bits.astype(np.uint32) << 16).view(np.float32)
    return orc.conv1d_f32(inp.x, inp.conv_w, inp.cu_seqlens, window=inp.conv_state0)
