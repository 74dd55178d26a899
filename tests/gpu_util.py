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

from linear_attention_delta_amd import synth

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
    [N][H][dk][dv] (slices by leading two axes).  Vectorised over heads (and
    over sequences when they all have one length), so every (sequence, head)
    slice of a large workload is checked in seconds."""
    x = np.asarray(x)
    ref = np.asarray(ref)
    assert x.shape == ref.shape, (x.shape, ref.shape)

    def ratio(num, den):
        return float(np.max(np.where(den > 0, num / np.where(den > 0, den, 1.0), num))) if num.size else 0.0

    if x.ndim == 4:
        d = np.abs(x.astype(np.float64) - ref)
        return ratio(np.max(d, axis=(2, 3)), np.max(np.abs(ref), axis=(2, 3)).astype(np.float64))
    cu = np.array([0, x.shape[0]]) if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int64)
    lens = np.diff(cu)
    if lens.size and np.all(lens == lens[0]) and lens[0] > 0 and cu[0] == 0:
        n, L = lens.size, int(lens[0])
        xs = x[:n * L].reshape(n, L, *x.shape[1:])
        rs = ref[:n * L].reshape(n, L, *ref.shape[1:])
        d = np.abs(xs.astype(np.float64) - rs)
        return ratio(np.max(d, axis=(1, 3)), np.max(np.abs(rs), axis=(1, 3)).astype(np.float64))
    worst = 0.0
    for i in range(len(cu) - 1):
        a, b = int(cu[i]), int(cu[i + 1])
        if a == b:
            continue
        d = np.abs(x[a:b].astype(np.float64) - ref[a:b])
        worst = max(worst, ratio(np.max(d, axis=(0, 2)), np.max(np.abs(ref[a:b]), axis=(0, 2)).astype(np.float64)))
    return worst


def oracle_scan_all(orc, inp, y, *, state0="inp", heads_tiled=False, scale=None, l2norm=True):
    """The oracle's token scan over every (sequence, v-head) of a workload in
    one threaded call, on the q/k/v column blocks of the conv output y.
    Returns (o [N_tok][H_v][d_v], S [N][H_v][d_k][d_v]) in fp64."""
    q, k, v = synth.split_qkv(y, inp.shape)
    s0 = inp.state0 if isinstance(state0, str) else state0
    return orc.scan(q, k, v, inp.g, inp.beta, inp.cu_seqlens, state0=s0,
                    scale=inp.scale if scale is None else scale, l2norm=l2norm, heads_tiled=heads_tiled)


def conv_inputs(orc, inp, *, gpu_dtype=None):
    """Run the oracle's fp32 conv (+SiLU) on a workload's raw inputs, returning
    y as fp32 numpy holding exactly the dtype's values (bf16-rounded for bf16)."""
    if inp.dtype == "bf16":
        bits = orc.conv1d_f32(inp.x, inp.conv_w, inp.cu_seqlens, window=inp.conv_state0, out_bf16=True)
        return (bits.astype(np.uint32) << 16).view(np.float32)
    return orc.conv1d_f32(inp.x, inp.conv_w, inp.cu_seqlens, window=inp.conv_state0)
