"""GPU gated RMS norm (gdn_gated_rmsnorm) through the C ABI against the fp64
oracle: the 4096-token layer's output shape in bf16, fp32 with strided
rows, in place, and rows where eps or the gate decide the result."""
import numpy as np
import pytest

from linear_attention_delta_amd import synth
from tests.gpu_util import TOL, note, to_dev, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def G():
    import torch
    assert torch.cuda.is_available()
    from linear_attention_delta_amd import gdn
    return gdn


def _row_err(y, ref):
    """Worst (token, head) row of max|y - ref| / max|ref| (rows of zeros use 1)."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.maximum(np.max(np.abs(ref), axis=-1), 1e-30)
    return float(np.max(np.max(np.abs(y - ref), axis=-1) / den))


@pytest.mark.parametrize("dtype,n,h,d", [("bf16", 4096, 32, 128), ("bf16", 37, 3, 64), ("f32", 300, 5, 128),
                                         ("f32", 1, 1, 64), ("bf16", 1001, 7, 128)])
def test_gated_norm_matches_oracle(G, orc, dtype, n, h, d):
    note(f"gated norm dtype={dtype} n={n} h={h} d={d}")
    r = np.random.default_rng(n + h + d)
    o = r.normal(size=(n, h, d)).astype(np.float32) * np.exp(r.normal(size=(n, h, 1))).astype(np.float32)
    o = synth.round_bf16(o) if dtype == "bf16" else o
    z, w = synth.gate_inputs(7, n, h, d, dtype)
    y = G.gated_rmsnorm(to_dev(o, dtype), to_dev(z, dtype), to_dev(w))
    ref = orc.gated_rmsnorm(o, z, w)
    err = _row_err(to_np(y), ref)
    note(f"  worst row error {err:.2e}")
    assert err <= TOL[dtype]


def test_gated_norm_strided_and_in_place(G, orc):
    """Token rows inside wider buffers (as the carry's o and a fused
    projection's z would be), and y written over o."""
    import torch
    r = np.random.default_rng(3)
    n, h, d = 129, 4, 128
    big_o = r.normal(size=(n, h * d + 64)).astype(np.float32)
    big_z = r.normal(size=(n, h * d + 32)).astype(np.float32)
    w = (1 + 0.1 * r.normal(size=d)).astype(np.float32)
    big_o_dev = to_dev(big_o)
    o_dev = big_o_dev[:, 16:16 + h * d].view(n, h, d)
    z_dev = to_dev(big_z)[:, :h * d].view(n, h, d)
    ref = orc.gated_rmsnorm(big_o[:, 16:16 + h * d].reshape(n, h, d), big_z[:, :h * d].reshape(n, h, d), w)
    y = G.gated_rmsnorm(o_dev, z_dev, to_dev(w))
    assert _row_err(to_np(y), ref) <= 1e-5
    G.GatedNorm(o_dev, z_dev, to_dev(w), y=o_dev)(o_dev, z_dev, o_dev)     # in place, through the bound call
    torch.cuda.synchronize()
    assert _row_err(to_np(o_dev), ref) <= 1e-5
    after = to_np(big_o_dev)
    assert np.array_equal(after[:, :16], big_o[:, :16]) and np.array_equal(after[:, 16 + h * d:], big_o[:, 16 + h * d:])


def test_gated_norm_edge_rows(G, orc):
    """Zero rows (y = 0), rows so small that eps sets the scale, a zero gate,
    large gates of both signs, and a row dominated by one large value."""
    n, h, d = 6, 1, 64
    o = np.zeros((n, h, d), np.float32)
    z = np.ones((n, h, d), np.float32)
    o[1] = 1e-5
    o[2] = np.linspace(-1, 1, d)
    z[2] = 0.0
    o[3] = np.linspace(-2, 3, d)
    z[3] = np.where(np.arange(d) % 2, 30.0, -30.0)
    o[4, 0, 5] = 1e15
    o[5] = np.linspace(0.5, 1.5, d)
    w = np.linspace(0.5, 2.0, d).astype(np.float32)
    y = to_np(G.gated_rmsnorm(to_dev(o), to_dev(z), to_dev(w)))
    ref = orc.gated_rmsnorm(o, z, w)
    assert np.all(y[0] == 0.0) and np.all(y[2] == 0.0)
    assert np.all(np.isfinite(y))
    assert _row_err(y, ref) <= 1e-5
