"""GPU gates from the raw projections (gdn_gating) through the C ABI against
the fp64 oracle: the 4096-token layer's shape with a and b as column blocks
of one projection, fp32 inputs, and the tails of softplus and the sigmoid."""
import numpy as np
import pytest

from linear_attention_delta_amd import synth
from tests.gpu_util import note, to_dev, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def G():
    import torch
    assert torch.cuda.is_available()
    from linear_attention_delta_amd import gdn
    return gdn


def _rel(x, ref):
    """Worst elementwise relative error (fp32 arithmetic: a few ulp)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(x - ref) / np.maximum(np.abs(ref), 1e-300)))


@pytest.mark.parametrize("dtype,n,h", [("bf16", 4096, 32), ("f32", 333, 5), ("bf16", 1, 1)])
def test_gating_matches_oracle(G, orc, dtype, n, h):
    note(f"gating dtype={dtype} n={n} h={h}")
    ab, A_log, dt_bias = synth.gating_inputs(9, n, h, dtype)
    ab_dev = to_dev(ab, dtype)
    g, beta = G.gating(ab_dev[:, :h], ab_dev[:, h:], to_dev(A_log), to_dev(dt_bias))
    g_ref, b_ref = orc.gating(ab[:, :h], ab[:, h:], A_log, dt_bias)
    eg, eb = _rel(to_np(g), g_ref), _rel(to_np(beta), b_ref)
    note(f"  g rel err {eg:.2e}, beta rel err {eb:.2e}")
    assert eg <= 1e-5 and eb <= 1e-5


def test_gating_tails(G, orc):
    """Large |a + dt_bias| and |b|: softplus -> x and -> e^x, the sigmoid
    -> 1 and -> e^b, with no overflow and no loss of the small side."""
    x = np.array([[-80.0, -30.0, -5.0, 0.0, 5.0, 30.0, 80.0, 1e-7]], np.float32)
    h = x.shape[1]
    A_log = np.linspace(-1, 1, h).astype(np.float32)
    dt_bias = np.zeros(h, np.float32)
    g, beta = G.gating(to_dev(x), to_dev(x), to_dev(A_log), to_dev(dt_bias))
    g_ref, b_ref = orc.gating(x, x, A_log, dt_bias)
    gn, bn = to_np(g), to_np(beta)
    assert np.all(np.isfinite(gn)) and np.all(gn < 0) and np.all((bn > 0) & (bn <= 1))
    assert _rel(gn, g_ref) <= 1e-5 and _rel(bn, b_ref) <= 1e-5
