"""GDN_DEBUG=1: every entry point synchronises after its launches and scans
its outputs for NaN/Inf, returning GDN_ERR_NONFINITE when it finds one (the
per-stage NaN/Inf probe of the oxydllm 0.0.0-alpha.12.2 notes, "New
Features", GDN debug aids).  Without the variable the same calls succeed."""
import os

import pytest

from linear_attention_delta_amd import synth
from tests.gpu_util import note, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def G():
    import torch
    assert torch.cuda.is_available()
    from linear_attention_delta_amd import gdn
    return gdn


@pytest.fixture
def debug_env():
    old = os.environ.get("GDN_DEBUG")
    yield
    if old is None:
        os.environ.pop("GDN_DEBUG", None)
    else:
        os.environ["GDN_DEBUG"] = old


def _expect(G, fn, status):
    try:
        fn()
    except G.GdnError as e:
        assert e.status == status, (e.status, str(e))
        return
    assert status == G.GDN_OK, "expected an error"


def test_debug_probe_flags_nonfinite_outputs(G, debug_env):
    import torch
    sh = synth.LayerShape(2, 4, 64, 64)
    inp = synth.make_prefill(91, sh, [70, 33], "bf16", name="debug")
    cu = torch.from_numpy(inp.cu_seqlens).cuda()
    w = to_dev(inp.conv_w)
    x = to_dev(inp.x, "bf16")
    bad = x.clone()
    bad[5, 3] = float("nan")
    g, beta = to_dev(inp.g), to_dev(inp.beta)
    a = sh.num_qk_heads * sh.head_dim_k
    n = x.shape[0]

    def prefill(xx):
        y = G.conv1d(xx, w, cu_seqlens=cu)
        q = y[:, :a].view(n, 2, 64)
        k = y[:, a:2 * a].view(n, 2, 64)
        v = y[:, 2 * a:].view(n, 4, 64)
        G.prefill(q, k, v, g, beta, cu_seqlens=cu)
        torch.cuda.synchronize()

    GDN_ERR_NONFINITE = 5
    for flag in ("0", "1"):
        os.environ["GDN_DEBUG"] = flag
        note(f"GDN_DEBUG={flag}")
        _expect(G, lambda: prefill(x), G.GDN_OK)
        _expect(G, lambda: G.conv1d(bad, w, cu_seqlens=cu), GDN_ERR_NONFINITE if flag == "1" else G.GDN_OK)
        # the scan's probe: finite q, k, v with one NaN gate
        y = G.conv1d(x, w, cu_seqlens=cu)
        q = y[:, :a].view(n, 2, 64)
        k = y[:, a:2 * a].view(n, 2, 64)
        v = y[:, 2 * a:].view(n, 4, 64)
        gbad = g.clone()
        gbad[40, 1] = float("nan")
        _expect(G, lambda: G.prefill(q, k, v, gbad, beta, cu_seqlens=cu), GDN_ERR_NONFINITE if flag == "1" else G.GDN_OK)
        torch.cuda.synchronize()
