"""gdn_prefill_chunked_noalloc through the C ABI: the same results as
gdn_prefill_chunked with a caller workspace, bit for bit, on two calls in a
row (the second on a smaller problem, so the library's array holds the first
call's contents when the second starts)."""
import ctypes

import numpy as np
import pytest

from linear_attention_delta_amd import synth
from tests.gpu_util import conv_inputs, note, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def G():
    import torch
    assert torch.cuda.is_available()
    from linear_attention_delta_amd import gdn
    return gdn


def _views(y, sh, dtype):
    yd = to_dev(y, dtype)
    n, a = y.shape[0], sh.num_qk_heads * sh.head_dim_k
    return (yd[:, :a].view(n, sh.num_qk_heads, sh.head_dim_k), yd[:, a:2 * a].view(n, sh.num_qk_heads, sh.head_dim_k),
            yd[:, 2 * a:].view(n, sh.num_v_heads, sh.head_dim_v))


def _both(G, orc, inp):
    import torch
    sh = inp.shape
    y = conv_inputs(orc, inp)
    q, k, v = _views(y, sh, inp.dtype)
    g, beta = to_dev(inp.g), to_dev(inp.beta)
    cu = None if inp.dense_T else torch.from_numpy(inp.cu_seqlens).cuda()
    s0 = None if inp.state0 is None else torch.from_numpy(inp.state0).cuda()
    kw = dict(cu_seqlens=cu, seqlen=inp.dense_T or None, num_seqs=inp.num_seqs, chunk_size=inp.chunk_size)
    o_ref, S_ref = G.prefill(q, k, v, g, beta, state_in=s0, **kw)
    n, hv, dv = v.shape
    o = torch.full((n, hv, dv), float("nan"), dtype=q.dtype, device="cuda")
    S = torch.full((inp.num_seqs, hv, sh.head_dim_k, dv), float("nan"), dtype=torch.float32, device="cuda")
    G.prefill_noalloc(q, k, v, g, beta, o, S, state_in=s0, **kw)
    torch.cuda.synchronize()
    return o, S, o_ref, S_ref


def test_noalloc_equals_workspace_call_twice(G, orc):
    """The 4096-token bf16 layer (62.9 MB of workspace), then a smaller ragged
    batch with initial states: each equals the workspace call bit for bit."""
    import torch
    big = synth.prefill_4k_bf16()
    small = synth.make_prefill(12, synth.LayerShape(2, 4, 128, 64), [300, 0, 17, 1000, 64], "bf16",
                               state0_std=0.05, chunk_size=32, name="noalloc-small")
    for inp in (big, small):
        note(f"noalloc {inp.name}")
        o, S, o_ref, S_ref = _both(G, orc, inp)
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), inp.name
        assert torch.equal(S, S_ref), inp.name
    # and the large one again after the small one (stale small-call contents)
    o, S, o_ref, S_ref = _both(G, orc, big)
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)) and torch.equal(S, S_ref)


def test_noalloc_rejects_problems_beyond_its_array(G):
    d = G.make_dims(num_seqs=1, total_tokens=8192, seqlen=8192, num_qk_heads=16, num_v_heads=32, head_dim_k=128,
                    head_dim_v=128)
    assert G.workspace_size(d) > 64 << 20
    st = G.lib.gdn_prefill_chunked_noalloc(ctypes.byref(d), 16, 16, 16, 16, 16, None, None, 16, None, None)
    assert st == 2 and "no-allocation" in G.last_error()
