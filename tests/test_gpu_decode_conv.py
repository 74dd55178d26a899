"""GPU decode step fused with the conv step (gdn_decode_conv_step) through the
C ABI: bit for bit the conv step followed by the plain decode step, and
within the layer's tolerance of the fp64 oracle on the 64-sequence decode
workload."""
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


def _bits(t):
    import torch
    t = t.detach().contiguous()
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


def _two_calls(G, x, w, bias, g, beta, S, cs, slots, *, hk, hv, dk, dv, tiled, scale, l2):
    """The conv step on the slots' windows (gathered, then scattered back),
    then the plain decode step on the q, k, v it stored."""
    import torch
    B = x.shape[0]
    idx = torch.arange(B, device=x.device) if slots is None else slots.long()
    win = cs[idx].contiguous()
    y = G.conv1d(x, w, seqlen=1, num_seqs=B, bias=bias, conv_state=win)
    cs[idx] = win
    a = hk * dk
    q = y[:, :a].view(B, hk, dk)
    k = y[:, a:2 * a].view(B, hk, dk)
    v = y[:, 2 * a:].view(B, hv, dv)
    return G.decode_step(q, k, v, g, beta, S, state_slots=slots, l2norm=l2, heads_tiled=tiled, scale=scale)


@pytest.mark.parametrize("dtype,dk,dv,hk,hv,width,tiled,scale,l2,use_bias,use_slots", [
    ("bf16", 128, 128, 2, 4, 4, False, 1.0, True, False, False),
    ("bf16", 128, 128, 2, 4, 4, True, 0.088, True, True, True),
    ("bf16", 64, 128, 3, 3, 2, False, 1.0, True, True, True),     # one v-head per q/k head
    ("bf16", 128, 64, 1, 3, 8, False, 1.0, False, False, True),   # three per q/k head
    ("bf16", 64, 64, 2, 8, 5, True, 0.5, True, True, False),      # four per q/k head
    ("f32", 128, 128, 2, 4, 4, False, 1.0, True, True, True),
    ("f32", 64, 64, 1, 4, 3, True, 2.0, True, False, False),
    # wide windows with 128 x 128 heads load the conv inputs after the state
    ("bf16", 128, 128, 1, 2, 8, False, 1.0, True, True, True),
    ("f32", 128, 128, 2, 2, 6, True, 1.0, True, False, True),
])
def test_fused_equals_conv_then_decode(G, dtype, dk, dv, hk, hv, width, tiled, scale, l2, use_bias, use_slots):
    import torch
    note(f"decode_conv dtype={dtype} dk={dk} dv={dv} hk={hk} hv={hv} W={width} tiled={tiled} slots={use_slots}")
    r = np.random.default_rng(1000 * width + dk + dv + hv)
    B, nslots = 5, 9
    cc = 2 * hk * dk + hv * dv
    w = to_dev((0.5 * r.normal(size=(cc, width))).astype(np.float32))
    bias = to_dev((0.2 * r.normal(size=cc)).astype(np.float32)) if use_bias else None
    win0 = r.normal(size=(nslots, width - 1, cc)).astype(np.float32)
    S0 = (0.05 * r.normal(size=(nslots, hv, dk, dv))).astype(np.float32)
    cs_a, cs_b = to_dev(win0, dtype), to_dev(win0, dtype)
    S_a, S_b = torch.from_numpy(S0).cuda(), torch.from_numpy(S0).cuda()
    slots = torch.tensor([7, 2, 0, 5, 3], dtype=torch.int32).cuda() if use_slots else None
    fused = G.DecodeConv(torch.empty((B, cc), dtype=cs_a.dtype, device="cuda"), w, num_qk_heads=hk,
                         num_v_heads=hv, head_dim_k=dk, head_dim_v=dv, num_slots=nslots, bias=bias, l2norm=l2,
                         heads_tiled=tiled, scale=scale)
    o_a = torch.empty((B, hv, dv), dtype=cs_a.dtype, device="cuda")
    for step in range(4):
        # every other step reads its rows from a wider buffer (strided x)
        xs = r.normal(size=(B, cc + (8 if step % 2 else 0))).astype(np.float32)
        x = to_dev(xs, dtype)[:, :cc] if step % 2 else to_dev(xs, dtype)
        g = to_dev((-np.logaddexp(0, r.normal(size=(B, hv))) * 0.5).astype(np.float32))
        beta = to_dev((1 / (1 + np.exp(-r.normal(size=(B, hv))))).astype(np.float32))
        if step % 2:
            G.decode_conv_step(x, w, g, beta, S_a, cs_a, num_qk_heads=hk, num_v_heads=hv, head_dim_k=dk,
                               head_dim_v=dv, bias=bias, state_slots=slots, l2norm=l2, heads_tiled=tiled,
                               scale=scale, out=o_a)
        else:
            fused(x, g, beta, S_a, cs_a, o_a, state_slots=slots)
        o_b = _two_calls(G, x, w, bias, g, beta, S_b, cs_b, slots, hk=hk, hv=hv, dk=dk, dv=dv, tiled=tiled,
                         scale=scale, l2=l2)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(o_a), _bits(o_b)), f"o differs at step {step}"
        assert np.array_equal(_bits(S_a), _bits(S_b)), f"state differs at step {step}"
        assert np.array_equal(_bits(cs_a), _bits(cs_b)), f"conv window differs at step {step}"
    assert np.all(np.isfinite(to_np(o_a)))
    if use_slots:  # slots no sequence names keep their state and window
        for s in (1, 4, 6, 8):
            assert np.array_equal(to_np(S_a)[s], S0[s])
            assert np.array_equal(to_np(cs_a)[s], to_np(to_dev(win0, dtype))[s])


def test_fused_bad_slot(G):
    """A slot index out of range gives NaN outputs for that sequence only and
    leaves every state and window alone."""
    import torch
    r = np.random.default_rng(5)
    B, hk, hv, d, width, nslots = 4, 2, 4, 64, 4, 6
    cc = 2 * hk * d + hv * d
    w = to_dev((0.5 * r.normal(size=(cc, width))).astype(np.float32))
    cs = to_dev(r.normal(size=(nslots, width - 1, cc)).astype(np.float32), "bf16")
    S = torch.from_numpy((0.05 * r.normal(size=(nslots, hv, d, d))).astype(np.float32)).cuda()
    x = to_dev(r.normal(size=(B, cc)).astype(np.float32), "bf16")
    g = to_dev(np.full((B, hv), -0.1, np.float32))
    beta = to_dev(np.full((B, hv), 0.5, np.float32))
    slots = torch.tensor([1, 6, 3, -2], dtype=torch.int32).cuda()
    S_before, cs_before = _bits(S), _bits(cs)
    o = G.decode_conv_step(x, w, g, beta, S, cs, num_qk_heads=hk, num_v_heads=hv, head_dim_k=d, head_dim_v=d,
                           state_slots=slots)
    torch.cuda.synchronize()
    on = to_np(o)
    assert np.all(np.isnan(on[1])) and np.all(np.isnan(on[3]))
    assert np.all(np.isfinite(on[0])) and np.all(np.isfinite(on[2]))
    S_after, cs_after = _bits(S), _bits(cs)
    for s in set(range(nslots)) - {1, 3}:
        assert np.array_equal(S_after[s], S_before[s]) and np.array_equal(cs_after[s], cs_before[s])
    for s in (1, 3):
        assert not np.array_equal(cs_after[s], cs_before[s])


# The fused step on the 64-sequence decode workload against the oracle (every
# sequence, 1000 steps) is tests/test_gpu_decode.py::test_decode_b64_1000_steps.
