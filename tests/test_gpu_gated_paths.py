"""GPU prefill and decode with the gates computed inside the kernels from
their raw projections (gdn_prefill_conv_gated, gdn_decode_conv_gated_step),
through the C ABI: bit for bit gdn_gating followed by the calls that take g
and beta, on the 4096-token bf16 layer, an fp32 varlen batch and the
64-sequence decode workload; and g, beta themselves against the oracle."""
import numpy as np
import pytest
import torch

from linear_attention_delta_amd import synth
from tests.gpu_util import note, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def G():
    assert torch.cuda.is_available()
    from linear_attention_delta_amd import gdn
    return gdn


def _bits(t):
    t = t.detach().contiguous()
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


@pytest.mark.parametrize("which", ["4k-bf16", "varlen-f32", "varlen-bf16-c32"])
def test_gated_prefill_equals_gating_then_prefill(G, which):
    if which == "4k-bf16":
        inp, dtype, cu, chunk = synth.prefill_4k_bf16(), "bf16", None, 64
    elif which == "varlen-bf16-c32":
        # the segment-parallel carry over several sequences, chunk 32, ragged tails
        lens = [5, 300, 1031, 64]
        inp = synth.make_prefill(13, synth.QWEN35_4B, lens, "bf16", name="gated-varlen-bf16")
        dtype, chunk = "bf16", 32
        cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).cuda()
    else:
        inp = synth.make_prefill(12, synth.TINY, [1, 70, 33, 128], "f32", name="gated-varlen")
        dtype, chunk = "f32", 16
        cu = torch.from_numpy(np.concatenate([[0], np.cumsum([1, 70, 33, 128])]).astype(np.int32)).cuda()
    sh = inp.shape
    T = inp.total_tokens
    hv = sh.num_v_heads
    note(f"gated prefill {which}: T={T}")
    ab, A_log, dt_bias = synth.gating_inputs(21, T, hv, dtype)
    ab_d = to_dev(ab, dtype)
    a_, b_ = ab_d[:, :hv], ab_d[:, hv:]
    A_d, D_d = to_dev(A_log), to_dev(dt_bias)
    x = to_dev(inp.x, dtype)
    w = to_dev(inp.conv_w)
    kw = dict(num_qk_heads=sh.num_qk_heads, num_v_heads=hv, head_dim_k=sh.head_dim_k, head_dim_v=sh.head_dim_v,
              chunk_size=chunk)
    if cu is None:
        p = G.ConvPrefill(x, w, seqlen=T, **kw)
        nseq = 1
    else:
        p = G.ConvPrefill(x, w, cu_seqlens=cu, **kw)
        nseq = cu.numel() - 1
    cc = sh.conv_channels
    S0 = torch.from_numpy((0.02 * np.random.default_rng(5).normal(size=(nseq, hv, sh.head_dim_k, sh.head_dim_v)))
                          .astype(np.float32)).cuda()
    win0 = to_dev(np.random.default_rng(6).normal(size=(nseq, 3, cc)).astype(np.float32), dtype)
    outs = []
    for gated in (False, True):
        y = torch.empty((T, cc), dtype=x.dtype, device="cuda")
        o = torch.empty((T, hv, sh.head_dim_v), dtype=x.dtype, device="cuda")
        st = torch.empty_like(S0)
        win = win0.clone()
        if gated:
            G.conv_prefill_gated(p, x, y, G.gate_inputs(a_, b_, A_d, D_d), o, state_in=S0, state_out=st,
                                 conv_state=win)
        else:
            g, beta = G.gating(a_, b_, A_d, D_d)
            p(x, y, g, beta, o, S0, st, win)
        torch.cuda.synchronize()
        outs.append((y, o, st, win))
    for name, u, v in zip(("y", "o", "state", "window"), outs[0], outs[1]):
        assert np.array_equal(_bits(u), _bits(v)), f"{name} differs"
    assert np.all(np.isfinite(outs[1][1].float().cpu().numpy()))


def test_gated_decode_equals_gating_then_decode(G):
    inp = synth.decode_b64_bf16()
    sh = inp.shape
    B, hv = inp.batch, sh.num_v_heads
    note(f"gated decode {inp.name}")
    w = to_dev(inp.conv_w)
    step = G.DecodeConv(to_dev(inp.x[0], "bf16"), w, num_qk_heads=sh.num_qk_heads, num_v_heads=hv,
                        head_dim_k=sh.head_dim_k, head_dim_v=sh.head_dim_v, num_slots=B + 3)
    r = np.random.default_rng(8)
    S0 = torch.from_numpy((0.02 * r.normal(size=(B + 3, hv, sh.head_dim_k, sh.head_dim_v))).astype(np.float32)).cuda()
    win0 = to_dev(r.normal(size=(B + 3, 3, sh.conv_channels)).astype(np.float32), "bf16")
    slots = torch.from_numpy(r.permutation(B + 3)[:B].astype(np.int32)).cuda()
    S_a, S_b, W_a, W_b = S0.clone(), S0.clone(), win0.clone(), win0.clone()
    o_a = torch.empty((B, hv, sh.head_dim_v), dtype=torch.bfloat16, device="cuda")
    o_b = torch.empty_like(o_a)
    for i in range(5):
        ab, A_log, dt_bias = synth.gating_inputs(30 + i, B, hv, "bf16")
        ab_d = to_dev(ab, "bf16")
        a_, b_ = ab_d[:, :hv], ab_d[:, hv:]
        A_d, D_d = to_dev(A_log), to_dev(dt_bias)
        x = to_dev(inp.x[i % inp.pool], "bf16")
        G.decode_conv_gated_step(step, x, G.gate_inputs(a_, b_, A_d, D_d), S_a, W_a, o_a, state_slots=slots)
        g, beta = G.gating(a_, b_, A_d, D_d)
        step(x, g, beta, S_b, W_b, o_b, state_slots=slots)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(o_a), _bits(o_b)), f"o differs at step {i}"
        assert np.array_equal(_bits(S_a), _bits(S_b)), f"state differs at step {i}"
        assert np.array_equal(_bits(W_a), _bits(W_b)), f"window differs at step {i}"


def test_gated_decode_tiled_heads_group4(G, orc):
    """The gated, fused decode step with tiled head order and four v-heads per
    q/k head, against gating + conv step + plain decode step in fp64."""
    hk, hv, d, B, W = 2, 8, 64, 3, 4
    cc = 2 * hk * d + hv * d
    r = np.random.default_rng(44)
    x = r.normal(size=(B, cc)).astype(np.float32)
    w = (0.5 * r.normal(size=(cc, W))).astype(np.float32)
    win = r.normal(size=(B, W - 1, cc)).astype(np.float32)
    S0 = (0.05 * r.normal(size=(B, hv, d, d))).astype(np.float32)
    ab, A_log, dt_bias = synth.gating_inputs(45, B, hv, "f32")
    S = torch.from_numpy(S0).cuda()
    Wd = to_dev(win)
    step = G.DecodeConv(to_dev(x), to_dev(w), num_qk_heads=hk, num_v_heads=hv, head_dim_k=d, head_dim_v=d,
                        num_slots=B, heads_tiled=True)
    abd = to_dev(ab)
    o = torch.empty((B, hv, d), dtype=torch.float32, device="cuda")
    G.decode_conv_gated_step(step, to_dev(x), G.gate_inputs(abd[:, :hv], abd[:, hv:], to_dev(A_log), to_dev(dt_bias)),
                             S, Wd, o)
    torch.cuda.synchronize()
    g, beta = orc.gating(ab[:, :hv], ab[:, hv:], A_log, dt_bias)
    cu1 = np.arange(B + 1).astype(np.int32)
    y = orc.conv1d_f32(x, w, cu1, window=win)
    q, k, v = y[:, :hk * d].reshape(B, hk, d), y[:, hk * d:2 * hk * d].reshape(B, hk, d), y[:, 2 * hk * d:].reshape(B, hv, d)
    o_ref, S_ref = orc.decode_step(q, k, v, g, beta, S0, heads_tiled=True)
    eo = float(np.max(np.abs(o.cpu().numpy() - o_ref)) / np.max(np.abs(o_ref)))
    es = float(np.max(np.abs(S.cpu().numpy() - S_ref)) / np.max(np.abs(S_ref)))
    note(f"  gated tiled decode: o err {eo:.2e}, S err {es:.2e}")
    assert eo <= 2e-3 and es <= 2e-3
    assert np.array_equal(Wd[:, -1].cpu().numpy(), x)
