"""The prefill from raw rows (gdn_prefill_conv_prepare + gdn_prefill_scan,
and gdn_prefill_conv_chunked) on the GPU, through the C ABI.

The results must equal, bit for bit, those of gdn_conv1d followed by
gdn_prefill_chunked on the q/k/v column views of its output: y, o, the
final state and the advanced conv window.  y is also checked bit for bit
against the oracle's fp32 convolution, and o / state against the oracle's
token scan within the dtype's tolerance.  Cases: the 4096-token bf16
layer, ragged varlen batches with windows, bias and initial states (empty,
1-3 token and multi-chunk sequences), chunk 16/32/64, d_k != d_v, one and
four v-heads per q/k head, tiled heads, strided x rows, and the fallback
cases (fp32, width 3)."""
import numpy as np
import pytest

from linear_attention_delta_amd import synth
from tests.gpu_util import TOL, note, rel_err_slices, to_dev, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def G():
    import torch
    assert torch.cuda.is_available()
    from linear_attention_delta_amd import gdn
    return gdn


def _bits(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy().view(np.uint32)


def _x_dev(inp, pad):
    """Device copy of the raw rows, with `pad` extra columns per row (a
    strided view, like a slice of a wider projection)."""
    import torch
    n, cc = inp.x.shape
    xs = torch.zeros((n, cc + pad), dtype=torch.float32)
    xs[:, :cc] = torch.from_numpy(inp.x)
    dt = torch.bfloat16 if inp.dtype == "bf16" else torch.float32
    return xs.to(dt).cuda()[:, :cc]


def _run(G, inp, w, *, fused, chunk, bias=None, heads_tiled=False, pad=0, split=False):
    """One prefill from raw rows.  Returns (y, o, state, window) on the host
    as raw bits (y, o, window) and fp32 (state)."""
    import torch
    sh = inp.shape
    n, cc = inp.x.shape
    dt = torch.bfloat16 if inp.dtype == "bf16" else torch.float32
    x = _x_dev(inp, pad)
    wd = to_dev(w)
    bd = None if bias is None else to_dev(bias)
    cu = None if inp.dense_T else torch.from_numpy(inp.cu_seqlens).cuda()
    seqlen = inp.dense_T if inp.dense_T else None
    win = None if inp.conv_state0 is None else to_dev(inp.conv_state0, inp.dtype)
    s0 = None if inp.state0 is None else torch.from_numpy(inp.state0).cuda()
    hv, dk, dv = sh.num_v_heads, sh.head_dim_k, sh.head_dim_v
    # outputs and workspace start as NaN / -1 bytes: anything left unwritten shows
    o = torch.full((n, hv, dv), float("nan"), dtype=dt, device="cuda")
    S = torch.full((inp.num_seqs, hv, dk, dv), float("nan"), dtype=torch.float32, device="cuda")
    if fused:
        y = torch.full((n, cc), float("nan"), dtype=dt, device="cuda")
        p = G.ConvPrefill(x, wd, num_qk_heads=sh.num_qk_heads, num_v_heads=hv, head_dim_k=dk, head_dim_v=dv,
                          cu_seqlens=cu, seqlen=seqlen, num_seqs=inp.num_seqs, chunk_size=chunk,
                          heads_tiled=heads_tiled, scale=inp.scale, bias=bd)
        p.ws.fill_(-1)
        g, beta = to_dev(inp.g), to_dev(inp.beta)
        if split:
            p.conv_prepare(x, y, g, beta, conv_state=win)
            p.scan(y, g, beta, o, s0, S)
        else:
            p(x, y, g, beta, o, s0, S, conv_state=win)
    else:
        y = G.conv1d(x, wd, cu_seqlens=cu, seqlen=seqlen, num_seqs=inp.num_seqs, bias=bd, conv_state=win)
        a = sh.num_qk_heads * dk
        q = y[:, :a].view(n, sh.num_qk_heads, dk)
        k = y[:, a:2 * a].view(n, sh.num_qk_heads, dk)
        v = y[:, 2 * a:].view(n, hv, dv)
        pp = G.Prefill(q, k, v, cu_seqlens=cu, seqlen=seqlen, num_seqs=inp.num_seqs, chunk_size=chunk,
                       heads_tiled=heads_tiled, scale=inp.scale)
        pp.ws.fill_(-1)
        pp(q, k, v, to_dev(inp.g), to_dev(inp.beta), o, s0, S)
    torch.cuda.synchronize()
    return _bits(y), _bits(o), S.cpu().numpy(), None if win is None else _bits(win)


def _oracle_check(orc, inp, w, bias, y_bits, o_bits, S, heads_tiled=False):
    """y bit-exact against the oracle's fp32 convolution; o and state within
    tolerance of the oracle's token scan on that y."""
    sh = inp.shape
    bf = inp.dtype == "bf16"
    ref = orc.conv1d_f32(inp.x, w, inp.cu_seqlens, window=inp.conv_state0, bias=bias, out_bf16=bf)
    assert np.array_equal(y_bits, ref if bf else ref.view(np.uint32)), "y differs from the oracle's convolution"
    y = (ref.astype(np.uint32) << 16).view(np.float32) if bf else ref
    q, k, v = synth.split_qkv(y, sh)
    o = (o_bits.astype(np.uint32) << 16).view(np.float32) if bf else o_bits.view(np.float32)
    o_ref, S_ref = orc.scan(q, k, v, inp.g, inp.beta, inp.cu_seqlens, state0=inp.state0, scale=inp.scale,
                            heads_tiled=heads_tiled)
    return rel_err_slices(o, o_ref, inp.cu_seqlens), rel_err_slices(S, S_ref)


def _check_equal(fu, un, what):
    for name, a, b in zip(("y", "o", "state", "window"), fu, un):
        if a is None and b is None:
            continue
        assert a.shape == b.shape and np.array_equal(a.view(np.uint8), b.view(np.uint8)), \
            f"{what}: raw-row entry point {name} differs from conv1d + prefill"


LENS = [0, 1, 2, 3, 5, 15, 16, 17, 63, 64, 65, 130, 200]


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_raw_rows_ragged_windows_bias(G, orc, chunk):
    sh = synth.LayerShape(2, 4, 128, 128)
    inp = synth.make_prefill(40 + chunk, sh, LENS, "bf16", state0_std=0.05, conv_state=True, chunk_size=chunk,
                             name="fused-ragged")
    bias = (0.3 * np.random.default_rng(chunk).standard_normal(sh.conv_channels)).astype(np.float32)
    note(f"raw-row ragged chunk={chunk}")
    fu = _run(G, inp, inp.conv_w, fused=True, chunk=chunk, bias=bias, pad=24)
    un = _run(G, inp, inp.conv_w, fused=False, chunk=chunk, bias=bias, pad=24)
    _check_equal(fu, un, f"chunk {chunk}")
    eo, es = _oracle_check(orc, inp, inp.conv_w, bias, fu[0], fu[1], fu[2])
    note(f"  o err {eo:.2e}  S err {es:.2e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


@pytest.mark.parametrize("hk,hv,dk,dv,tiled,chunk", [
    (4, 4, 128, 128, False, 64),    # one v-head per q/k head
    (2, 8, 64, 128, False, 32),     # four per head: two workgroups share a q/k head
    (2, 8, 128, 64, True, 64),      # tiled heads
    (3, 6, 64, 64, True, 16),
])
def test_raw_rows_head_layouts(G, orc, hk, hv, dk, dv, tiled, chunk):
    sh = synth.LayerShape(hk, hv, dk, dv)
    inp = synth.make_prefill(50 + hk + hv + dk // 8 + dv, sh, [70, 0, 129, 3, 64], "bf16", state0_std=0.05,
                             conv_state=True, chunk_size=chunk, name="fused-heads")
    note(f"raw-row heads hk={hk} hv={hv} dk={dk} dv={dv} tiled={tiled} chunk={chunk}")
    fu = _run(G, inp, inp.conv_w, fused=True, chunk=chunk, heads_tiled=tiled, split=True)
    un = _run(G, inp, inp.conv_w, fused=False, chunk=chunk, heads_tiled=tiled)
    _check_equal(fu, un, "heads")
    eo, es = _oracle_check(orc, inp, inp.conv_w, None, fu[0], fu[1], fu[2], heads_tiled=tiled)
    note(f"  o err {eo:.2e}  S err {es:.2e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


def test_raw_rows_qwen35_4k(G, orc):
    """The 4096-token bf16 layer (one sequence, 64 chunks, several carry
    segments), no window: equal to conv1d + prefill and within tolerance of the oracle."""
    inp = synth.prefill_4k_bf16()
    note(f"raw-row {inp.name}")
    fu = _run(G, inp, inp.conv_w, fused=True, chunk=64)
    un = _run(G, inp, inp.conv_w, fused=False, chunk=64)
    _check_equal(fu, un, inp.name)
    eo, es = _oracle_check(orc, inp, inp.conv_w, None, fu[0], fu[1], fu[2])
    note(f"  o err {eo:.2e}  S err {es:.2e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


def test_raw_rows_long_multi_segment(G, orc):
    """Three 1537-token sequences with windows and initial states: several
    carry segments per sequence and a ragged last chunk."""
    sh = synth.LayerShape(2, 4, 128, 128)
    inp = synth.make_prefill(61, sh, [1537, 1537, 1537], "bf16", state0_std=0.05, conv_state=True,
                             name="fused-long")
    note("raw-row long multi-segment")
    fu = _run(G, inp, inp.conv_w, fused=True, chunk=64)
    un = _run(G, inp, inp.conv_w, fused=False, chunk=64)
    _check_equal(fu, un, "long")
    eo, es = _oracle_check(orc, inp, inp.conv_w, None, fu[0], fu[1], fu[2])
    note(f"  o err {eo:.2e}  S err {es:.2e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


def test_raw_rows_fp32_and_width3(G, orc):
    """fp32, and bf16 with a width-3 convolution."""
    sh = synth.LayerShape(2, 4, 64, 64)
    inp = synth.make_prefill(71, sh, [40, 0, 3, 100], "f32", state0_std=0.05, conv_state=True, name="fused-f32")
    note("raw-row prefill fp32")
    fu = _run(G, inp, inp.conv_w, fused=True, chunk=32)
    un = _run(G, inp, inp.conv_w, fused=False, chunk=32)
    _check_equal(fu, un, "fp32")
    eo, es = _oracle_check(orc, inp, inp.conv_w, None, fu[0], fu[1], fu[2])
    assert eo <= TOL["f32"] and es <= TOL["f32"]

    inp = synth.make_prefill(72, sh, [40, 0, 3, 100], "bf16", state0_std=0.05, name="fused-w3")
    w3 = (0.5 * np.random.default_rng(3).standard_normal((sh.conv_channels, 3))).astype(np.float32)
    note("raw-row prefill width 3")
    fu = _run(G, inp, w3, fused=True, chunk=64)
    un = _run(G, inp, w3, fused=False, chunk=64)
    _check_equal(fu, un, "width 3")
    eo, es = _oracle_check(orc, inp, w3, None, fu[0], fu[1], fu[2])
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


def test_raw_rows_repeat_is_bitwise(G):
    """Two runs of the raw-row path on the same inputs give the same bits."""
    sh = synth.LayerShape(2, 4, 128, 128)
    inp = synth.make_prefill(81, sh, [300, 7, 64], "bf16", state0_std=0.05, conv_state=True, name="fused-rep")
    a = _run(G, inp, inp.conv_w, fused=True, chunk=64)
    b = _run(G, inp, inp.conv_w, fused=True, chunk=64)
    _check_equal(a, b, "repeat")
