"""GPU causal conv1d (+SiLU) through the C ABI against the oracle's fp32
evaluation: bit-exact outputs and windows."""
import numpy as np
import pytest

from linear_attention_delta_amd import synth
from tests.gpu_util import bits_to_dev, note, to_dev, to_np

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


def _oracle_bits(orc, x, w, cu, win, bias, silu, dtype):
    if dtype == "bf16":
        return orc.conv1d_f32(x, w, cu, window=win, bias=bias, silu=silu, out_bf16=True)
    return orc.conv1d_f32(x, w, cu, window=win, bias=bias, silu=silu).view(np.uint32)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("width", [2, 4, 5, 8])
def test_conv_varlen_bitexact(G, orc, dtype, width):
    import torch
    note(f"conv varlen dtype={dtype} W={width}")
    r = np.random.default_rng(width)
    C = 96 if dtype == "f32" else 160
    lens = [1, 0, 2, 3, 37, 16, 5, 70]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    N = int(cu[-1])
    x = synth.round_bf16(r.normal(size=(N, C)).astype(np.float32)) if dtype == "bf16" else r.normal(size=(N, C)).astype(np.float32)
    w = (0.5 * r.normal(size=(C, width))).astype(np.float32)
    bias = r.normal(size=C).astype(np.float32)
    win = r.normal(size=(len(lens), width - 1, C)).astype(np.float32)
    if dtype == "bf16":
        win = synth.round_bf16(win)
    for use_win in (False, True):
        for b in (None, bias):
            for silu in (True, False):
                # strided x (rows padded) like a slice of a wider projection
                xs = torch.zeros((N, C + 16), dtype=torch.float32)
                xs[:, :C] = torch.from_numpy(x)
                xd = xs.to(torch.bfloat16 if dtype == "bf16" else torch.float32).cuda()[:, :C]
                cs = to_dev(win, dtype) if use_win else None
                y = G.conv1d(xd, to_dev(w), cu_seqlens=torch.from_numpy(cu).cuda(),
                             bias=to_dev(b) if b is not None else None, conv_state=cs, activation=silu)
                torch.cuda.synchronize()
                ref = _oracle_bits(orc, x, w, cu, win if use_win else None, b, silu, dtype)
                assert np.array_equal(_bits(y), ref), f"conv mismatch win={use_win} bias={b is not None} silu={silu}"
                if use_win:
                    _, wref = orc.conv1d(x, w, cu, window=win)
                    got = to_np(cs)
                    for i, L in enumerate(lens):
                        if L == 0:
                            assert np.array_equal(got[i], win[i])
                    assert np.array_equal(got, wref.astype(np.float32)), "window update"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [33, 32])
def test_conv_dense_and_step(G, orc, dtype, T):
    """T = 32: every sequence starts on a 16-token span boundary, so each
    span at a sequence start reads its halo from that sequence's window;
    T = 33: sequence starts fall inside spans."""
    import torch
    note(f"conv dense + decode step dtype={dtype} T={T}")
    r = np.random.default_rng(5)
    B, C, W = 3, 64, 4
    x = r.normal(size=(B * T, C)).astype(np.float32)
    if dtype == "bf16":
        x = synth.round_bf16(x)
    w = (0.5 * r.normal(size=(C, W))).astype(np.float32)
    cu = (np.arange(B + 1) * T).astype(np.int32)
    win = r.normal(size=(B, W - 1, C)).astype(np.float32)
    if dtype == "bf16":
        win = synth.round_bf16(win)
    cs = to_dev(win, dtype)
    y = G.conv1d(to_dev(x, dtype), to_dev(w), seqlen=T, conv_state=cs)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(y), _oracle_bits(orc, x, w, cu, win, None, True, dtype))
    _, wref = orc.conv1d(x, w, cu, window=win)
    assert np.array_equal(to_np(cs), wref.astype(np.float32))
    # decode-time step: one token per sequence, window carried
    win_np = wref.astype(np.float32)
    for step in range(5):
        xt = r.normal(size=(B, C)).astype(np.float32)
        if dtype == "bf16":
            xt = synth.round_bf16(xt)
        yt = G.conv1d(to_dev(xt, dtype), to_dev(w), seqlen=1, num_seqs=B, conv_state=cs)
        torch.cuda.synchronize()
        cu1 = np.arange(B + 1).astype(np.int32)
        assert np.array_equal(_bits(yt), _oracle_bits(orc, xt, w, cu1, win_np, None, True, dtype)), f"step {step}"
        _, win_np = orc.conv1d(xt, w, cu1, window=win_np)
        win_np = win_np.astype(np.float32)
        assert np.array_equal(to_np(cs), win_np), f"window after step {step}"


def test_conv_qwen35_4k_bitexact(G, orc):
    """The 4096-token, 8192-channel bf16 layer conv (as the prefill bench runs it)."""
    import torch
    inp = synth.prefill_4k_bf16()
    note(f"conv {inp.name}: {inp.x.shape}")
    y = G.conv1d(to_dev(inp.x, "bf16"), to_dev(inp.conv_w), seqlen=4096)
    torch.cuda.synchronize()
    ref = orc.conv1d_f32(inp.x, inp.conv_w, inp.cu_seqlens, out_bf16=True)
    got = _bits(y)
    bad = int(np.sum(got != ref))
    assert bad == 0, f"{bad} mismatching elements"


def test_conv_special_values_bitexact(G, orc):
    """Zeros, bf16 subnormals, the largest finite values, infinities and NaNs
    (both signs, with payloads) through conv + SiLU: the output bits still
    equal the oracle's fp32 definition (NaN results are the canonical 0x7fc0)."""
    import torch
    note("conv special values bf16")
    r = np.random.default_rng(11)
    T, C, W = 48, 64, 4
    specials = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x007f, 0x807f, 0x0080, 0x8080, 0x7f7f, 0xff7f,
                         0x7f80, 0xff80, 0x7fc0, 0xffc0, 0x7fa1, 0xffc1, 0x3f80, 0xbf80, 0x4200, 0xc2b1,
                         0x42b2, 0xc2b2, 0x42ae, 0xc2ae], dtype=np.uint16)
    normal = synth.bf16_bits(r.normal(size=(T, C)).astype(np.float32))
    bits = np.where(r.random((T, C)) < 0.35, specials[r.integers(0, len(specials), (T, C))], normal).astype(np.uint16)
    x = (bits.astype(np.uint32) << 16).view(np.float32)
    w = np.array([1.0, -1.0, 0.5, 2.0, 1e-3, -3.0, 0.0, 1e20], dtype=np.float32)[r.integers(0, 8, (C, W))]
    cu = np.array([0, 17, T], dtype=np.int32)
    y = G.conv1d(bits_to_dev(bits), to_dev(w), cu_seqlens=torch.from_numpy(cu).cuda())
    torch.cuda.synchronize()
    ref = orc.conv1d_f32(x, w, cu, out_bf16=True)
    got = _bits(y)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[0]}: got {got[tuple(bad[0])]:#06x} want {ref[tuple(bad[0])]:#06x}"


def test_silu_bf16_pre_activation_sweep(G, orc):
    """SiLU of chosen fp32 pre-activations, rounded to bf16, equals the
    oracle's fp32 definition bit for bit.  A width-2 conv with taps
    (a_c, 1) over the rows x = (1, 0) gives pre-activation exactly a_c at the
    second token, so the sweep covers every bf16 value, a million random
    fp32 values in [-12, 12] (about 0.05% of which land near a bf16 rounding
    midpoint, where the kernel switches to the exact division), arbitrary
    fp32 bit patterns (NaN, infinities, subnormals, large negatives)."""
    import torch
    note("conv SiLU pre-activation sweep bf16")
    r = np.random.default_rng(12)
    n_uni, n_bits = 1 << 20, 1 << 19
    a = np.concatenate([
        (np.arange(1 << 16, dtype=np.uint32) << 16).view(np.float32),
        r.uniform(-12.0, 12.0, n_uni).astype(np.float32),
        r.integers(0, 1 << 32, n_bits, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ])
    C = len(a)
    assert C % 8 == 0
    w = np.stack([a, np.ones_like(a)], axis=1).astype(np.float32)
    x = np.zeros((2, C), dtype=np.float32)
    x[0] = 1.0
    y = G.conv1d(to_dev(x, "bf16"), torch.from_numpy(w).cuda(), seqlen=2)
    torch.cuda.synchronize()
    got = _bits(y)[1]
    ref = orc.conv1d_f32(x, w, np.array([0, 2], dtype=np.int32), out_bf16=True)[1]
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, f"{bad.size} mismatches, first a={a[bad[0]]!r}: got {got[bad[0]]:#06x} want {ref[bad[0]]:#06x}"


@pytest.mark.slow
def test_silu_bf16_every_fp32_preactivation(G, orc):
    """Every fp32 pre-activation, through the bf16 convolution kernel: with
    all taps zero the pre-activation is exactly the channel's fp32 bias
    (fma(0, 0, b) = b), so 1024 launches of 2^22 channels, each channel's
    bias one of the 2^32 bit patterns, give SiLU rounded to bf16 for every
    fp32 value -- on each of the kernel's three walks over two 36-token
    sequences: a full 32-token span from the first sequence's start (zero
    halo, rows 0 and 20), the token-by-token walk of the span that the
    second sequence starts inside (row 33) and the ragged last span
    (row 70).  Each must equal the oracle's fp32 definition (Cody-Waite
    exponential, exact division, round to nearest even) bit for bit; the
    test stops at the
    first launch with a mismatch and names its input.  About 16 s on one
    MI355X with 16 host threads for the oracle."""
    import threading

    import torch
    C, S, NSEQ, NBLK = 1 << 22, 36, 2, 1 << 10
    T = S * NSEQ
    rows = [0, 20, 33, 70]
    x = torch.zeros((T, C), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((C, 4), dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    x1 = np.zeros((1, C), dtype=np.float32)
    w1 = np.zeros((C, 4), dtype=np.float32)
    cu1 = np.array([0, 1], dtype=np.int32)
    n_thr = 16
    for blk in range(NBLK):
        a = (np.arange(C, dtype=np.uint64) + np.uint64(blk) * np.uint64(C)).astype(np.uint32).view(np.float32)
        bias = torch.from_numpy(a).cuda()
        conv = G.Conv1d(x, w, seqlen=S, num_seqs=NSEQ, bias=bias)
        conv(x, y)
        got = _bits(y[rows])
        ref = np.empty(C, dtype=np.uint16)

        def part(i):
            s = slice(i * C // n_thr, (i + 1) * C // n_thr)
            ref[s] = orc.conv1d_f32(x1[:, s], w1[s], cu1, bias=a[s], out_bf16=True)[0]

        th = [threading.Thread(target=part, args=(i,)) for i in range(n_thr)]
        for t in th:
            t.start()
        for t in th:
            t.join()
        for row, path in enumerate(("full span, sequence start", "full span", "token-by-token", "ragged span")):
            bad = np.flatnonzero(got[row] != ref)
            assert bad.size == 0, (f"block {blk}, {path} path: {bad.size} "
                                   f"mismatches, first a bits {a.view(np.uint32)[bad[0]]:#010x}: "
                                   f"got {got[row][bad[0]]:#06x} want {ref[bad[0]]:#06x}")
        if blk % 64 == 0:
            note(f"  exhaustive SiLU: {blk + 1} of {NBLK} blocks of 2^22 inputs match")
    note("  exhaustive SiLU: all 2^32 fp32 pre-activations match")
