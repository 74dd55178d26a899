"""GPU chunked prefill through the C ABI against the fp64 token-by-token
oracle, on the five workloads and the edge cases (ragged tails, empty and
short sequences, chunk 16/32/64, d_k != d_v, tiled heads, state in/out,
prefix continuation, packing and repeat-run bit equality)."""
import numpy as np
import pytest

from linear_attention_delta_amd import synth
from tests.gpu_util import TOL, conv_inputs, note, oracle_scan_all, rel_err_slices, to_dev, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def G():
    import torch
    assert torch.cuda.is_available()
    from linear_attention_delta_amd import gdn
    return gdn


def _dev_qkv(y, sh, dtype):
    """Device copy of the conv output and strided q/k/v views into it."""
    yd = to_dev(y, dtype)
    n = y.shape[0]
    a = sh.num_qk_heads * sh.head_dim_k
    q = yd[:, :a].view(n, sh.num_qk_heads, sh.head_dim_k)
    k = yd[:, a:2 * a].view(n, sh.num_qk_heads, sh.head_dim_k)
    v = yd[:, 2 * a:].view(n, sh.num_v_heads, sh.head_dim_v)
    return q, k, v


def _run_gpu(G, inp, y, *, chunk=None, state0=None, heads_tiled=False, scale=None, l2norm=True):
    import torch
    sh = inp.shape
    q, k, v = _dev_qkv(y, sh, inp.dtype)
    cu = None if inp.dense_T else torch.from_numpy(inp.cu_seqlens).cuda()
    s0 = None if state0 is None else torch.from_numpy(np.ascontiguousarray(state0, dtype=np.float32)).cuda()
    # workspace and outputs start as NaN bytes: anything the library reads
    # without having written it, or fails to write, shows up as NaN
    p = G.Prefill(q, k, v, cu_seqlens=cu, seqlen=inp.dense_T if inp.dense_T else None, num_seqs=inp.num_seqs,
                  chunk_size=chunk or inp.chunk_size, heads_tiled=heads_tiled,
                  scale=inp.scale if scale is None else scale, l2norm=l2norm)
    p.ws.fill_(-1)
    n, hv, dv = v.shape
    o = torch.full((n, hv, dv), float("nan"), dtype=q.dtype, device=q.device)
    S = torch.full((inp.num_seqs, hv, q.shape[2], dv), float("nan"), dtype=torch.float32, device=q.device)
    p(q, k, v, to_dev(inp.g), to_dev(inp.beta), o, s0, S)
    torch.cuda.synchronize()
    return to_np(o), to_np(S)


def _oracle(orc, inp, y, *, state0="inp", heads_tiled=False, scale=None, l2norm=True):
    """The oracle on every (sequence, v-head) of the workload, one threaded call."""
    return oracle_scan_all(orc, inp, y, state0=state0, heads_tiled=heads_tiled, scale=scale, l2norm=l2norm)


def _compare(inp, o_gpu, S_gpu, o_ref, S_ref):
    """Worst per-(sequence, v-head) relative error of o and of the final state."""
    return rel_err_slices(o_gpu, o_ref, inp.cu_seqlens), rel_err_slices(S_gpu, S_ref)


def test_tiny_fp32_workload(G, orc):
    """B=1, T=64 (one chunk), 2 q/k heads, 4 v heads, d=64, fp32: the GPU
    conv feeds the GPU scan; checked against oracle conv + oracle scan."""
    import torch
    inp = synth.tiny_fp32()
    note(f"prefill {inp.name}")
    x = to_dev(inp.x)
    y_dev = G.conv1d(x, to_dev(inp.conv_w), seqlen=64)
    sh = inp.shape
    a = sh.num_qk_heads * sh.head_dim_k
    q = y_dev[:, :a].view(64, 2, 64)
    k = y_dev[:, a:2 * a].view(64, 2, 64)
    v = y_dev[:, 2 * a:].view(64, 4, 64)
    o, S = G.prefill(q, k, v, to_dev(inp.g), to_dev(inp.beta), seqlen=64)
    torch.cuda.synchronize()
    yref, _ = orc.conv1d(inp.x, inp.conv_w)
    qr, kr, vr = synth.split_qkv(yref, sh)
    o_ref, S_ref = orc.scan(qr, kr, vr, inp.g, inp.beta)
    eo, es = rel_err_slices(to_np(o), o_ref), rel_err_slices(to_np(S), S_ref)
    note(f"  o err {eo:.2e}  S err {es:.2e}")
    assert eo <= TOL["f32"] and es <= TOL["f32"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_ragged_varlen_all_heads(G, orc, dtype, chunk):
    """Several tiles and ragged tails: lengths 0, 1, 15, 16, 17, 63, 64, 65,
    200 packed by cu_seqlens, nonzero initial states."""
    sh = synth.LayerShape(2, 4, 128, 128)
    inp = synth.make_prefill(7 + chunk, sh, [0, 1, 15, 16, 17, 63, 64, 65, 200], dtype, state0_std=0.05,
                             chunk_size=chunk, name="ragged")
    note(f"prefill ragged dtype={dtype} chunk={chunk}")
    y = conv_inputs(orc, inp)
    o, S = _run_gpu(G, inp, y, state0=inp.state0)
    o_ref, S_ref = _oracle(orc, inp, y)
    eo, es = _compare(inp, o, S, o_ref, S_ref)
    note(f"  o err {eo:.2e}  S err {es:.2e}")
    assert eo <= TOL[dtype] and es <= TOL[dtype]


@pytest.mark.parametrize("dtype,chunk,dk,dv", [
    ("f32", 16, 64, 128), ("f32", 32, 64, 64), ("f32", 16, 64, 64), ("f32", 32, 128, 64),
    ("bf16", 16, 64, 128), ("bf16", 16, 64, 64)])
def test_ragged_sequential_carry_shapes(G, orc, dtype, chunk, dk, dv):
    """The sequential carry (fp32, and bf16 chunk 16) at d_k = 64 and small
    chunks, where a thread's staged K/Q vectors cover rows of both matrices
    and its loads split differently over the chunk: odd and even chunk
    counts, a lone chunk, ragged tails and an empty sequence, with nonzero
    initial states."""
    sh = synth.LayerShape(2, 4, dk, dv)
    inp = synth.make_prefill(31 + chunk + dk + dv, sh, [1, 17, 0, 33, 96, 130], dtype, state0_std=0.05,
                             chunk_size=chunk, name="ragged-seq")
    note(f"prefill ragged sequential carry dtype={dtype} chunk={chunk} dk={dk} dv={dv}")
    y = conv_inputs(orc, inp)
    o, S = _run_gpu(G, inp, y, state0=inp.state0)
    o_ref, S_ref = _oracle(orc, inp, y)
    eo, es = _compare(inp, o, S, o_ref, S_ref)
    note(f"  o err {eo:.2e}  S err {es:.2e}")
    assert eo <= TOL[dtype] and es <= TOL[dtype]


@pytest.mark.parametrize("dtype,dk,dv,tiled,l2,scale", [
    ("f32", 64, 128, True, True, 0.0883883), ("bf16", 128, 64, False, True, 1.0),
    ("f32", 64, 64, False, False, 1.0), ("bf16", 64, 128, True, True, 0.5)])
def test_shapes_and_flags(G, orc, dtype, dk, dv, tiled, l2, scale):
    sh = synth.LayerShape(2, 6, dk, dv)
    inp = synth.make_prefill(21, sh, [130, 77], dtype, state0_std=0.05 if l2 else 0.01, name="shapes")
    note(f"prefill shapes dtype={dtype} dk={dk} dv={dv} tiled={tiled} l2={l2}")
    y = conv_inputs(orc, inp)
    if not l2:   # unnormalised keys: keep the recurrence contractive (|k|^2 beta <= 2)
        y = y.copy()
        a = sh.num_qk_heads * dk
        y[:, :2 * a] *= 0.9 / np.sqrt(dk) / max(1.0, float(np.max(np.abs(y[:, :2 * a]))))
        if dtype == "bf16":
            y = synth.round_bf16(y)
    o, S = _run_gpu(G, inp, y, state0=inp.state0, heads_tiled=tiled, scale=scale, l2norm=l2)
    o_ref, S_ref = _oracle(orc, inp, y, heads_tiled=tiled, scale=scale, l2norm=l2)
    eo, es = _compare(inp, o, S, o_ref, S_ref)
    note(f"  o err {eo:.2e}  S err {es:.2e}")
    assert eo <= TOL[dtype] and es <= TOL[dtype]


@pytest.mark.parametrize("chunk,dk,dv,tiled,lens", [
    (64, 128, 128, False, [1100, 0, 1, 700, 2050, 513]),
    (32, 128, 128, True, [1100, 0, 1, 700, 2050, 513]),
    (64, 64, 128, False, [1100, 0, 1, 700, 2050, 513]),
    (32, 128, 64, False, [1100, 0, 1, 700, 2050, 513]),
    (64, 64, 64, True, [1100, 0, 1, 700, 2050, 513]),
    (64, 128, 128, False, [1100, 1100]),       # dense, three segments per sequence
    (32, 128, 128, False, [1537, 1537, 1537]),  # dense, ragged last chunk and segment
])
def test_multi_segment_bf16(G, orc, chunk, dk, dv, tiled, lens):
    """bf16 sequences long enough that the carry runs in several segments
    (segment starts chained across segments), with empty, one-token and
    ragged sequences in the same batch and nonzero initial states."""
    sh = synth.LayerShape(2, 4, dk, dv)
    inp = synth.make_prefill(31 + chunk + dk + dv, sh, lens, "bf16", state0_std=0.05, chunk_size=chunk,
                             name="multiseg")
    note(f"prefill multi-segment chunk={chunk} dk={dk} dv={dv} tiled={tiled} lens={lens}")
    y = conv_inputs(orc, inp)
    o, S = _run_gpu(G, inp, y, state0=inp.state0, heads_tiled=tiled)
    o_ref, S_ref = _oracle(orc, inp, y, heads_tiled=tiled)
    eo, es = _compare(inp, o, S, o_ref, S_ref)
    note(f"  o err {eo:.2e}  S err {es:.2e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


@pytest.mark.parametrize("nseq", [1000, 1100])
def test_many_segments_bf16(G, orc, nseq):
    """Many short sequences on the segment path: the passes take up to 1024
    segments longest first and more in index order (1000 and 1100 segments,
    lengths 0..150 with empty ones among them)."""
    sh = synth.LayerShape(1, 2, 64, 64)
    lens = [int(x) for x in np.random.default_rng(nseq).integers(0, 151, size=nseq)]
    inp = synth.make_prefill(nseq, sh, lens, "bf16", state0_std=0.05, chunk_size=64, name="many-seg")
    note(f"prefill many segments nseq={nseq} tokens={sum(lens)}")
    y = conv_inputs(orc, inp)
    o, S = _run_gpu(G, inp, y, state0=inp.state0)
    o_ref, S_ref = _oracle(orc, inp, y)
    eo, es = _compare(inp, o, S, o_ref, S_ref)
    note(f"  o err {eo:.2e}  S err {es:.2e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


def test_qwen35_4k_bf16(G, orc):
    """B=1, T=4096, 16/32 heads, d=128, bf16, chunk 64 -- the benchmark's
    launch configuration; every v-head against the oracle."""
    inp = synth.prefill_4k_bf16()
    note(f"prefill {inp.name}")
    y = conv_inputs(orc, inp)
    o, S = _run_gpu(G, inp, y)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))
    o_ref, S_ref = _oracle(orc, inp, y)
    eo, es = _compare(inp, o, S, o_ref, S_ref)
    note(f"  o err {eo:.2e}  S err {es:.2e} (all 32 heads)")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


@pytest.mark.parametrize("T", [16384, 32768])
def test_long_single_sequence_bf16(G, orc, T):
    """One bf16 sequence of 16384 or 32768 tokens with the 4096-token layer's
    heads: the carry runs in 8 segments of 32 or 64 chunks, so the bf16
    segment transitions span 4x or 8x the chunks of the 4096-token layer.
    Every v-head against the oracle."""
    inp = synth.make_prefill(90 + T // 1024, synth.QWEN35_4B, [T], "bf16", name=f"long-T{T}-bf16")
    note(f"prefill {inp.name}")
    y = conv_inputs(orc, inp)
    o, S = _run_gpu(G, inp, y)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))
    o_ref, S_ref = _oracle(orc, inp, y)
    eo, es = _compare(inp, o, S, o_ref, S_ref)
    note(f"  o err {eo:.2e}  S err {es:.2e} (all 32 heads, T={T})")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


def test_adversarial_8k_fp32(G, orc):
    """Repeated tokens in runs up to 512, beta ~ U(0.9, 1), decay near 1, fp32:
    the blockwise inverse must stay finite and accurate."""
    inp = synth.adversarial_8k_fp32()
    note(f"prefill {inp.name}")
    y = conv_inputs(orc, inp)
    o, S = _run_gpu(G, inp, y)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))
    o_ref, S_ref = _oracle(orc, inp, y)
    eo, es = _compare(inp, o, S, o_ref, S_ref)
    note(f"  o err {eo:.2e}  S err {es:.2e} (all 32 heads)")
    assert eo <= TOL["f32"] and es <= TOL["f32"]


def test_varlen_16seq_bf16(G, orc):
    """16 sequences of U{128..8192} tokens packed (59,908 tokens), initial
    states ~N(0, 0.02): all 512 (sequence, v-head) pairs against the oracle."""
    inp = synth.varlen_bf16()
    note(f"prefill {inp.name}: {inp.total_tokens} tokens")
    y = conv_inputs(orc, inp)
    o, S = _run_gpu(G, inp, y, state0=inp.state0)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))
    o_ref, S_ref = _oracle(orc, inp, y)
    eo, es = _compare(inp, o, S, o_ref, S_ref)
    note(f"  o err {eo:.2e}  S err {es:.2e} (all {inp.num_seqs * inp.shape.num_v_heads} pairs)")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


def test_packing_and_repeat_are_bitwise(G, orc):
    """A packed batch equals each sequence run alone, bit for bit; two runs of
    the same call are bit-identical; state_out may alias state_in."""
    import torch
    sh = synth.LayerShape(2, 4, 128, 128)
    inp = synth.make_prefill(31, sh, [100, 64, 1, 190], "bf16", state0_std=0.02, name="pack")
    y = conv_inputs(orc, inp)
    o, S = _run_gpu(G, inp, y, state0=inp.state0)
    o2, S2 = _run_gpu(G, inp, y, state0=inp.state0)
    assert np.array_equal(o, o2) and np.array_equal(S, S2), "repeat run differs"
    cu = inp.cu_seqlens
    for i in range(inp.num_seqs):
        a, b = int(cu[i]), int(cu[i + 1])
        one = synth.PrefillInputs("one", sh, "bf16", np.array([0, b - a], dtype=np.int32), b - a, inp.x[a:b],
                                  inp.conv_w, inp.g[a:b], inp.beta[a:b], inp.state0[i:i + 1])
        oi, Si = _run_gpu(G, one, y[a:b], state0=inp.state0[i:i + 1])
        assert np.array_equal(oi, o[a:b]) and np.array_equal(Si[0], S[i]), f"seq {i} differs when packed"
    # in-place state
    q, k, v = _dev_qkv(y, sh, "bf16")
    st = torch.from_numpy(inp.state0).cuda()
    G.prefill(q, k, v, to_dev(inp.g), to_dev(inp.beta), state_in=st, state_out=st,
              cu_seqlens=torch.from_numpy(cu).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(to_np(st), S)


def test_prefix_continuation_and_decode_handoff(G, orc):
    """prefill(t tokens) -> state -> prefill(rest) matches one prefill of all
    tokens (within tolerance), and decode steps continue from a prefill state."""
    import torch
    sh = synth.LayerShape(2, 4, 128, 128)
    T = 300
    inp = synth.make_prefill(41, sh, [T], "bf16", name="cont")
    y = conv_inputs(orc, inp)
    o_ref, S_ref = orc.scan(*synth.split_qkv(y, sh), inp.g, inp.beta)
    for cut in (1, 64, 100):
        first = synth.PrefillInputs("p1", sh, "bf16", np.array([0, cut], dtype=np.int32), cut, None, None,
                                    inp.g[:cut], inp.beta[:cut], None)
        second = synth.PrefillInputs("p2", sh, "bf16", np.array([0, T - cut], dtype=np.int32), T - cut, None, None,
                                     inp.g[cut:], inp.beta[cut:], None)
        o1, S1 = _run_gpu(G, first, y[:cut])
        o2, S2 = _run_gpu(G, second, y[cut:], state0=S1)
        eo = rel_err_slices(np.concatenate([o1, o2]), o_ref)
        es = rel_err_slices(S2, S_ref)
        note(f"  continuation at {cut}: o err {eo:.2e}  S err {es:.2e}")
        assert eo <= TOL["bf16"] and es <= TOL["bf16"]
    # handoff: decode 8 more tokens from the prefill state
    o, S = _run_gpu(G, inp, y)
    Sd = torch.from_numpy(S).cuda()
    Sr = S_ref.copy()
    r = np.random.default_rng(3)
    for step in range(8):
        q = synth.round_bf16(r.normal(size=(1, 2, 128)).astype(np.float32))
        k = synth.round_bf16(r.normal(size=(1, 2, 128)).astype(np.float32))
        v = synth.round_bf16(r.normal(size=(1, 4, 128)).astype(np.float32))
        g = (-0.5 * np.logaddexp(0, r.normal(size=(1, 4)))).astype(np.float32)
        b = (1 / (1 + np.exp(-r.normal(size=(1, 4))))).astype(np.float32)
        od = G.decode_step(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), to_dev(g), to_dev(b), Sd)
        torch.cuda.synchronize()
        orf, Sr = orc.decode_step(q, k, v, g, b, Sr)
        eo = rel_err_slices(to_np(od), orf, np.arange(2))
        assert eo <= TOL["bf16"], f"handoff step {step}: {eo:.2e}"
    assert rel_err_slices(to_np(Sd), Sr) <= TOL["bf16"]


def test_side_stream_call_keeps_its_buffers(G, orc):
    """prefill() on a side stream: its temporary workspace (and fresh outputs)
    are allocated on the current stream and dropped at return, while the side
    stream's kernels may still run.  Allocations made right afterwards on the
    current stream, and filled there, must not land on them: the result equals
    the same call on the current stream, bit for bit."""
    import torch
    sh = synth.LayerShape(2, 4, 128, 128)
    inp = synth.make_prefill(77, sh, [2048], "bf16", name="side-stream")
    y = conv_inputs(orc, inp)
    q, k, v = _dev_qkv(y, sh, "bf16")
    g, beta = to_dev(inp.g), to_dev(inp.beta)
    o_ref, S_ref = G.prefill(q, k, v, g, beta, seqlen=2048)
    torch.cuda.synchronize()
    ws_elems = G.workspace_size(G.Prefill(q, k, v, seqlen=2048).dims) // 4 + 64
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    o, S = G.prefill(q, k, v, g, beta, seqlen=2048, stream=side)
    junk = [torch.full((ws_elems,), -1, dtype=torch.int32, device="cuda") for _ in range(3)]
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    del junk
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)) and torch.equal(S, S_ref)
