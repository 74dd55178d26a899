"""Multi-layer decode captured in one HIP graph: the library's decode calls
launch kernels only (no allocation, no memset, no synchronisation), so a
token's step over several layers records into a graph.  Every replay, with
new inputs copied in and eager work between replays, must equal the same
calls made eagerly, bit for bit."""
import numpy as np
import pytest
import torch

from linear_attention_delta_amd import synth
from tests.gpu_util import note, to_dev

pytestmark = pytest.mark.gpu

L, B = 3, 4


def _bits(t):
    t = t.detach().contiguous()
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


def _layers(G, sh, seed):
    """Per layer: conv taps, gate parameters, state pool, window; and the
    static input buffers a graph reads."""
    r = np.random.default_rng(seed)
    cc, hv = sh.conv_channels, sh.num_v_heads
    out = []
    for l in range(L):
        out.append(dict(
            w=to_dev((0.5 * r.normal(size=(cc, 4))).astype(np.float32)),
            A_log=to_dev(r.uniform(-1, 1.5, size=hv).astype(np.float32)),
            dt_bias=to_dev((0.5 * r.normal(size=hv)).astype(np.float32)),
            S=torch.from_numpy((0.02 * r.normal(size=(B, hv, sh.head_dim_k, sh.head_dim_v))).astype(np.float32)).cuda(),
            W=to_dev(r.normal(size=(B, 3, cc)).astype(np.float32), "bf16"),
            x=torch.empty((B, cc), dtype=torch.bfloat16, device="cuda"),
            ab=torch.empty((B, 2 * hv), dtype=torch.bfloat16, device="cuda"),
            o=torch.empty((B, hv, sh.head_dim_v), dtype=torch.bfloat16, device="cuda")))
    return out


def _token(G, sh, layers, steps, gates):
    for l, ly in enumerate(layers):
        G.decode_conv_gated_step(steps[l], ly["x"], gates[l], ly["S"], ly["W"], ly["o"])


def _bind(G, sh, layers):
    hv = sh.num_v_heads
    steps = [G.DecodeConv(ly["x"], ly["w"], num_qk_heads=sh.num_qk_heads, num_v_heads=hv, head_dim_k=sh.head_dim_k,
                          head_dim_v=sh.head_dim_v, num_slots=B) for ly in layers]
    gates = [G.gate_inputs(ly["ab"][:, :hv], ly["ab"][:, hv:], ly["A_log"], ly["dt_bias"]) for ly in layers]
    return steps, gates


def test_multilayer_decode_graph_replays_equal_eager():
    from linear_attention_delta_amd import gdn as G
    sh = synth.QWEN35_4B
    eager = _layers(G, sh, 1)
    graphed = _layers(G, sh, 1)
    steps_e, gates_e = _bind(G, sh, eager)
    r = np.random.default_rng(2)
    inputs = [[(to_dev(r.normal(size=(B, sh.conv_channels)).astype(np.float32), "bf16"),
                to_dev(r.normal(size=(B, 2 * sh.num_v_heads)).astype(np.float32), "bf16")) for _ in range(L)]
              for _ in range(5)]

    def load(layers, i):
        for ly, (x, ab) in zip(layers, inputs[i]):
            ly["x"].copy_(x)
            ly["ab"].copy_(ab)

    # capture token 0 on a side stream (warm-up launches first, as capture requires)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    scratch = _layers(G, sh, 3)          # warm-up target, so the compared states stay untouched
    with torch.cuda.stream(side):
        steps_w, gates_w = _bind(G, sh, scratch)
        _token(G, sh, scratch, steps_w, gates_w)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        steps_g, gates_g = _bind(G, sh, graphed)   # bound to the capture stream
        _token(G, sh, graphed, steps_g, gates_g)
    torch.cuda.synchronize()
    for i in range(5):
        note(f"decode graph replay {i}")
        load(graphed, i)
        graph.replay()
        load(eager, i)
        _token(G, sh, eager, steps_e, gates_e)
        _ = torch.ones(1 << 20, device="cuda").sum()   # eager work between replays
        torch.cuda.synchronize()
        for l in range(L):
            for key in ("o", "S", "W"):
                assert np.array_equal(_bits(graphed[l][key]), _bits(eager[l][key])), (i, l, key)
    assert np.all(np.isfinite(graphed[-1]["o"].float().cpu().numpy()))
