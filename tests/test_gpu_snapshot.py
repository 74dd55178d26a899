"""State snapshots for prefix caching (gdn_snapshot_push / gdn_snapshot_restore)
through the C ABI.  A decode graph that pushes every layer's state and conv
window into a device ring every fourth token is replayed; restoring an
entry and continuing from it must reproduce the uninterrupted run bit for
bit (outputs, states, windows), and leave every other slot alone."""
import numpy as np
import pytest
import torch

from linear_attention_delta_amd import synth
from tests.gpu_util import note, to_dev

pytestmark = pytest.mark.gpu

L, B, NSLOTS, RING = 3, 4, 6, 3
SLOTS = [4, 1, 5, 0]          # live slot of each sequence; slots 2 and 3 belong to no one


def _bits(t):
    t = t.detach().contiguous()
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


def _layers(G, sh, seed, slots):
    r = np.random.default_rng(seed)
    cc, hv = sh.conv_channels, sh.num_v_heads
    out = []
    for _ in range(L):
        ly = dict(
            w=to_dev((0.5 * r.normal(size=(cc, 4))).astype(np.float32)),
            A_log=to_dev(r.uniform(-1, 1.5, size=hv).astype(np.float32)),
            dt_bias=to_dev((0.5 * r.normal(size=hv)).astype(np.float32)),
            S=torch.from_numpy((0.02 * r.normal(size=(NSLOTS, hv, sh.head_dim_k, sh.head_dim_v)))
                               .astype(np.float32)).cuda(),
            W=to_dev(r.normal(size=(NSLOTS, 3, cc)).astype(np.float32), "bf16"),
            x=torch.empty((B, cc), dtype=torch.bfloat16, device="cuda"),
            ab=torch.empty((B, 2 * hv), dtype=torch.bfloat16, device="cuda"),
            o=torch.empty((B, hv, sh.head_dim_v), dtype=torch.bfloat16, device="cuda"))
        ly["ring"] = G.SnapshotRing(ly["S"], ly["W"], B, RING, slots=slots)
        out.append(ly)
    return out


def _bind(G, sh, layers):
    hv = sh.num_v_heads
    steps = [G.DecodeConv(ly["x"], ly["w"], num_qk_heads=sh.num_qk_heads, num_v_heads=hv, head_dim_k=sh.head_dim_k,
                          head_dim_v=sh.head_dim_v, num_slots=NSLOTS) for ly in layers]
    gates = [G.gate_inputs(ly["ab"][:, :hv], ly["ab"][:, hv:], ly["A_log"], ly["dt_bias"]) for ly in layers]
    return steps, gates


def _token(G, layers, steps, gates, slots, push):
    for l, ly in enumerate(layers):
        G.decode_conv_gated_step(steps[l], ly["x"], gates[l], ly["S"], ly["W"], ly["o"], state_slots=slots)
        if push:
            ly["ring"].push(ly["S"], ly["W"])


def test_restore_and_continue_equals_uninterrupted_run():
    from linear_attention_delta_amd import gdn as G
    sh = synth.QWEN35_4B
    slots = torch.tensor(SLOTS, dtype=torch.int32, device="cuda")
    live = _layers(G, sh, 7, slots)
    r = np.random.default_rng(8)
    T = 16
    inputs = [[(to_dev(r.normal(size=(B, sh.conv_channels)).astype(np.float32), "bf16"),
                to_dev(r.normal(size=(B, 2 * sh.num_v_heads)).astype(np.float32), "bf16")) for _ in range(L)]
              for _ in range(T)]

    def load(t):
        for ly, (x, ab) in zip(live, inputs[t]):
            ly["x"].copy_(x)
            ly["ab"].copy_(ab)

    # warm-up launches on throw-away layers, then capture a plain token and a
    # token that pushes every layer's slots into its ring
    scratch = _layers(G, sh, 9, slots)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st_w, ga_w = _bind(G, sh, scratch)
        _token(G, scratch, st_w, ga_w, slots, True)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    plain, pushing = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(plain):
        st_p, ga_p = _bind(G, sh, live)
        _token(G, live, st_p, ga_p, slots, False)
    with torch.cuda.graph(pushing):
        st_q, ga_q = _bind(G, sh, live)
        _token(G, live, st_q, ga_q, slots, True)
    torch.cuda.synchronize()

    push_after = (3, 7, 11)      # entries 0, 1, 2
    o_hist = []
    for t in range(T):
        load(t)
        (pushing if t in push_after else plain).replay()
        o_hist.append([_bits(ly["o"]) for ly in live])
        _ = torch.ones(1 << 16, device="cuda").sum()   # eager work between replays
    torch.cuda.synchronize()
    end_S = [_bits(ly["S"]) for ly in live]
    end_W = [_bits(ly["W"]) for ly in live]
    for ly in live:
        assert int(ly["ring"].head.item()) == len(push_after)

    # restore the snapshot taken after token 7 and run tokens 8.. again, eagerly
    entry, t0 = 1, push_after[1] + 1
    before = [(_bits(ly["S"]), _bits(ly["W"])) for ly in live]
    for ly in live:
        ly["ring"].restore(entry, ly["S"], ly["W"])
    torch.cuda.synchronize()
    for l, ly in enumerate(live):
        for s in (2, 3):     # slots no sequence names are untouched
            assert np.array_equal(_bits(ly["S"])[s], before[l][0][s]) and np.array_equal(_bits(ly["W"])[s],
                                                                                       before[l][1][s])
    st_e, ga_e = _bind(G, sh, live)
    for t in range(t0, T):
        note(f"snapshot: continue token {t}")
        load(t)
        _token(G, live, st_e, ga_e, slots, False)
        torch.cuda.synchronize()
        for l, ly in enumerate(live):
            assert np.array_equal(_bits(ly["o"]), o_hist[t][l]), (t, l)
    for l, ly in enumerate(live):
        assert np.array_equal(_bits(ly["S"]), end_S[l]) and np.array_equal(_bits(ly["W"]), end_W[l]), l
    # entry 2 holds the states after token 11: restoring it and replaying
    # 12.. through the graph gives the same end again
    for ly in live:
        ly["ring"].restore(2, ly["S"], ly["W"])
    for t in range(push_after[2] + 1, T):
        load(t)
        plain.replay()
    torch.cuda.synchronize()
    for l, ly in enumerate(live):
        assert np.array_equal(_bits(ly["S"]), end_S[l]) and np.array_equal(_bits(ly["o"]), o_hist[T - 1][l]), l
