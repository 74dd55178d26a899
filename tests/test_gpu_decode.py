"""GPU decode step through the C ABI against the fp64 oracle."""
import numpy as np
import pytest

from linear_attention_delta_amd import synth
from tests.gpu_util import TOL, bits_to_dev, note, rel_err_slices, to_dev, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def G():
    import torch
    assert torch.cuda.is_available()
    from linear_attention_delta_amd import gdn
    return gdn


def _random_step(r, B, hk, hv, dk, dv, dtype):
    q = r.normal(size=(B, hk, dk)).astype(np.float32)
    k = r.normal(size=(B, hk, dk)).astype(np.float32)
    v = r.normal(size=(B, hv, dv)).astype(np.float32)
    if dtype == "bf16":
        q, k, v = synth.round_bf16(q), synth.round_bf16(k), synth.round_bf16(v)
    g = (-np.logaddexp(0, r.normal(size=(B, hv))) * 0.5).astype(np.float32)
    beta = (1 / (1 + np.exp(-r.normal(size=(B, hv))))).astype(np.float32)
    return q, k, v, g, beta


@pytest.mark.parametrize("dtype,dk,dv,tiled,scale,l2", [
    ("bf16", 128, 128, False, 1.0, True), ("f32", 128, 128, False, 1.0, True),
    ("f32", 64, 128, True, 0.125, True), ("bf16", 128, 64, False, 1.0, False), ("f32", 64, 64, False, 2.0, True)])
def test_decode_matches_oracle(G, orc, dtype, dk, dv, tiled, scale, l2):
    import torch
    note(f"decode dtype={dtype} dk={dk} dv={dv} tiled={tiled}")
    r = np.random.default_rng(dk + dv)
    B, hk, hv = 6, 2, 6
    S0 = (0.02 * r.normal(size=(B, hv, dk, dv))).astype(np.float32)
    S = torch.from_numpy(S0).cuda()
    Sref = S0.astype(np.float64)
    for step in range(3):
        q, k, v, g, beta = _random_step(r, B, hk, hv, dk, dv, dtype)
        o = G.decode_step(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), to_dev(g), to_dev(beta), S,
                          l2norm=l2, heads_tiled=tiled, scale=scale)
        torch.cuda.synchronize()
        oref, Sref = orc.decode_step(q, k, v, g, beta, Sref, scale=scale, l2norm=l2, heads_tiled=tiled)
        eo = rel_err_slices(to_np(o), oref, np.arange(B + 1))
        es = rel_err_slices(to_np(S), Sref)
        note(f"  step {step}: o err {eo:.2e}  S err {es:.2e}")
        assert eo <= TOL[dtype] and es <= TOL[dtype]


def test_decode_state_slots(G, orc):
    """Sequences read and write the slots named by state_slots; other slots
    are untouched; a slot index out of range poisons that output only."""
    import torch
    r = np.random.default_rng(11)
    B, hk, hv, d, nslots = 4, 1, 2, 64, 7
    S0 = (0.1 * r.normal(size=(nslots, hv, d, d))).astype(np.float32)
    S = torch.from_numpy(S0).cuda()
    slots = np.array([5, 0, 3, 6], dtype=np.int32)
    q, k, v, g, beta = _random_step(r, B, hk, hv, d, d, "f32")
    o = G.decode_step(to_dev(q), to_dev(k), to_dev(v), to_dev(g), to_dev(beta), S,
                      state_slots=torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    oref, Snew = orc.decode_step(q, k, v, g, beta, S0[slots])
    assert rel_err_slices(to_np(o), oref, np.arange(B + 1)) <= 1e-5
    got = to_np(S)
    for i, s in enumerate(slots):
        assert rel_err_slices(got[s:s + 1], Snew[i:i + 1]) <= 1e-5
    for s in set(range(nslots)) - set(slots.tolist()):
        assert np.array_equal(got[s], S0[s])
    bad = np.array([1, 9, 2, -1], dtype=np.int32)
    before = to_np(S).copy()
    o2 = G.decode_step(to_dev(q), to_dev(k), to_dev(v), to_dev(g), to_dev(beta), S,
                       state_slots=torch.from_numpy(bad).cuda())
    torch.cuda.synchronize()
    o2n = to_np(o2)
    assert np.all(np.isnan(o2n[1])) and np.all(np.isnan(o2n[3]))
    assert np.all(np.isfinite(o2n[0])) and np.all(np.isfinite(o2n[2]))
    after = to_np(S)
    for s in set(range(nslots)) - {1, 2}:
        assert np.array_equal(after[s], before[s])


class DecodePipelineOracle:
    """conv step + recurrent step of the decode workload, one step at a time,
    in fp64 with the fp32 conv (q, k, v rounded to bf16 exactly as the GPU's
    conv stores them), on the sequences `seqs` (all heads).  The fp64 state
    is stepped in place."""

    def __init__(self, orc, inp, seqs):
        self.orc, self.inp, self.seqs = orc, inp, np.asarray(seqs)
        self.win = inp.conv_state0[self.seqs].astype(np.float32)
        self.S = np.ascontiguousarray(inp.state0[self.seqs], dtype=np.float64)
        self.cu1 = np.arange(len(self.seqs) + 1).astype(np.int32)
        self.i = 0

    def step(self):
        inp, orc = self.inp, self.orc
        p = self.i % inp.pool
        xt = inp.x[p][self.seqs]
        bits = orc.conv1d_f32(xt, inp.conv_w, self.cu1, window=self.win, out_bf16=True)
        y = (bits.astype(np.uint32) << 16).view(np.float32)
        _, win = orc.conv1d(xt, inp.conv_w, self.cu1, window=self.win)
        self.win = win.astype(np.float32)
        q, k, v = synth.split_qkv(y, inp.shape)
        o, _ = orc.decode_step(q, k, v, inp.g[p][self.seqs], inp.beta[p][self.seqs], self.S, in_place=True)
        self.i += 1
        return o


def test_decode_b64_1000_steps(G, orc):
    """The 64-sequence Qwen3.5-4B-shaped decode workload for 1000 steps
    (cycling 16 input sets), through both decode paths: conv step + decode
    step (two calls), and the fused gdn_decode_conv_step.  Against one fp64
    oracle pass: o of every sequence and head at every step, and the whole
    state at steps 1, 16 and 1000."""
    import torch
    inp = synth.decode_b64_bf16()
    sh = inp.shape
    B, steps = inp.batch, 1000
    note(f"decode workload {inp.name}: B={B}, {steps} steps, both paths")
    x_dev = [to_dev(inp.x[p], "bf16") for p in range(inp.pool)]
    g_dev = [to_dev(inp.g[p]) for p in range(inp.pool)]
    b_dev = [to_dev(inp.beta[p]) for p in range(inp.pool)]
    w = to_dev(inp.conv_w)
    a = sh.num_qk_heads * sh.head_dim_k
    keep = (1, 16, steps)
    hist, kept = {}, {}
    for path in ("two_calls", "fused"):
        cs = to_dev(inp.conv_state0, "bf16")
        S = torch.from_numpy(inp.state0).cuda()
        o_all = torch.empty((steps, B, sh.num_v_heads, sh.head_dim_v), dtype=torch.bfloat16, device="cuda")
        fused = G.DecodeConv(x_dev[0], w, num_qk_heads=sh.num_qk_heads, num_v_heads=sh.num_v_heads,
                             head_dim_k=sh.head_dim_k, head_dim_v=sh.head_dim_v, num_slots=B)
        kept[path] = {}
        for i in range(steps):
            p = i % inp.pool
            if path == "fused":
                fused(x_dev[p], g_dev[p], b_dev[p], S, cs, o_all[i])
            else:
                y = G.conv1d(x_dev[p], w, seqlen=1, num_seqs=B, conv_state=cs)
                q = y[:, :a].view(B, sh.num_qk_heads, sh.head_dim_k)
                k = y[:, a:2 * a].view(B, sh.num_qk_heads, sh.head_dim_k)
                v = y[:, 2 * a:].view(B, sh.num_v_heads, sh.head_dim_v)
                G.decode_step(q, k, v, g_dev[p], b_dev[p], S, out=o_all[i])
            if i + 1 in keep:
                kept[path][i + 1] = S.cpu().numpy()
        torch.cuda.synchronize()
        hist[path] = o_all.view(torch.int16).cpu().numpy().view(np.uint16)  # bf16 bits, 0.5 GB
        del o_all
    note("  gpu done; running the oracle over every sequence")
    ref = DecodePipelineOracle(orc, inp, np.arange(B))
    cu = np.arange(B + 1)
    worst = {path: 0.0 for path in hist}
    for i in range(steps):
        o_ref = ref.step()
        for path in hist:
            o_gpu = (hist[path][i].astype(np.uint32) << 16).view(np.float32)
            worst[path] = max(worst[path], rel_err_slices(o_gpu, o_ref, cu))
        if i + 1 in keep:
            for path in hist:
                es = rel_err_slices(kept[path][i + 1], ref.S)
                note(f"  {path}: S err at step {i + 1}: {es:.2e}")
                assert es <= TOL["bf16"], f"{path}: state at step {i + 1}"
    for path in hist:
        note(f"  {path}: worst o err over {steps} steps, all {B} sequences: {worst[path]:.2e}")
        assert worst[path] <= TOL["bf16"], path
