"""The prefill with the gated RMS norm fused into the carry's output
(gdn_prefill_chunked_gated_norm / gdn_prefill_scan_gated_norm) through the C
ABI: against the oracle (token scan, then the gated norm in fp64) on every
(sequence, v-head), and against the unfused calls (prefill, then
gdn_gated_rmsnorm): the same final state bit for bit, and y within one
rounding of the output dtype (only the order of each row's sum differs)."""
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


def _views(yd, sh):
    n, a = yd.shape[0], sh.num_qk_heads * sh.head_dim_k
    return (yd[:, :a].view(n, sh.num_qk_heads, sh.head_dim_k), yd[:, a:2 * a].view(n, sh.num_qk_heads, sh.head_dim_k),
            yd[:, 2 * a:].view(n, sh.num_v_heads, sh.head_dim_v))


def _run(G, orc, inp, *, heads_tiled=False, z_pad=0, seed=3):
    import torch
    sh = inp.shape
    y = conv_inputs(orc, inp)
    q, k, v = _views(to_dev(y, inp.dtype), sh)
    g, beta = to_dev(inp.g), to_dev(inp.beta)
    cu = None if inp.dense_T else torch.from_numpy(inp.cu_seqlens).cuda()
    s0 = None if inp.state0 is None else torch.from_numpy(inp.state0).cuda()
    n, hv, dv = v.shape
    z, wn = synth.gate_inputs(seed, n, hv, dv, inp.dtype)
    zw = np.zeros((n, hv * dv + z_pad), dtype=np.float32)      # z rows inside a wider buffer
    zw[:, :hv * dv] = z.reshape(n, -1)
    zd = to_dev(zw, inp.dtype)[:, :hv * dv].view(n, hv, dv)
    wd = to_dev(wn)
    p = G.Prefill(q, k, v, cu_seqlens=cu, seqlen=inp.dense_T or None, num_seqs=inp.num_seqs,
                  chunk_size=inp.chunk_size, heads_tiled=heads_tiled, scale=inp.scale)
    p.ws.fill_(-1)
    dt = q.dtype
    yf = torch.full((n, hv, dv), float("nan"), dtype=dt, device="cuda")
    Sf = torch.full((inp.num_seqs, hv, sh.head_dim_k, dv), float("nan"), dtype=torch.float32, device="cuda")
    p.gated_norm(q, k, v, g, beta, zd, wd, yf, s0, Sf)
    o = torch.empty((n, hv, dv), dtype=dt, device="cuda")
    Su = torch.empty_like(Sf)
    p(q, k, v, g, beta, o, s0, Su)
    yu = G.gated_rmsnorm(o, zd, wd)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_scan_all(orc, inp, y, heads_tiled=heads_tiled)
    y_ref = orc.gated_rmsnorm(o_ref, z, wn)
    return dict(yf=to_np(yf), yu=to_np(yu), Sf=Sf.cpu().numpy(), Su=Su.cpu().numpy(), y_ref=y_ref, S_ref=S_ref)


def _check(inp, r):
    tol = TOL[inp.dtype]
    ey = rel_err_slices(r["yf"], r["y_ref"], inp.cu_seqlens)
    es = rel_err_slices(r["Sf"], r["S_ref"])
    note(f"  fused y err {ey:.2e}  S err {es:.2e}")
    assert ey <= tol and es <= tol
    assert np.array_equal(r["Sf"].view(np.uint32), r["Su"].view(np.uint32)), "state differs from the unfused call"
    # y against the unfused norm: the same o bits, the row sums added in
    # another order -> at most one rounding of the output dtype apart
    ulp = 2.0 ** -7 if inp.dtype == "bf16" else 2.0 ** -20
    d = np.abs(r["yf"] - r["yu"])
    assert np.all(d <= ulp * np.abs(r["yu"]) + 1e-30), float(np.max(d / (np.abs(r["yu"]) + 1e-30)))


def test_fused_norm_qwen35_4k(G, orc):
    """The 4096-token bf16 layer: the norm runs inside the segment carry."""
    inp = synth.prefill_4k_bf16()
    note(f"fused gated norm {inp.name}")
    _check(inp, _run(G, orc, inp, z_pad=64))


@pytest.mark.parametrize("dtype,chunk,dk,dv,tiled", [
    ("bf16", 64, 128, 128, False), ("bf16", 32, 128, 64, True), ("bf16", 64, 64, 128, False),
    ("bf16", 32, 64, 64, False),
    ("bf16", 16, 128, 128, False),   # sequential carry, then the norm in place
    ("f32", 64, 128, 128, True), ("f32", 32, 64, 64, False)])
def test_fused_norm_ragged(G, orc, dtype, chunk, dk, dv, tiled):
    """Ragged varlen batches with initial states (empty, 1-token, partial
    chunks, several segments), every head layout and carry path."""
    sh = synth.LayerShape(2, 4, dk, dv)
    lens = [0, 1, 17, 64, 65, 200, 1100, 0, 513]
    inp = synth.make_prefill(60 + chunk + dk + dv, sh, lens, dtype, state0_std=0.05, chunk_size=chunk,
                             name="fused-norm-ragged")
    note(f"fused gated norm ragged dtype={dtype} chunk={chunk} dk={dk} dv={dv} tiled={tiled}")
    _check(inp, _run(G, orc, inp, heads_tiled=tiled, z_pad=8 if dtype == "bf16" else 4))
