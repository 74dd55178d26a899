"""The chunked algorithm (as the kernels run it) against the oracle, on the CPU."""
import numpy as np
import pytest

from linear_attention_delta_amd import synth
from tests import chunk_model


def _rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("tiled", [False, True])
def test_chunked_equals_token_recurrence(orc, chunk, tiled):
    r = np.random.default_rng(chunk + 7 * tiled)
    lens = [1, 70, 129, 16, 0, 33]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, Hk, Hv, dk, dv = int(cu[-1]), 2, 4, 16, 8
    q = r.normal(size=(T, Hk, dk)); k = r.normal(size=(T, Hk, dk)); v = r.normal(size=(T, Hv, dv))
    g = -np.logaddexp(0, r.normal(size=(T, Hv))) * 0.5
    beta = 1 / (1 + np.exp(-r.normal(size=(T, Hv))))
    S0 = r.normal(size=(len(lens), Hv, dk, dv)) * 0.1
    o_ref, S_ref = orc.scan(q, k, v, g, beta, cu, state0=S0, scale=0.3, heads_tiled=tiled)
    o, S = chunk_model.chunked_scan(q, k, v, g, beta, cu, state0=S0, chunk=chunk, scale=0.3, heads_tiled=tiled)
    assert _rel(o, o_ref) < 1e-11 and _rel(S, S_ref) < 1e-11


def test_blockwise_inverse_matches_solve():
    r = np.random.default_rng(3)
    for C in (16, 32, 64):
        K = r.normal(size=(C, 32)); K /= np.linalg.norm(K, axis=1, keepdims=True)
        beta = r.uniform(0, 1, C)
        gam = np.cumsum(-r.uniform(0, 0.2, C))
        A = np.tril(beta[:, None] * np.exp(gam[:, None] - gam[None, :]) * (K @ K.T), -1)
        inv = chunk_model.inverse_blockwise(A)
        fs = chunk_model.inverse_forward_substitution(A)
        assert np.max(np.abs(inv @ (np.eye(C) + A) - np.eye(C))) < 1e-10
        assert np.max(np.abs(inv - fs)) < 1e-10 * max(1.0, np.max(np.abs(fs)))


def test_repeated_key_inverse_closed_form():
    """One unit key repeated with beta = 1, g = 0: A = strictly-lower ones, and
    (I + A)^{-1} = I - (ones on the first subdiagonal).  Plain doubling of the
    whole 64x64 block forms A^32-sized powers (entries ~ C(62,31)); the
    blockwise form never does."""
    C = 64
    A = np.tril(np.ones((C, C)), -1)
    inv = chunk_model.inverse_blockwise(A)
    expect = np.eye(C) - np.eye(C, k=-1)
    assert np.array_equal(inv, expect)


def test_tiny_workload_through_chunk_model(orc):
    """The tiny fp32 workload (conv -> SiLU -> chunked scan) agrees with the oracle."""
    inp = synth.tiny_fp32()
    y, _ = orc.conv1d(inp.x, inp.conv_w, inp.cu_seqlens)
    q, k, v = synth.split_qkv(y, inp.shape)
    o_ref, S_ref = orc.scan(q, k, v, inp.g, inp.beta, inp.cu_seqlens)
    o, S = chunk_model.chunked_scan(q, k, v, inp.g, inp.beta, inp.cu_seqlens, chunk=64)
    assert _rel(o, o_ref) < 1e-11 and _rel(S, S_ref) < 1e-11
