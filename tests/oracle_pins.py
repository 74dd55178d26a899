"""Pins for the CPU oracle: facts fixed by the mathematics, checked against
the oracle without reusing its code.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError when the
oracle disagrees.  The recurrence pins follow the gated delta rule as the
oxydllm 0.0.0-alpha.12.2 release notes ("New Features", Gated DeltaNet
runtime) use it, written here in the orientation of the layer's usual
formula: a d_v x d_k memory M_t = alpha_t M_{t-1} (I - beta_t k_t k_t^T) +
beta_t v_t k_t^T read as o_t = M_t q_t.  The oracle stores S = M^T
([d_k][d_v]); tests use d_k != d_v so a transposed state cannot pass.
They are also run against deliberately broken copies of the oracle
(tests/test_oracle_mutants.py) to show that each planted mistake fails at
least one of them.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import expit
from scipy.stats import ortho_group

EPS = 1e-6


def _rng(i):
    return np.random.default_rng(1000 + i)


def _unit_rows(a):
    return a / np.linalg.norm(a, axis=-1, keepdims=True)


def _close(a, b, rtol, atol=0.0, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    err = np.max(np.abs(a - b)) if a.size else 0.0
    ref = max(np.max(np.abs(b)) if b.size else 0.0, 1e-300)
    assert err <= rtol * ref + atol, f"{what}: max err {err:.3e} vs ref {ref:.3e}"


# --------------------------------------------------------------- recurrence

def _unrolled_memory(M0, qs, ks, vs, alphas, betas):
    """Brute force in the d_v x d_k orientation, from the explicit unrolled
    product: M_t = M_0 A_1...A_t + sum_{s<=t} beta_s v_s k_s^T A_{s+1}...A_t,
    A_j = alpha_j (I - beta_j k_j k_j^T).  Returns (o [T][d_v], M_T)."""
    dk = ks.shape[1]
    T = ks.shape[0]
    A = [a * (np.eye(dk) - b * np.outer(k, k)) for a, b, k in zip(alphas, betas, ks)]
    outs = []
    M_t = M0
    for t in range(T):
        prod = np.eye(dk)
        for j in range(t + 1):
            prod = prod @ A[j]
        M_t = M0 @ prod
        for s in range(t + 1):
            tail = np.eye(dk)
            for j in range(s + 1, t + 1):
                tail = tail @ A[j]
            M_t = M_t + betas[s] * np.outer(vs[s], ks[s]) @ tail
        outs.append(M_t @ qs[t])
    return np.array(outs), M_t


def pin_bruteforce(orc):
    """Tiny cases (d <= 4, T <= 6), d_k != d_v, grouped heads, nonzero state,
    T = 1 included: the oracle equals the unrolled product."""
    cases = [(3, 2, 5, 1, 1), (2, 4, 6, 1, 2), (4, 4, 1, 2, 2), (4, 3, 6, 2, 4), (1, 3, 4, 1, 1)]
    for ci, (dk, dv, T, Hk, Hv) in enumerate(cases):
        r = _rng(ci)
        q = r.normal(size=(T, Hk, dk))
        k = _unit_rows(r.normal(size=(T, Hk, dk)))
        v = r.normal(size=(T, Hv, dv))
        g = -r.uniform(0.0, 1.0, (T, Hv))
        beta = r.uniform(0.0, 1.0, (T, Hv))
        S0 = r.normal(size=(1, Hv, dk, dv))
        o, S = orc.scan(q, k, v, g, beta, state0=S0, scale=1.0, l2norm=False)
        G = Hv // Hk
        for h in range(Hv):
            hk = h // G
            oo, MT = _unrolled_memory(S0[0, h].T, q[:, hk], k[:, hk], v[:, h], np.exp(g[:, h]), beta[:, h])
            _close(o[:, h], oo, 1e-12, what=f"bruteforce o case {ci} head {h}")
            _close(S[0, h], MT.T, 1e-12, what=f"bruteforce S case {ci} head {h}")


def pin_beta_zero(orc):
    """beta = 0: nothing is written; the memory only decays.
    S_T = e^{sum g} S_0 and o_t = e^{g_1+...+g_t} S_0^T q_t."""
    r = _rng(10)
    T, Hk, Hv, dk, dv = 7, 2, 4, 5, 3
    q = r.normal(size=(T, Hk, dk))
    k = r.normal(size=(T, Hk, dk))
    v = r.normal(size=(T, Hv, dv))
    g = -r.uniform(0, 0.5, (T, Hv))
    beta = np.zeros((T, Hv))
    S0 = r.normal(size=(1, Hv, dk, dv))
    o, S = orc.scan(q, k, v, g, beta, state0=S0, l2norm=False)
    cum = np.cumsum(g, axis=0)
    for h in range(Hv):
        hk = h // 2
        for t in range(T):
            _close(o[t, h], math.exp(cum[t, h]) * S0[0, h].T @ q[t, hk], 1e-12, what="beta=0 o")
        _close(S[0, h], math.exp(cum[-1, h]) * S0[0, h], 1e-12, what="beta=0 S")


def pin_orthonormal_keys(orc):
    """Keys drawn (with repeats) from an orthonormal basis {e_1..e_d}: the
    memory splits into one slot m_e = S^T e per basis vector.  A token with
    key e_i does m_{e_i} <- alpha (1 - beta) m_{e_i} + beta v and m_f <- alpha m_f
    for every other slot; o_t = sum_e (q_t . e) m_e.  With alpha = beta = 1
    this is exact retrieval: querying with k_j returns v_j."""
    r = _rng(20)
    dk, dv, T = 6, 4, 12
    E = ortho_group.rvs(dk, random_state=7)       # rows are the basis
    for variant in ("general", "retrieval"):
        idx = r.integers(0, dk, size=T)
        k = E[idx][:, None, :]
        q = r.normal(size=(T, 1, dk))
        v = r.normal(size=(T, 1, dv))
        if variant == "general":
            g = -r.uniform(0, 0.3, (T, 1))
            beta = r.uniform(0, 1, (T, 1))
            S0 = r.normal(size=(1, 1, dk, dv))
        else:
            g = np.zeros((T, 1))
            beta = np.ones((T, 1))
            S0 = np.zeros((1, 1, dk, dv))
            q = k.copy()
        o, S = orc.scan(q, k, v, g, beta, state0=S0, l2norm=False)
        m = E @ S0[0, 0]                          # slot e_i = S^T e_i
        for t in range(T):
            a, b = math.exp(g[t, 0]), beta[t, 0]
            m = a * m
            m[idx[t]] = (1 - b) * m[idx[t]] + b * v[t, 0]
            _close(o[t, 0], (E @ q[t, 0]) @ m, 1e-12, what=f"orthonormal {variant} o[{t}]")
            if variant == "retrieval":
                _close(o[t, 0], v[t, 0], 1e-12, what="exact retrieval")
        _close(S[0, 0], E.T @ m, 1e-12, what=f"orthonormal {variant} S")


def pin_repeated_key(orc):
    """One unit key repeated, beta = 1, g = 0: each token overwrites the slot,
    S_t = (I - k k^T) S_0 + k v_t^T and o_t = S_t^T q_t."""
    r = _rng(30)
    dk, dv, T = 5, 3, 9
    kk = _unit_rows(r.normal(size=dk))
    k = np.tile(kk, (T, 1, 1))
    q = r.normal(size=(T, 1, dk))
    v = r.normal(size=(T, 1, dv))
    S0 = r.normal(size=(1, 1, dk, dv))
    o, S = orc.scan(q, k, v, np.zeros((T, 1)), np.ones((T, 1)), state0=S0, l2norm=False)
    P = np.eye(dk) - np.outer(kk, kk)
    for t in range(T):
        St = P @ S0[0, 0] + np.outer(kk, v[t, 0])
        _close(o[t, 0], St.T @ q[t, 0], 1e-12, what="repeated key o")
    _close(S[0, 0], P @ S0[0, 0] + np.outer(kk, v[-1, 0]), 1e-12, what="repeated key S")


def pin_zero_key(orc):
    """k = 0 writes nothing: S_t = alpha_t S_{t-1} and o_t = S_t^T q_t (with
    the L2 norm on, the epsilon keeps 0/|0| at 0)."""
    r = _rng(35)
    dk, dv, T = 4, 6, 5
    q = r.normal(size=(T, 1, dk))
    k = np.zeros((T, 1, dk))
    v = r.normal(size=(T, 1, dv))
    g = -r.uniform(0, 1, (T, 1))
    beta = r.uniform(0, 1, (T, 1))
    S0 = r.normal(size=(1, 1, dk, dv))
    o, S = orc.scan(q, k, v, g, beta, state0=S0, l2norm=True)
    St = S0[0, 0].copy()
    for t in range(T):
        St = math.exp(g[t, 0]) * St
        qn = q[t, 0] / np.linalg.norm(q[t, 0])
        _close(o[t, 0], St.T @ qn, 1e-6, what="zero key o")
    _close(S[0, 0], St, 1e-12, what="zero key S")


def pin_linearity(orc):
    """o and S are jointly linear in (V, S_0) for fixed q, k, g, beta."""
    r = _rng(40)
    T, Hk, Hv, dk, dv = 9, 1, 2, 4, 5
    q = r.normal(size=(T, Hk, dk))
    k = r.normal(size=(T, Hk, dk))
    g = -r.uniform(0, 1, (T, Hv))
    beta = r.uniform(0, 1, (T, Hv))
    V1, V2 = r.normal(size=(2, T, Hv, dv))
    A1, A2 = r.normal(size=(2, 1, Hv, dk, dv))
    c = -1.75
    o1, S1 = orc.scan(q, k, V1, g, beta, state0=A1)
    o2, S2 = orc.scan(q, k, V2, g, beta, state0=A2)
    o3, S3 = orc.scan(q, k, V1 + c * V2, g, beta, state0=A1 + c * A2)
    _close(o3, o1 + c * o2, 1e-12, what="linearity o")
    _close(S3, S1 + c * S2, 1e-12, what="linearity S")


def pin_segments_and_packing(orc):
    """Running a sequence in two segments (state passed across) is bitwise
    the same as one run; packing sequences with cu_seqlens is bitwise the
    same as running each alone."""
    r = _rng(50)
    T, Hk, Hv, dk, dv = 23, 2, 4, 6, 5
    q = r.normal(size=(T, Hk, dk))
    k = r.normal(size=(T, Hk, dk))
    v = r.normal(size=(T, Hv, dv))
    g = -r.uniform(0, 1, (T, Hv))
    beta = r.uniform(0, 1, (T, Hv))
    S0 = r.normal(size=(1, Hv, dk, dv))
    o, S = orc.scan(q, k, v, g, beta, state0=S0)
    for cut in (1, 7, 16, 22):
        oa, Sa = orc.scan(q[:cut], k[:cut], v[:cut], g[:cut], beta[:cut], state0=S0)
        ob, Sb = orc.scan(q[cut:], k[cut:], v[cut:], g[cut:], beta[cut:], state0=Sa)
        assert np.array_equal(np.concatenate([oa, ob]), o), f"segment split at {cut} (o)"
        assert np.array_equal(Sb, S), f"segment split at {cut} (S)"
    cu = np.array([0, 5, 5, 17, 23], dtype=np.int32)     # includes an empty sequence
    S0s = r.normal(size=(4, Hv, dk, dv))
    op, Sp = orc.scan(q, k, v, g, beta, cu, state0=S0s)
    for i in range(4):
        a, b = cu[i], cu[i + 1]
        oi, Si = orc.scan(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b], state0=S0s[i:i + 1])
        assert np.array_equal(op[a:b], oi), f"packing seq {i} (o)"
        assert np.array_equal(Sp[i:i + 1], Si), f"packing seq {i} (S)"


def pin_head_mapping(orc):
    """Grouped heads: v-head h reads q/k head h // G (interleaved), or h % H_k
    (tiled).  Permuting v-heads from one order to the other permutes the
    results exactly."""
    r = _rng(60)
    T, Hk, Hv, dk, dv = 6, 2, 6, 4, 3
    G = Hv // Hk
    q = r.normal(size=(T, Hk, dk))
    k = r.normal(size=(T, Hk, dk))
    v = r.normal(size=(T, Hv, dv))
    g = -r.uniform(0, 1, (T, Hv))
    beta = r.uniform(0, 1, (T, Hv))
    S0 = r.normal(size=(1, Hv, dk, dv))
    # tiled head h reads qk head h % Hk; interleaved head h' reads h' // G.
    # perm[h] = the interleaved slot that reads the same qk head with the same rank.
    perm = np.array([(h % Hk) * G + h // Hk for h in range(Hv)])
    ot, St = orc.scan(q, k, v, g, beta, state0=S0, heads_tiled=True)
    inv = np.argsort(perm)
    vi, gi, bi, Si0 = np.empty_like(v), np.empty_like(g), np.empty_like(beta), np.empty_like(S0)
    vi[:, perm], gi[:, perm], bi[:, perm], Si0[:, perm] = v, g, beta, S0
    oi, Si = orc.scan(q, k, vi, gi, bi, state0=Si0, heads_tiled=False)
    assert np.array_equal(oi[:, perm], ot), "tiled vs interleaved (o)"
    assert np.array_equal(Si[:, perm], St), "tiled vs interleaved (S)"
    assert len(inv) == Hv
    # and each v-head really uses its own qk head: a single-head run agrees
    for h in range(Hv):
        o1, S1 = orc.scan(q[:, h // G:h // G + 1], k[:, h // G:h // G + 1], v[:, h:h + 1], g[:, h:h + 1],
                          beta[:, h:h + 1], state0=S0[:, h:h + 1])
        oi2, _ = orc.scan(q, k, v, g, beta, state0=S0)
        assert np.array_equal(oi2[:, h], o1[:, 0]), f"head {h} reads the wrong q/k head"


def pin_normalisation_and_scale(orc):
    """The L2 norm makes q and k scale-free (up to epsilon); `scale`
    multiplies every output and leaves the state alone."""
    r = _rng(70)
    T, Hk, Hv, dk, dv = 8, 1, 2, 16, 8
    q = r.normal(size=(T, Hk, dk))
    k = r.normal(size=(T, Hk, dk))
    v = r.normal(size=(T, Hv, dv))
    g = -r.uniform(0, 1, (T, Hv))
    beta = r.uniform(0, 1, (T, Hv))
    o, S = orc.scan(q, k, v, g, beta, l2norm=True)
    o2, S2 = orc.scan(3.0 * q, 0.25 * k, v, g, beta, l2norm=True)
    _close(o2, o, 1e-6, what="norm scale-free o")
    _close(S2, S, 1e-6, what="norm scale-free S")
    qn = q / np.linalg.norm(q, axis=-1, keepdims=True)
    kn = k / np.linalg.norm(k, axis=-1, keepdims=True)
    o3, S3 = orc.scan(qn, kn, v, g, beta, l2norm=False)
    _close(o3, o, 1e-6, what="norm vs unit rows o")
    _close(S3, S, 1e-6, what="norm vs unit rows S")
    o4, S4 = orc.scan(q, k, v, g, beta, l2norm=True, scale=2.0)
    assert np.array_equal(o4, 2.0 * o) and np.array_equal(S4, S), "scale=2 is an exact doubling of o"
    # epsilon sits inside the square root: a key of squared norm 1e-6 is scaled by 1/sqrt(2e-6)
    kt = np.zeros((1, 1, dk)); kt[0, 0, 0] = 1e-3
    vt = np.ones((1, 1, 1)); qt = np.zeros((1, 1, dk)); qt[0, 0, 0] = 1.0
    ot, St = orc.scan(qt, kt, vt, np.zeros((1, 1)), np.ones((1, 1)), l2norm=True)
    khat = 1e-3 / math.sqrt(1e-6 + EPS)
    _close(St[0, 0, 0, 0], khat, 1e-12, what="epsilon placement")


def pin_state_bound(orc):
    """Unit keys, beta in [0,1], alpha <= 1: |I - beta k k^T| <= 1, so
    |S_t|_2 <= |S_0|_2 + sum_s beta_s |v_s|.  A growing map breaks it."""
    r = _rng(80)
    T, dk, dv = 200, 8, 8
    k = r.normal(size=(T, 1, dk))
    q = r.normal(size=(T, 1, dk))
    v = r.normal(size=(T, 1, dv))
    g = -r.uniform(0, 0.01, (T, 1))
    beta = r.uniform(0.5, 1.0, (T, 1))
    S0 = r.normal(size=(1, 1, dk, dv))
    _, S = orc.scan(q, k, v, g, beta, state0=S0, l2norm=True)
    bound = np.linalg.norm(S0[0, 0], 2) + np.sum(beta[:, 0] * np.linalg.norm(v[:, 0], axis=-1))
    assert np.linalg.norm(S[0, 0], 2) <= bound * (1 + 1e-12)
    # and the state is not trivially small: with beta ~ 1 it tracks recent values
    assert np.linalg.norm(S[0, 0], 2) > 0.5


def pin_decode_is_one_token(orc):
    """The decode step on B sequences equals B one-token scans."""
    r = _rng(90)
    B, Hk, Hv, dk, dv = 5, 2, 4, 6, 4
    q = r.normal(size=(B, Hk, dk))
    k = r.normal(size=(B, Hk, dk))
    v = r.normal(size=(B, Hv, dv))
    g = -r.uniform(0, 1, (B, Hv))
    beta = r.uniform(0, 1, (B, Hv))
    S0 = r.normal(size=(B, Hv, dk, dv))
    o, S = orc.decode_step(q, k, v, g, beta, S0)
    for b in range(B):
        ob, Sb = orc.scan(q[b:b + 1], k[b:b + 1], v[b:b + 1], g[b:b + 1], beta[b:b + 1], state0=S0[b:b + 1])
        assert np.array_equal(o[b:b + 1], ob) and np.array_equal(S[b:b + 1], Sb)
    # one token from a given state, against the unrolled product (T = 1)
    for h in range(Hv):
        oo, M1 = _unrolled_memory(S0[0, h].T, q[0:1, h // 2], k[0:1, h // 2] / np.linalg.norm(k[0, h // 2]),
                                  v[0:1, h], np.exp(g[0:1, h]), beta[0:1, h])
        qn = q[0, h // 2] / np.linalg.norm(q[0, h // 2])
        _close(o[0, h], M1 @ qn, 1e-6, what="decode vs unrolled")
        _close(S[0, h], M1.T, 1e-6, what="decode state vs unrolled")


RECURRENCE_PINS = [pin_bruteforce, pin_beta_zero, pin_orthonormal_keys, pin_repeated_key, pin_zero_key,
                   pin_linearity, pin_segments_and_packing, pin_head_mapping, pin_normalisation_and_scale,
                   pin_state_bound, pin_decode_is_one_token]


# --------------------------------------------------------------------- conv

def _conv_numpy(x, w, window=None):
    """Reference causal depthwise conv of one sequence via numpy.convolve:
    prepend the window (or zeros) and correlate with the taps."""
    T, C = x.shape
    W = w.shape[1]
    ctx = np.zeros((W - 1, C)) if window is None else window
    xp = np.concatenate([ctx, x], axis=0)
    y = np.empty((T, C))
    if T == 0:
        return y
    for c in range(C):
        y[:, c] = np.convolve(xp[:, c], w[c, ::-1], mode="valid")
    return y


def pin_conv_numpy(orc):
    """Pre-activation equals numpy.convolve per channel; SiLU equals
    a * expit(a); varlen resets the context at each sequence start."""
    r = _rng(100)
    C, W = 7, 4
    lens = [5, 1, 2, 9, 0, 3]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    x = r.normal(size=(cu[-1], C))
    w = r.normal(size=(C, W))
    win = r.normal(size=(len(lens), W - 1, C))
    for use_win in (False, True):
        ya, _ = orc.conv1d(x, w, cu, window=win if use_win else None, silu=False)
        ys, _ = orc.conv1d(x, w, cu, window=win if use_win else None, silu=True)
        for i in range(len(lens)):
            a, b = cu[i], cu[i + 1]
            ref = _conv_numpy(x[a:b], w, win[i] if use_win else None)
            _close(ya[a:b], ref, 1e-13, what=f"conv seq {i} window={use_win}")
            _close(ys[a:b], ref * expit(ref), 1e-13, what=f"silu seq {i}")
    # bias
    bias = r.normal(size=C)
    yb, _ = orc.conv1d(x, w, cu, bias=bias, silu=False)
    ya, _ = orc.conv1d(x, w, cu, silu=False)
    _close(yb, ya + bias, 1e-13, what="bias")


def pin_conv_window(orc):
    """The window carries the last W-1 raw inputs: convolving a sequence in
    two pieces (window passed on) is bitwise one convolution, and the new
    window of a short sequence mixes old window rows and new tokens."""
    r = _rng(110)
    C, W = 5, 4
    x = r.normal(size=(11, C))
    w = r.normal(size=(C, W))
    win0 = r.normal(size=(1, W - 1, C))
    y, wout = orc.conv1d(x, w, window=win0)
    for cut in (1, 2, 3, 6, 10):
        y1, w1 = orc.conv1d(x[:cut], w, window=win0)
        y2, w2 = orc.conv1d(x[cut:], w, window=w1)
        assert np.array_equal(np.concatenate([y1, y2]), y), f"conv split at {cut}"
        assert np.array_equal(w2, wout), f"window after split at {cut}"
        hist = np.concatenate([win0[0], x[:cut]], axis=0)
        assert np.array_equal(w1[0], hist[-(W - 1):]), f"window content after {cut} tokens"


def pin_conv_f32(orc):
    """The fp32 evaluation stays within 4 fp32 ulps of the fp64 result, its
    exponential within 2 ulps of math.exp, and its bf16 output is the
    round-to-nearest-even of its fp32 output."""
    import torch
    r = _rng(120)
    C, W = 64, 4
    lens = [40, 3, 17]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    x = r.normal(size=(cu[-1], C)).astype(np.float32)
    w = (0.5 * r.normal(size=(C, W))).astype(np.float32)
    win = r.normal(size=(3, W - 1, C)).astype(np.float32)
    bias = r.normal(size=C).astype(np.float32)
    for silu in (False, True):
        for b in (None, bias):
            y32 = orc.conv1d_f32(x, w, cu, window=win, bias=b, silu=silu)
            y64, _ = orc.conv1d(x, w, cu, window=win, bias=b, silu=silu)
            # Error bound of a W-term fused dot product in fp32 (Higham, "Accuracy and
            # Stability of Numerical Algorithms", 3.1): |err| <= W u sum|w_j x_j| + u |bias|,
            # u = 2^-24; SiLU has slope <= 1.1 and adds a few rounding steps of its own.
            absdot, _ = orc.conv1d(np.abs(x), np.abs(w), cu, window=np.abs(win),
                                   bias=None if b is None else np.abs(b), silu=False)
            u = 2.0 ** -24
            bound = 1.1 * (W + 1) * u * absdot + 4 * u * np.abs(y64) + 1e-37
            err = np.abs(y32.astype(np.float64) - y64)
            assert np.all(err <= bound), f"f32 conv off by {np.max(err / bound):.2f} x its bound (silu={silu})"
            bits = orc.conv1d_f32(x, w, cu, window=win, bias=b, silu=silu, out_bf16=True)
            tb = torch.from_numpy(y32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            assert np.array_equal(bits, tb), "bf16 output is RNE of fp32 output"
    xs = np.concatenate([np.linspace(-86.0, 88.5, 20001), r.normal(size=2000) * 5, [0.0, -0.0, 1e-30, -1e-30]])
    for xv in xs.astype(np.float32):
        e = orc.exp_f32(float(xv))
        ref = math.exp(float(xv))
        u = float(np.spacing(np.float32(ref)))
        assert abs(e - ref) <= 2 * u, f"exp_f32({xv}) = {e}, exp = {ref}"
    assert orc.exp_f32(0.0) == 1.0 and orc.exp_f32(100.0) == math.inf and orc.exp_f32(-100.0) == 0.0


# --------------------------------------------------------------- gated norm
# y_j = w_j o_j / sqrt(mean(o^2) + eps) silu(z_j) per (token, v-head) row.

def _silu(a):
    return a * expit(a)


def pin_gated_norm_closed_forms(orc):
    """Rows whose root mean square is known by hand."""
    d = 4
    w = np.array([1.0, 2.0, 3.0, 4.0])
    g = 0.75 * math.log(3.0)                 # silu(ln 3) = ln 3 / (1 + 1/3)
    z = np.full((1, d), math.log(3.0))
    # [3, 4, 0, 0]: mean square 25/4, rms 2.5 (eps 0)
    y = orc.gated_rmsnorm(np.array([[3.0, 4.0, 0.0, 0.0]]), z, w, eps=0.0)
    _close(y, [[1.2 * g, 3.2 * g, 0.0, 0.0]], 1e-14, what="[3,4,0,0] row")
    # a constant row c: o / rms = c / sqrt(c^2 + eps), weight and gate by element
    c, eps = 0.37, 1e-6
    y = orc.gated_rmsnorm(np.full((1, d), c), z, w, eps=eps)
    _close(y, [w * c / math.sqrt(c * c + eps) * g], 1e-14, what="constant row")
    # a tiny row, where eps decides the scale: delta / sqrt(delta^2 + eps)
    dl = 1e-5
    y = orc.gated_rmsnorm(np.full((1, d), -dl), np.full((1, d), 2.0), w, eps=eps)
    _close(y, [-w * dl / math.sqrt(dl * dl + eps) * (2.0 / (1.0 + math.exp(-2.0)))], 1e-13, what="eps-dominated row")


def pin_gated_norm_gate(orc):
    """The gate: z = 0 gives 0; silu(z) - silu(-z) = z, so y(z) - y(-z) is the
    normalised, weighted row times z."""
    r = _rng(40)
    rows, d = 5, 16
    o = r.normal(size=(rows, d))
    z = r.normal(size=(rows, d)) * 3
    w = r.normal(size=d)
    assert np.all(orc.gated_rmsnorm(o, np.zeros_like(z), w) == 0.0)
    diff = orc.gated_rmsnorm(o, z, w) - orc.gated_rmsnorm(o, -z, w)
    rms = np.sqrt(np.mean(o * o, axis=1, keepdims=True) + EPS)
    _close(diff, w * o / rms * z, 1e-12, what="odd part of the gate")


def pin_gated_norm_rows_independent(orc):
    """Each (token, v-head) row is normalised on its own: changing one row
    changes no other, and with eps = 0 scaling a row by l > 0 leaves it
    unchanged."""
    r = _rng(41)
    T, H, d = 3, 4, 8
    o = r.normal(size=(T, H, d))
    z = r.normal(size=(T, H, d))
    w = r.normal(size=d)
    y0 = orc.gated_rmsnorm(o, z, w)
    o2 = o.copy()
    o2[1, 2] *= 7.0
    o2[2, 0] += 1.0
    y1 = orc.gated_rmsnorm(o2, z, w)
    changed = np.any(y1 != y0, axis=-1)
    assert changed[1, 2] and changed[2, 0] and changed.sum() == 2, changed
    ys = orc.gated_rmsnorm(o2 * 3.5, z, w, eps=0.0)
    _close(ys, orc.gated_rmsnorm(o2, z, w, eps=0.0), 1e-14, what="scale invariance")


# ------------------------------------------------------------------ gating
# g = -exp(A_log[h]) softplus(a + dt_bias[h]), beta = sigmoid(b), per (token, v-head).

def pin_gating_closed_forms(orc):
    """Points where softplus and the sigmoid are known: softplus(0) = ln 2,
    softplus(ln(e - 1)) = 1, softplus(x) -> x and -> e^x at the ends;
    sigmoid(0) = 1/2, sigmoid(+-ln 3) = 3/4, 1/4."""
    H = 3
    A_log = np.array([0.0, math.log(2.0), -1.0])
    dt_bias = np.array([0.0, 0.5, -0.25])
    pre = np.array([[0.0, math.log(math.e - 1.0), 50.0], [-50.0, 0.0, 0.0]])   # a + dt_bias
    a = pre - dt_bias
    b = np.array([[0.0, math.log(3.0), -math.log(3.0)], [0.0, 0.0, 0.0]])
    g, beta = orc.gating(a, b, A_log, dt_bias)
    decay = np.exp(A_log)
    sp = np.array([[math.log(2.0), 1.0, 50.0], [math.exp(-50.0), math.log(2.0), math.log(2.0)]])
    _close(g, -decay * sp, 1e-12, what="g closed forms")
    assert abs(g[1, 0] / (-math.exp(-50.0)) - 1.0) < 1e-12, g[1, 0]     # relative, far below 1
    _close(beta, [[0.5, 0.75, 0.25], [0.5, 0.5, 0.5]], 1e-14, what="beta closed forms")
    assert H == g.shape[1]


def pin_gating_heads_and_ranges(orc):
    """Each head takes its own A_log and dt_bias (a head's gates move with its
    own parameters only); g <= 0 and 0 < beta < 1; g is monotone decreasing
    in a and beta increasing in b."""
    r = _rng(50)
    T, H = 7, 5
    a = r.normal(size=(T, H)) * 3
    b = r.normal(size=(T, H)) * 3
    A_log = r.normal(size=H)
    dt_bias = r.normal(size=H)
    g0, b0 = orc.gating(a, b, A_log, dt_bias)
    assert np.all(g0 < 0) and np.all((b0 > 0) & (b0 < 1))
    A2, d2 = A_log.copy(), dt_bias.copy()
    A2[3] += 0.7
    d2[1] -= 1.3
    g1, b1 = orc.gating(a, b, A2, d2)
    moved = np.any(g1 != g0, axis=0)
    assert moved[1] and moved[3] and moved.sum() == 2, moved
    assert np.array_equal(b1, b0)
    _close(g1[:, 3], g0[:, 3] * math.exp(0.7), 1e-13, what="A_log scales the decay rate")
    ga, _ = orc.gating(a + 0.5, b, A_log, dt_bias)
    _, bb = orc.gating(a, b + 0.5, A_log, dt_bias)
    assert np.all(ga < g0) and np.all(bb > b0)


CONV_PINS = [pin_conv_numpy, pin_conv_window, pin_conv_f32]
NORM_PINS = [pin_gated_norm_closed_forms, pin_gated_norm_gate, pin_gated_norm_rows_independent]
GATING_PINS = [pin_gating_closed_forms, pin_gating_heads_and_ranges]
ALL_PINS = RECURRENCE_PINS + CONV_PINS + NORM_PINS + GATING_PINS
