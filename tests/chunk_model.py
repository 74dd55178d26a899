"""fp64 numpy model of the chunked algorithm the GPU kernels run.

Test-side only: it checks the algebra of the chunked form against the
token-by-token oracle before (and independently of) any HIP code.  It is
not the oracle and the oracle does not use it.

Within a chunk of C tokens (tokens r = 0..C'-1, gamma_r = g_0 + ... + g_r,
state S_0 at the chunk start, k_hat = rk * k, q_hat = rq * q):

  A[r,s]  = beta_r e^{gamma_r - gamma_s} (k_hat_r . k_hat_s)     s < r
  Tinv    = (I + A)^{-1}     (unit lower triangular)
  Tt      = Tinv diag(beta)
  X       = K_hat S_0
  U       = Tt (V - diag(e^gamma) X)                      (the new values)
  P[r,s]  = e^{gamma_r - gamma_s} (q_hat_r . k_hat_s)    s <= r
  O       = diag(e^gamma) Q_hat S_0 + P U
  S_next  = e^{gamma_last} S_0 + K_hat^T diag(e^{gamma_last - gamma}) U

(the WY/UT form of the delta rule; the oxydllm 0.0.0-alpha.12.2 release
notes, "New Features", run prefill as such a chunked parallel scan).  The
inverse is taken blockwise, as the same notes describe: each 16x16 diagonal
block N (strictly lower, so N^16 = 0) by the doubling product
(I+N)^{-1} = (I-N)(I+N^2)(I+N^4)(I+N^8), then diagonal blocks are merged
pairwise 16 -> 32 -> 64 with [[X,0],[Y,Z]]^{-1} = [[X^-1,0],[-Z^-1 Y X^-1, Z^-1]].
"""
from __future__ import annotations

import numpy as np

EPS = 1e-6


def inverse_doubling16(N):
    """(I + N)^{-1} for a strictly lower-triangular 16x16 (or smaller) N."""
    n = N.shape[0]
    I = np.eye(n)
    N2 = N @ N
    N4 = N2 @ N2
    N8 = N4 @ N4
    return (I - N) @ (I + N2) @ (I + N4) @ (I + N8)


def inverse_blockwise(A, block=16):
    """(I + A)^{-1} for strictly lower-triangular A (C x C, C in {16,32,64})."""
    C = A.shape[0]
    inv = np.zeros_like(A)
    for b in range(0, C, block):
        inv[b:b + block, b:b + block] = inverse_doubling16(A[b:b + block, b:b + block])
    w = block
    while w < C:
        for b in range(0, C, 2 * w):
            X = inv[b:b + w, b:b + w]
            Z = inv[b + w:b + 2 * w, b + w:b + 2 * w]
            Y = A[b + w:b + 2 * w, b:b + w]
            inv[b + w:b + 2 * w, b:b + w] = -Z @ (Y @ X)
        w *= 2
    return inv


def inverse_forward_substitution(A):
    """The row-by-row solve: Tinv[r] = e_r - sum_{s<r} A[r,s] Tinv[s]."""
    C = A.shape[0]
    inv = np.zeros_like(A)
    for r in range(C):
        inv[r] = np.eye(C)[r] - A[r, :r] @ inv[:r]
    return inv


def chunked_scan(q, k, v, g, beta, cu_seqlens=None, *, state0=None, chunk=64, scale=1.0, l2norm=True,
                 heads_tiled=False):
    n_tok, Hk, dk = q.shape
    _, Hv, dv = v.shape
    G = Hv // Hk
    cu = np.array([0, n_tok]) if cu_seqlens is None else np.asarray(cu_seqlens)
    n_seq = len(cu) - 1
    o = np.zeros((n_tok, Hv, dv))
    S_out = np.zeros((n_seq, Hv, dk, dv))
    for s in range(n_seq):
        for h in range(Hv):
            hk = h % Hk if heads_tiled else h // G
            S = np.zeros((dk, dv)) if state0 is None else np.array(state0[s, h], dtype=np.float64)
            for c0 in range(int(cu[s]), int(cu[s + 1]), chunk):
                c1 = min(c0 + chunk, int(cu[s + 1]))
                n = c1 - c0
                K = k[c0:c1, hk].astype(np.float64)
                Q = q[c0:c1, hk].astype(np.float64)
                V = v[c0:c1, h].astype(np.float64)
                gg = g[c0:c1, h].astype(np.float64)
                bb = beta[c0:c1, h].astype(np.float64)
                if l2norm:
                    rk = 1.0 / np.sqrt(np.sum(K * K, axis=1) + EPS)
                    rq = scale / np.sqrt(np.sum(Q * Q, axis=1) + EPS)
                else:
                    rk = np.ones(n)
                    rq = np.full(n, scale)
                Kh = K * rk[:, None]
                Qh = Q * rq[:, None]
                gam = np.cumsum(gg)
                D = np.exp(np.minimum(gam[:, None] - gam[None, :], 0.0))
                A = np.tril(bb[:, None] * D * (Kh @ Kh.T), -1)
                Cp = chunk if chunk >= 16 else n
                Ap = np.zeros((Cp, Cp))
                Ap[:n, :n] = A
                Tinv = inverse_blockwise(Ap)[:n, :n]
                Tt = Tinv * bb[None, :]
                X = Kh @ S
                U = Tt @ (V - np.exp(gam)[:, None] * X)
                P = np.tril(D * (Qh @ Kh.T))
                o[c0:c1, h] = np.exp(gam)[:, None] * (Qh @ S) + P @ U
                S = np.exp(gam[-1]) * S + Kh.T @ (np.exp(gam[-1] - gam)[:, None] * U)
            S_out[s, h] = S
    return o, S_out
