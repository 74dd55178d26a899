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

from linear_attention_delta_amd import synth

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


# ---------------------------------------------------------------------------
# Segment form of the carry (what the bf16 kernels run for one long sequence).
#
# Per chunk the state map is affine, S' = M S + B, with
#   M = e^{gamma_last} I - K_hat^T diag(e^{gamma_last - gamma}) Tt diag(e^gamma) K_hat.
# A sequence is cut into segments of L chunks.  Pass 1 carries Z = [S | Phi]
# through every segment but the last (S from zero -- from the true initial
# state for segment 0 -- and Phi from the identity), giving the segment's
# affine part B_p and transition Phi_p = M_last ... M_first.  The segment
# starts are chained, S_start[p+1] = Phi_p S_start[p] + B_p, and pass 2 re-runs
# every segment from its true start, producing the outputs.  In exact
# arithmetic this is the same product as the chunk-by-chunk loop, reassociated.
#
# With bf16=True the model rounds to bf16 exactly the operands that the GPU
# kernels feed to the bf16 matrix cores (raw q/k/v are bf16 already; the
# state and transition, the residual V - a X, the inverse Tt, the scaled U
# of the state update, the unscaled U and P of the output, the stored
# transition Phi and the state fed to the chain), accumulating in fp64
# instead of fp32.  It predicts how the error grows with the segment length
# without reproducing the kernels' bits.


def _rb(a, on):
    """a rounded to the nearest bf16 (ties to even) when `on`, as fp64."""
    return synth.round_bf16(np.asarray(a, dtype=np.float32)).astype(np.float64) if on else a


def _chunk_factors(Q, K, gg, bb, chunk, scale, l2norm):
    """Per-chunk, state-independent factors in the kernels' form (raw K, Q)."""
    n = K.shape[0]
    if l2norm:
        rk = 1.0 / np.sqrt(np.sum(K * K, axis=1) + EPS)
        rq = scale / np.sqrt(np.sum(Q * Q, axis=1) + EPS)
    else:
        rk = np.ones(n)
        rq = np.full(n, scale)
    gam = np.cumsum(gg)
    D = np.exp(np.minimum(gam[:, None] - gam[None, :], 0.0))
    Kh = K * rk[:, None]
    A = np.tril(bb[:, None] * D * (Kh @ Kh.T), -1)
    Ap = np.zeros((chunk, chunk))
    Ap[:n, :n] = A
    Tt = inverse_blockwise(Ap)[:n, :n] * bb[None, :]
    P = np.tril(D * rq[:, None] * rk[None, :] * (Q @ K.T))
    return dict(a=np.exp(gam) * rk, c=np.exp(gam[-1] - gam) * rk, gl=np.exp(gam[-1]), b=rq * np.exp(gam),
                Tt=Tt, P=P)


def _carry(Z, Vpad, K, Q, f, bf):
    """One chunk: Z <- gl Z + K^T (c U), U = Tt (V - a K Z); returns (Z, O or None).
    Vpad: the values term per column of Z (zeros for transition columns)."""
    zb = _rb(Z, bf)
    X = K @ zb
    U = _rb(f["Tt"], bf) @ _rb(Vpad - f["a"][:, None] * X, bf)
    O = None
    if Q is not None:
        O = f["b"][:, None] * (Q @ zb) + _rb(f["P"], bf) @ _rb(U, bf)
        O = _rb(O, bf)
    Z = f["gl"] * Z + K.T @ _rb(f["c"][:, None] * U, bf)
    return Z, O


def segmented_scan(q, k, v, g, beta, cu_seqlens=None, *, state0=None, chunk=64, seg_len=8, scale=1.0,
                   l2norm=True, heads_tiled=False, bf16=False):
    n_tok, Hk, dk = q.shape
    _, Hv, dv = v.shape
    G = Hv // Hk
    cu = np.array([0, n_tok]) if cu_seqlens is None else np.asarray(cu_seqlens)
    n_seq = len(cu) - 1
    o = np.zeros((n_tok, Hv, dv))
    S_out = np.zeros((n_seq, Hv, dk, dv))
    for s in range(n_seq):
        t0, t1 = int(cu[s]), int(cu[s + 1])
        starts = list(range(t0, t1, chunk))
        nseg = max(1, -(-len(starts) // seg_len))
        for h in range(Hv):
            hk = h % Hk if heads_tiled else h // G
            S0 = np.zeros((dk, dv)) if state0 is None else np.array(state0[s, h], dtype=np.float64)
            ch = []
            for c0 in starts:
                c1 = min(c0 + chunk, t1)
                K = k[c0:c1, hk].astype(np.float64)
                Q = q[c0:c1, hk].astype(np.float64)
                ch.append((c0, c1, K, Q, v[c0:c1, h].astype(np.float64),
                           _chunk_factors(Q, K, g[c0:c1, h].astype(np.float64), beta[c0:c1, h].astype(np.float64),
                                          chunk, scale, l2norm)))
            # pass 1: B_p and Phi_p for every segment but the last
            B, Phi = [], []
            for p in range(nseg - 1):
                Z = np.concatenate([S0 if p == 0 else np.zeros((dk, dv)), np.eye(dk)], axis=1)
                for (c0, c1, K, Q, V, f) in ch[p * seg_len:(p + 1) * seg_len]:
                    Z, _ = _carry(Z, np.concatenate([V, np.zeros((c1 - c0, dk))], axis=1), K, None, f, bf16)
                B.append(Z[:, :dv].copy())
                Phi.append(_rb(Z[:, dv:], bf16))
            # chain of segment starts
            start = [S0]
            if nseg > 1:
                start.append(B[0])
            for p in range(1, nseg - 1):
                start.append(Phi[p] @ _rb(start[p], bf16) + B[p])
            # pass 2: every segment from its true start
            for p in range(nseg):
                Z = start[p]
                for (c0, c1, K, Q, V, f) in ch[p * seg_len:(p + 1) * seg_len]:
                    Z, O = _carry(Z, V, K, Q, f, bf16)
                    o[c0:c1, h] = O
                if p == nseg - 1:
                    S_out[s, h] = Z
    return o, S_out
