"""CPU checker (oracle) for the Gated DeltaNet layer core.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline import this package; the product path (the GPU library and its
binding) never does.  It shares no code with the GPU path.

The arithmetic lives in ``gdn_oracle.c`` (plain fp64 C, threaded over
independent (sequence, v-head) pairs).  This module only marshals numpy
arrays into it.  Parity status of each function is listed at the bottom.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libgdn_oracle.so")

L2NORM = 1
HEADS_TILED = 2


def build(force: bool = True) -> str:
    """Compile gdn_oracle.c with gcc into oracle/libgdn_oracle.so."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
               "-pthread", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class Oracle:
    """The oracle's entry points bound to one compiled copy of gdn_oracle.c."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32 = ctypes.c_int
        lib.gdn_oracle_conv1d_f64.argtypes = [i32, P, i32, i32, P, P, P, P, i32, P, P]
        lib.gdn_oracle_conv1d_f64.restype = None
        lib.gdn_oracle_conv1d_f32.argtypes = [i32, P, i32, i32, P, P, P, P, i32, P, i32, P]
        lib.gdn_oracle_conv1d_f32.restype = None
        lib.gdn_oracle_exp_f32.argtypes = [ctypes.c_float]
        lib.gdn_oracle_exp_f32.restype = ctypes.c_float
        lib.gdn_oracle_scan.argtypes = [i32, P, i32, i32, i32, i32, ctypes.c_double, ctypes.c_uint,
                                        P, P, P, P, P, P, P, P, i32]
        lib.gdn_oracle_scan.restype = i32
        lib.gdn_oracle_gated_rmsnorm.argtypes = [ctypes.c_long, i32, P, P, P, ctypes.c_double, P]
        lib.gdn_oracle_gated_rmsnorm.restype = None
        lib.gdn_oracle_gating.argtypes = [ctypes.c_long, i32, P, P, P, P, P, P]
        lib.gdn_oracle_gating.restype = None
        lib.gdn_oracle_available_cores.argtypes = []
        lib.gdn_oracle_available_cores.restype = i32
        self.lib = lib
        self.path = path

    def available_cores(self) -> int:
        return int(self.lib.gdn_oracle_available_cores())

    def conv1d(self, x, w, cu_seqlens=None, *, bias=None, window=None, silu=True):
        """fp64 causal depthwise conv (+SiLU).  x [N][C], w [C][W], window
        [n_seq][W-1][C] or None.  Returns (y [N][C] fp64, new window [n_seq][W-1][C])."""
        x = _f64(x)
        w = _f64(w)
        n_tok, C = x.shape
        W = w.shape[1]
        cu = _cu(cu_seqlens, n_tok)
        n_seq = len(cu) - 1
        y = np.empty((n_tok, C), dtype=np.float64)
        wo = np.empty((n_seq, W - 1, C), dtype=np.float64)
        self.lib.gdn_oracle_conv1d_f64(n_seq, _ptr(cu), C, W, _ptr(x), _ptr(w), _ptr(_f64(bias)),
                                       _ptr(_f64(window)), int(bool(silu)), _ptr(y), _ptr(wo))
        return y, wo

    def conv1d_f32(self, x, w, cu_seqlens=None, *, bias=None, window=None, silu=True, out_bf16=False):
        """fp32 conv in its defining evaluation order (the bit-exact target).
        Returns fp32 [N][C], or bf16 bit patterns (uint16) when out_bf16."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        w = np.ascontiguousarray(w, dtype=np.float32)
        n_tok, C = x.shape
        W = w.shape[1]
        cu = _cu(cu_seqlens, n_tok)
        n_seq = len(cu) - 1
        b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
        win = None if window is None else np.ascontiguousarray(window, dtype=np.float32)
        if out_bf16:
            out = np.empty((n_tok, C), dtype=np.uint16)
            self.lib.gdn_oracle_conv1d_f32(n_seq, _ptr(cu), C, W, _ptr(x), _ptr(w), _ptr(b), _ptr(win),
                                           int(bool(silu)), None, 1, _ptr(out))
        else:
            out = np.empty((n_tok, C), dtype=np.float32)
            self.lib.gdn_oracle_conv1d_f32(n_seq, _ptr(cu), C, W, _ptr(x), _ptr(w), _ptr(b), _ptr(win),
                                           int(bool(silu)), _ptr(out), 0, None)
        return out

    def exp_f32(self, x: float) -> float:
        return float(self.lib.gdn_oracle_exp_f32(ctypes.c_float(x)))

    def scan(self, q, k, v, g, beta, cu_seqlens=None, *, state0=None, scale=1.0, l2norm=True,
             heads_tiled=False, n_threads=0, return_threads=False, state_out=None):
        """Token-by-token gated delta rule in fp64.

        q, k [N][H_k][d_k]; v [N][H_v][d_v]; g, beta [N][H_v]; state0
        [n_seq][H_v][d_k][d_v] or None.  Returns (o [N][H_v][d_v], S [n_seq][H_v][d_k][d_v]).
        state_out: optional C-contiguous fp64 array of S's shape to write S
        into; it may be state0 itself (each (sequence, head) slice is read
        before it is written), which steps a large state without copies."""
        q, k, v, g, beta = (_f64(a) for a in (q, k, v, g, beta))
        n_tok, Hk, dk = q.shape
        _, Hv, dv = v.shape
        assert k.shape == q.shape and v.shape[0] == n_tok and g.shape == (n_tok, Hv) and beta.shape == (n_tok, Hv)
        cu = _cu(cu_seqlens, n_tok)
        assert int(cu[-1]) == n_tok
        n_seq = len(cu) - 1
        s0 = _f64(state0)
        if s0 is not None:
            assert s0.shape == (n_seq, Hv, dk, dv)
        o = np.zeros((n_tok, Hv, dv), dtype=np.float64)
        if state_out is not None:
            assert state_out.dtype == np.float64 and state_out.flags.c_contiguous
            assert state_out.shape == (n_seq, Hv, dk, dv)
            if state0 is not None and np.shares_memory(state_out, state0):
                assert s0 is state0, "state_out may alias state0 only when state0 is contiguous fp64"
            S = state_out
        else:
            S = np.zeros((n_seq, Hv, dk, dv), dtype=np.float64)
        flags = (L2NORM if l2norm else 0) | (HEADS_TILED if heads_tiled else 0)
        nt = self.lib.gdn_oracle_scan(n_seq, _ptr(cu), Hk, Hv, dk, dv, float(scale), flags,
                                      _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(s0),
                                      _ptr(o), _ptr(S), int(n_threads))
        if nt < 0:
            raise ValueError("oracle scan rejected the shapes")
        return (o, S, nt) if return_threads else (o, S)

    def gated_rmsnorm(self, o, z, w, *, eps=1e-6):
        """Gated RMS norm in fp64: o, z [..., d] (the last axis is one v-head's
        values), w [d].  Returns y of o's shape."""
        o, z, w = _f64(o), _f64(z), _f64(w)
        assert o.shape == z.shape and w.shape == (o.shape[-1],)
        d = o.shape[-1]
        y = np.zeros(o.shape, dtype=np.float64)
        self.lib.gdn_oracle_gated_rmsnorm(o.size // d if d else 0, d, _ptr(o), _ptr(z), _ptr(w), float(eps), _ptr(y))
        return y

    def gating(self, a, b, A_log, dt_bias):
        """Gates in fp64 from the raw projections a, b [N][H] and the per-head
        A_log, dt_bias [H].  Returns (g, beta), each [N][H]."""
        a, b, A_log, dt_bias = (_f64(x) for x in (a, b, A_log, dt_bias))
        assert a.ndim == 2 and b.shape == a.shape and A_log.shape == dt_bias.shape == (a.shape[1],)
        g = np.zeros(a.shape, dtype=np.float64)
        beta = np.zeros(a.shape, dtype=np.float64)
        self.lib.gdn_oracle_gating(a.shape[0], a.shape[1], _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias),
                                   _ptr(g), _ptr(beta))
        return g, beta

    def decode_step(self, q, k, v, g, beta, state, *, scale=1.0, l2norm=True, heads_tiled=False,
                    n_threads=0, in_place=False):
        """One recurrent step for B sequences (one token each): q, k [B][H_k][d_k],
        v [B][H_v][d_v], g, beta [B][H_v], state [B][H_v][d_k][d_v].
        Returns (o [B][H_v][d_v], new state); with in_place the new state is
        written over `state` (C-contiguous fp64) and that array is returned."""
        B = q.shape[0]
        cu = np.arange(B + 1, dtype=np.int32)
        return self.scan(q, k, v, g, beta, cu, state0=state, scale=scale, l2norm=l2norm,
                         heads_tiled=heads_tiled, n_threads=n_threads, state_out=state if in_place else None)


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def _cu(cu_seqlens, n_tok):
    if cu_seqlens is None:
        return np.array([0, n_tok], dtype=np.int32)
    return np.ascontiguousarray(cu_seqlens, dtype=np.int32)


_default: Optional[Oracle] = None


def default() -> Oracle:
    global _default
    if _default is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        _default = Oracle(_LIB_PATH)
    return _default


def available_cores() -> int:
    return default().available_cores()


def conv1d(*a, **kw):
    return default().conv1d(*a, **kw)


def conv1d_f32(*a, **kw):
    return default().conv1d_f32(*a, **kw)


def exp_f32(x: float) -> float:
    return default().exp_f32(x)


def scan(*a, **kw):
    return default().scan(*a, **kw)


def decode_step(*a, **kw):
    return default().decode_step(*a, **kw)


def gated_rmsnorm(*a, **kw):
    return default().gated_rmsnorm(*a, **kw)


def gating(*a, **kw):
    return default().gating(*a, **kw)


def source_text() -> str:
    with open(_SRC) as f:
        return f.read()


def build_variant(source: str, out_path: str) -> Oracle:
    """Compile a (patched) copy of the oracle source to out_path and bind it.
    The tests use this to check that their pins reject planted mistakes."""
    src = out_path + ".c"
    with open(src, "w") as f:
        f.write(source)
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
                    "-pthread", src, "-o", out_path, "-lm"], check=True)
    return Oracle(out_path)


# Parity status (what pins each function; the tests under tests/ hold them):
#   conv1d        pinned: numpy.convolve per channel, SiLU closed forms, window
#                 carry / segment split, varlen reset.
#   conv1d_f32    pinned: within 4 fp32 ulp of conv1d (fp64) and bitwise
#                 self-consistent; exp_f32 within 2 ulp of math.exp.
#   scan          pinned: brute-force unrolled transition products, beta=0 and
#                 alpha=1 orthonormal-key closed forms, repeated-key closed form,
#                 linearity, segment invariance, head mapping, d_k != d_v.
#   decode_step   pinned through scan (it is scan with one token per sequence).
