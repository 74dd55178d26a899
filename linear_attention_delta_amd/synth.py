"""Seeded synthetic inputs for the Gated DeltaNet layer core.

This module only draws random numbers and packs them into arrays.  It holds
none of the layer's arithmetic (no convolution, no normalisation, no state
update): the GPU path and the CPU checker both take their inputs from here and
from nowhere else.

Shapes follow a Qwen3.5-style hybrid layer: the short causal convolution runs
over C_conv = 2*H_k*d_k + H_v*d_v channels ordered [q | k | v]; the gates are
one value per token and v-head, kept in fp32 (the oxydllm 0.0.0-alpha.12.2
release notes, "New Features": DeltaNet scalar parameters stay F32 end to
end).

Distributions (standard deviations, not variances):
  raw x ~ N(0, 1); conv taps ~ N(0, 0.5);
  beta = sigmoid(N(0, 1)); g = -softplus(N(0, 1)) * 0.5   (log-decay, alpha = e^g)
  adversarial variant: beta ~ U(0.9, 1.0), g ~ U(-0.01, 0), x rows drawn from a
  4-symbol alphabet in runs of 1..512 identical tokens;
  initial states ~ N(0, 0.02) where a workload asks for them.

Every array comes from its own numpy PCG64 stream keyed by (seed, name), so
that changing one size never changes another array's values.
"""
from __future__ import annotations

import dataclasses
import hashlib
import zlib
from typing import Optional

import numpy as np

CONV_WIDTH = 4


def _rng(seed: int, name: str) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([int(seed), zlib.crc32(name.encode())]))


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even; NaN -> quiet NaN."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact fp32 values."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def round_bf16(a: np.ndarray) -> np.ndarray:
    """fp32 values rounded (RNE) to the nearest bf16, returned as fp32."""
    return bf16_bits_to_f32(bf16_bits(a))


@dataclasses.dataclass
class LayerShape:
    num_qk_heads: int
    num_v_heads: int
    head_dim_k: int
    head_dim_v: int

    @property
    def conv_channels(self) -> int:
        return 2 * self.num_qk_heads * self.head_dim_k + self.num_v_heads * self.head_dim_v


TINY = LayerShape(2, 4, 64, 64)
QWEN35_4B = LayerShape(16, 32, 128, 128)


@dataclasses.dataclass
class PrefillInputs:
    """One prefill workload.  ``x`` holds the raw conv inputs, already rounded
    to ``dtype`` (so both sides see identical values), as fp32 numpy."""

    name: str
    shape: LayerShape
    dtype: str                      # "f32" or "bf16" (the q/k/v/o dtype)
    cu_seqlens: np.ndarray          # int32 [N+1]
    dense_T: int                    # T when every sequence has the same length, else 0
    x: np.ndarray                   # [N_tok][C_conv] fp32 (bf16-representable when dtype == "bf16")
    conv_w: np.ndarray              # [C_conv][W] fp32
    g: np.ndarray                   # [N_tok][H_v] fp32
    beta: np.ndarray                # [N_tok][H_v] fp32
    state0: Optional[np.ndarray]    # [N][H_v][d_k][d_v] fp32 or None (zeros)
    conv_state0: Optional[np.ndarray] = None  # [N][W-1][C_conv] (dtype-representable) or None
    chunk_size: int = 64
    scale: float = 1.0

    @property
    def num_seqs(self) -> int:
        return int(len(self.cu_seqlens) - 1)

    @property
    def total_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    def digest(self) -> str:
        h = hashlib.sha256()
        for a in (self.cu_seqlens, self.x, self.conv_w, self.g, self.beta):
            h.update(np.ascontiguousarray(a).tobytes())
        if self.state0 is not None:
            h.update(np.ascontiguousarray(self.state0).tobytes())
        return h.hexdigest()[:16]


def _gates(seed: int, n_tok: int, hv: int):
    b = _rng(seed, "beta").standard_normal((n_tok, hv))
    gg = _rng(seed, "g").standard_normal((n_tok, hv))
    beta = 1.0 / (1.0 + np.exp(-b))
    g = -np.logaddexp(0.0, gg) * 0.5
    return g.astype(np.float32), beta.astype(np.float32)


def _quant(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    return round_bf16(x) if dtype == "bf16" else x


def make_prefill(seed: int, shape: LayerShape, seqlens, dtype: str, *, state0_std: float = 0.0,
                 conv_state: bool = False, chunk_size: int = 64, scale: float = 1.0,
                 name: str = "custom") -> PrefillInputs:
    seqlens = [int(s) for s in seqlens]
    cu = np.zeros(len(seqlens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(seqlens)
    n_tok = int(cu[-1])
    cc = shape.conv_channels
    x = _quant(_rng(seed, "x").standard_normal((n_tok, cc), dtype=np.float32), dtype)
    w = (_rng(seed, "conv_w").standard_normal((cc, CONV_WIDTH)) * 0.5).astype(np.float32)
    g, beta = _gates(seed, n_tok, shape.num_v_heads)
    s0 = None
    if state0_std > 0:
        s0 = (_rng(seed, "state0").standard_normal(
            (len(seqlens), shape.num_v_heads, shape.head_dim_k, shape.head_dim_v), dtype=np.float32)
            * np.float32(state0_std)).astype(np.float32)
    cs0 = None
    if conv_state:
        cs0 = _quant(_rng(seed, "conv_state0").standard_normal(
            (len(seqlens), CONV_WIDTH - 1, cc), dtype=np.float32), dtype)
    dense_T = seqlens[0] if len(set(seqlens)) == 1 else 0
    return PrefillInputs(name, shape, dtype, cu, dense_T, x, w, g, beta, s0, cs0, chunk_size, scale)


def adversarial_prefill(seed: int, shape: LayerShape, T: int, dtype: str = "f32", *,
                        chunk_size: int = 64, max_run: int = 512, n_symbols: int = 4,
                        name: str = "adversarial") -> PrefillInputs:
    """Token rows drawn from a small alphabet in long runs, so that (after the
    conv warm-up of each run) keys repeat exactly; beta near 1, decay near 1."""
    cc = shape.conv_channels
    rows = _rng(seed, "symbols").standard_normal((n_symbols, cc), dtype=np.float32)
    r = _rng(seed, "runs")
    ids = np.empty(T, dtype=np.int64)
    t = 0
    while t < T:
        n = int(r.integers(1, max_run + 1))
        ids[t:t + n] = int(r.integers(0, n_symbols))
        t += n
    x = _quant(rows[ids], dtype)
    w = (_rng(seed, "conv_w").standard_normal((cc, CONV_WIDTH)) * 0.5).astype(np.float32)
    beta = _rng(seed, "beta").uniform(0.9, 1.0, (T, shape.num_v_heads)).astype(np.float32)
    g = _rng(seed, "g").uniform(-0.01, 0.0, (T, shape.num_v_heads)).astype(np.float32)
    cu = np.array([0, T], dtype=np.int32)
    return PrefillInputs(name, shape, dtype, cu, T, x, w, g, beta, None, None, chunk_size, 1.0)


def varlen_lengths(seed: int, n: int = 16, lo: int = 128, hi: int = 8192) -> list:
    return [int(v) for v in _rng(seed, "seqlens").integers(lo, hi + 1, size=n)]


# ---- the five workloads ---------------------------------------------------

def tiny_fp32(seed: int = 0) -> PrefillInputs:
    """B=1, T=64 (one chunk), 2 q/k heads, 4 v heads, d=64, fp32, zero state."""
    return make_prefill(seed, TINY, [64], "f32", name="tiny-fp32-T64")


def prefill_4k_bf16(seed: int = 1) -> PrefillInputs:
    """B=1, T=4096, 16 q/k heads, 32 v heads, d=128, bf16 in, zero state."""
    return make_prefill(seed, QWEN35_4B, [4096], "bf16", name="qwen35-4b-prefill-T4096-bf16")


def adversarial_8k_fp32(seed: int = 3) -> PrefillInputs:
    """B=1, T=8192, 4-symbol runs up to 512, beta~U(0.9,1), g~U(-0.01,0), fp32."""
    return adversarial_prefill(seed, QWEN35_4B, 8192, "f32", name="adversarial-keys-T8192-fp32")


def varlen_bf16(seed: int = 4, n: int = 16) -> PrefillInputs:
    """16 sequences, lengths ~U{128..8192} packed, nonzero initial states ~N(0,0.02)."""
    return make_prefill(seed, QWEN35_4B, varlen_lengths(seed, n), "bf16", state0_std=0.02,
                        name="varlen-16seq-bf16")


@dataclasses.dataclass
class DecodeInputs:
    """Batched one-token decode: a pool of ``pool`` input sets cycled over steps."""

    name: str
    shape: LayerShape
    dtype: str
    batch: int
    pool: int
    x: np.ndarray             # [pool][B][C_conv] fp32 (dtype-representable)
    g: np.ndarray             # [pool][B][H_v] fp32
    beta: np.ndarray          # [pool][B][H_v] fp32
    conv_w: np.ndarray        # [C_conv][W] fp32
    conv_state0: np.ndarray   # [B][W-1][C_conv] (dtype-representable)
    state0: np.ndarray        # [B][H_v][d_k][d_v] fp32
    scale: float = 1.0


def make_decode(seed: int, shape: LayerShape, batch: int, dtype: str, *, pool: int = 16,
                state_std: float = 0.02, name: str = "custom-decode") -> DecodeInputs:
    cc = shape.conv_channels
    x = _quant(_rng(seed, "x").standard_normal((pool, batch, cc), dtype=np.float32), dtype)
    g, beta = _gates(seed, pool * batch, shape.num_v_heads)
    g = g.reshape(pool, batch, -1)
    beta = beta.reshape(pool, batch, -1)
    w = (_rng(seed, "conv_w").standard_normal((cc, CONV_WIDTH)) * 0.5).astype(np.float32)
    cs0 = _quant(_rng(seed, "conv_state0").standard_normal((batch, CONV_WIDTH - 1, cc), dtype=np.float32), dtype)
    s0 = (_rng(seed, "state0").standard_normal(
        (batch, shape.num_v_heads, shape.head_dim_k, shape.head_dim_v), dtype=np.float32)
        * np.float32(state_std)).astype(np.float32)
    return DecodeInputs(name, shape, dtype, batch, pool, x, g, beta, w, cs0, s0)


def decode_b64_bf16(seed: int = 2) -> DecodeInputs:
    """B=64 sequences, 32 v heads, fp32 state ~N(0,0.02), bf16 projections, pool of 16 input sets."""
    return make_decode(seed, QWEN35_4B, 64, "bf16", name="qwen35-4b-decode-B64-bf16")


def split_qkv(y: np.ndarray, shape: LayerShape):
    """Views of the conv output [N][C_conv] as q [N][H_k][d_k], k [N][H_k][d_k], v [N][H_v][d_v]."""
    n = y.shape[0]
    a = shape.num_qk_heads * shape.head_dim_k
    q = y[:, :a].reshape(n, shape.num_qk_heads, shape.head_dim_k)
    k = y[:, a:2 * a].reshape(n, shape.num_qk_heads, shape.head_dim_k)
    v = y[:, 2 * a:].reshape(n, shape.num_v_heads, shape.head_dim_v)
    return q, k, v


def gate_inputs(seed: int, n_tok: int, hv: int, dv: int, dtype: str):
    """The gated norm's other inputs: the gate projection z ~ N(0, 1) in the
    input dtype [n_tok][hv][dv], and an fp32 weight [dv] ~ 1 + N(0, 0.1)."""
    r = _rng(seed, "gate")
    z = _quant(r.normal(size=(n_tok, hv, dv)).astype(np.float32), dtype)
    w = (1.0 + 0.1 * r.normal(size=dv)).astype(np.float32)
    return z, w


def gating_inputs(seed: int, n_tok: int, hv: int, dtype: str):
    """The gates' raw inputs: the decay and beta projections a, b ~ N(0, 1)
    as the two column blocks of one [n_tok][2 hv] projection output in the
    input dtype, and fp32 per-head A_log ~ U(-1, 1.5) and dt_bias ~ N(0, 0.5)."""
    r = _rng(seed, "gating")
    ab = _quant(r.normal(size=(n_tok, 2 * hv)).astype(np.float32), dtype)
    A_log = r.uniform(-1.0, 1.5, size=hv).astype(np.float32)
    dt_bias = (0.5 * r.normal(size=hv)).astype(np.float32)
    return ab, A_log, dt_bias
