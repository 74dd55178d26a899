"""Thin ctypes binding of libgdn (include/gdn.h).

Argument marshalling only: every step of the layer runs in the library's
HIP kernels.  Tensors are torch CUDA (HIP) tensors used for device memory;
the binding passes their data pointers and the current stream.  If
libgdn.so is missing this module raises at import -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

GDN_OK = 0
GDN_F32 = 0
GDN_BF16 = 1
GDN_QK_L2NORM = 1
GDN_HEADS_TILED = 2
OP_PREFILL = 0
OP_DECODE = 1

STATUS_NAMES = {0: "GDN_OK", 1: "GDN_ERR_INVALID_ARG", 2: "GDN_ERR_UNSUPPORTED", 3: "GDN_ERR_WORKSPACE",
                4: "GDN_ERR_HIP", 5: "GDN_ERR_NONFINITE"}

EXPORTED = ["gdn_status_string", "gdn_last_error", "gdn_version", "gdn_validate_dims", "gdn_validate", "gdn_conv1d",
            "gdn_prefill_workspace_size", "gdn_prefill_chunked", "gdn_prefill_chunked_noalloc", "gdn_prefill_prepare",
            "gdn_prefill_scan",
            "gdn_prefill_conv_prepare", "gdn_prefill_conv_chunked", "gdn_decode_step", "gdn_decode_conv_step",
            "gdn_gated_rmsnorm", "gdn_gating", "gdn_prefill_conv_gated", "gdn_decode_conv_gated_step",
            "gdn_snapshot_push", "gdn_snapshot_restore", "gdn_prefill_scan_gated_norm",
            "gdn_prefill_chunked_gated_norm"]


class GdnDims(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32), ("total_tokens", ctypes.c_int32), ("seqlen", ctypes.c_int32),
        ("num_qk_heads", ctypes.c_int32), ("num_v_heads", ctypes.c_int32),
        ("head_dim_k", ctypes.c_int32), ("head_dim_v", ctypes.c_int32), ("chunk_size", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("flags", ctypes.c_uint32), ("scale", ctypes.c_float),
        ("reserved", ctypes.c_int32),
        ("stride_q", ctypes.c_int64), ("stride_k", ctypes.c_int64), ("stride_v", ctypes.c_int64),
    ]


class GdnGateInputs(ctypes.Structure):
    _fields_ = [("a", ctypes.c_void_p), ("stride_a", ctypes.c_int64), ("b", ctypes.c_void_p),
                ("stride_b", ctypes.c_int64), ("A_log", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p)]


class GdnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m linear_attention_delta_amd.build` "
                          "(or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    D = ctypes.POINTER(GdnDims)
    GI = ctypes.POINTER(GdnGateInputs)
    sig = {
        "gdn_status_string": ([i32], ctypes.c_char_p),
        "gdn_last_error": ([], ctypes.c_char_p),
        "gdn_version": ([], ctypes.c_char_p),
        "gdn_validate_dims": ([D, i32], i32),
        "gdn_validate": ([D, i32, ctypes.POINTER(P), i32, i64], i32),
        "gdn_conv1d": ([i32, i32, i32, P, i32, i32, i32, P, i64, P, P, P, i32, P, i64, P], i32),
        "gdn_prefill_workspace_size": ([D], sz),
        "gdn_prefill_chunked": ([D, P, P, P, P, P, P, P, P, P, P, sz, P], i32),
        "gdn_prefill_chunked_noalloc": ([D, P, P, P, P, P, P, P, P, P, P], i32),
        "gdn_prefill_prepare": ([D, P, P, P, P, P, P, sz, P], i32),
        "gdn_prefill_scan": ([D, P, P, P, P, P, P, P, P, P, P, sz, P], i32),
        "gdn_prefill_conv_prepare": ([D, i32, P, i64, P, P, P, P, P, P, P, i64, P, sz, P], i32),
        "gdn_prefill_conv_chunked": ([D, i32, P, i64, P, P, P, P, P, P, P, P, i64, P, P, P, sz, P], i32),
        "gdn_decode_step": ([D, P, P, P, P, P, P, i32, P, P, P], i32),
        "gdn_decode_conv_step": ([D, i32, P, i64, P, P, P, P, P, P, i32, P, P, P], i32),
        "gdn_gated_rmsnorm": ([i32, i32, i32, i32, P, i64, P, i64, P, ctypes.c_float, P, i64, P], i32),
        "gdn_gating": ([i32, i32, i32, P, i64, P, i64, P, P, P, P, P], i32),
        "gdn_prefill_conv_gated": ([D, GI, i32, P, i64, P, P, P, P, P, P, i64, P, P, P, sz, P], i32),
        "gdn_decode_conv_gated_step": ([D, GI, i32, P, i64, P, P, P, P, i32, P, P, P], i32),
        "gdn_snapshot_push": ([i32, P, i32, i64, P, i64, P, i32, P, P, P, P], i32),
        "gdn_prefill_scan_gated_norm": ([D, P, P, P, P, P, P, P, P, i64, P, ctypes.c_float, P, P, P, sz, P], i32),
        "gdn_prefill_chunked_gated_norm": ([D, P, P, P, P, P, P, P, P, i64, P, ctypes.c_float, P, P, P, sz, P], i32),
        "gdn_snapshot_restore": ([i32, P, i32, i64, P, i64, P, i32, P, P, i32, P], i32),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    return lib


lib = _load()


def last_error() -> str:
    return lib.gdn_last_error().decode()


def _check(status: int):
    if status != GDN_OK:
        raise GdnError(status, last_error())


def make_dims(*, num_seqs, total_tokens, seqlen, num_qk_heads, num_v_heads, head_dim_k, head_dim_v,
              chunk_size=64, dtype=GDN_BF16, l2norm=True, heads_tiled=False, scale=1.0,
              stride_q=0, stride_k=0, stride_v=0) -> GdnDims:
    flags = (GDN_QK_L2NORM if l2norm else 0) | (GDN_HEADS_TILED if heads_tiled else 0)
    return GdnDims(num_seqs, total_tokens, seqlen, num_qk_heads, num_v_heads, head_dim_k, head_dim_v,
                   chunk_size, dtype, flags, scale, 0, stride_q, stride_k, stride_v)


def validate_dims(d: GdnDims, op: int) -> int:
    return int(lib.gdn_validate_dims(ctypes.byref(d), op))


def validate(d: GdnDims, op: int, ptrs, extent: int) -> int:
    """Host-only check of a prefill (op 0) or decode (op 1) call's arguments:
    ptrs are integer addresses (or None) in the order gdn_validate lists."""
    arr = (ctypes.c_void_p * len(ptrs))(*[None if p is None else int(p) for p in ptrs])
    return int(lib.gdn_validate(ctypes.byref(d), op, arr, len(ptrs), int(extent)))


# ---- torch helpers (memory and streams only) -----------------------------

def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream=None) -> Optional[int]:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _keep_for_stream(stream, *tensors):
    """Tensors allocated here on the current stream but used by kernels queued
    on another `stream`: tell torch's caching allocator, so that a block
    dropped at return (the temporary workspace) is not handed out again
    before that stream's kernels are done with it."""
    if stream is None:
        return
    import torch
    if stream == torch.cuda.current_stream():
        return
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    if t.dtype == torch.float32:
        return GDN_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _row_stride(t) -> int:
    """Elements between consecutive tokens of a [N, H, d] (or [N, H*d]) view
    whose inner dims are packed."""
    return t.stride(0)


def conv1d(x, weight, *, cu_seqlens=None, seqlen=None, num_seqs=None, bias=None, conv_state=None,
           activation=True, out=None, stream=None):
    """Causal depthwise conv (+SiLU).  x [N_tok, C] (rows may be strided),
    weight fp32 [C, W].  Dense if seqlen is given (num_seqs = N_tok // seqlen),
    varlen if cu_seqlens (device int32 [N+1]) is given.  Returns y [N_tok, C]."""
    import torch
    n_tok, C = x.shape
    if out is None:
        out = torch.empty((n_tok, C), dtype=x.dtype, device=x.device)
    if cu_seqlens is not None:
        n_seq = cu_seqlens.numel() - 1
        sl = 0
    else:
        sl = int(seqlen if seqlen is not None else n_tok)
        n_seq = int(num_seqs if num_seqs is not None else (n_tok // sl if sl else 1))
    _check(lib.gdn_conv1d(n_seq, n_tok, sl, _ptr(cu_seqlens), C, weight.shape[1], _dtype_code(x),
                          _ptr(x), x.stride(0), _ptr(weight), _ptr(bias), _ptr(conv_state),
                          1 if activation else 0, _ptr(out), out.stride(0), _stream(stream)))
    _keep_for_stream(stream, out)
    return out


class Conv1d:
    """Bound convolution call: sizes, weight and stream fixed at construction,
    so that a loop of calls pays only the library call itself."""

    def __init__(self, x, weight, *, cu_seqlens=None, seqlen=None, num_seqs=None, bias=None,
                 activation=True, stride_y=None, stream=None):
        n_tok, C = x.shape
        if cu_seqlens is not None:
            n_seq, sl = cu_seqlens.numel() - 1, 0
        else:
            sl = int(seqlen if seqlen is not None else n_tok)
            n_seq = int(num_seqs if num_seqs is not None else (n_tok // sl if sl else 1))
        self.shape = (n_tok, C)
        self._fixed = (n_seq, n_tok, sl, _ptr(cu_seqlens), C, weight.shape[1], _dtype_code(x))
        self._w = (_ptr(weight), _ptr(bias))
        self._act = 1 if activation else 0
        self._stride_x = x.stride(0)
        self._stride_y = C if stride_y is None else stride_y
        self._stream = _stream(stream)
        self._keep = (weight, bias, cu_seqlens)

    def __call__(self, x, y, conv_state=None):
        _check(lib.gdn_conv1d(*self._fixed, x.data_ptr(), self._stride_x, *self._w, _ptr(conv_state),
                              self._act, y.data_ptr(), self._stride_y, self._stream))
        return y


def _dims_for(q, k, v, *, num_seqs, seqlen, chunk_size, l2norm, heads_tiled, scale):
    n_tok, hk, dk = q.shape
    _, hv, dv = v.shape
    return make_dims(num_seqs=num_seqs, total_tokens=n_tok, seqlen=seqlen, num_qk_heads=hk, num_v_heads=hv,
                     head_dim_k=dk, head_dim_v=dv, chunk_size=chunk_size, dtype=_dtype_code(q),
                     l2norm=l2norm, heads_tiled=heads_tiled, scale=scale,
                     stride_q=_row_stride(q), stride_k=_row_stride(k), stride_v=_row_stride(v))


def workspace_size(d: GdnDims) -> int:
    n = int(lib.gdn_prefill_workspace_size(ctypes.byref(d)))
    if n == 0 and validate_dims(d, OP_PREFILL) != GDN_OK:
        raise GdnError(validate_dims(d, OP_PREFILL), last_error())
    return n


def alloc_workspace(d: GdnDims, device="cuda"):
    import torch
    n = workspace_size(d)
    return torch.empty(max(n, 256) // 4 + 64, dtype=torch.int32, device=device)  # 256-aligned by torch


class Prefill:
    """Bound prefill problem: dims + workspace, reusable across calls."""

    def __init__(self, q, k, v, *, cu_seqlens=None, seqlen=None, num_seqs=None, chunk_size=64,
                 l2norm=True, heads_tiled=False, scale=1.0, workspace=None):
        n_tok = q.shape[0]
        if cu_seqlens is not None:
            num_seqs = cu_seqlens.numel() - 1
            seqlen = 0
        else:
            seqlen = int(seqlen if seqlen is not None else n_tok)
            num_seqs = int(num_seqs if num_seqs is not None else (n_tok // seqlen if seqlen else 1))
        self.dims = _dims_for(q, k, v, num_seqs=num_seqs, seqlen=seqlen, chunk_size=chunk_size,
                              l2norm=l2norm, heads_tiled=heads_tiled, scale=scale)
        self.cu_seqlens = cu_seqlens
        self.ws = workspace if workspace is not None else alloc_workspace(self.dims, q.device)
        self.ws_bytes = self.ws.numel() * self.ws.element_size()

    def prepare(self, q, k, g, beta, stream=None):
        _check(lib.gdn_prefill_prepare(ctypes.byref(self.dims), _ptr(q), _ptr(k), _ptr(g), _ptr(beta),
                                       _ptr(self.cu_seqlens), _ptr(self.ws), self.ws_bytes, _stream(stream)))

    def scan(self, q, k, v, g, beta, o, state_in=None, state_out=None, stream=None):
        _check(lib.gdn_prefill_scan(ctypes.byref(self.dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                    _ptr(state_in), _ptr(self.cu_seqlens), _ptr(o), _ptr(state_out),
                                    _ptr(self.ws), self.ws_bytes, _stream(stream)))

    def __call__(self, q, k, v, g, beta, o, state_in=None, state_out=None, stream=None):
        _check(lib.gdn_prefill_chunked(ctypes.byref(self.dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                       _ptr(state_in), _ptr(self.cu_seqlens), _ptr(o), _ptr(state_out),
                                       _ptr(self.ws), self.ws_bytes, _stream(stream)))

    def gated_norm(self, q, k, v, g, beta, z, norm_weight, y, state_in=None, state_out=None, eps=1e-6,
                   stream=None):
        """The prefill with the gated norm fused (gdn_prefill_chunked_gated_norm):
        y [N_tok, H_v, d_v] = weight * o / rms(o) * silu(z) instead of o."""
        _check(lib.gdn_prefill_chunked_gated_norm(
            ctypes.byref(self.dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_in),
            _ptr(self.cu_seqlens), _ptr(z), _row_stride(z), _ptr(norm_weight), ctypes.c_float(eps), _ptr(y),
            _ptr(state_out), _ptr(self.ws), self.ws_bytes, _stream(stream)))

    def scan_gated_norm(self, q, k, v, g, beta, z, norm_weight, y, state_in=None, state_out=None, eps=1e-6,
                        stream=None):
        """The carry half with the gated norm fused (gdn_prefill_scan_gated_norm)."""
        _check(lib.gdn_prefill_scan_gated_norm(
            ctypes.byref(self.dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_in),
            _ptr(self.cu_seqlens), _ptr(z), _row_stride(z), _ptr(norm_weight), ctypes.c_float(eps), _ptr(y),
            _ptr(state_out), _ptr(self.ws), self.ws_bytes, _stream(stream)))


def prefill(q, k, v, g, beta, *, state_in=None, cu_seqlens=None, seqlen=None, num_seqs=None, chunk_size=64,
            l2norm=True, heads_tiled=False, scale=1.0, want_state=True, out=None, state_out=None, stream=None):
    """Chunked prefill.  q, k [N_tok, H_k, d_k]; v [N_tok, H_v, d_v] (token
    rows may be strided views); g, beta fp32 [N_tok, H_v].  Returns (o, state)."""
    import torch
    p = Prefill(q, k, v, cu_seqlens=cu_seqlens, seqlen=seqlen, num_seqs=num_seqs, chunk_size=chunk_size,
                l2norm=l2norm, heads_tiled=heads_tiled, scale=scale)
    n_tok, hv, dv = v.shape
    if out is None:
        out = torch.empty((n_tok, hv, dv), dtype=q.dtype, device=q.device)
    if state_out is None and want_state:
        state_out = torch.empty((p.dims.num_seqs, hv, q.shape[2], dv), dtype=torch.float32, device=q.device)
    p(q, k, v, g, beta, out, state_in, state_out, stream)
    _keep_for_stream(stream, p.ws, out, state_out)
    return out, state_out


def prefill_noalloc(q, k, v, g, beta, o, state_out, *, state_in=None, cu_seqlens=None, seqlen=None,
                    num_seqs=None, chunk_size=64, l2norm=True, heads_tiled=False, scale=1.0, stream=None):
    """gdn_prefill_chunked_noalloc: the chunked prefill with the library's own
    device workspace (no workspace argument).  o and state_out are the
    caller's; nothing is allocated here or in the library."""
    n_tok = q.shape[0]
    if cu_seqlens is not None:
        num_seqs, seqlen = cu_seqlens.numel() - 1, 0
    else:
        seqlen = int(seqlen if seqlen is not None else n_tok)
        num_seqs = int(num_seqs if num_seqs is not None else (n_tok // seqlen if seqlen else 1))
    d = _dims_for(q, k, v, num_seqs=num_seqs, seqlen=seqlen, chunk_size=chunk_size, l2norm=l2norm,
                  heads_tiled=heads_tiled, scale=scale)
    _check(lib.gdn_prefill_chunked_noalloc(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                           _ptr(state_in), _ptr(cu_seqlens), _ptr(o), _ptr(state_out),
                                           _stream(stream)))
    return o, state_out


class ConvPrefill:
    """Bound prefill from raw rows: x [N_tok, C_conv] (channels [q | k | v],
    rows may be strided) -> y = SiLU(conv(x)) [N_tok, C_conv] -> o, state.
    Dims + workspace, reusable across calls."""

    def __init__(self, x, weight, *, num_qk_heads, num_v_heads, head_dim_k, head_dim_v, y_stride=None,
                 cu_seqlens=None, seqlen=None, num_seqs=None, chunk_size=64, l2norm=True, heads_tiled=False,
                 scale=1.0, bias=None, workspace=None):
        n_tok, cc = x.shape
        if cc != 2 * num_qk_heads * head_dim_k + num_v_heads * head_dim_v:
            raise ValueError("x must have 2 H_k d_k + H_v d_v channels")
        if cu_seqlens is not None:
            num_seqs = cu_seqlens.numel() - 1
            seqlen = 0
        else:
            seqlen = int(seqlen if seqlen is not None else n_tok)
            num_seqs = int(num_seqs if num_seqs is not None else (n_tok // seqlen if seqlen else 1))
        ys = int(y_stride if y_stride is not None else cc)
        self.dims = make_dims(num_seqs=num_seqs, total_tokens=n_tok, seqlen=seqlen, num_qk_heads=num_qk_heads,
                              num_v_heads=num_v_heads, head_dim_k=head_dim_k, head_dim_v=head_dim_v,
                              chunk_size=chunk_size, dtype=_dtype_code(x), l2norm=l2norm, heads_tiled=heads_tiled,
                              scale=scale, stride_q=ys, stride_k=ys, stride_v=ys)
        self.y_stride = ys
        self.weight, self.bias, self.cu_seqlens = weight, bias, cu_seqlens
        self.width = weight.shape[1]
        self.ws = workspace if workspace is not None else alloc_workspace(self.dims, x.device)
        self.ws_bytes = self.ws.numel() * self.ws.element_size()

    def views(self, y):
        """q, k, v column views of y."""
        d = self.dims
        a = d.num_qk_heads * d.head_dim_k
        n = y.shape[0]
        return (y[:, :a].view(n, d.num_qk_heads, d.head_dim_k), y[:, a:2 * a].view(n, d.num_qk_heads, d.head_dim_k),
                y[:, 2 * a:2 * a + d.num_v_heads * d.head_dim_v].view(n, d.num_v_heads, d.head_dim_v))

    def conv_prepare(self, x, y, g, beta, conv_state=None, stream=None):
        _check(lib.gdn_prefill_conv_prepare(ctypes.byref(self.dims), self.width, _ptr(x), _row_stride(x),
                                            _ptr(self.weight), _ptr(self.bias), _ptr(conv_state), _ptr(g),
                                            _ptr(beta), _ptr(self.cu_seqlens), _ptr(y), self.y_stride,
                                            _ptr(self.ws), self.ws_bytes, _stream(stream)))

    def scan(self, y, g, beta, o, state_in=None, state_out=None, stream=None):
        q, k, v = self.views(y)
        _check(lib.gdn_prefill_scan(ctypes.byref(self.dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                    _ptr(state_in), _ptr(self.cu_seqlens), _ptr(o), _ptr(state_out),
                                    _ptr(self.ws), self.ws_bytes, _stream(stream)))

    def scan_gated_norm(self, y, g, beta, z, norm_weight, out, state_in=None, state_out=None, eps=1e-6,
                        stream=None):
        """The carry on the q, k, v column blocks of the conv output y, with
        the gated norm fused: out = weight * o / rms(o) * silu(z)."""
        q, k, v = self.views(y)
        _check(lib.gdn_prefill_scan_gated_norm(
            ctypes.byref(self.dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_in),
            _ptr(self.cu_seqlens), _ptr(z), _row_stride(z), _ptr(norm_weight), ctypes.c_float(eps), _ptr(out),
            _ptr(state_out), _ptr(self.ws), self.ws_bytes, _stream(stream)))

    def __call__(self, x, y, g, beta, o, state_in=None, state_out=None, conv_state=None, stream=None):
        _check(lib.gdn_prefill_conv_chunked(ctypes.byref(self.dims), self.width, _ptr(x), _row_stride(x),
                                            _ptr(self.weight), _ptr(self.bias), _ptr(conv_state), _ptr(g),
                                            _ptr(beta), _ptr(state_in), _ptr(self.cu_seqlens), _ptr(y),
                                            self.y_stride, _ptr(o), _ptr(state_out), _ptr(self.ws), self.ws_bytes,
                                            _stream(stream)))


def conv_prefill(x, weight, g, beta, *, num_qk_heads, num_v_heads, head_dim_k, head_dim_v, state_in=None,
                 conv_state=None, cu_seqlens=None, seqlen=None, num_seqs=None, chunk_size=64, l2norm=True,
                 heads_tiled=False, scale=1.0, bias=None, want_state=True, stream=None):
    """Prefill from raw rows x [N_tok, 2 H_k d_k + H_v d_v] through the conv
    (+SiLU) and the chunked scan in one library call.  conv_state, if given,
    is advanced in place.  Returns (y, o, state)."""
    import torch
    p = ConvPrefill(x, weight, num_qk_heads=num_qk_heads, num_v_heads=num_v_heads, head_dim_k=head_dim_k,
                    head_dim_v=head_dim_v, cu_seqlens=cu_seqlens, seqlen=seqlen, num_seqs=num_seqs,
                    chunk_size=chunk_size, l2norm=l2norm, heads_tiled=heads_tiled, scale=scale, bias=bias)
    n_tok = x.shape[0]
    y = torch.empty((n_tok, x.shape[1]), dtype=x.dtype, device=x.device)
    o = torch.empty((n_tok, num_v_heads, head_dim_v), dtype=x.dtype, device=x.device)
    st = torch.empty((p.dims.num_seqs, num_v_heads, head_dim_k, head_dim_v), dtype=torch.float32,
                     device=x.device) if want_state else None
    p(x, y, g, beta, o, state_in, st, conv_state, stream)
    _keep_for_stream(stream, p.ws, y, o, st)
    return y, o, st


class Decode:
    """Bound decode step: dims and stream fixed at construction (q, k, v of
    the given shapes and token strides), reusable across steps and state
    pools of num_slots slots."""

    def __init__(self, q, k, v, *, num_slots, l2norm=True, heads_tiled=False, scale=1.0, stream=None):
        self.dims = _dims_for(q, k, v, num_seqs=q.shape[0], seqlen=1, chunk_size=64, l2norm=l2norm,
                              heads_tiled=heads_tiled, scale=scale)
        self._d = ctypes.byref(self.dims)
        self.num_slots = int(num_slots)
        self._stream = _stream(stream)

    def __call__(self, q, k, v, g, beta, state, out, state_slots=None):
        _check(lib.gdn_decode_step(self._d, q.data_ptr(), k.data_ptr(), v.data_ptr(), g.data_ptr(),
                                   beta.data_ptr(), state.data_ptr(), self.num_slots, _ptr(state_slots),
                                   out.data_ptr(), self._stream))
        return out


def decode_step(q, k, v, g, beta, state, *, state_slots=None, l2norm=True, heads_tiled=False, scale=1.0,
                out=None, stream=None):
    """One token per sequence.  q, k [B, H_k, d_k]; v [B, H_v, d_v]; g, beta
    fp32 [B, H_v]; state fp32 [slots, H_v, d_k, d_v] updated in place."""
    import torch
    B, hk, dk = q.shape
    _, hv, dv = v.shape
    d = _dims_for(q, k, v, num_seqs=B, seqlen=1, chunk_size=64, l2norm=l2norm, heads_tiled=heads_tiled,
                  scale=scale)
    if out is None:
        out = torch.empty((B, hv, dv), dtype=q.dtype, device=q.device)
    _check(lib.gdn_decode_step(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state),
                               state.shape[0], _ptr(state_slots), _ptr(out), _stream(stream)))
    _keep_for_stream(stream, out)
    return out


def _decode_conv_dims(x, *, num_qk_heads, num_v_heads, head_dim_k, head_dim_v, l2norm, heads_tiled, scale):
    B, cc = x.shape
    if cc != 2 * num_qk_heads * head_dim_k + num_v_heads * head_dim_v:
        raise ValueError("x must have 2 H_k d_k + H_v d_v channels")
    return make_dims(num_seqs=B, total_tokens=B, seqlen=1, num_qk_heads=num_qk_heads, num_v_heads=num_v_heads,
                     head_dim_k=head_dim_k, head_dim_v=head_dim_v, chunk_size=64, dtype=_dtype_code(x),
                     l2norm=l2norm, heads_tiled=heads_tiled, scale=scale)


class DecodeConv:
    """Bound decode step from raw rows x [B, C_conv] (channels [q | k | v],
    rows may be strided): conv step + SiLU and the recurrent step in one
    library call.  Sizes, conv weights and stream fixed at construction."""

    def __init__(self, x, weight, *, num_qk_heads, num_v_heads, head_dim_k, head_dim_v, num_slots, bias=None,
                 l2norm=True, heads_tiled=False, scale=1.0, stream=None):
        self.dims = _decode_conv_dims(x, num_qk_heads=num_qk_heads, num_v_heads=num_v_heads,
                                      head_dim_k=head_dim_k, head_dim_v=head_dim_v, l2norm=l2norm,
                                      heads_tiled=heads_tiled, scale=scale)
        self._d = ctypes.byref(self.dims)
        self.width = weight.shape[1]
        self._w = (_ptr(weight), _ptr(bias))
        self._keep = (weight, bias)
        self.num_slots = int(num_slots)
        self._stream = _stream(stream)

    def __call__(self, x, g, beta, state, conv_state, out, state_slots=None):
        _check(lib.gdn_decode_conv_step(self._d, self.width, x.data_ptr(), x.stride(0), *self._w,
                                        conv_state.data_ptr(), g.data_ptr(), beta.data_ptr(), state.data_ptr(),
                                        self.num_slots, _ptr(state_slots), out.data_ptr(), self._stream))
        return out


def decode_conv_step(x, weight, g, beta, state, conv_state, *, num_qk_heads, num_v_heads, head_dim_k, head_dim_v,
                     bias=None, state_slots=None, l2norm=True, heads_tiled=False, scale=1.0, out=None, stream=None):
    """One token per sequence from raw rows x [B, 2 H_k d_k + H_v d_v]; weight
    fp32 [C_conv, W]; conv_state [slots, W-1, C_conv] and state fp32
    [slots, H_v, d_k, d_v] are advanced in place.  Returns o [B, H_v, d_v]."""
    import torch
    d = _decode_conv_dims(x, num_qk_heads=num_qk_heads, num_v_heads=num_v_heads, head_dim_k=head_dim_k,
                          head_dim_v=head_dim_v, l2norm=l2norm, heads_tiled=heads_tiled, scale=scale)
    if out is None:
        out = torch.empty((x.shape[0], num_v_heads, head_dim_v), dtype=x.dtype, device=x.device)
    _check(lib.gdn_decode_conv_step(ctypes.byref(d), weight.shape[1], _ptr(x), x.stride(0), _ptr(weight), _ptr(bias),
                                    _ptr(conv_state), _ptr(g), _ptr(beta), _ptr(state), state.shape[0],
                                    _ptr(state_slots), _ptr(out), _stream(stream)))
    _keep_for_stream(stream, out)
    return out


class GatedNorm:
    """Bound gated-norm call: sizes, strides, weight and stream fixed at
    construction from example o, z and y views, so that a loop of calls pays
    only the library call itself."""

    def __init__(self, o, z, weight, *, y=None, eps=1e-6, stream=None):
        n, h, d = o.shape
        ys = _row_stride(y) if y is not None else h * d
        self._fixed = (n, h, d, _dtype_code(o))
        self._strides = (_row_stride(o), _row_stride(z), ys)
        self._w = (_ptr(weight), ctypes.c_float(eps))
        self._keep = weight
        self._stream = _stream(stream)

    def __call__(self, o, z, y):
        so, sz, sy = self._strides
        _check(lib.gdn_gated_rmsnorm(*self._fixed, o.data_ptr(), so, z.data_ptr(), sz, *self._w, y.data_ptr(), sy,
                                     self._stream))
        return y


def gated_rmsnorm(o, z, weight, *, eps=1e-6, out=None, stream=None):
    """Gated RMS norm of the layer output: o, z [N_tok, H_v, d_v] (token rows
    may be strided views), weight fp32 [d_v].  out may be o (in place).
    Returns y = weight * o / rms(o) * silu(z) per (token, head)."""
    import torch
    n, h, d = o.shape
    if out is None:
        out = torch.empty((n, h, d), dtype=o.dtype, device=o.device)
    _check(lib.gdn_gated_rmsnorm(n, h, d, _dtype_code(o), _ptr(o), _row_stride(o), _ptr(z), _row_stride(z),
                                 _ptr(weight), float(eps), _ptr(out), _row_stride(out), _stream(stream)))
    _keep_for_stream(stream, out)
    return out


class Gating:
    """Bound gating call: sizes, strides, parameters and stream fixed at
    construction from example a, b views [N_tok, H_v]."""

    def __init__(self, a, b, A_log, dt_bias, *, stream=None):
        n, h = a.shape
        self._fixed = (n, h, _dtype_code(a))
        self._strides = (a.stride(0), b.stride(0))
        self._p = (_ptr(A_log), _ptr(dt_bias))
        self._keep = (A_log, dt_bias)
        self._stream = _stream(stream)

    def __call__(self, a, b, g, beta):
        sa, sb = self._strides
        _check(lib.gdn_gating(*self._fixed, a.data_ptr(), sa, b.data_ptr(), sb, *self._p, g.data_ptr(),
                              beta.data_ptr(), self._stream))
        return g, beta


def gating(a, b, A_log, dt_bias, *, g=None, beta=None, stream=None):
    """g = -exp(A_log) softplus(a + dt_bias), beta = sigmoid(b) from the raw
    projections a, b [N_tok, H_v] (rows may be strided); A_log, dt_bias fp32
    [H_v].  Returns (g, beta), fp32 [N_tok, H_v]."""
    import torch
    n, h = a.shape
    if g is None:
        g = torch.empty((n, h), dtype=torch.float32, device=a.device)
    if beta is None:
        beta = torch.empty((n, h), dtype=torch.float32, device=a.device)
    Gating(a, b, A_log, dt_bias, stream=stream)(a, b, g, beta)
    _keep_for_stream(stream, g, beta)
    return g, beta


def gate_inputs(a, b, A_log, dt_bias) -> GdnGateInputs:
    """The gates' raw inputs for the gated calls: a, b [N_tok, H_v] views in
    the problem's dtype (rows may be strided), A_log, dt_bias fp32 [H_v]."""
    return GdnGateInputs(_ptr(a), a.stride(0), _ptr(b), b.stride(0), _ptr(A_log), _ptr(dt_bias))


def conv_prefill_gated(p: "ConvPrefill", x, y, gates: GdnGateInputs, o, *, state_in=None, state_out=None,
                       conv_state=None, stream=None):
    """The whole prefill of a bound ConvPrefill problem with the gates computed
    in the prepare from their raw projections (gdn_prefill_conv_gated)."""
    _check(lib.gdn_prefill_conv_gated(ctypes.byref(p.dims), ctypes.byref(gates), p.width, _ptr(x), _row_stride(x),
                                      _ptr(p.weight), _ptr(p.bias), _ptr(conv_state), _ptr(state_in),
                                      _ptr(p.cu_seqlens), _ptr(y), p.y_stride, _ptr(o), _ptr(state_out), _ptr(p.ws),
                                      p.ws_bytes, _stream(stream)))


def decode_conv_gated_step(step: "DecodeConv", x, gates: GdnGateInputs, state, conv_state, out, state_slots=None):
    """One decode step of a bound DecodeConv problem with the gates computed
    in the step's kernel from their raw projections."""
    _check(lib.gdn_decode_conv_gated_step(step._d, ctypes.byref(gates), step.width, x.data_ptr(), x.stride(0),
                                          *step._w, conv_state.data_ptr(), state.data_ptr(), step.num_slots,
                                          _ptr(state_slots), out.data_ptr(), step._stream))
    return out


class SnapshotRing:
    """A device ring of `ring_len` snapshots of the live state (and conv
    window) slots of one layer, for num_seqs sequences: push() copies the
    slots into entry (*head mod ring_len) and advances the device counter
    `head`; restore(e) copies entry e back.  Memory is torch's; the copies
    are the library's kernels."""

    def __init__(self, state, conv_state, num_seqs, ring_len, *, slots=None):
        import torch
        self.num_slots = state.shape[0]
        self.state_elems = state[0].numel()
        self.window_bytes = 0 if conv_state is None else conv_state[0].numel() * conv_state.element_size()
        self.num_seqs, self.ring_len, self.slots = int(num_seqs), int(ring_len), slots
        dev = state.device
        self.ring_state = torch.empty((ring_len, num_seqs) + tuple(state.shape[1:]), dtype=torch.float32, device=dev)
        self.ring_window = None if conv_state is None else torch.empty(
            (ring_len, num_seqs) + tuple(conv_state.shape[1:]), dtype=conv_state.dtype, device=dev)
        self.head = torch.zeros(1, dtype=torch.int32, device=dev)

    def push(self, state, conv_state, stream=None):
        _check(lib.gdn_snapshot_push(self.num_seqs, _ptr(self.slots), self.num_slots, self.state_elems, _ptr(state),
                                     self.window_bytes, _ptr(conv_state), self.ring_len, _ptr(self.ring_state),
                                     _ptr(self.ring_window), _ptr(self.head), _stream(stream)))

    def restore(self, entry, state, conv_state, stream=None):
        _check(lib.gdn_snapshot_restore(self.num_seqs, _ptr(self.slots), self.num_slots, self.state_elems,
                                        _ptr(state), self.window_bytes, _ptr(conv_state), self.ring_len,
                                        _ptr(self.ring_state), _ptr(self.ring_window), int(entry), _stream(stream)))
