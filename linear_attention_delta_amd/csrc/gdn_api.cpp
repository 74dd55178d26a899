// gdn_api.cpp -- the C ABI of libgdn (declared in include/gdn.h): argument
// validation, workspace carving and kernel dispatch.  Every check runs on
// the host before any HIP call, so an invalid call queues nothing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "gdn.h"
#include "gdn_internal.h"

namespace {

thread_local std::string g_last_error;

gdn_status fail(gdn_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
gdn_status fail(gdn_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

gdn_status ok() {
  g_last_error.clear();
  return GDN_OK;
}

// Read on every call, so a process can switch the probe on and off.
bool debug_enabled() {
  const char* e = getenv("GDN_DEBUG");
  return e && e[0] == '1';
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t elem_size(int dtype) { return dtype == GDN_BF16 ? 2 : 4; }

constexpr int64_t kMaxTokens = 1LL << 30;

gdn_status check_dims(const gdn_dims* d, int op) {
  if (!d) return fail(GDN_ERR_INVALID_ARG, "dims is NULL");
  if (d->reserved != 0) return fail(GDN_ERR_INVALID_ARG, "dims.reserved must be 0");
  if (d->num_seqs < 1) return fail(GDN_ERR_INVALID_ARG, "num_seqs must be >= 1 (got %d)", d->num_seqs);
  if (d->total_tokens < 0 || d->total_tokens > kMaxTokens)
    return fail(GDN_ERR_INVALID_ARG, "total_tokens out of range (got %d)", d->total_tokens);
  if (d->seqlen < 0) return fail(GDN_ERR_INVALID_ARG, "seqlen must be >= 0 (got %d)", d->seqlen);
  if (d->seqlen > 0 && (int64_t)d->num_seqs * d->seqlen != d->total_tokens)
    return fail(GDN_ERR_INVALID_ARG, "dense layout needs total_tokens == num_seqs * seqlen (%d != %d * %d)",
                d->total_tokens, d->num_seqs, d->seqlen);
  if (d->num_qk_heads < 1) return fail(GDN_ERR_INVALID_ARG, "num_qk_heads must be >= 1");
  if (d->num_v_heads < d->num_qk_heads || d->num_v_heads % d->num_qk_heads != 0)
    return fail(GDN_ERR_INVALID_ARG, "num_v_heads (%d) must be a positive multiple of num_qk_heads (%d)",
                d->num_v_heads, d->num_qk_heads);
  if (d->num_v_heads > 4096) return fail(GDN_ERR_UNSUPPORTED, "num_v_heads > 4096");
  if (d->head_dim_k <= 0 || d->head_dim_v <= 0)
    return fail(GDN_ERR_INVALID_ARG, "head dims must be positive");
  if ((d->head_dim_k != 64 && d->head_dim_k != 128) || (d->head_dim_v != 64 && d->head_dim_v != 128))
    return fail(GDN_ERR_UNSUPPORTED, "head dims must be 64 or 128 (got d_k=%d, d_v=%d)", d->head_dim_k,
                d->head_dim_v);
  if (d->dtype != GDN_F32 && d->dtype != GDN_BF16) return fail(GDN_ERR_INVALID_ARG, "dtype must be GDN_F32 or GDN_BF16");
  if (d->flags & ~(uint32_t)(GDN_QK_L2NORM | GDN_HEADS_TILED))
    return fail(GDN_ERR_INVALID_ARG, "unknown flag bits 0x%x", d->flags);
  if (!std::isfinite(d->scale)) return fail(GDN_ERR_INVALID_ARG, "scale must be finite");
  const int64_t vec = d->dtype == GDN_BF16 ? 8 : 4;
  const int64_t qk_row = (int64_t)d->num_qk_heads * d->head_dim_k;
  const int64_t v_row = (int64_t)d->num_v_heads * d->head_dim_v;
  const int64_t sq = d->stride_q ? d->stride_q : qk_row;
  const int64_t sk = d->stride_k ? d->stride_k : qk_row;
  const int64_t sv = d->stride_v ? d->stride_v : v_row;
  if (sq < qk_row || sk < qk_row || sv < v_row)
    return fail(GDN_ERR_INVALID_ARG, "token strides must cover a whole row (q %lld, k %lld >= %lld; v %lld >= %lld)",
                (long long)sq, (long long)sk, (long long)qk_row, (long long)sv, (long long)v_row);
  if (sq % vec || sk % vec || sv % vec)
    return fail(GDN_ERR_INVALID_ARG, "token strides must be multiples of %lld elements", (long long)vec);
  if (sq > (1 << 24) || sk > (1 << 24) || sv > (1 << 24))
    return fail(GDN_ERR_UNSUPPORTED, "token strides above 2^24 elements are not supported");
  if (op == 0) {
    if (d->chunk_size != 16 && d->chunk_size != 32 && d->chunk_size != 64)
      return fail(GDN_ERR_UNSUPPORTED, "chunk_size must be 16, 32 or 64 (got %d)", d->chunk_size);
  } else if (op == 1) {
    if (d->seqlen != 1 || d->total_tokens != d->num_seqs)
      return fail(GDN_ERR_INVALID_ARG, "decode needs seqlen == 1 and total_tokens == num_seqs");
  } else {
    return fail(GDN_ERR_INVALID_ARG, "op must be 0 (prefill) or 1 (decode)");
  }
  return ok();
}

int64_t max_chunks(const gdn_dims* d) {
  const int64_t C = d->chunk_size;
  if (d->seqlen > 0) return (int64_t)d->num_seqs * ((d->seqlen + C - 1) / C);
  return (int64_t)d->total_tokens / C + d->num_seqs;
}

// Segment-parallel carry (bf16 operands, chunk 32 or 64): the library's
// choice of segment length, in chunks.  About one segment per compute unit
// for a single long sequence (the prefill then has 8 + (segments - 1) + 8
// dependent chunk steps instead of 64); for batches that already fill the
// GPU the segments grow so the extra carry of pass 1 stays small.
bool seg_enabled(const gdn_dims* d) {
  return d->dtype == GDN_BF16 && (d->chunk_size == 32 || d->chunk_size == 64);
}

int seg_len(const gdn_dims* d) {
  const int64_t units = max_chunks(d) * d->num_v_heads;
  return (int)std::max<int64_t>(8, (units + 255) / 256);
}

int64_t max_segs(const gdn_dims* d) {
  const int64_t L = seg_len(d);
  if (d->seqlen > 0) {
    const int64_t cps = (d->seqlen + d->chunk_size - 1) / d->chunk_size;
    return (int64_t)d->num_seqs * std::max<int64_t>(1, (cps + L - 1) / L);
  }
  return max_chunks(d) / L + d->num_seqs;
}

// Workspace: [chunk table (varlen only)] [Tt, P per chunk and v-head]
// [a, b, c, e^{gamma_last} per chunk and v-head], and on the segment path
// [segment table and dispatch order (varlen only)] [segment start states, fp32]
// [segment transitions, bf16]; each part 256-byte aligned.
struct WsLayout {
  size_t table_off, table_bytes, mats_off, mats_bytes, scal_off, scal_bytes;
  size_t segt_off, segt_bytes, sst_off, sst_bytes, phi_off, phi_bytes, total;
};

size_t align256(size_t n) { return (n + 255) / 256 * 256; }

WsLayout ws_layout(const gdn_dims* d) {
  WsLayout w;
  const size_t units = (size_t)max_chunks(d) * d->num_v_heads;
  const size_t C = d->chunk_size;
  w.table_off = 0;
  // varlen: chunk offsets [num_seqs + 1], and on the sequential carry its
  // dispatch order [num_seqs] (the segment path keeps its own below)
  w.table_bytes = d->seqlen > 0 ? 0 : align256((size_t)(d->num_seqs + 1 + (seg_enabled(d) ? 0 : d->num_seqs)) * 4);
  w.mats_off = w.table_bytes;
  w.mats_bytes = align256(units * 2 * C * C * elem_size(d->dtype));
  w.scal_off = w.mats_off + w.mats_bytes;
  w.scal_bytes = align256(units * gdn::kScalRows * C * 4);
  w.segt_off = w.scal_off + w.scal_bytes;
  w.segt_bytes = w.sst_bytes = w.phi_bytes = 0;
  if (seg_enabled(d)) {
    const size_t segs = (size_t)max_segs(d) * d->num_v_heads;
    // varlen: segment offsets [num_seqs + 1], then the dispatch order [max_segs]
    w.segt_bytes = d->seqlen > 0 ? 0 : align256((size_t)(d->num_seqs + 1 + max_segs(d)) * 4);
    w.sst_bytes = align256(segs * d->head_dim_k * d->head_dim_v * 4);
    w.phi_bytes = align256(segs * d->head_dim_k * d->head_dim_k * 2);
  }
  w.sst_off = w.segt_off + w.segt_bytes;
  w.phi_off = w.sst_off + w.sst_bytes;
  w.total = w.phi_off + w.phi_bytes;
  return w;
}

gdn::ScanArgs make_args(const gdn_dims* d) {
  gdn::ScanArgs a;
  memset(&a, 0, sizeof(a));
  a.num_seqs = d->num_seqs;
  a.total_tokens = d->total_tokens;
  a.seqlen = d->seqlen;
  a.hk = d->num_qk_heads;
  a.hv = d->num_v_heads;
  a.dk = d->head_dim_k;
  a.dv = d->head_dim_v;
  a.chunk = d->chunk_size;
  a.dtype = d->dtype;
  a.l2norm = (d->flags & GDN_QK_L2NORM) ? 1 : 0;
  a.tiled = (d->flags & GDN_HEADS_TILED) ? 1 : 0;
  a.scale = d->scale;
  a.stride_q = d->stride_q ? d->stride_q : (long)d->num_qk_heads * d->head_dim_k;
  a.stride_k = d->stride_k ? d->stride_k : (long)d->num_qk_heads * d->head_dim_k;
  a.stride_v = d->stride_v ? d->stride_v : (long)d->num_v_heads * d->head_dim_v;
  return a;
}

gdn_status hip_fail(hipError_t e, const char* what) {
  return fail(GDN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// ---- GDN_DEBUG probe: the count lives in a file-scope device variable (one
// per device).  A probe zeroes it, counts into it and reads it back, then
// synchronises its stream; probes from several host threads (on any
// streams) take turns under a mutex, so no probe sees another's count.
__device__ int g_nonfinite_count;
std::mutex g_debug_mu;

gdn_status debug_check(hipStream_t s, const char* what, const void* p, long n, int dtype) {
  if (!debug_enabled() || !p || n <= 0) return GDN_OK;
  std::lock_guard<std::mutex> lock(g_debug_mu);
  int* dcount = nullptr;
  hipError_t e = hipGetSymbolAddress(reinterpret_cast<void**>(&dcount), HIP_SYMBOL(g_nonfinite_count));
  if (e != hipSuccess) return hip_fail(e, "GDN_DEBUG symbol");
  int zero = 0, count = 0;
  if ((e = hipMemcpyAsync(dcount, &zero, sizeof(int), hipMemcpyHostToDevice, s)) != hipSuccess ||
      (e = gdn::launch_nonfinite_probe(p, n, dtype, dcount, s)) != hipSuccess ||
      (e = hipMemcpyAsync(&count, dcount, sizeof(int), hipMemcpyDeviceToHost, s)) != hipSuccess ||
      (e = hipStreamSynchronize(s)) != hipSuccess)
    return hip_fail(e, "GDN_DEBUG probe");
  if (count) return fail(GDN_ERR_NONFINITE, "GDN_DEBUG: %d non-finite values in %s", count, what);
  return GDN_OK;
}

// need_gb: g and beta are arrays (false where the gates come from the raw
// projections, checked by check_gates)
gdn_status check_scan_ptrs(const gdn_dims* d, const void* q, const void* k, const void* v, const float* g,
                           const float* beta, const int32_t* cu, bool need_qv, bool need_gb = true) {
  if (d->total_tokens > 0) {
    if (!k || (need_gb && (!g || !beta)) || (need_qv && (!q || !v)))
      return fail(GDN_ERR_INVALID_ARG, "q, k, v, g and beta must be non-NULL");
    if (!aligned(k, 16) || (need_qv && (!aligned(q, 16) || !aligned(v, 16))))
      return fail(GDN_ERR_INVALID_ARG, "q, k and v must be 16-byte aligned");
    if (need_gb && (!aligned(g, 4) || !aligned(beta, 4)))
      return fail(GDN_ERR_INVALID_ARG, "g and beta must be 4-byte aligned");
  }
  if (d->seqlen == 0 && (!cu || !aligned(cu, 4)))
    return fail(GDN_ERR_INVALID_ARG, "varlen (seqlen == 0) needs a 4-byte aligned cu_seqlens");
  return GDN_OK;
}

gdn_status check_gates(const gdn_dims* d, const gdn_gate_inputs* G) {
  if (!G) return fail(GDN_ERR_INVALID_ARG, "gates is NULL");
  if (G->stride_a < d->num_v_heads || G->stride_b < d->num_v_heads)
    return fail(GDN_ERR_INVALID_ARG, "gate strides must be >= num_v_heads (%d)", d->num_v_heads);
  if (!G->A_log || !G->dt_bias || !aligned(G->A_log, 4) || !aligned(G->dt_bias, 4))
    return fail(GDN_ERR_INVALID_ARG, "A_log and dt_bias must be non-NULL and 4-byte aligned");
  if (d->total_tokens > 0) {
    if (!G->a || !G->b) return fail(GDN_ERR_INVALID_ARG, "gate projections a and b must be non-NULL");
    if (!aligned(G->a, elem_size(d->dtype)) || !aligned(G->b, elem_size(d->dtype)))
      return fail(GDN_ERR_INVALID_ARG, "gate projections must be aligned to their element size");
  }
  return GDN_OK;
}

void set_gates(gdn::ScanArgs& a, const gdn_gate_inputs* G) {
  if (!G) return;
  a.gate_a = G->a;
  a.gate_b = G->b;
  a.stride_ga = G->stride_a;
  a.stride_gb = G->stride_b;
  a.A_log = G->A_log;
  a.dt_bias = G->dt_bias;
}

// state_out may be state_in itself (in place) but must not partially overlap it
gdn_status check_state_overlap(const gdn_dims* d, const float* state_in, const float* state_out) {
  if (state_in && state_out && state_in != state_out) {
    const size_t sbytes = (size_t)d->num_seqs * d->num_v_heads * d->head_dim_k * d->head_dim_v * 4;
    const char* a0 = reinterpret_cast<const char*>(state_in);
    const char* b0 = reinterpret_cast<const char*>(state_out);
    if (a0 < b0 + sbytes && b0 < a0 + sbytes)
      return fail(GDN_ERR_INVALID_ARG, "state_out may alias state_in exactly but not partially overlap it");
  }
  return GDN_OK;
}

gdn_status check_workspace(const gdn_dims* d, const void* ws, size_t ws_bytes) {
  const WsLayout L = ws_layout(d);
  if (L.total > 0 && !ws) return fail(GDN_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", L.total);
  if (ws && !aligned(ws, 256)) return fail(GDN_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < L.total) return fail(GDN_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, L.total);
  return GDN_OK;
}

void carve(gdn::ScanArgs& a, const gdn_dims* d, const void* ws) {
  const WsLayout L = ws_layout(d);
  char* base = reinterpret_cast<char*>(const_cast<void*>(ws));
  a.chunk_offsets = L.table_bytes ? reinterpret_cast<int32_t*>(base + L.table_off) : nullptr;
  a.tinv = base ? base + L.mats_off : nullptr;
  a.scal = base ? reinterpret_cast<float*>(base + L.scal_off) : nullptr;
  a.max_chunks = (int)max_chunks(d);
  if (seg_enabled(d)) {
    a.seg_len = seg_len(d);
    a.max_segs = (int)max_segs(d);
    a.seg_offsets = L.segt_bytes ? reinterpret_cast<int32_t*>(base + L.segt_off) : nullptr;
    a.seg_perm = a.seg_offsets ? a.seg_offsets + (d->num_seqs + 1) : nullptr;
    a.seg_state = base ? reinterpret_cast<float*>(base + L.sst_off) : nullptr;
    a.seg_phi = base ? reinterpret_cast<uint16_t*>(base + L.phi_off) : nullptr;
  } else if (a.chunk_offsets) {
    a.seg_perm = a.chunk_offsets + (d->num_seqs + 1);
  }
}

gdn_status run_prepare(gdn::ScanArgs& a, hipStream_t s) {
  hipError_t e;
  if (a.seqlen == 0 && (e = gdn::launch_chunk_table(a, s)) != hipSuccess) return hip_fail(e, "chunk table launch");
  if (a.total_tokens > 0 && (e = gdn::launch_prepare(a, s)) != hipSuccess) return hip_fail(e, "prepare launch");
  return GDN_OK;
}

gdn_status run_scan(gdn::ScanArgs& a, const gdn_dims* d, hipStream_t s) {
  hipError_t e = gdn::launch_scan(a, s);
  if (e != hipSuccess) return hip_fail(e, "scan launch");
  if (a.norm_z && !gdn::seg_path(a) && d->total_tokens > 0) {
    // the carry paths without the fused norm wrote o into y: the gated norm
    // follows in place
    gdn::NormArgs n;
    n.rows = (long)d->total_tokens * d->num_v_heads;
    n.heads = d->num_v_heads;
    n.dv = d->head_dim_v;
    n.dtype = d->dtype;
    n.o = a.o;
    n.z = a.norm_z;
    n.weight = a.norm_w;
    n.y = a.o;
    n.stride_o = n.stride_y = (long)d->num_v_heads * d->head_dim_v;
    n.stride_z = a.stride_z;
    n.eps = a.norm_eps;
    if ((e = gdn::launch_gated_norm(n, s)) != hipSuccess) return hip_fail(e, "gated norm launch");
  }
  gdn_status st = debug_check(s, "o", a.o, (long)d->total_tokens * d->num_v_heads * d->head_dim_v, d->dtype);
  if (st != GDN_OK) return st;
  return debug_check(s, "state_out", a.state_out, (long)d->num_seqs * d->num_v_heads * d->head_dim_k * d->head_dim_v,
                     GDN_F32);
}

// ---- The no-allocation prefill's workspace: a file-scope device array.
// Each GPU the library runs on holds its own copy until the process ends.
// Host code never passes the array's name to a kernel or a copy: the name
// is a host-side stand-in, not a device address.  The address comes from
// hipGetSymbolAddress, once per device with that device current.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

gdn_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(GDN_ERR_UNSUPPORTED, "device index %d is not below %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p || !aligned(p, 256)) return fail(GDN_ERR_HIP, "scratch array address is not 256-byte aligned");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return GDN_OK;
}

// The gated norm fused into the carry's output (NULL: plain o).
struct NormIn {
  const void* z;
  int64_t stride_z;
  const float* weight;
  float eps;
};

gdn_status check_norm(const gdn_dims* d, const NormIn* n, const void* y) {
  if (!n) return GDN_OK;
  const int64_t row = (int64_t)d->num_v_heads * d->head_dim_v;
  const int vec = d->dtype == GDN_BF16 ? 8 : 4;
  if (n->stride_z < row || n->stride_z % vec)
    return fail(GDN_ERR_INVALID_ARG, "stride_z must be >= H_v d_v (%lld) and a multiple of %d elements", (long long)row, vec);
  if (!n->weight || !aligned(n->weight, 4)) return fail(GDN_ERR_INVALID_ARG, "norm weight must be non-NULL and 4-byte aligned");
  if (!(n->eps >= 0.0f) || !std::isfinite(n->eps)) return fail(GDN_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (d->total_tokens > 0) {
    if (!n->z || !aligned(n->z, 16)) return fail(GDN_ERR_INVALID_ARG, "z must be non-NULL and 16-byte aligned");
    const size_t esz = elem_size(d->dtype);
    const size_t zb = ((size_t)(d->total_tokens - 1) * n->stride_z + row) * esz, yb = (size_t)d->total_tokens * row * esz;
    const char* z0 = reinterpret_cast<const char*>(n->z);
    const char* y0 = reinterpret_cast<const char*>(y);
    if (y0 && z0 < y0 + yb && y0 < z0 + zb) return fail(GDN_ERR_INVALID_ARG, "y must not overlap z");
  }
  return GDN_OK;
}

}  // namespace

extern "C" {

const char* gdn_status_string(gdn_status s) {
  switch (s) {
    case GDN_OK: return "GDN_OK";
    case GDN_ERR_INVALID_ARG: return "GDN_ERR_INVALID_ARG";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED";
    case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE";
    case GDN_ERR_HIP: return "GDN_ERR_HIP";
    case GDN_ERR_NONFINITE: return "GDN_ERR_NONFINITE";
  }
  return "GDN_ERR_UNKNOWN";
}

const char* gdn_last_error(void) { return g_last_error.c_str(); }

const char* gdn_version(void) { return "0.1.0"; }

gdn_status gdn_validate_dims(const gdn_dims* d, int32_t op) { return check_dims(d, op); }


gdn_status gdn_conv1d(int32_t num_seqs, int32_t total_tokens, int32_t seqlen, const int32_t* cu_seqlens,
                      int32_t channels, int32_t width, int32_t dtype, const void* x, int64_t stride_x,
                      const float* weight, const float* bias, void* conv_state, int32_t activation, void* y,
                      int64_t stride_y, void* stream) {
  if (num_seqs < 1) return fail(GDN_ERR_INVALID_ARG, "num_seqs must be >= 1");
  if (total_tokens < 0 || total_tokens > kMaxTokens) return fail(GDN_ERR_INVALID_ARG, "total_tokens out of range");
  if (seqlen < 0) return fail(GDN_ERR_INVALID_ARG, "seqlen must be >= 0");
  if (seqlen > 0 && (int64_t)num_seqs * seqlen != total_tokens)
    return fail(GDN_ERR_INVALID_ARG, "dense layout needs total_tokens == num_seqs * seqlen");
  if (dtype != GDN_F32 && dtype != GDN_BF16) return fail(GDN_ERR_INVALID_ARG, "dtype must be GDN_F32 or GDN_BF16");
  const int vec = dtype == GDN_BF16 ? 8 : 4;
  if (channels < 1 || channels % vec) return fail(GDN_ERR_INVALID_ARG, "channels must be a positive multiple of %d", vec);
  if (width < 2 || width > 8) return fail(GDN_ERR_UNSUPPORTED, "width must be in [2, 8] (got %d)", width);
  if (activation != 0 && activation != 1) return fail(GDN_ERR_INVALID_ARG, "activation must be 0 or 1");
  if (stride_x < channels || stride_y < channels || stride_x % vec || stride_y % vec)
    return fail(GDN_ERR_INVALID_ARG, "strides must be >= channels and multiples of %d", vec);
  if (total_tokens > 0) {
    if (!x || !y) return fail(GDN_ERR_INVALID_ARG, "x and y must be non-NULL");
    if (!aligned(x, 16) || !aligned(y, 16)) return fail(GDN_ERR_INVALID_ARG, "x and y must be 16-byte aligned");
  }
  if (!weight || !aligned(weight, 4)) return fail(GDN_ERR_INVALID_ARG, "weight must be non-NULL and 4-byte aligned");
  if (bias && !aligned(bias, 4)) return fail(GDN_ERR_INVALID_ARG, "bias must be 4-byte aligned");
  if (conv_state && !aligned(conv_state, 16)) return fail(GDN_ERR_INVALID_ARG, "conv_state must be 16-byte aligned");
  if (seqlen == 0 && (!cu_seqlens || !aligned(cu_seqlens, 4)))
    return fail(GDN_ERR_INVALID_ARG, "varlen (seqlen == 0) needs a 4-byte aligned cu_seqlens");
  {
    // the kernels read x and the window while they write y (and then the
    // window from x): no two of them may share bytes
    const size_t esz = dtype == GDN_BF16 ? 2 : 4;
    auto overlap = [](const void* p, size_t pn, const void* q, size_t qn) {
      const char* a0 = static_cast<const char*>(p);
      const char* b0 = static_cast<const char*>(q);
      return pn && qn && a0 < b0 + qn && b0 < a0 + pn;
    };
    const size_t xb = total_tokens > 0 ? ((size_t)(total_tokens - 1) * stride_x + channels) * esz : 0;
    const size_t yb = total_tokens > 0 ? ((size_t)(total_tokens - 1) * stride_y + channels) * esz : 0;
    const size_t wb = conv_state ? (size_t)num_seqs * (width - 1) * channels * esz : 0;
    if (overlap(x, xb, y, yb)) return fail(GDN_ERR_INVALID_ARG, "x and y must not overlap");
    if (overlap(conv_state, wb, x, xb) || overlap(conv_state, wb, y, yb))
      return fail(GDN_ERR_INVALID_ARG, "conv_state must not overlap x or y");
  }
  gdn::ConvArgs a;
  a.num_seqs = num_seqs;
  a.total_tokens = total_tokens;
  a.seqlen = seqlen;
  a.cu_seqlens = cu_seqlens;
  a.channels = channels;
  a.width = width;
  a.dtype = dtype;
  a.activation = activation;
  a.x = x;
  a.stride_x = stride_x;
  a.weight = weight;
  a.bias = bias;
  a.conv_state = conv_state;
  a.y = y;
  a.stride_y = stride_y;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = gdn::launch_conv1d(a, s);
  if (e != hipSuccess) return hip_fail(e, "conv1d launch");
  if (debug_enabled() && total_tokens > 0) {
    // y rows may be strided: probe the whole span (padding included)
    gdn_status st = debug_check(s, "conv y", y, (long)(total_tokens - 1) * stride_y + channels, dtype);
    if (st != GDN_OK) return st;
  }
  return ok();
}

size_t gdn_prefill_workspace_size(const gdn_dims* d) {
  if (check_dims(d, 0) != GDN_OK) return 0;
  return ws_layout(d).total;
}

gdn_status gdn_prefill_prepare(const gdn_dims* d, const void* q, const void* k, const float* g, const float* beta,
                               const int32_t* cu_seqlens, void* workspace, size_t ws_bytes, void* stream) {
  gdn_status st = check_dims(d, 0);
  if (st != GDN_OK) return st;
  if ((st = check_scan_ptrs(d, q, k, nullptr, g, beta, cu_seqlens, false)) != GDN_OK) return st;
  if (d->total_tokens > 0 && (!q || !aligned(q, 16))) return fail(GDN_ERR_INVALID_ARG, "q must be non-NULL and 16-byte aligned");
  if ((st = check_workspace(d, workspace, ws_bytes)) != GDN_OK) return st;
  gdn::ScanArgs a = make_args(d);
  a.q = q;
  a.k = k;
  a.g = g;
  a.beta = beta;
  a.cu_seqlens = cu_seqlens;
  carve(a, d, workspace);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if ((st = run_prepare(a, s)) != GDN_OK) return st;
  return ok();
}

// need_gb false: the carry after a prepare that computed the gates itself
// (the carry kernels read neither g nor beta)
static gdn_status scan_impl(const gdn_dims* d, const void* q, const void* k, const void* v, const float* g,
                            const float* beta, const float* state_in, const int32_t* cu_seqlens, void* o,
                            float* state_out, const void* workspace, size_t ws_bytes, void* stream, bool need_gb,
                            const NormIn* norm = nullptr) {
  gdn_status st = check_dims(d, 0);
  if (st != GDN_OK) return st;
  if ((st = check_norm(d, norm, o)) != GDN_OK) return st;
  if ((st = check_scan_ptrs(d, q, k, v, g, beta, cu_seqlens, true, need_gb)) != GDN_OK) return st;
  if ((st = check_workspace(d, workspace, ws_bytes)) != GDN_OK) return st;
  if (d->total_tokens > 0 && (!o || !aligned(o, 16))) return fail(GDN_ERR_INVALID_ARG, "o must be non-NULL and 16-byte aligned");
  if ((state_in && !aligned(state_in, 16)) || (state_out && !aligned(state_out, 16)))
    return fail(GDN_ERR_INVALID_ARG, "states must be 16-byte aligned");
  if ((st = check_state_overlap(d, state_in, state_out)) != GDN_OK) return st;
  gdn::ScanArgs a = make_args(d);
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.state_in = state_in;
  a.cu_seqlens = cu_seqlens;
  a.o = o;
  a.state_out = state_out;
  if (norm) {
    a.norm_z = norm->z;
    a.stride_z = norm->stride_z;
    a.norm_w = norm->weight;
    a.norm_eps = norm->eps;
  }
  carve(a, d, workspace);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if ((st = run_scan(a, d, s)) != GDN_OK) return st;
  return ok();
}

gdn_status gdn_prefill_scan(const gdn_dims* d, const void* q, const void* k, const void* v, const float* g,
                            const float* beta, const float* state_in, const int32_t* cu_seqlens, void* o,
                            float* state_out, const void* workspace, size_t ws_bytes, void* stream) {
  return scan_impl(d, q, k, v, g, beta, state_in, cu_seqlens, o, state_out, workspace, ws_bytes, stream, true);
}

// Every check of gdn_prefill_chunked (both halves), host only.
static gdn_status validate_prefill(const gdn_dims* d, const void* q, const void* k, const void* v, const float* g,
                                   const float* beta, const float* state_in, const int32_t* cu_seqlens,
                                   const void* o, const float* state_out, const void* workspace, size_t ws_bytes) {
  gdn_status st = check_dims(d, 0);
  if (st != GDN_OK) return st;
  if ((st = check_scan_ptrs(d, q, k, v, g, beta, cu_seqlens, true)) != GDN_OK) return st;
  if ((st = check_workspace(d, workspace, ws_bytes)) != GDN_OK) return st;
  if (d->total_tokens > 0 && (!o || !aligned(o, 16))) return fail(GDN_ERR_INVALID_ARG, "o must be non-NULL and 16-byte aligned");
  if ((state_in && !aligned(state_in, 16)) || (state_out && !aligned(state_out, 16)))
    return fail(GDN_ERR_INVALID_ARG, "states must be 16-byte aligned");
  return check_state_overlap(d, state_in, state_out);
}

gdn_status gdn_prefill_chunked(const gdn_dims* d, const void* q, const void* k, const void* v, const float* g,
                               const float* beta, const float* state_in, const int32_t* cu_seqlens, void* o,
                               float* state_out, void* workspace, size_t ws_bytes, void* stream) {
  // validate the scan half fully before queuing the prepare half
  gdn_status st = validate_prefill(d, q, k, v, g, beta, state_in, cu_seqlens, o, state_out, workspace, ws_bytes);
  if (st != GDN_OK) return st;
  if ((st = gdn_prefill_prepare(d, q, k, g, beta, cu_seqlens, workspace, ws_bytes, stream)) != GDN_OK) return st;
  return gdn_prefill_scan(d, q, k, v, g, beta, state_in, cu_seqlens, o, state_out, workspace, ws_bytes, stream);
}

gdn_status gdn_prefill_chunked_noalloc(const gdn_dims* d, const void* q, const void* k, const void* v,
                                       const float* g, const float* beta, const float* state_in,
                                       const int32_t* cu_seqlens, void* o, float* state_out, void* stream) {
  gdn_status st = check_dims(d, 0);
  if (st != GDN_OK) return st;
  const size_t need = ws_layout(d).total;
  if (need > kScratchBytes)
    return fail(GDN_ERR_UNSUPPORTED,
                "this problem needs %zu bytes of workspace, more than the %zu the no-allocation prefill holds; "
                "call gdn_prefill_chunked with a workspace instead", need, kScratchBytes);
  // every argument check first (a stand-in workspace address: the real one
  // is known only after a HIP call), so an invalid call makes none
  if ((st = validate_prefill(d, q, k, v, g, beta, state_in, cu_seqlens, o, state_out,
                             reinterpret_cast<void*>(uintptr_t(256)), kScratchBytes)) != GDN_OK)
    return st;
  void* ws = nullptr;
  if ((st = scratch_of_current_device(&ws)) != GDN_OK) return st;
  return gdn_prefill_chunked(d, q, k, v, g, beta, state_in, cu_seqlens, o, state_out, ws, kScratchBytes, stream);
}

gdn_status gdn_prefill_scan_gated_norm(const gdn_dims* d, const void* q, const void* k, const void* v, const float* g,
                                      const float* beta, const float* state_in, const int32_t* cu_seqlens,
                                      const void* z, int64_t stride_z, const float* norm_weight, float eps, void* y,
                                      float* state_out, const void* workspace, size_t ws_bytes, void* stream) {
  const NormIn n{z, stride_z, norm_weight, eps};
  return scan_impl(d, q, k, v, g, beta, state_in, cu_seqlens, y, state_out, workspace, ws_bytes, stream, true, &n);
}

gdn_status gdn_prefill_chunked_gated_norm(const gdn_dims* d, const void* q, const void* k, const void* v,
                                         const float* g, const float* beta, const float* state_in,
                                         const int32_t* cu_seqlens, const void* z, int64_t stride_z,
                                         const float* norm_weight, float eps, void* y, float* state_out,
                                         void* workspace, size_t ws_bytes, void* stream) {
  // both halves validated before the prepare is queued
  gdn_status st = validate_prefill(d, q, k, v, g, beta, state_in, cu_seqlens, y, state_out, workspace, ws_bytes);
  if (st != GDN_OK) return st;
  const NormIn n{z, stride_z, norm_weight, eps};
  if ((st = check_norm(d, &n, y)) != GDN_OK) return st;
  if ((st = gdn_prefill_prepare(d, q, k, g, beta, cu_seqlens, workspace, ws_bytes, stream)) != GDN_OK) return st;
  return gdn_prefill_scan_gated_norm(d, q, k, v, g, beta, state_in, cu_seqlens, z, stride_z, norm_weight, eps, y,
                                     state_out, workspace, ws_bytes, stream);
}

static gdn_status conv_prepare_impl(const gdn_dims* d, const gdn_gate_inputs* gates, int32_t conv_width,
                                    const void* x, int64_t stride_x, const float* conv_weight,
                                    const float* conv_bias, void* conv_state, const float* g, const float* beta,
                                    const int32_t* cu_seqlens, void* y, int64_t stride_y, void* workspace,
                                    size_t ws_bytes, void* stream) {
  gdn_status st = check_dims(d, 0);
  if (st != GDN_OK) return st;
  const int64_t cc = 2LL * d->num_qk_heads * d->head_dim_k + (int64_t)d->num_v_heads * d->head_dim_v;
  const int vec = d->dtype == GDN_BF16 ? 8 : 4;
  if (conv_width < 2 || conv_width > 8) return fail(GDN_ERR_UNSUPPORTED, "conv_width must be in [2, 8] (got %d)", conv_width);
  if (stride_x < cc || stride_y < cc || stride_x % vec || stride_y % vec)
    return fail(GDN_ERR_INVALID_ARG, "stride_x and stride_y must be >= %lld channels and multiples of %d", (long long)cc, vec);
  if (d->stride_q != stride_y || d->stride_k != stride_y || d->stride_v != stride_y)
    return fail(GDN_ERR_INVALID_ARG, "q, k and v are the column blocks of y: d's strides must equal stride_y");
  if (d->total_tokens > 0) {
    if (!x || !y) return fail(GDN_ERR_INVALID_ARG, "x and y must be non-NULL");
    if (!aligned(x, 16) || !aligned(y, 16)) return fail(GDN_ERR_INVALID_ARG, "x and y must be 16-byte aligned");
    const size_t esz = d->dtype == GDN_BF16 ? 2 : 4;
    const char* x0 = reinterpret_cast<const char*>(x);
    const char* y0 = reinterpret_cast<const char*>(y);
    const size_t xb = ((size_t)(d->total_tokens - 1) * stride_x + cc) * esz;
    const size_t yb = ((size_t)(d->total_tokens - 1) * stride_y + cc) * esz;
    if (x0 < y0 + yb && y0 < x0 + xb) return fail(GDN_ERR_INVALID_ARG, "x and y must not overlap");
  }
  if (!conv_weight || !aligned(conv_weight, 4))
    return fail(GDN_ERR_INVALID_ARG, "conv_weight must be non-NULL and 4-byte aligned");
  if (conv_bias && !aligned(conv_bias, 4)) return fail(GDN_ERR_INVALID_ARG, "conv_bias must be 4-byte aligned");
  if (conv_state && !aligned(conv_state, 16)) return fail(GDN_ERR_INVALID_ARG, "conv_state must be 16-byte aligned");
  const void* q = y;
  const void* k = reinterpret_cast<const char*>(y) + (size_t)d->num_qk_heads * d->head_dim_k * (d->dtype == GDN_BF16 ? 2 : 4);
  if ((st = check_scan_ptrs(d, q, k, nullptr, g, beta, cu_seqlens, false, !gates)) != GDN_OK) return st;
  if (gates && (st = check_gates(d, gates)) != GDN_OK) return st;
  if ((st = check_workspace(d, workspace, ws_bytes)) != GDN_OK) return st;

  gdn::ConvArgs ca;
  ca.num_seqs = d->num_seqs;
  ca.total_tokens = d->total_tokens;
  ca.seqlen = d->seqlen;
  ca.cu_seqlens = cu_seqlens;
  ca.channels = (int)cc;
  ca.width = conv_width;
  ca.dtype = d->dtype;
  ca.activation = 1;
  ca.x = x;
  ca.stride_x = stride_x;
  ca.weight = conv_weight;
  ca.bias = conv_bias;
  ca.conv_state = conv_state;
  ca.y = y;
  ca.stride_y = stride_y;

  gdn::ScanArgs a = make_args(d);
  a.q = q;
  a.k = k;
  a.g = g;
  a.beta = beta;
  a.cu_seqlens = cu_seqlens;
  set_gates(a, gates);
  carve(a, d, workspace);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  // The two kernels back to back: folding the convolution into the prepare
  // kernel was measured slower (both are bound by vector-instruction issue,
  // and the stand-alone convolution overlaps its arithmetic with its memory
  // traffic across many more waves).
  if ((e = gdn::launch_conv1d(ca, s)) != hipSuccess) return hip_fail(e, "conv1d launch");
  if ((st = run_prepare(a, s)) != GDN_OK) return st;
  if (debug_enabled() && d->total_tokens > 0) {
    st = debug_check(s, "conv y", y, (long)(d->total_tokens - 1) * stride_y + cc, d->dtype);
    if (st != GDN_OK) return st;
  }
  return ok();
}

gdn_status gdn_prefill_conv_prepare(const gdn_dims* d, int32_t conv_width, const void* x, int64_t stride_x,
                                    const float* conv_weight, const float* conv_bias, void* conv_state, const float* g,
                                    const float* beta, const int32_t* cu_seqlens, void* y, int64_t stride_y,
                                    void* workspace, size_t ws_bytes, void* stream) {
  return conv_prepare_impl(d, nullptr, conv_width, x, stride_x, conv_weight, conv_bias, conv_state, g, beta,
                           cu_seqlens, y, stride_y, workspace, ws_bytes, stream);
}

static gdn_status conv_chunked_impl(const gdn_dims* d, const gdn_gate_inputs* gates, int32_t conv_width,
                                    const void* x, int64_t stride_x, const float* conv_weight,
                                    const float* conv_bias, void* conv_state, const float* g, const float* beta,
                                    const float* state_in, const int32_t* cu_seqlens, void* y, int64_t stride_y,
                                    void* o, float* state_out, void* workspace, size_t ws_bytes, void* stream) {
  gdn_status st = check_dims(d, 0);
  if (st != GDN_OK) return st;
  // validate the scan half before queuing anything
  if (d->total_tokens > 0 && (!o || !aligned(o, 16))) return fail(GDN_ERR_INVALID_ARG, "o must be non-NULL and 16-byte aligned");
  if ((state_in && !aligned(state_in, 16)) || (state_out && !aligned(state_out, 16)))
    return fail(GDN_ERR_INVALID_ARG, "states must be 16-byte aligned");
  if ((st = check_state_overlap(d, state_in, state_out)) != GDN_OK) return st;
  if ((st = conv_prepare_impl(d, gates, conv_width, x, stride_x, conv_weight, conv_bias, conv_state, g, beta,
                              cu_seqlens, y, stride_y, workspace, ws_bytes, stream)) != GDN_OK)
    return st;
  const size_t esz = d->dtype == GDN_BF16 ? 2 : 4;
  const char* y0 = reinterpret_cast<const char*>(y);
  const void* q = y0;
  const void* k = y0 + (size_t)d->num_qk_heads * d->head_dim_k * esz;
  const void* v = y0 + (size_t)2 * d->num_qk_heads * d->head_dim_k * esz;
  return scan_impl(d, q, k, v, g, beta, state_in, cu_seqlens, o, state_out, workspace, ws_bytes, stream, !gates);
}

gdn_status gdn_prefill_conv_chunked(const gdn_dims* d, int32_t conv_width, const void* x, int64_t stride_x,
                                    const float* conv_weight, const float* conv_bias, void* conv_state, const float* g,
                                    const float* beta, const float* state_in, const int32_t* cu_seqlens, void* y,
                                    int64_t stride_y, void* o, float* state_out, void* workspace, size_t ws_bytes,
                                    void* stream) {
  return conv_chunked_impl(d, nullptr, conv_width, x, stride_x, conv_weight, conv_bias, conv_state, g, beta, state_in,
                           cu_seqlens, y, stride_y, o, state_out, workspace, ws_bytes, stream);
}

gdn_status gdn_prefill_conv_gated(const gdn_dims* d, const gdn_gate_inputs* gates, int32_t conv_width, const void* x,
                                  int64_t stride_x, const float* conv_weight, const float* conv_bias, void* conv_state,
                                  const float* state_in, const int32_t* cu_seqlens, void* y, int64_t stride_y, void* o,
                                  float* state_out, void* workspace, size_t ws_bytes, void* stream) {
  gdn_status st = check_dims(d, 0);
  if (st != GDN_OK) return st;
  if ((st = check_gates(d, gates)) != GDN_OK) return st;
  return conv_chunked_impl(d, gates, conv_width, x, stride_x, conv_weight, conv_bias, conv_state, nullptr, nullptr,
                           state_in, cu_seqlens, y, stride_y, o, state_out, workspace, ws_bytes, stream);
}

// Every check of gdn_decode_step, host only.
static gdn_status validate_decode(const gdn_dims* d, const void* q, const void* k, const void* v, const float* g,
                                  const float* beta, const float* state, int64_t num_slots,
                                  const int32_t* state_slots, const void* o) {
  gdn_status st = check_dims(d, 1);
  if (st != GDN_OK) return st;
  if ((st = check_scan_ptrs(d, q, k, v, g, beta, nullptr, true)) != GDN_OK) return st;
  if (!o || !aligned(o, 16)) return fail(GDN_ERR_INVALID_ARG, "o must be non-NULL and 16-byte aligned");
  if (!state || !aligned(state, 16)) return fail(GDN_ERR_INVALID_ARG, "state must be non-NULL and 16-byte aligned");
  if (num_slots < 1 || num_slots > INT32_MAX) return fail(GDN_ERR_INVALID_ARG, "num_slots must be in [1, 2^31)");
  if (!state_slots && num_slots < d->num_seqs)
    return fail(GDN_ERR_INVALID_ARG, "without state_slots, num_slots (%lld) must be >= num_seqs (%d)",
                (long long)num_slots, d->num_seqs);
  if (state_slots && !aligned(state_slots, 4)) return fail(GDN_ERR_INVALID_ARG, "state_slots must be 4-byte aligned");
  return GDN_OK;
}

gdn_status gdn_decode_step(const gdn_dims* d, const void* q, const void* k, const void* v, const float* g,
                           const float* beta, float* state, int32_t num_slots, const int32_t* state_slots, void* o,
                           void* stream) {
  gdn_status st = validate_decode(d, q, k, v, g, beta, state, num_slots, state_slots, o);
  if (st != GDN_OK) return st;
  gdn::ScanArgs a = make_args(d);
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.o = o;
  a.state = state;
  a.state_slots = state_slots;
  a.num_slots = num_slots;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = gdn::launch_decode(a, s);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  if ((st = debug_check(s, "o", o, (long)d->num_seqs * d->num_v_heads * d->head_dim_v, d->dtype)) != GDN_OK) return st;
  return ok();
}

static gdn_status decode_conv_impl(const gdn_dims* d, const gdn_gate_inputs* gates, int32_t conv_width,
                                   const void* x, int64_t stride_x, const float* conv_weight, const float* conv_bias,
                                   void* conv_state, const float* g, const float* beta, float* state,
                                   int32_t num_slots, const int32_t* state_slots, void* o, void* stream) {
  gdn_status st = check_dims(d, 1);
  if (st != GDN_OK) return st;
  const int64_t cc = 2LL * d->num_qk_heads * d->head_dim_k + (int64_t)d->num_v_heads * d->head_dim_v;
  const int vec = d->dtype == GDN_BF16 ? 8 : 4;
  const size_t esz = elem_size(d->dtype);
  if (conv_width < 2 || conv_width > 8) return fail(GDN_ERR_UNSUPPORTED, "conv_width must be in [2, 8] (got %d)", conv_width);
  if (d->num_v_heads / d->num_qk_heads > 4)
    return fail(GDN_ERR_UNSUPPORTED, "the fused step takes at most 4 v-heads per q/k head (got %d)",
                d->num_v_heads / d->num_qk_heads);
  if (stride_x < cc || stride_x % vec)
    return fail(GDN_ERR_INVALID_ARG, "stride_x must be >= %lld channels and a multiple of %d", (long long)cc, vec);
  if (!x || !aligned(x, 16)) return fail(GDN_ERR_INVALID_ARG, "x must be non-NULL and 16-byte aligned");
  if (!conv_weight || !aligned(conv_weight, 4))
    return fail(GDN_ERR_INVALID_ARG, "conv_weight must be non-NULL and 4-byte aligned");
  if (conv_bias && !aligned(conv_bias, 4)) return fail(GDN_ERR_INVALID_ARG, "conv_bias must be 4-byte aligned");
  if (!conv_state || !aligned(conv_state, 16))
    return fail(GDN_ERR_INVALID_ARG, "conv_state must be non-NULL and 16-byte aligned");
  if (gates) {
    if ((st = check_gates(d, gates)) != GDN_OK) return st;
  } else if (!g || !beta || !aligned(g, 4) || !aligned(beta, 4)) {
    return fail(GDN_ERR_INVALID_ARG, "g and beta must be non-NULL and 4-byte aligned");
  }
  if (!o || !aligned(o, 16)) return fail(GDN_ERR_INVALID_ARG, "o must be non-NULL and 16-byte aligned");
  if (!state || !aligned(state, 16)) return fail(GDN_ERR_INVALID_ARG, "state must be non-NULL and 16-byte aligned");
  if (num_slots < 1) return fail(GDN_ERR_INVALID_ARG, "num_slots must be >= 1");
  if (!state_slots && num_slots < d->num_seqs)
    return fail(GDN_ERR_INVALID_ARG, "without state_slots, num_slots (%d) must be >= num_seqs (%d)", num_slots,
                d->num_seqs);
  if (state_slots && !aligned(state_slots, 4)) return fail(GDN_ERR_INVALID_ARG, "state_slots must be 4-byte aligned");
  {
    const char* x0 = reinterpret_cast<const char*>(x);
    const char* w0 = reinterpret_cast<const char*>(conv_state);
    const size_t xb = ((size_t)(d->num_seqs - 1) * stride_x + cc) * esz;
    const size_t wb = (size_t)num_slots * (conv_width - 1) * cc * esz;
    if (x0 < w0 + wb && w0 < x0 + xb) return fail(GDN_ERR_INVALID_ARG, "x and conv_state must not overlap");
  }
  gdn::ConvArgs c;
  c.num_seqs = d->num_seqs;
  c.total_tokens = d->num_seqs;
  c.seqlen = 1;
  c.cu_seqlens = nullptr;
  c.channels = (int)cc;
  c.width = conv_width;
  c.dtype = d->dtype;
  c.activation = 1;
  c.x = x;
  c.stride_x = stride_x;
  c.weight = conv_weight;
  c.bias = conv_bias;
  c.conv_state = conv_state;
  c.y = nullptr;
  c.stride_y = 0;
  gdn::ScanArgs a = make_args(d);
  a.g = g;
  a.beta = beta;
  a.o = o;
  a.state = state;
  a.state_slots = state_slots;
  a.num_slots = num_slots;
  set_gates(a, gates);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = gdn::launch_decode_conv(a, c, s);
  if (e != hipSuccess) return hip_fail(e, "decode conv launch");
  if ((st = debug_check(s, "o", o, (long)d->num_seqs * d->num_v_heads * d->head_dim_v, d->dtype)) != GDN_OK) return st;
  return ok();
}

gdn_status gdn_decode_conv_step(const gdn_dims* d, int32_t conv_width, const void* x, int64_t stride_x,
                                const float* conv_weight, const float* conv_bias, void* conv_state, const float* g,
                                const float* beta, float* state, int32_t num_slots, const int32_t* state_slots,
                                void* o, void* stream) {
  return decode_conv_impl(d, nullptr, conv_width, x, stride_x, conv_weight, conv_bias, conv_state, g, beta, state,
                          num_slots, state_slots, o, stream);
}

gdn_status gdn_decode_conv_gated_step(const gdn_dims* d, const gdn_gate_inputs* gates, int32_t conv_width,
                                      const void* x, int64_t stride_x, const float* conv_weight,
                                      const float* conv_bias, void* conv_state, float* state, int32_t num_slots,
                                      const int32_t* state_slots, void* o, void* stream) {
  gdn_status st = check_dims(d, 1);
  if (st != GDN_OK) return st;
  if ((st = check_gates(d, gates)) != GDN_OK) return st;
  return decode_conv_impl(d, gates, conv_width, x, stride_x, conv_weight, conv_bias, conv_state, nullptr, nullptr,
                          state, num_slots, state_slots, o, stream);
}

gdn_status gdn_gated_rmsnorm(int32_t total_tokens, int32_t num_heads, int32_t head_dim, int32_t dtype,
                             const void* o, int64_t stride_o, const void* z, int64_t stride_z, const float* weight,
                             float eps, void* y, int64_t stride_y, void* stream) {
  if (total_tokens < 0 || total_tokens > kMaxTokens) return fail(GDN_ERR_INVALID_ARG, "total_tokens out of range");
  if (num_heads < 1 || num_heads > 4096) return fail(GDN_ERR_INVALID_ARG, "num_heads must be in [1, 4096]");
  if (head_dim != 64 && head_dim != 128) return fail(GDN_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", head_dim);
  if (dtype != GDN_F32 && dtype != GDN_BF16) return fail(GDN_ERR_INVALID_ARG, "dtype must be GDN_F32 or GDN_BF16");
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return fail(GDN_ERR_INVALID_ARG, "eps must be finite and >= 0");
  const int vec = dtype == GDN_BF16 ? 8 : 4;
  const int64_t row = (int64_t)num_heads * head_dim;
  if (stride_o < row || stride_z < row || stride_y < row || stride_o % vec || stride_z % vec || stride_y % vec)
    return fail(GDN_ERR_INVALID_ARG, "token strides must be >= %lld and multiples of %d elements", (long long)row, vec);
  if (!weight || !aligned(weight, 4)) return fail(GDN_ERR_INVALID_ARG, "weight must be non-NULL and 4-byte aligned");
  if (total_tokens > 0) {
    if (!o || !z || !y) return fail(GDN_ERR_INVALID_ARG, "o, z and y must be non-NULL");
    if (!aligned(o, 16) || !aligned(z, 16) || !aligned(y, 16))
      return fail(GDN_ERR_INVALID_ARG, "o, z and y must be 16-byte aligned");
    const size_t esz = elem_size(dtype);
    auto span = [&](int64_t stride) { return ((size_t)(total_tokens - 1) * stride + row) * esz; };
    auto overlap = [](const void* p, size_t pn, const void* q, size_t qn) {
      const char* a = reinterpret_cast<const char*>(p);
      const char* b = reinterpret_cast<const char*>(q);
      return a < b + qn && b < a + pn;
    };
    if (overlap(y, span(stride_y), z, span(stride_z))) return fail(GDN_ERR_INVALID_ARG, "y must not overlap z");
    if (!(y == o && stride_y == stride_o) && overlap(y, span(stride_y), o, span(stride_o)))
      return fail(GDN_ERR_INVALID_ARG, "y may be o itself (same stride) but must not partially overlap it");
  }
  gdn::NormArgs a;
  a.rows = (long)total_tokens * num_heads;
  a.heads = num_heads;
  a.dv = head_dim;
  a.dtype = dtype;
  a.o = o;
  a.z = z;
  a.weight = weight;
  a.y = y;
  a.stride_o = stride_o;
  a.stride_z = stride_z;
  a.stride_y = stride_y;
  a.eps = eps;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = gdn::launch_gated_norm(a, s);
  if (e != hipSuccess) return hip_fail(e, "gated norm launch");
  if (debug_enabled() && total_tokens > 0) {
    gdn_status st = debug_check(s, "gated norm y", y, (long)(total_tokens - 1) * stride_y + row, dtype);
    if (st != GDN_OK) return st;
  }
  return ok();
}

gdn_status gdn_gating(int32_t total_tokens, int32_t num_heads, int32_t dtype, const void* a, int64_t stride_a,
                      const void* b, int64_t stride_b, const float* A_log, const float* dt_bias, float* g, float* beta,
                      void* stream) {
  if (total_tokens < 0 || total_tokens > kMaxTokens) return fail(GDN_ERR_INVALID_ARG, "total_tokens out of range");
  if (num_heads < 1 || num_heads > 4096) return fail(GDN_ERR_INVALID_ARG, "num_heads must be in [1, 4096]");
  if (dtype != GDN_F32 && dtype != GDN_BF16) return fail(GDN_ERR_INVALID_ARG, "dtype must be GDN_F32 or GDN_BF16");
  if (stride_a < num_heads || stride_b < num_heads)
    return fail(GDN_ERR_INVALID_ARG, "token strides must be >= num_heads (%d)", num_heads);
  if (!A_log || !dt_bias || !aligned(A_log, 4) || !aligned(dt_bias, 4))
    return fail(GDN_ERR_INVALID_ARG, "A_log and dt_bias must be non-NULL and 4-byte aligned");
  if (total_tokens > 0) {
    const size_t esz = elem_size(dtype);
    if (!a || !b || !g || !beta) return fail(GDN_ERR_INVALID_ARG, "a, b, g and beta must be non-NULL");
    if (!aligned(a, esz) || !aligned(b, esz) || !aligned(g, 4) || !aligned(beta, 4))
      return fail(GDN_ERR_INVALID_ARG, "a, b, g and beta must be aligned to their element size");
    const size_t out = (size_t)total_tokens * num_heads * 4;
    const size_t ab = ((size_t)(total_tokens - 1) * stride_a + num_heads) * esz;
    const size_t bb = ((size_t)(total_tokens - 1) * stride_b + num_heads) * esz;
    auto overlap = [](const void* p, size_t pn, const void* q, size_t qn) {
      const char* x = reinterpret_cast<const char*>(p);
      const char* y = reinterpret_cast<const char*>(q);
      return x < y + qn && y < x + pn;
    };
    if (overlap(g, out, beta, out) || overlap(g, out, a, ab) || overlap(g, out, b, bb) || overlap(beta, out, a, ab) ||
        overlap(beta, out, b, bb))
      return fail(GDN_ERR_INVALID_ARG, "g and beta must not overlap each other, a or b");
  }
  gdn::GatingArgs ga;
  ga.rows = total_tokens;
  ga.heads = num_heads;
  ga.dtype = dtype;
  ga.gate_a = a;
  ga.gate_b = b;
  ga.stride_ga = stride_a;
  ga.stride_gb = stride_b;
  ga.A_log = A_log;
  ga.dt_bias = dt_bias;
  ga.g = g;
  ga.beta = beta;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = gdn::launch_gating(ga, s);
  if (e != hipSuccess) return hip_fail(e, "gating launch");
  if (debug_enabled() && total_tokens > 0) {
    gdn_status st = debug_check(s, "g", g, (long)total_tokens * num_heads, GDN_F32);
    if (st != GDN_OK) return st;
    if ((st = debug_check(s, "beta", beta, (long)total_tokens * num_heads, GDN_F32)) != GDN_OK) return st;
  }
  return ok();
}

static gdn_status snapshot_impl(int32_t num_seqs, const int32_t* slots, int32_t num_slots, int64_t state_elems,
                                const void* state, int64_t window_bytes, const void* conv_state, int32_t ring_len,
                                const void* ring_state, const void* ring_window, int32_t* ring_head, int32_t entry,
                                int to_ring, void* stream) {
  if (num_seqs < 0) return fail(GDN_ERR_INVALID_ARG, "num_seqs must be >= 0");
  if (num_slots < 1) return fail(GDN_ERR_INVALID_ARG, "num_slots must be >= 1");
  if (!slots && num_slots < num_seqs)
    return fail(GDN_ERR_INVALID_ARG, "without slots, num_slots (%d) must be >= num_seqs (%d)", num_slots, num_seqs);
  if (slots && !aligned(slots, 4)) return fail(GDN_ERR_INVALID_ARG, "slots must be 4-byte aligned");
  if (ring_len < 1) return fail(GDN_ERR_INVALID_ARG, "ring_len must be >= 1");
  if (state_elems < 0 || state_elems % 4 || window_bytes < 0 || window_bytes % 16)
    return fail(GDN_ERR_INVALID_ARG, "state_elems must be a multiple of 4 and window_bytes of 16 (both >= 0)");
  if (state_elems > (1LL << 36) || window_bytes > (1LL << 38))
    return fail(GDN_ERR_UNSUPPORTED, "per-slot sizes above 2^36 elements / 2^38 bytes are not supported");
  if (state_elems > 0 && (!state || !ring_state || !aligned(state, 16) || !aligned(ring_state, 16)))
    return fail(GDN_ERR_INVALID_ARG, "state and ring_state must be non-NULL and 16-byte aligned");
  if (window_bytes > 0 && (!conv_state || !ring_window || !aligned(conv_state, 16) || !aligned(ring_window, 16)))
    return fail(GDN_ERR_INVALID_ARG, "conv_state and ring_window must be non-NULL and 16-byte aligned");
  if (to_ring) {
    if (!ring_head || !aligned(ring_head, 4)) return fail(GDN_ERR_INVALID_ARG, "ring_head must be non-NULL and 4-byte aligned");
  } else if (entry < 0 || entry >= ring_len) {
    return fail(GDN_ERR_INVALID_ARG, "entry (%d) must be in [0, ring_len = %d)", entry, ring_len);
  }
  auto overlap = [](const void* p, size_t pn, const void* q, size_t qn) {
    const char* x = reinterpret_cast<const char*>(p);
    const char* y = reinterpret_cast<const char*>(q);
    return pn && qn && x < y + qn && y < x + pn;
  };
  const size_t sb = (size_t)state_elems * 4, wb = (size_t)window_bytes;
  const size_t live_s = (size_t)num_slots * sb, live_w = (size_t)num_slots * wb;
  const size_t ring_s = (size_t)ring_len * num_seqs * sb, ring_w = (size_t)ring_len * num_seqs * wb;
  if (overlap(state, live_s, ring_state, ring_s) || overlap(conv_state, live_w, ring_window, ring_w) ||
      overlap(state, live_s, ring_window, ring_w) || overlap(conv_state, live_w, ring_state, ring_s))
    return fail(GDN_ERR_INVALID_ARG, "the live slots and the ring must not overlap");
  if (num_seqs == 0 || (sb == 0 && wb == 0)) {
    if (!to_ring) return ok();
  }
  gdn::SnapArgs a;
  a.num_seqs = num_seqs;
  a.num_slots = num_slots;
  a.ring_len = ring_len;
  a.entry = entry;
  a.slots = slots;
  a.state_bytes = (long)sb;
  a.window_bytes = (long)wb;
  a.state = const_cast<void*>(state);
  a.window = const_cast<void*>(conv_state);
  a.ring_state = const_cast<void*>(ring_state);
  a.ring_window = const_cast<void*>(ring_window);
  a.head = to_ring ? ring_head : nullptr;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = gdn::launch_snapshot(a, to_ring, s);
  if (e != hipSuccess) return hip_fail(e, to_ring ? "snapshot push launch" : "snapshot restore launch");
  return ok();
}

gdn_status gdn_snapshot_push(int32_t num_seqs, const int32_t* slots, int32_t num_slots, int64_t state_elems,
                             const float* state, int64_t window_bytes, const void* conv_state, int32_t ring_len,
                             float* ring_state, void* ring_window, int32_t* ring_head, void* stream) {
  return snapshot_impl(num_seqs, slots, num_slots, state_elems, state, window_bytes, conv_state, ring_len, ring_state,
                       ring_window, ring_head, 0, 1, stream);
}

gdn_status gdn_snapshot_restore(int32_t num_seqs, const int32_t* slots, int32_t num_slots, int64_t state_elems,
                                float* state, int64_t window_bytes, void* conv_state, int32_t ring_len,
                                const float* ring_state, const void* ring_window, int32_t entry, void* stream) {
  return snapshot_impl(num_seqs, slots, num_slots, state_elems, state, window_bytes, conv_state, ring_len, ring_state,
                       ring_window, nullptr, entry, 0, stream);
}

gdn_status gdn_validate(const gdn_dims* d, int32_t op, const void* const* ptrs, int32_t n_ptrs, int64_t extent) {
  if (op != 0 && op != 1) return fail(GDN_ERR_INVALID_ARG, "op must be 0 (prefill) or 1 (decode)");
  const int32_t need = op == 0 ? 10 : 8;
  if (!ptrs || n_ptrs != need)
    return fail(GDN_ERR_INVALID_ARG, "%s takes %d pointers (got %d)", op == 0 ? "prefill" : "decode", need, n_ptrs);
  const float* const* fp = reinterpret_cast<const float* const*>(ptrs);
  gdn_status st;
  if (op == 0) {
    if (extent < 0) return fail(GDN_ERR_INVALID_ARG, "workspace bytes must be >= 0");
    st = validate_prefill(d, ptrs[0], ptrs[1], ptrs[2], fp[3], fp[4], fp[5], reinterpret_cast<const int32_t*>(ptrs[6]),
                          ptrs[7], fp[8], ptrs[9], (size_t)extent);
  } else {
    st = validate_decode(d, ptrs[0], ptrs[1], ptrs[2], fp[3], fp[4], fp[5], extent,
                         reinterpret_cast<const int32_t*>(ptrs[6]), ptrs[7]);
  }
  return st == GDN_OK ? ok() : st;
}

}  // extern "C"
