// gdn_internal.h -- argument blocks and kernel launchers shared between the
// C-ABI layer (gdn_api.cpp) and the kernels (*.hip).  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

struct ConvArgs {
  int num_seqs, total_tokens, seqlen;
  const int32_t* cu_seqlens;
  int channels, width, dtype, activation;
  const void* x;
  long stride_x;
  const float* weight;
  const float* bias;
  void* conv_state;
  void* y;
  long stride_y;
};

// Rows of the per-(chunk, v-head) scalar block written by the prepare, each
// `chunk` fp32 values, one per token of the chunk:
//   0 a = e^{gamma} rk      1 b = scale e^{gamma} rq (sequential carry only)
//   2 c = e^{gamma_last - gamma} rk                  3 e^{gamma_last} (first element)
//   4 gamma                 5 rk = 1/|k| (1 without the L2 norm)
//   6 (free: the segment-parallel carry puts scale rq there in LDS)
//   7 e^{gamma}
constexpr int kScalRows = 8;

// Everything the scan kernels need; pointers are device pointers.
struct ScanArgs {
  int num_seqs, total_tokens, seqlen;  // seqlen > 0: dense
  int hk, hv, dk, dv, chunk;           // heads, head dims, chunk size
  int dtype;                           // 0 f32, 1 bf16
  int l2norm, tiled;
  float scale;
  long stride_q, stride_k, stride_v;   // elements between tokens
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  const float* state_in;
  const int32_t* cu_seqlens;  // varlen only
  void* o;
  float* state_out;
  // workspace carve-up
  int32_t* chunk_offsets;     // [num_seqs + 1], varlen only
  void* tinv;                 // [max_chunks][hv][2][chunk][chunk] in the operand type: Tt, P, each as
                              // its lower 16x16 blocks packed at the front (block i(i+1)/2+j at 256 n)
  float* scal;                // [max_chunks][hv][kScalRows][chunk] fp32 per-row scalars (see kScalRows)
  int max_chunks;
  // segment-parallel scan (bf16, chunk 32/64): every sequence is cut into
  // segments of seg_len chunks (at least one segment per sequence)
  int seg_len;
  int max_segs;               // bound on the number of segments, all sequences
  int32_t* seg_offsets;       // [num_seqs + 1], varlen only
  int32_t* seg_perm;          // varlen only: the carry's units (segments, or sequences on the sequential
                              // carry) in the order its workgroups take them, longest first
  float* seg_state;           // [max_segs][hv][dk][dv] fp32: start state of each segment
  uint16_t* seg_phi;          // [max_segs][hv][dk][dk] bf16: transition of each segment
  // decode only
  float* state;
  const int32_t* state_slots;
  int num_slots;
  // gates from the raw projections (gate_math.h) instead of g and beta,
  // where gate_a is set: the prepare and the fused decode step compute them
  const void* gate_a;
  const void* gate_b;
  long stride_ga, stride_gb;
  const float* A_log;
  const float* dt_bias;
  // the gated RMS norm fused into the carry's output write, where norm_z is
  // set: o then receives y = w * o / sqrt(mean(o^2) + eps) * silu(z) per
  // (token, v-head) row, z [N_tok][H_v][d_v] with token stride stride_z
  const void* norm_z;
  long stride_z;
  const float* norm_w;
  float norm_eps;
};

// Gated RMS norm over rows of d_v values (one row per token and v-head;
// heads packed inside a token row); device pointers.
struct NormArgs {
  long rows;       // tokens * heads
  int heads, dv, dtype;
  const void* o;
  const void* z;
  const float* weight;
  void* y;
  long stride_o, stride_z, stride_y;  // elements between tokens
  float eps;
};

// The gates from the raw projections: g, beta fp32 [rows][heads] (packed).
struct GatingArgs {
  long rows;  // tokens
  int heads, dtype;
  const void* gate_a;
  const void* gate_b;
  long stride_ga, stride_gb;  // elements between tokens
  const float* A_log;
  const float* dt_bias;
  float* g;
  float* beta;
};

// A push or restore of state snapshots: per sequence b, live slot slots[b]
// (or b) of state [num_slots][state_bytes] and window [num_slots][window_bytes]
// against ring entry e of ring_state [ring_len][num_seqs][state_bytes] and
// ring_window [ring_len][num_seqs][window_bytes]; e = *head mod ring_len
// (push, then the counter is advanced) or `entry`.
struct SnapArgs {
  int num_seqs, num_slots, ring_len, entry;
  const int32_t* slots;
  long state_bytes, window_bytes;  // multiples of 16
  void* state;
  void* window;
  void* ring_state;
  void* ring_window;
  int* head;
};

hipError_t launch_conv1d(const ConvArgs& a, hipStream_t s);
hipError_t launch_snapshot(const SnapArgs& a, int to_ring, hipStream_t s);
hipError_t launch_gated_norm(const NormArgs& a, hipStream_t s);
hipError_t launch_gating(const GatingArgs& a, hipStream_t s);
hipError_t launch_chunk_table(const ScanArgs& a, hipStream_t s);
hipError_t launch_prepare(const ScanArgs& a, hipStream_t s);
hipError_t launch_scan(const ScanArgs& a, hipStream_t s);
// true if launch_scan takes the segment-parallel path for these arguments
bool seg_path(const ScanArgs& a);
hipError_t launch_seg(const ScanArgs& a, hipStream_t s);
hipError_t launch_decode(const ScanArgs& a, hipStream_t s);
// decode step with the conv step fused in (c.x, c.stride_x, c.weight, c.bias,
// c.conv_state, c.channels and c.width are used; the window is per slot)
hipError_t launch_decode_conv(const ScanArgs& a, const ConvArgs& c, hipStream_t s);
// GDN_DEBUG: count non-finite values (fp32 or bf16) into *count (device int).
hipError_t launch_nonfinite_probe(const void* p, long n, int dtype, int* count, hipStream_t s);

}  // namespace gdn
