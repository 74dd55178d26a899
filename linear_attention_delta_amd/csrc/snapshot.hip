// snapshot.hip -- a ring of recurrent-state snapshots for prefix caching.
//
// The pages keep each sequence's state (the d_k x d_v fp32 memories of all
// v-heads and the causal-conv window) in a per-(sequence, layer) slot, and
// reuse a prompt prefix by restoring the state saved at its end instead of
// recomputing it (Vallmo.jl README, "What's here": recurrent state
// snapshot/restore gives prefix caching; PicoLM fork changelog, "SSM State
// Checkpointing": the state is saved periodically during prefill and
// generation, and on partial reuse the nearest saved state is restored and
// only the remaining tokens are processed).  Here a snapshot is a copy of
// the live slots into one entry of a caller-owned ring; restore copies an
// entry back.  Push takes its entry from a device counter, which it then
// advances, so a captured decode graph can push every N tokens with no host
// work.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kSnapThreads = 256;
constexpr int kSnapVecs = 4;                                  // 16-byte vectors per thread
constexpr long kSnapTile = 16L * kSnapThreads * kSnapVecs;    // bytes per workgroup

// One workgroup copies one 16 KB tile of one sequence's state or window.
// to_ring: live slot -> ring entry (push), else ring entry -> live slot.
__global__ void __launch_bounds__(kSnapThreads) k_snapshot(SnapArgs a, int to_ring) {
  const long st_tiles = (a.state_bytes + kSnapTile - 1) / kSnapTile;
  const long win_tiles = (a.window_bytes + kSnapTile - 1) / kSnapTile;
  const long per_seq = st_tiles + win_tiles;
  const long b = blockIdx.x / per_seq, t = blockIdx.x % per_seq;
  if (b >= a.num_seqs) return;
  const int slot = a.slots ? a.slots[b] : (int)b;
  if (slot < 0 || slot >= a.num_slots) return;  // not a live slot: leave both sides alone
  const int entry = a.head ? (int)(((long)*a.head % a.ring_len + a.ring_len) % a.ring_len) : a.entry;
  const bool win = t >= st_tiles;
  const long bytes = win ? a.window_bytes : a.state_bytes;
  char* live = reinterpret_cast<char*>(win ? a.window : a.state) + slot * bytes;
  char* ring = reinterpret_cast<char*>(win ? a.ring_window : a.ring_state) + ((long)entry * a.num_seqs + b) * bytes;
  const long off = (win ? t - st_tiles : t) * kSnapTile;
  const char* src = to_ring ? live : ring;
  char* dst = to_ring ? ring : live;
  u32x4 v[kSnapVecs];
#pragma unroll
  for (int j = 0; j < kSnapVecs; j++) {
    const long o = off + 16L * (threadIdx.x + kSnapThreads * j);
    if (o < bytes) v[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + o));
  }
#pragma unroll
  for (int j = 0; j < kSnapVecs; j++) {
    const long o = off + 16L * (threadIdx.x + kSnapThreads * j);
    if (o < bytes) __builtin_nontemporal_store(v[j], reinterpret_cast<u32x4*>(dst + o));
  }
}

// After every tile of a push has read the counter: advance it.
__global__ void k_ring_advance(int* head) {
  if (threadIdx.x == 0) *head += 1;
}

}  // namespace

hipError_t launch_snapshot(const SnapArgs& a, int to_ring, hipStream_t s) {
  const long per_seq = (a.state_bytes + kSnapTile - 1) / kSnapTile + (a.window_bytes + kSnapTile - 1) / kSnapTile;
  const long blocks = per_seq * a.num_seqs;
  if (blocks > 0) {
    if (blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(k_snapshot, dim3((unsigned)blocks), dim3(kSnapThreads), 0, s, a, to_ring);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (to_ring && a.head) {
    hipLaunchKernelGGL(k_ring_advance, dim3(1), dim3(64), 0, s, a.head);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace gdn
