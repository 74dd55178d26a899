// Drives the C ABI's host-side paths that need no GPU -- validation of every
// entry point, workspace sizing, status strings, the no-allocation prefill's
// size check -- so that an AddressSanitizer / UndefinedBehaviorSanitizer
// build of the ABI layer can check them.  Calls that pass validation reach
// the HIP runtime, which has no device here and reports an error.  Exit
// status 0 when every call returned the expected status class.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "gdn.h"

static int bad = 0;
static void expect(bool ok, const char* what) {
  if (!ok) {
    std::printf("unexpected: %s (%s)\n", what, gdn_last_error());
    bad = 1;
  }
}
static const void* P(uintptr_t a) { return reinterpret_cast<const void*>(a); }
static void* M(uintptr_t a) { return reinterpret_cast<void*>(a); }

int main() {
  gdn_dims d;
  std::memset(&d, 0, sizeof d);
  d.num_seqs = 1; d.total_tokens = 4096; d.seqlen = 4096; d.num_qk_heads = 16; d.num_v_heads = 32;
  d.head_dim_k = 128; d.head_dim_v = 128; d.chunk_size = 64; d.dtype = GDN_BF16; d.flags = GDN_QK_L2NORM;
  d.scale = 1.0f;
  expect(gdn_validate_dims(&d, 0) == GDN_OK, "valid dims");
  const size_t ws = gdn_prefill_workspace_size(&d);
  expect(ws > 0, "workspace size");
  for (int s = 0; s <= 6; s++) expect(std::strlen(gdn_status_string((gdn_status)s)) > 0, "status string");
  expect(std::strlen(gdn_version()) > 0, "version");
  // every field out of range, one at a time
  gdn_dims e = d; e.num_seqs = 0; expect(gdn_validate_dims(&e, 0) == GDN_ERR_INVALID_ARG, "num_seqs");
  e = d; e.num_v_heads = 24; expect(gdn_validate_dims(&e, 0) == GDN_ERR_INVALID_ARG, "heads");
  e = d; e.head_dim_k = 96; expect(gdn_validate_dims(&e, 0) == GDN_ERR_UNSUPPORTED, "head dim");
  e = d; e.chunk_size = 48; expect(gdn_validate_dims(&e, 0) == GDN_ERR_UNSUPPORTED, "chunk");
  e = d; e.stride_q = 100; expect(gdn_validate_dims(&e, 0) == GDN_ERR_INVALID_ARG, "stride");
  e = d; e.flags = 8; expect(gdn_validate_dims(&e, 0) == GDN_ERR_INVALID_ARG, "flags");
  e = d; e.reserved = 1; expect(gdn_validate_dims(&e, 0) == GDN_ERR_INVALID_ARG, "reserved");
  e = d; e.total_tokens = -1; expect(gdn_prefill_workspace_size(&e) == 0, "bad workspace size");
  expect(gdn_validate_dims(nullptr, 0) == GDN_ERR_INVALID_ARG, "null dims");
  // whole calls through gdn_validate
  const void* pre[10] = {P(16), P(32), P(48), P(64), P(80), P(1 << 26), nullptr, P(96), P(1 << 26), P(256)};
  expect(gdn_validate(&d, 0, pre, 10, (int64_t)ws) == GDN_OK, "validate prefill");
  expect(gdn_validate(&d, 0, pre, 10, (int64_t)ws - 256) == GDN_ERR_WORKSPACE, "small workspace");
  expect(gdn_validate(&d, 0, pre, 9, (int64_t)ws) == GDN_ERR_INVALID_ARG, "pointer count");
  expect(gdn_validate(&d, 0, nullptr, 10, (int64_t)ws) == GDN_ERR_INVALID_ARG, "null pointers");
  gdn_dims dd = d; dd.num_seqs = 64; dd.total_tokens = 64; dd.seqlen = 1;
  const void* dec[8] = {P(16), P(32), P(48), P(64), P(80), P(1 << 26), nullptr, P(96)};
  expect(gdn_validate(&dd, 1, dec, 8, 64) == GDN_OK, "validate decode");
  expect(gdn_validate(&dd, 1, dec, 8, 63) == GDN_ERR_INVALID_ARG, "decode slots");
  // entry points rejecting bad arguments before any HIP call
  expect(gdn_prefill_chunked(&d, P(16), P(16), P(16), (const float*)P(16), (const float*)P(16), nullptr, nullptr,
                             M(16), nullptr, M(256), 1024, nullptr) == GDN_ERR_WORKSPACE, "chunked workspace");
  expect(gdn_prefill_chunked(&d, P(16), P(16), P(16), (const float*)P(16), (const float*)P(16),
                             (const float*)P(1 << 26), nullptr, M(16), (float*)M((1 << 26) + 16), M(256), ws,
                             nullptr) == GDN_ERR_INVALID_ARG, "state overlap");
  expect(gdn_conv1d(1, 10, 10, nullptr, 60, 4, GDN_BF16, P(16), 64, (const float*)P(16), nullptr, nullptr, 1, M(16),
                    64, nullptr) == GDN_ERR_INVALID_ARG, "conv channels");
  expect(gdn_gated_rmsnorm(4, 2, 96, GDN_BF16, P(16), 256, P(16), 256, (const float*)P(16), 1e-6f, M(16), 256,
                           nullptr) == GDN_ERR_UNSUPPORTED, "norm head dim");
  expect(gdn_gating(4, 2, GDN_BF16, P(16), 1, P(16), 2, (const float*)P(16), (const float*)P(16), (float*)M(64),
                    (float*)M(128), nullptr) == GDN_ERR_INVALID_ARG, "gating stride");
  expect(gdn_snapshot_restore(4, nullptr, 4, 16, (float*)M(1 << 20), 0, nullptr, 3, (const float*)P(1 << 24),
                              nullptr, 3, nullptr) == GDN_ERR_INVALID_ARG, "snapshot entry");
  expect(gdn_decode_step(&dd, P(16), P(16), P(16), (const float*)P(16), (const float*)P(16), nullptr, 64, nullptr,
                         M(16), nullptr) == GDN_ERR_INVALID_ARG, "decode state");
  gdn_dims big = d; big.total_tokens = big.seqlen = 8192;
  expect(gdn_prefill_chunked_noalloc(&big, P(16), P(16), P(16), (const float*)P(16), (const float*)P(16), nullptr,
                                     nullptr, M(16), nullptr, nullptr) == GDN_ERR_UNSUPPORTED, "noalloc size");
  // valid calls reach the runtime, which has no device here
  const gdn_status st = gdn_prefill_chunked(&d, P(16), P(16), P(16), (const float*)P(16), (const float*)P(16), nullptr,
                                            nullptr, M(16), nullptr, M(256), ws, nullptr);
  expect(st == GDN_ERR_HIP || st == GDN_OK, "valid call");
  std::printf(bad ? "abi driver: FAILED\n" : "abi driver: ok\n");
  return bad;
}
