// Direct-call timing of the decode entry point: gqa_decode_split is called
// back to back from C (no Python, no graph), rotating over several input
// sets, between two HIP events on the call's stream -- optionally queued
// behind a long read of device memory, during which the host enqueues the
// calls, so that the events bracket exactly the calls.  The entry point comes
// in as a function pointer, so this measurement library does not link
// libgqa.so.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../../include/gqa_probe.h"

namespace {

typedef int (*decode_split_fn)(const void*, const void*, const void*, const int32_t*, void*, int, int, int, int,
                               int, float, int, int, void*, size_t, void*);

}  // namespace

extern "C" int gqa_probe_time_decode_calls(void* fn, const void* const* q, const void* const* k_cache,
                                           const void* const* v_cache, const int32_t* const* seqlens,
                                           int n_inputs, void* out, int B, int H, int G, int d, int n_max,
                                           float scale, int dtype, int num_splits, void* workspace,
                                           size_t workspace_bytes, int warmup, int calls,
                                           const void* lead_buf, size_t lead_bytes, uint32_t* sink,
                                           void* stream, float* ms) {
  if (!fn || !q || !k_cache || !v_cache || !seqlens || !ms || n_inputs < 1 || calls < 1 || warmup < 0 ||
      (lead_buf && !sink))
    return 1;
  const decode_split_fn call = reinterpret_cast<decode_split_fn>(fn);
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto one = [&](int i) {
    const int r = i % n_inputs;
    return call(q[r], k_cache[r], v_cache[r], seqlens[r], out, B, H, G, d, n_max, scale, dtype, num_splits,
                workspace, workspace_bytes, stream);
  };
  for (int i = 0; i < warmup; ++i)
    if (one(i) != 0) return 2;
  hipEvent_t a = nullptr, b = nullptr;
  if (hipEventCreate(&a) != hipSuccess) return 4;
  if (hipEventCreate(&b) != hipSuccess) {
    (void)hipEventDestroy(a);
    return 4;
  }
  int rc = 0;
  if (hipStreamSynchronize(s) != hipSuccess) rc = 4;
  // the lead read keeps the device busy while the calls below are enqueued, so
  // that the start event is taken when the first timed call can start
  if (rc == 0 && lead_buf) rc = gqa_probe_hbm_read(lead_buf, lead_bytes, sink, 2048, 8, stream) == 0 ? 0 : 1;
  if (rc == 0 && hipEventRecord(a, s) != hipSuccess) rc = 4;
  for (int i = 0; rc == 0 && i < calls; ++i)
    if (one(i) != 0) rc = 2;
  if (rc == 0 && (hipEventRecord(b, s) != hipSuccess || hipEventSynchronize(b) != hipSuccess ||
                  hipEventElapsedTime(ms, a, b) != hipSuccess))
    rc = 4;
  (void)hipEventDestroy(a);
  (void)hipEventDestroy(b);
  return rc;
}
