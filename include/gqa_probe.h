/*
 * gqa_probe.h - C ABI of libgqa_probe.so: measurement probes for the
 * benchmark (not part of the attention library).
 *
 * gqa_probe_hbm_read - read `bytes` of device memory once with 16-byte
 * non-temporal loads (every lane keeps `unroll` loads in flight, `blocks`
 * workgroups of 256 threads stride over the buffer) and fold them into one
 * value that is written to sink[0] only if it equals a fixed key.  Timing
 * calls over a buffer much larger than the 256 MB last-level cache gives the
 * HBM read rate a streaming kernel can reach: the measured ceiling against
 * which the memory-bound kernels are also reported.
 *
 *   buf     device pointer, 16-byte aligned; bytes a positive multiple of 16.
 *   sink    device pointer to at least 4 writable bytes.
 *   blocks  1 .. 2^20;  unroll  4, 8 or 16.
 *   stream  hipStream_t as void* (enqueued asynchronously).
 * Returns 0, 1 for an invalid argument (nothing enqueued), 4 if the launch
 * was refused.
 */
#ifndef GQA_PROBE_H_
#define GQA_PROBE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int gqa_probe_hbm_read(const void* buf, size_t bytes, uint32_t* sink, int blocks, int unroll,
                       void* stream);

/*
 * gqa_probe_valu_rate - vector-unit issue rate: `blocks` workgroups of 256
 * threads, every lane running 8 independent chains of 4096 steps of one
 * instruction kind -- kind 0: v_fma_f32, 1: v_exp_f32 (on -|x|, so values stay
 * in (0, 1]), 2: one of each per step.  The launch time over the whole chip
 * gives the SIMD cycles per wave64 instruction of that kind, and kind 2 shows
 * whether an exp overlaps an FMA.  out: device, blocks * 256 floats (written).
 * Returns 0, 1 for an invalid argument (nothing enqueued), 4 if the launch was
 * refused.
 */
int gqa_probe_valu_rate(float* out, int kind, int blocks, void* stream);

/*
 * gqa_probe_lds_rate - LDS read rate: `blocks` workgroups of 256 threads,
 * each filling a 64 KB LDS array and reading it with 8 x 4096 instructions
 * per wave of one kind -- kind 0: ds_read_b128 (16 bytes per lane, each
 * 16-lane quarter covering the 64 banks once); 1: ds_read_b64_tr_b16 (8
 * bytes per lane) at the addresses from which the causal prefill kernel reads
 * its transposed V operand at d = 128.  Two workgroups share a compute unit,
 * so 512 blocks fill the chip; the launch time gives the LDS cycles per wave
 * instruction of that kind.  sink: device, 4 bytes, written only if the
 * folded data equals a fixed key.  Returns 0, 1 for an invalid argument
 * (nothing enqueued), 4 if the launch was refused.
 */
int gqa_probe_lds_rate(uint32_t* sink, int kind, int blocks, void* stream);

/*
 * gqa_probe_time_decode_calls - timing of the decode step by direct calls:
 * `warmup` untimed calls, then `calls` back-to-back calls of `fn` -- a
 * pointer to libgqa.so's gqa_decode_split, passed in so that this library
 * does not link the attention library -- made directly from C, call i
 * reading input set i % n_inputs, between two HIP events recorded on
 * `stream`.  With lead_buf, a read of lead_bytes of it (gqa_probe_hbm_read,
 * 2048 blocks, unroll 8; sink as there) is queued just before the start
 * event: the host enqueues the calls while it runs, so the events bracket
 * exactly the calls.  The elapsed milliseconds of the timed calls go to *ms.
 *
 *   q, k_cache, v_cache, seqlens  host arrays of n_inputs device pointers
 *   other arguments               passed through to gqa_decode_split
 * Returns 0; 1 for an invalid argument (nothing called; an invalid lead read
 * after the warmup calls also returns 1); 2 if a call returned a non-zero
 * status (its detail: gqa_last_error in libgqa.so); 4 for a failed HIP
 * event or synchronisation call.
 */
int gqa_probe_time_decode_calls(void* fn, const void* const* q, const void* const* k_cache,
                                const void* const* v_cache, const int32_t* const* seqlens,
                                int n_inputs, void* out, int B, int H, int G, int d, int n_max,
                                float scale, int dtype, int num_splits, void* workspace,
                                size_t workspace_bytes, int warmup, int calls,
                                const void* lead_buf, size_t lead_bytes, uint32_t* sink,
                                void* stream, float* ms);

#ifdef __cplusplus
}
#endif

#endif /* GQA_PROBE_H_ */
