/*
 * mqa_probe.h - a measurement probe shipped with libmqa; not part of the operation.
 *
 * mqa_probe_gather reads the bytes that mqa_paged_logits reads for a list of 132-byte
 * cache rows (each row's 128 key bytes and 4-byte scale, with the same per-lane access
 * pattern) and nothing else, so its time is the ceiling of the gather step of the
 * logits on this GPU for that row order. The row format is the cache row of the
 * stepcodex.com pa_mqa_logits issue, section "Minimal reproduction" (128 e4m3fn key
 * bytes followed by one fp32 scale).
 *
 *   kv_cache            device, [num_rows_in_cache, 132] bytes, 4-byte aligned
 *   num_rows_in_cache   >= 1; a listed row outside [0, num_rows_in_cache) reads row 0
 *   rows                device int32 [n], the cache rows in the order they are visited
 *   n                   >= 0 (0 enqueues nothing)
 *   groups_per_cu       1..8 workgroups of 256 threads (4 waves) per compute unit; each
 *                       wave walks a contiguous share of the list
 *   stages_in_flight    2 or 4 stages of 64 rows each wave keeps loading ahead
 *   sink                device int32 [sink_words], written (one folded word per lane),
 *                       4-byte aligned; sink_words >= mqa_probe_gather_sink_words(groups_per_cu)
 * Returns 0 on success, 1 for a NULL pointer, 2 for a bad size, 3 for a bad
 * groups_per_cu or stages_in_flight or a misaligned pointer, 4 for a short sink, 5 for a launch error. The
 * work is enqueued on `stream`; nothing is allocated or synchronised.
 *
 * mqa_probe_gather_lds gathers the same rows straight into LDS (global_load_lds_dwordx4, no
 * registers held by the loads in flight): each row's 16-byte-aligned 144-byte window, which
 * contains its 132 bytes, as nine 16-byte pieces, 64 rows per stage, each wave into its own
 * LDS area, then one dword per piece is read back from LDS and folded into the sink.
 * Arguments and returns as mqa_probe_gather, except: stages_in_flight is 2 or 3 (9 KB of
 * LDS per wave per stage; a workgroup holds about 80 KB with 2 stages, 116 KB with 3, so at
 * most 2 or 1 workgroups share a compute unit whatever groups_per_cu asks), and kv_cache
 * must be 16-byte aligned.
 */
#ifndef MQA_PROBE_H
#define MQA_PROBE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

size_t mqa_probe_gather_sink_words(int32_t groups_per_cu);

int mqa_probe_gather(const uint8_t* kv_cache, int64_t num_rows_in_cache, const int32_t* rows, int64_t n,
                     int32_t groups_per_cu, int32_t stages_in_flight, int32_t* sink, size_t sink_words,
                     hipStream_t stream);

int mqa_probe_gather_lds(const uint8_t* kv_cache, int64_t num_rows_in_cache, const int32_t* rows, int64_t n,
                         int32_t groups_per_cu, int32_t stages_in_flight, int32_t* sink, size_t sink_words,
                         hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MQA_PROBE_H */
