/*
 * mla_verify_probe.h — measurement aids shipped in libmla_verify.so beside the
 * attention path (include/mla_verify.h). Neither is a step of the method: they
 * measure what this GPU sustains (matrix-core rate and clock, row-gather
 * rate), the ceilings against which the attention kernels' achieved rates are
 * read next to the published peaks. Same conventions as mla_verify.h: device
 * pointers, caller-owned memory, work enqueued on `stream`, 0 or a negative
 * MLA_ERR_* code (all checks before any HIP call).
 */
#ifndef MLA_VERIFY_PROBE_H
#define MLA_VERIFY_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Measurement aid, not a step of the attention path: the bf16 matrix-core rate
 * this GPU sustains under full load, against which the split kernel's achieved
 * TFLOP/s can be read next to the published dense peak (clocks under a full
 * matrix-core load sit well below the peak's). Launches `blocks` workgroups of
 * 4 waves; every wave runs `iters` rounds of 16 independent
 * v_mfma_f32_32x32x16_bf16 (32,768 flops each), so one launch performs
 * blocks x 4 x iters x 16 x 32,768 flops. Each thread writes one float of
 * `sink` (device memory, at least blocks x 256 floats); in each workgroup's
 * 256, element 0 holds the shader-clock cycles (s_memtime) and element 1 the
 * 100 MHz real-time ticks (s_memrealtime) that its MFMA loop took, so
 * sum(element 0) / sum(element 1) x 100 MHz is the clock under that load. Checks
 * (MLA_ERR_INVALID): 1 <= blocks <= 65,536, 1 <= iters <= 1,000,000, sink
 * non-NULL and 4-byte aligned. Enqueued on `stream`; time it with events. */
int mla_probe_mfma_bf16(int32_t blocks, int32_t iters, float* sink, void* stream);

/* Measurement aid, not a step of the attention path: gathers cache rows by index
 * with no compute, the rate against which the sparse path's gathered bytes can be
 * read. For group g and k < per_group, index i = indices[g * per_group + k]
 * selects row (g / tokens_per_seq) * kv_seq_stride + i of c_kv (1,024 bytes) and
 * of k_rope (128 bytes) when 0 <= i < kv_seq_stride (any i >= 0 when
 * kv_seq_stride is 0) and the row is below kv_rows; other indices are skipped. One
 * workgroup of 256 threads per (group, 64 indices), each thread writing one float
 * of `sink` (at least groups x ceil(per_group / 64) x 256 floats). Checks
 * (MLA_ERR_INVALID): pointers non-NULL, c_kv and k_rope 16-byte aligned, indices
 * and sink 4-byte aligned, kv_rows >= 1, 0 <= kv_seq_stride <= 2^21 (kv_rows <=
 * 2^21 when it is 0), groups, per_group, tokens_per_seq >= 1. Enqueued on
 * `stream`; time it with events. */
int mla_probe_gather_rows(const uint16_t* c_kv, const uint16_t* k_rope, int64_t kv_rows,
                          int64_t kv_seq_stride, const int32_t* indices, int32_t groups,
                          int32_t per_group, int32_t tokens_per_seq, float* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_VERIFY_PROBE_H */
