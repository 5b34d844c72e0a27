/*
 * rlk_probes.h -- measurement probes of the two resources the logprob kernels are bound by,
 * for the benchmark's "achievable ceiling" figures.  They are not part of the logprob API
 * (rlk_logprob.h) and live in their own library, librlk_probes.so, built from
 * entropy_rlk_logprob_amd/csrc/rlk_probes.hip for gfx950.
 *
 * Conventions as in rlk_logprob.h: device pointers owned by the caller, asynchronous on
 * `stream` (a hipStream_t passed as void*), no allocation, no synchronization.  Both return
 * 0 on success, a hipError_t value if the launch fails, and -1 (nothing launched) for bad
 * arguments.
 */
#ifndef RLK_PROBES_H
#define RLK_PROBES_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Streaming read: `bytes` of device memory at `buf` (16-byte aligned, bytes a positive
 * multiple of 16) read once with 16-byte non-temporal loads by 2048 workgroups of 256
 * threads in a grid-stride loop -- the access pattern of a plain bandwidth test.  `sink`
 * ([2048 * 256] floats) is written only if a lane's sum of the values it read equals
 * 1234.5 exactly, which keeps the loads from being removed.  Rate = bytes / time. */
int rlk_probe_stream_read(const void* buf, size_t bytes, float* sink, void* stream);

/* Register-only MFMA loop: `blocks` workgroups of 4 waves; each wave keeps 8 accumulators
 * of v_mfma_f32_32x32x16_bf16 and runs `iters` (a positive multiple of 4) steps of 8 MFMAs
 * on operands held in registers: 4 + 2 fragments of pseudo-random finite bf16 values drawn
 * from `seed`, rotated from step to step so that every MFMA sees changing data, as a GEMM's
 * do.  Each thread writes the sum of its accumulators to sink[block * 256 + thread].
 * Work = blocks * 4 * iters * 8 * 32768 flop. */
int rlk_probe_mfma(int32_t blocks, int32_t iters, uint32_t seed, float* sink, void* stream);

/* Properties of the current device behind the peak figures (host only, launches nothing):
 * the compute-unit count, the peak engine clock and the memory clock in kHz, the memory bus
 * width in bits, and the architecture name (NUL-terminated, truncated to arch_len - 1).  The
 * dense bf16 MFMA peak is compute_units x engine clock x 4096 flop per clock.  Returns 0, a
 * hipError_t value if the query fails, or -1 for a null pointer. */
int rlk_probe_device_info(int32_t* compute_units, int32_t* engine_clock_khz,
                          int32_t* memory_clock_khz, int32_t* memory_bus_bits, char* arch,
                          size_t arch_len);

#ifdef __cplusplus
}
#endif

#endif /* RLK_PROBES_H */
