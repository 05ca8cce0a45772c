/*
 * streamkl_probes.h - calibration probes for MI355X (gfx950), in their own
 * library (libstreamkl_probes.so) beside the attention-KL library.
 *
 * Each probe is one kernel with an exactly known amount of work; the caller
 * times it on `stream` with HIP events and divides.  They measure what the
 * hardware delivers to simple code on this GPU, the ceilings that the
 * attention-KL kernels are compared with:
 *   streamkl_probe_mfma    bf16 matrix-core rate (v_mfma_f32_32x32x16_bf16,
 *                          32768 flop per wave instruction, 4 per loop trip);
 *   streamkl_probe_mfma_data  the same with realistic operands (caller data,
 *                          changing on every instruction), from registers or
 *                          with the A operand from LDS;
 *   streamkl_probe_exp     v_exp_f32 issue rate (8 per lane per loop trip);
 *   streamkl_probe_exp_fma whether exp and FMA from two waves of a SIMD
 *                          issue in the same cycles;
 *   streamkl_probe_read    HBM read rate (16-byte loads, grid-stride, with or
 *                          without the non-temporal cache policy);
 *   streamkl_probe_atomic  fp32 atomic-add rate (4-byte payload per add).
 * They compute nothing of the method itself.
 *
 * Pointers are caller-owned device memory; nothing is allocated.  Returns 0,
 * -1 for invalid arguments (nothing launched) or -6 for a launch error.
 */
#ifndef STREAMKL_PROBES_H
#define STREAMKL_PROBES_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Threads per workgroup of every probe (sink arrays hold one value per thread). */
int streamkl_probe_threads(void);

/* workgroups x 4 waves, each `iters` trips of 4 independent MFMAs on constant
 * register operands.  waves_per_simd (1 to 3): each workgroup reserves enough
 * LDS that at most that many share a compute unit, i.e. that many waves per
 * SIMD.  sink: >= workgroups * threads floats (written, meaningless). */
int streamkl_probe_mfma(int waves_per_simd, int workgroups, int iters, float* sink, size_t sink_floats,
                        hipStream_t stream);

/* As streamkl_probe_mfma, but each lane cycles through 8 A and 8 B operand
 * chunks read from src (src_bytes >= workgroups * threads * 256, 16-byte
 * aligned); from_lds = 1 takes the A operand from a 32 KB LDS tile of that
 * data instead (one ds_read_b128 per lane per MFMA), from_lds = 2 the same
 * bytes through two transposing reads (ds_read_b64_tr_b16).  Operand reuse:
 * from_lds = 3 is mode 1 with each B chunk used by two consecutive MFMAs,
 * 4 the same pairing with both operands in registers, 5 one B chunk for four
 * consecutive MFMAs (registers).  Any other value is rejected (-1).  8 MFMAs
 * of 32768 flop per wave per loop trip in every mode. */
int streamkl_probe_mfma_data(const void* src, size_t src_bytes, int from_lds, int waves_per_simd, int workgroups,
                             int iters, float* sink, size_t sink_floats, hipStream_t stream);

/* workgroups x 256 threads, each `iters` trips of 8 independent v_exp_f32.
 * sink: >= workgroups * threads floats. */
int streamkl_probe_exp(int workgroups, int iters, float* sink, size_t sink_floats, hipStream_t stream);

/* Whether v_exp_f32 and v_fma_f32 from two waves on one SIMD issue together:
 * workgroups x 8 waves (512 threads), one workgroup per compute unit, each wave
 * `iters` trips of 8 independent chains.  mode 0: all waves exp; 1: all FMA;
 * 2: four waves exp and four FMA (one of each per SIMD).
 * sink: >= workgroups * 512 floats. */
int streamkl_probe_exp_fma(int mode, int workgroups, int iters, float* sink, size_t sink_floats,
                           hipStream_t stream);

/* Reads `bytes` (a multiple of 16) of src (16-byte aligned) once; nontemporal
 * != 0 marks the loads non-temporal (the nt cache policy, for data read once).
 * sink: >= workgroups * threads * 4 bytes. */
int streamkl_probe_read(const void* src, size_t bytes, int nontemporal, int workgroups, void* sink,
                        size_t sink_bytes, hipStream_t stream);

/* Adds 1.0f to each of dst[0 .. n_floats) `reps` times with fp32 atomics. */
int streamkl_probe_atomic(float* dst, size_t n_floats, int workgroups, int reps, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* STREAMKL_PROBES_H */
