// Calibration probes for the ceilings quoted beside the attention-KL kernels:
// how fast this GPU runs a pure bf16 MFMA loop, a stream of v_exp_f32, a
// plain read of a large buffer and fp32 atomic adds.  Each probe is one
// kernel whose work is known exactly; the caller times it with HIP events.
// Every access stays inside the buffers the caller passes (sizes checked on
// the host), and every loop has a fixed trip count.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "streamkl_probes.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

// LDS a matrix-core probe workgroup reserves so that at most WPS of them fit in
// the 160 KB of a CU.  A workgroup is 4 waves, one per SIMD, so WPS is also the
// number of waves per SIMD (the registers of these kernels allow up to 3).
// How many waves share a SIMD changes what the matrix cores sustain.
template <int WPS>
constexpr int reserve_bytes() {
  static_assert(WPS >= 1 && WPS <= 3, "1 to 3 waves per SIMD");
  return WPS == 1 ? 96 * 1024 : WPS == 2 ? 64 * 1024 : 48 * 1024;
}

// The per-lane result goes through the reserved LDS on its way to sink[gid],
// so the reservation is part of the kernel and nothing is optimised away.
template <int WPS>
__device__ __forceinline__ void store_through_lds(u32x4* lds, float s, float* __restrict__ sink, int gid) {
  __syncthreads();
  lds[threadIdx.x] = u32x4{__float_as_uint(s), 0u, 0u, 0u};
  __syncthreads();
  sink[gid] = __uint_as_float(lds[(threadIdx.x + 1) % kThreads].x);
}

// Four independent accumulator chains of v_mfma_f32_32x32x16_bf16 per wave,
// operands in registers.  One lane's sum of the results goes to sink[gid] so
// that nothing is optimised away.
template <int WPS>
__global__ __launch_bounds__(kThreads) void mfma_loop(int iters, float* __restrict__ sink) {
  __shared__ u32x4 lds[reserve_bytes<WPS>() / 16];
  const int gid = blockIdx.x * kThreads + threadIdx.x;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * (float)((threadIdx.x + e) & 7));
    b[e] = (__bf16)(0.002f * (float)((threadIdx.x * 3 + e) & 7));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  store_through_lds<WPS>(lds, s, sink, gid);
}

// 16 bytes at tile[idx] (idx < 2048) through two transposing 8-byte reads.
__device__ __forceinline__ u32x4 read_tr_16(const u32x4* tile, int idx) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const __attribute__((address_space(3))) char* p = (const __attribute__((address_space(3))) char*)(tile + idx);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p + 8));
  const u32x2 l = __builtin_bit_cast(u32x2, lo), h = __builtin_bit_cast(u32x2, hi);
  return u32x4{l.x, l.y, h.x, h.y};
}

// The same MFMA loop with realistic operands: each lane holds 8 different A
// and B chunks loaded from `src` (caller-supplied data, 256 bytes per thread),
// so the multiplier inputs change on every instruction as they do on real
// tiles.  SRC 1: the A operand comes from a 32 KB LDS tile of the same data
// instead (one 16-byte ds_read_b128 per lane per MFMA, the score-MFMA access
// pattern); SRC 2: the same bytes through two transposing 8-byte reads
// (ds_read_b64_tr_b16, the gradient-MFMA access pattern of the backward).
// Operand reuse: SRC 3 is SRC 1 with each B chunk used by two consecutive
// MFMAs (two key blocks against one register-held query chunk); SRC 4 the
// same pairing from registers only; SRC 5 one B chunk for four consecutive
// MFMAs, from registers.  The MFMA count is the same in every mode.
template <int SRC, int WPS>
__global__ __launch_bounds__(kThreads) void mfma_data_loop(const u32x4* __restrict__ src, int iters,
                                                          float* __restrict__ sink) {
  constexpr bool LDS = SRC == 1 || SRC == 2 || SRC == 3;
  static_assert(reserve_bytes<WPS>() >= 2048 * 16, "the LDS tile lives in the reservation");
  __shared__ u32x4 tile[reserve_bytes<WPS>() / 16];
  const int gid = blockIdx.x * kThreads + threadIdx.x;
  const int lane = threadIdx.x & 63;
  u32x4 a[8], b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = src[(size_t)gid * 16 + i];
    b[i] = src[(size_t)gid * 16 + 8 + i];
  }
  if (LDS) {
    // this workgroup's 256 threads x 256 bytes = 64 KB of src; its first 32 KB fill the tile
    for (int i = threadIdx.x; i < 2048; i += kThreads) tile[i] = src[(size_t)blockIdx.x * kThreads * 16 + i];
    __syncthreads();
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; i += 4) {
      u32x4 x0 = a[i], x1 = a[i + 1], x2 = a[i + 2], x3 = a[i + 3];
      if (SRC == 1 || SRC == 3) {
        const int o = (it * 8 + i) * 64 + lane;
        x0 = tile[o & 2047];
        x1 = tile[(o + 64) & 2047];
        x2 = tile[(o + 128) & 2047];
        x3 = tile[(o + 192) & 2047];
      } else if (SRC == 2) {
        const int o = (it * 8 + i) * 64 + lane;
        x0 = read_tr_16(tile, o & 2047);
        x1 = read_tr_16(tile, (o + 64) & 2047);
        x2 = read_tr_16(tile, (o + 128) & 2047);
        x3 = read_tr_16(tile, (o + 192) & 2047);
      }
      constexpr bool PAIR = SRC == 3 || SRC == 4, QUAD = SRC == 5;
      const u32x4 y0 = b[i], y1 = (PAIR || QUAD) ? b[i] : b[i + 1];
      const u32x4 y2 = QUAD ? b[i] : b[i + 2], y3 = QUAD ? b[i] : PAIR ? b[i + 2] : b[i + 3];
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, x0), __builtin_bit_cast(bf16x8, y0),
                                                    c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, x1), __builtin_bit_cast(bf16x8, y1),
                                                    c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, x2), __builtin_bit_cast(bf16x8, y2),
                                                    c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, x3), __builtin_bit_cast(bf16x8, y3),
                                                    c3, 0, 0, 0);
      // Register operands: keep the loop's scalar bookkeeping out from between
      // the MFMAs.  With two or three waves per SIMD, a scalar instruction
      // between them measurably lowers the rate this loop sustains, below the
      // board's power limit, and the probe is meant to show the matrix cores'
      // own ceiling.
      if (!LDS) __builtin_amdgcn_sched_barrier(0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  store_through_lds<WPS>(tile, s, sink, gid);
}

// Eight independent chains x <- 2^(-x) of v_exp_f32 per lane (the negation is
// a free source modifier), so the loop is one transcendental instruction per
// element and its rate is the issue rate of v_exp_f32.
__global__ __launch_bounds__(kThreads) void exp_loop(int iters, float* __restrict__ sink) {
  const int gid = blockIdx.x * kThreads + threadIdx.x;
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = 0.01f * (float)((threadIdx.x + j) & 15);
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = __builtin_amdgcn_exp2f(-x[j]);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += x[j];
  sink[gid] = s;
}

// Eight waves per workgroup, one workgroup per CU (LDS reservation), so each
// SIMD holds two waves (waves w and w + 4 of a workgroup share a SIMD as the
// dispatcher deals them out).  MODE 0: every wave runs eight independent
// v_exp_f32 chains; MODE 1: eight independent v_fma_f32 chains; MODE 2: waves
// 0-3 run the exp chains and waves 4-7 the FMA chains, so each SIMD holds one
// of each.  Equal instruction counts per wave in every mode: comparing the
// three times shows whether a transcendental from one wave and an FMA from
// another issue in the same cycles or take turns.
constexpr int kMixThreads = 512;

template <int MODE>
__global__ __launch_bounds__(kMixThreads) void exp_fma_loop(int iters, float* __restrict__ sink) {
  __shared__ float lds[96 * 1024 / 4];
  const int gid = blockIdx.x * kMixThreads + threadIdx.x;
  const int wave = threadIdx.x / 64;
  const bool exp_wave = MODE == 0 || (MODE == 2 && wave < 4);
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = 0.01f * (float)((threadIdx.x + j) & 15);
  if (exp_wave) {
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = __builtin_amdgcn_exp2f(-x[j]);
    }
  } else {
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = __builtin_fmaf(x[j], 0.999f, 0.001f);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += x[j];
  // through the reserved LDS, so the reservation is part of the kernel
  __syncthreads();
  lds[threadIdx.x] = s;
  __syncthreads();
  sink[gid] = lds[(threadIdx.x + 1) % kMixThreads];
}

// Grid-stride read of n16 16-byte words, four independent loads in flight
// per thread; a per-thread XOR of what was read goes to sink[gid].  NT: the
// loads carry the non-temporal cache policy (data read once).
template <bool NT>
__global__ __launch_bounds__(kThreads) void read_loop(const u32x4* __restrict__ src, size_t n16,
                                                       uint32_t* __restrict__ sink) {
  const size_t gid = (size_t)blockIdx.x * kThreads + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * kThreads;
  auto load = [&](size_t i) { return NT ? __builtin_nontemporal_load(src + i) : src[i]; };
  uint32_t acc = 0;
  size_t i = gid;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 v0 = load(i), v1 = load(i + stride), v2 = load(i + 2 * stride), v3 = load(i + 3 * stride);
    acc ^= (v0.x ^ v0.y ^ v0.z ^ v0.w) ^ (v1.x ^ v1.y ^ v1.z ^ v1.w) ^ (v2.x ^ v2.y ^ v2.z ^ v2.w) ^
           (v3.x ^ v3.y ^ v3.z ^ v3.w);
  }
  for (; i < n16; i += stride) {
    const u32x4 v = load(i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  sink[gid] = acc;
}

// `reps` passes of one fp32 atomic add of 1.0 to each of the n floats of dst,
// consecutive lanes on consecutive addresses.
__global__ __launch_bounds__(kThreads) void atomic_loop(float* __restrict__ dst, size_t n, int reps) {
  const size_t gid = (size_t)blockIdx.x * kThreads + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * kThreads;
  for (int r = 0; r < reps; ++r)
    for (size_t i = gid; i < n; i += stride) atomicAdd(dst + i, 1.0f);
}

int status(hipError_t e) { return e == hipSuccess ? 0 : -6; }

template <int SRC>
hipError_t launch_mfma_data(int waves_per_simd, int workgroups, const u32x4* src, int iters, float* sink,
                            hipStream_t stream) {
  if (waves_per_simd == 1)
    hipLaunchKernelGGL((mfma_data_loop<SRC, 1>), dim3(workgroups), dim3(kThreads), 0, stream, src, iters, sink);
  else if (waves_per_simd == 2)
    hipLaunchKernelGGL((mfma_data_loop<SRC, 2>), dim3(workgroups), dim3(kThreads), 0, stream, src, iters, sink);
  else
    hipLaunchKernelGGL((mfma_data_loop<SRC, 3>), dim3(workgroups), dim3(kThreads), 0, stream, src, iters, sink);
  return hipGetLastError();
}

}  // namespace

extern "C" {

int streamkl_probe_threads(void) { return kThreads; }

int streamkl_probe_mfma(int waves_per_simd, int workgroups, int iters, float* sink, size_t sink_floats,
                        hipStream_t stream) {
  if (waves_per_simd < 1 || waves_per_simd > 3 || workgroups < 1 || iters < 1 || !sink ||
      sink_floats < (size_t)workgroups * kThreads)
    return -1;
  if (waves_per_simd == 1)
    hipLaunchKernelGGL(mfma_loop<1>, dim3(workgroups), dim3(kThreads), 0, stream, iters, sink);
  else if (waves_per_simd == 2)
    hipLaunchKernelGGL(mfma_loop<2>, dim3(workgroups), dim3(kThreads), 0, stream, iters, sink);
  else
    hipLaunchKernelGGL(mfma_loop<3>, dim3(workgroups), dim3(kThreads), 0, stream, iters, sink);
  return status(hipGetLastError());
}

int streamkl_probe_mfma_data(const void* src, size_t src_bytes, int from_lds, int waves_per_simd, int workgroups,
                             int iters, float* sink, size_t sink_floats, hipStream_t stream) {
  if (!src || from_lds < 0 || from_lds > 5 || waves_per_simd < 1 || waves_per_simd > 3 || workgroups < 1 ||
      iters < 1 || !sink ||
      sink_floats < (size_t)workgroups * kThreads || ((uintptr_t)src & 15) != 0 ||
      src_bytes < (size_t)workgroups * kThreads * 256)
    return -1;
  const u32x4* s = (const u32x4*)src;
  if (from_lds == 5) return status(launch_mfma_data<5>(waves_per_simd, workgroups, s, iters, sink, stream));
  if (from_lds == 4) return status(launch_mfma_data<4>(waves_per_simd, workgroups, s, iters, sink, stream));
  if (from_lds == 3) return status(launch_mfma_data<3>(waves_per_simd, workgroups, s, iters, sink, stream));
  if (from_lds == 2) return status(launch_mfma_data<2>(waves_per_simd, workgroups, s, iters, sink, stream));
  if (from_lds == 1) return status(launch_mfma_data<1>(waves_per_simd, workgroups, s, iters, sink, stream));
  return status(launch_mfma_data<0>(waves_per_simd, workgroups, s, iters, sink, stream));
}

int streamkl_probe_exp(int workgroups, int iters, float* sink, size_t sink_floats, hipStream_t stream) {
  if (workgroups < 1 || iters < 1 || !sink || sink_floats < (size_t)workgroups * kThreads) return -1;
  hipLaunchKernelGGL(exp_loop, dim3(workgroups), dim3(kThreads), 0, stream, iters, sink);
  return status(hipGetLastError());
}

int streamkl_probe_exp_fma(int mode, int workgroups, int iters, float* sink, size_t sink_floats,
                           hipStream_t stream) {
  if (mode < 0 || mode > 2 || workgroups < 1 || iters < 1 || !sink || sink_floats < (size_t)workgroups * kMixThreads)
    return -1;
  if (mode == 0)
    hipLaunchKernelGGL(exp_fma_loop<0>, dim3(workgroups), dim3(kMixThreads), 0, stream, iters, sink);
  else if (mode == 1)
    hipLaunchKernelGGL(exp_fma_loop<1>, dim3(workgroups), dim3(kMixThreads), 0, stream, iters, sink);
  else
    hipLaunchKernelGGL(exp_fma_loop<2>, dim3(workgroups), dim3(kMixThreads), 0, stream, iters, sink);
  return status(hipGetLastError());
}

int streamkl_probe_read(const void* src, size_t bytes, int nontemporal, int workgroups, void* sink,
                        size_t sink_bytes, hipStream_t stream) {
  if (!src || !sink || workgroups < 1 || bytes % 16 != 0 || ((uintptr_t)src & 15) != 0 ||
      sink_bytes < (size_t)workgroups * kThreads * sizeof(uint32_t))
    return -1;
  if (nontemporal)
    hipLaunchKernelGGL(read_loop<true>, dim3(workgroups), dim3(kThreads), 0, stream, (const u32x4*)src, bytes / 16,
                       (uint32_t*)sink);
  else
    hipLaunchKernelGGL(read_loop<false>, dim3(workgroups), dim3(kThreads), 0, stream, (const u32x4*)src, bytes / 16,
                       (uint32_t*)sink);
  return status(hipGetLastError());
}

int streamkl_probe_atomic(float* dst, size_t n_floats, int workgroups, int reps, hipStream_t stream) {
  if (!dst || n_floats < 1 || workgroups < 1 || reps < 1) return -1;
  hipLaunchKernelGGL(atomic_loop, dim3(workgroups), dim3(kThreads), 0, stream, dst, n_floats, reps);
  return status(hipGetLastError());
}

}  // extern "C"
