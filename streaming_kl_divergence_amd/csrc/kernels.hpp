// Launch interface between the C ABI (api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>

namespace skl {

// Forward / split-K partial kernel arguments.
struct FwdParams {
  const char* q1;
  const char* k1;
  const char* q2;
  const char* k2;
  int n_q, n_k, heads, causal;
  float scale;   // softmax scale
  float c;       // scale * log2(e): exponent factor for exp2
  float* kl;
  float* lse1;
  float* lse2;
  float* part;      // split-K: partial states [splits][heads][n_q][5]
  int splits;       // split-K: number of key ranges
  int split_keys;   // split-K: keys per range (a multiple of the key tile)
};

// Key tile of the forward kernel (keys per LDS tile).
constexpr int kFwdKeyTile = 64;

// Queries per workgroup of the forward kernel for a given wave count.
inline int fwd_queries_per_block(int nw) { return 32 * nw; }

// Waves per workgroup the forward uses for n_q queries.
inline int fwd_waves(int n_q) { return n_q <= 32 ? 1 : 4; }

hipError_t launch_fwd(const FwdParams& p, int dtype, int head_dim, int nw, bool split,
                      hipStream_t stream);
hipError_t launch_splitk_combine(const FwdParams& p, hipStream_t stream);

// Bytes of the fixed device scratch behind streamkl_fwd_splitk_noalloc (the
// split-K partial states, 20 bytes per (range, head, query)).
constexpr size_t kNoAllocScratchBytes = (size_t)8 << 20;
// Device address of that scratch on the current device (looked up on the
// first call per device and kept).
hipError_t noalloc_scratch(float** out);

// Backward kernel arguments (both settings).
struct BwdParams {
  const char* q1;
  const char* k1;
  const char* q2;
  const char* k2;
  int n_q, n_k, heads, causal;
  float scale, c;
  const float* lse1;
  const float* lse2;
  const float* kl;    // Setting 2 only
  const float* dkl;   // NULL = all ones
  float* dq;          // gradient of the setting's Q (fp32); both settings: dQ2
  float* dk;          // gradient of the setting's K (fp32); both settings: dK2
  float* dq1;         // both settings: dQ1 (Setting 2's gradients)
  float* dk1;         // both settings: dK1
  int setting;        // 1 or 2 (ignored by the both-settings launch)
  int dq_splits;      // separate path: key ranges of the dQ kernel (1 = plain stores)
};

hipError_t launch_bwd_separate(const BwdParams& p, int dtype, int head_dim, bool dk, bool dq, hipStream_t stream);
hipError_t launch_bwd_fused(const BwdParams& p, int dtype, int head_dim, hipStream_t stream);
// Both settings from one recomputation: dQ2, dK2 into p.dq, p.dk and dQ1, dK1
// into p.dq1, p.dk1 (needs p.kl); dk / dq select the key-block and the
// query-block kernel.  fp32 inputs run the two settings one after the other
// on the separate kernels.
hipError_t launch_bwd_both(const BwdParams& p, int dtype, int head_dim, bool dk, bool dq, hipStream_t stream);

// Whether the fused kernel's LDS footprint fits a workgroup for this dtype and head_dim.
bool fused_supported(int dtype, int head_dim);

// Queries per workgroup of the separate dQ kernel; keys per workgroup of the key-block kernels.
constexpr int kBwdQueriesPerBlock = 128;
constexpr int kBwdKeysPerBlock = 128;

}  // namespace skl
