// Backward pieces shared by the single-setting kernels (bwd.hip) and the
// both-settings kernels (bwd_both.hip): LDS tile geometry of the key-block and
// query-block kernels and the transposed-operand gradient MFMA.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace skl {

// ---- transposed LDS tiles ------------------------------------------------------
// XT[d][j] (d < D, j < R) of element T; row stride R*sizeof(T) + PAD bytes.
template <typename T, int D, int R, int PAD>
struct TGeom {
  static constexpr int kStride = R * (int)sizeof(T) + PAD;
  static constexpr int kBytes = D * kStride;
};

template <typename T, int D>
struct KvCfg {
  static constexpr int NW = 4;
  static constexpr int BKW = 32 * NW;                                    // keys per workgroup
  static constexpr int BT = (sizeof(T) == 4 && D == 128) ? 32 : 64;      // queries per tile
  static constexpr int NQB = BT / 32;
  static constexpr int TILE = BT * Geom<T, D>::kRowBytes;
  static constexpr bool TR = sizeof(T) == 2;   // bf16: transposing reads; fp32: a transposed copy
  using QT = TGeom<T, D, BT, 8>;
  using KT = TGeom<T, D, BKW, 16>;
  using DS = TGeom<T, BT, BKW, 16>;   // dS rows: [query][key]
  static constexpr int kQtBytes = TR ? 0 : QT::kBytes;
  static constexpr int kLdsBase = 4 * TILE + kQtBytes + 2 * 3 * BT * 4;
  // The fused kernel's dS block has a region of its own when it fits beside
  // the rest in a CU's 160 KB; otherwise (fp32 at d = 128) it reuses the two
  // Q tiles of the current buffer, dead once every wave has its scores (the
  // kernel adds one barrier before writing dS there).
  static constexpr bool kDsInTiles = kLdsBase + KT::kBytes + DS::kBytes > 160 * 1024;
  static_assert(!kDsInTiles || (DS::kBytes <= 2 * TILE && NQB == 1),
                "dS reuses one buffer's two Q tiles only with one query block per tile");
  static constexpr int kLdsFused = kLdsBase + KT::kBytes + (kDsInTiles ? 0 : DS::kBytes);
};

template <typename T, int D>
struct QCfg {
  static constexpr int NW = 4;
  static constexpr int BQ = 32 * NW;
  static constexpr int BK = (sizeof(T) == 4 && D == 128) ? 32 : 64;
  static constexpr int NKB = BK / 32;
  static constexpr int TILE = BK * Geom<T, D>::kRowBytes;
  static constexpr bool TR = sizeof(T) == 2;
  using KT = TGeom<T, D, BK, 8>;
  static constexpr int kLds = 4 * TILE + (TR ? 0 : KT::kBytes);
};

// dS of one 32 x 32 block in bf16, in MFMA operand order (k-steps 0 and 1).
struct PackedDS {
  bf16x8 b[2];
};
__device__ __forceinline__ PackedDS pack_ds(const float* v) {
  PackedDS r;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int e = 0; e < 8; ++e) r.b[t][e] = (__bf16)v[8 * t + e];
  return r;
}

// Fill n floats with zeros (n a multiple of 4, p 16-byte aligned); a kernel,
// not hipMemsetAsync, so the call can sit in a captured graph.
hipError_t zero_fill(float* p, size_t n, hipStream_t s);

}  // namespace skl
