// Recomputation backward of the attention KL divergence, both settings.
//
// "StreamKL: Fast and Memory-Efficient KL Divergence for Boosting Attention
// Distillation" (gist.science technical summary), Methodology 2,
// Recomputation Strategy: only KL, LSE1, LSE2 are kept from the forward; the
// probabilities are regenerated tile by tile as P_t = exp(S_t - LSE_t).
//   Setting 1 (P1 fixed, gradients to Q2, K2):  dS2 = g (P2 - P1)
//   Setting 2 (P2 fixed, gradients to Q1, K1):  dS1 = g P1 (r - KL),
//     r = (S1 - LSE1) - (S2 - LSE2), formed from logits and the saved LSEs
//     (Methodology 3, Numerical Stability)
//   dQ = scale dS K,  dK = scale dS^T Q.
// The fused kernel visits each (query tile, key block) pair once, keeps dK in
// registers and adds dQ with fp32 atomics; the separate path runs a dK kernel
// and a dQ kernel that each recompute P (Methodology 2, Kernel Fusion).
//
// gfx950 mapping
//   * The scores come from v_mfma_f32_32x32x16_bf16 exactly as in the
//     forward.  The dK kernel computes S = Q K^T with K (this wave's 32 keys)
//     held in VGPRs, so each lane owns one key; the dQ kernel computes
//     S^T = K Q^T with Q held in VGPRs, so each lane owns one query.
//   * dS is formed in fp32 and rounded once to bf16.  The 16 accumulator
//     registers of a 32 x 32 score block are, in order, exactly the k-operand
//     of the next MFMA (two runs of four consecutive indices per lane half),
//     so dS never leaves the registers for dK (dK^T += Q^T dS) or for the
//     separate dQ (dQ^T += K^T dS^T).  The other operand (Q^T or K^T) is a
//     transposed copy of the LDS tile whose rows are padded so the 8-byte
//     reads of 32 different rows hit all 64 banks once.
//   * Fused: the dQ tile needs dS with queries on lanes, so each wave writes
//     its dS block to LDS, and after a barrier the workgroup computes the
//     64 x d dQ tile over its 128 keys and adds it to dQ with one fp32 atomic
//     per element.
//   * Causal: the key-block kernels start at the first query tile that sees
//     their first key; tiles past a wave's frontier are skipped; only tiles
//     crossing the diagonal or a tail take the masked path.
#include <type_traits>

#include "bwd_shared.hpp"

namespace skl {

// Write XT from row-major source rows, four rows at a time: `fetch(row, c)`
// returns chunk c (16 bytes) of source row `row`.  NT threads share the work.
template <typename T, int D, int R, int PAD, int NT, typename Fetch>
__device__ __forceinline__ void build_transposed(SKL_LDS char* xt, int tid, Fetch fetch) {
  using G = Geom<T, D>;
  using TG = TGeom<T, D, R, PAD>;
  constexpr int kUnits = (R / 4) * G::kChunks;
#pragma unroll
  for (int u0 = 0; u0 < kUnits; u0 += NT) {
    const int u = u0 + tid;
    if (kUnits % NT != 0 && u >= kUnits) break;
    const int c = u % G::kChunks;
    const int j0 = (u / G::kChunks) * 4;
    const u32x4 w0 = fetch(j0 + 0, c), w1 = fetch(j0 + 1, c), w2 = fetch(j0 + 2, c), w3 = fetch(j0 + 3, c);
    if constexpr (sizeof(T) == 2) {
      // chunk c holds d = 8c .. 8c+7; dword k holds (d = 8c+2k, 8c+2k+1)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t lo01 = (w0[k] & 0xFFFFu) | (w1[k] << 16);
        const uint32_t lo23 = (w2[k] & 0xFFFFu) | (w3[k] << 16);
        const uint32_t hi01 = (w0[k] >> 16) | (w1[k] & 0xFFFF0000u);
        const uint32_t hi23 = (w2[k] >> 16) | (w3[k] & 0xFFFF0000u);
        const int d = 8 * c + 2 * k;
        *(SKL_LDS u32x2*)(xt + d * TG::kStride + j0 * 2) = u32x2{lo01, lo23};
        *(SKL_LDS u32x2*)(xt + (d + 1) * TG::kStride + j0 * 2) = u32x2{hi01, hi23};
      }
    } else {
      // chunk c holds d = 4c .. 4c+3
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int d = 4 * c + k;
        *(SKL_LDS u32x4*)(xt + d * TG::kStride + j0 * 4) = u32x4{w0[k], w1[k], w2[k], w3[k]};
      }
    }
  }
}

// acc(32 d-rows x 32 cols) += XT(d rows, k) * V(k, cols) where V is one 32 x 32
// score-layout block held as 16 fp32 registers per lane (register r of lane
// half h is index base + 8*(r/4) + 4*h + r%4 along k) and XT row d =
// (row block) + lane % 32 starts at `xrow`; `base` is the block's first k.
template <typename T>
__device__ __forceinline__ f32x16 kgroup_mfma(const SKL_LDS char* xrow, int base, int h, const float* v,
                                              f32x16 acc);

template <>
__device__ __forceinline__ f32x16 kgroup_mfma<__bf16>(const SKL_LDS char* xrow, int base, int h, const float* v,
                                                      f32x16 acc) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const u32x2 lo = *(const SKL_LDS u32x2*)(xrow + (base + 16 * t + 4 * h) * 2);
    const u32x2 hi = *(const SKL_LDS u32x2*)(xrow + (base + 16 * t + 8 + 4 * h) * 2);
    const u32x4 a = u32x4{lo.x, lo.y, hi.x, hi.y};
    bf16x8 b;
#pragma unroll
    for (int e = 0; e < 8; ++e) b[e] = (__bf16)v[8 * t + e];
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), b, acc, 0, 0, 0);
  }
  return acc;
}

template <>
__device__ __forceinline__ f32x16 kgroup_mfma<float>(const SKL_LDS char* xrow, int base, int h, const float* v,
                                                     f32x16 acc) {
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const f32x4 a = *(const SKL_LDS f32x4*)(xrow + (base + 8 * m + 4 * h) * 4);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, v[4 * m + 0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, v[4 * m + 1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, v[4 * m + 2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, v[4 * m + 3], acc, 0, 0, 0);
  }
  return acc;
}

// bf16 form of kgroup_mfma: the A operand (X^T rows = 32 columns of the
// row-major LDS tile starting at element column 32 db; k = tile rows rbase ..
// rbase+31) comes straight from the row-major tile through transposing reads
// (tb: the lane's tr_base for hi = 0 and 1).
template <int D>
__device__ __forceinline__ f32x16 kgroup_mfma_tr(const SKL_LDS char* tile, int rbase, int db, const int* tb,
                                                 const float* v, f32x16 acc) {
  constexpr int RB = D * 2;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const SKL_LDS char* rows = tile + (rbase + 16 * t) * RB;
    const u32x2 lo = read_tr4_at(rows + (tb[0] ^ (64 * db)));
    const u32x2 hi = read_tr4_at(rows + (tb[1] ^ (64 * db)));
    const u32x4 a = u32x4{lo.x, lo.y, hi.x, hi.y};
    bf16x8 b;
#pragma unroll
    for (int e = 0; e < 8; ++e) b[e] = (__bf16)v[8 * t + e];
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), b, acc, 0, 0, 0);
  }
  return acc;
}

// ---- per-row coefficients --------------------------------------------------------
// Setting 1: (LSE1 log2e, LSE2 log2e, g)            dS = g (2^(x2 c - b) - 2^(x1 c - a))
// Setting 2: (LSE1 log2e, g scale, -g (LSE1 - LSE2 + KL))
//                                                 dS = 2^(x1 c - a) (b (x1 - x2) + c3)
// HAS_G false: no upstream weights (g = 1), so Setting 1 needs no factor and
// Setting 2's b is the scale itself; only two per-row values vary.
// The saved per-row values are loaded raw and turned into coefficients only
// when needed: a load whose value is used at once makes the compiler wait for
// it, and that wait also covers any tile DMA issued just before it.
template <int SETTING, bool HAS_G>
struct RowVals {
  float l1 = 0.f, l2 = 0.f, kl = 0.f, g = 1.f;
  __device__ __forceinline__ void load(const BwdParams& p, size_t row) {
    l1 = p.lse1[row];
    l2 = p.lse2[row];
    if (SETTING == 2) kl = p.kl[row];
    if (HAS_G) g = p.dkl[row];
  }
  __device__ __forceinline__ void coefs(const BwdParams& p, float& a, float& b, float& c3) const {
    a = l1 * kLog2e;
    if (SETTING == 1) {
      b = l2 * kLog2e;
      c3 = g;
    } else {
      b = g * p.scale;
      c3 = -g * (l1 - l2 + kl);
    }
  }
};

template <int SETTING, bool HAS_G>
__device__ __forceinline__ void row_coefs(const BwdParams& p, size_t row, float& a, float& b, float& c3) {
  RowVals<SETTING, HAS_G> v;
  v.load(p, row);
  v.coefs(p, a, b, c3);
}

template <int SETTING, bool HAS_G>
__device__ __forceinline__ float dlogit(float x1, float x2, float c, float a, float b, float c3) {
  const float p1 = fast_exp2(fmaf(x1, c, -a));
  if (SETTING == 1) {
    const float p2 = fast_exp2(fmaf(x2, c, -b));
    return HAS_G ? c3 * (p2 - p1) : p2 - p1;
  }
  return p1 * fmaf(b, x1 - x2, c3);
}

// ---- key-block kernel: dK (separate path) or dK + atomic dQ (fused path) ---------

// bf16 separate path: two waves per SIMD (at most 256 VGPRs each); the fp32 and fused
// instantiations need more registers and run one wave per SIMD.
template <typename T, int D, int SETTING, bool FUSED, bool HAS_G>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu((sizeof(T) == 2 && !FUSED) ? 2 : 1)))
void bwd_kv_kernel(BwdParams p) {
  using G = Geom<T, D>;
  using C = KvCfg<T, D>;
  constexpr int NW = C::NW, BT = C::BT, NQB = C::NQB, TILE = C::TILE, DB = D / 32;
  __shared__ __attribute__((aligned(16))) char smem[FUSED ? C::kLdsFused : C::kLdsBase];
  SKL_LDS char* lds = (SKL_LDS char*)smem;
  SKL_LDS char* qt = lds + 4 * TILE;                                    // fp32 only
  SKL_LDS float* coef = (SKL_LDS float*)(qt + C::kQtBytes);             // [2][3][BT]
  SKL_LDS char* kt = (SKL_LDS char*)(coef + 2 * 3 * BT);
  SKL_LDS char* dst = kt + C::KT::kBytes;   // dS block (fused), unless it reuses the Q tiles

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int col = lane & 31;

  const int nkb = (p.n_k + C::BKW - 1) / C::BKW;
  const int w = xcd_work_index(blockIdx.x, p.heads * nkb);
  if (w >= p.heads * nkb) return;
  const int head = w / nkb;
  const int kb = w % nkb;   // key block 0 (heaviest when causal) first
  const int k0 = kb * C::BKW;
  const int kw0 = k0 + wave * 32;
  const int key = kw0 + col;
  const int off = p.n_k - p.n_q;
  const float c = p.c;
  const int pb = pair_base<T, D>(col, h);                              // operand reads of S
  const int tb[2] = {tr_base<D>(lane, 0), tr_base<D>(lane, 1)};        // transposing reads

  const size_t hq = (size_t)head * p.n_q;
  const size_t hk = (size_t)head * p.n_k;
  const char* q1 = p.q1 + hq * G::kRowBytes;
  const char* q2 = p.q2 + hq * G::kRowBytes;
  const char* ks = (SETTING == 1 ? p.k2 : p.k1) + hk * G::kRowBytes;

  // this lane's key row: chunks 2g + h of K1 and K2
  u32x4 kf1[G::kGroups], kf2[G::kGroups];
  {
    const int kr = min(key, p.n_k - 1);
    const char* a1 = p.k1 + (hk + kr) * G::kRowBytes + h * 16;
    const char* a2 = p.k2 + (hk + kr) * G::kRowBytes + h * 16;
#pragma unroll
    for (int g = 0; g < G::kGroups; ++g) {
      kf1[g] = *(const u32x4*)(a1 + g * 32);
      kf2[g] = *(const u32x4*)(a2 + g * 32);
    }
  }
  if (FUSED) {
    // K^T of this workgroup's keys, for the dQ tiles
    build_transposed<T, D, C::BKW, 16, NW * 64>(kt, tid, [&](int r, int cc) {
      const int kr = min(k0 + r, p.n_k - 1);
      return *(const u32x4*)(ks + (size_t)kr * G::kRowBytes + cc * 16);
    });
  }

  f32x16 dkt[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) dkt[i] = f32x16{};

  // query tiles that can see this block's keys
  const int qfirst = p.causal ? max(0, k0 - off) : 0;
  const int t0 = qfirst / BT;
  const int ntiles = (p.n_q + BT - 1) / BT - t0;
  const bool wave_idle = kw0 >= p.n_k;

  auto load_coefs = [&](int q0, SKL_LDS float* cf) {
    if (tid < BT) {
      float a = 0.f, b = 0.f, c3 = 0.f;
      if (q0 + tid < p.n_q) row_coefs<SETTING, HAS_G>(p, hq + q0 + tid, a, b, c3);
      cf[tid] = a;
      cf[BT + tid] = b;
      cf[2 * BT + tid] = c3;
    }
  };
  TileStream<T, D, BT, NW> ts;
  ts.init(tid);
  // Per-row coefficients run one tile ahead of use: the raw values of tile
  // t+1 are loaded into registers during tile t-1 and written to LDS right
  // after the barrier that opens tile t (by then the loop-top wait has seen
  // them land, so no wait ever covers a tile DMA in flight); the barrier that
  // opens tile t+1 publishes them.
  RowVals<SETTING, HAS_G> nv;
  bool nv_ok = false;
  if (ntiles > 0) {
    issue_tile_async<T, D, BT, NW>(q1, t0 * BT, p.n_q, lds, tid, wave);
    issue_tile_async<T, D, BT, NW>(q2, t0 * BT, p.n_q, lds + TILE, tid, wave);
    load_coefs(t0 * BT, coef);
    nv_ok = ntiles > 1 && tid < BT && (t0 + 1) * BT + tid < p.n_q;
    if (nv_ok) nv.load(p, hq + (t0 + 1) * BT + tid);
  }
  // Masking is needed only on tiles that cross the causal diagonal (the
  // first tiles of this block's query range) or hold a tail (the last tile,
  // or every tile of the last key block).  Three loops (leading masked,
  // unmasked, trailing masked) keep one straight-line body per loop, so the
  // compiler never holds both bodies' state at once.  Every iteration has
  // the same barriers, so waves of one workgroup may sit in different loops.
  auto tile_needs_mask = [&](int t) {
    const int q0 = (t0 + t) * BT;
    return (q0 + BT > p.n_q) || (kw0 + 32 > p.n_k) || (p.causal && kw0 + 31 > q0 + off);
  };
  auto tile = [&](int t, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int q0 = (t0 + t) * BT;
    const int buf = t & 1;
    const SKL_LDS char* t1 = lds + buf * 2 * TILE;
    const SKL_LDS char* t2 = t1 + TILE;
    const SKL_LDS float* cf = coef + buf * 3 * BT;
    SKL_LDS char* dsb = C::kDsInTiles ? lds + buf * 2 * TILE : dst;
    wait_async_loads();
    __syncthreads();  // tile t and its coefficients visible; tile t-1's readers done
    const bool has_next = t + 1 < ntiles;
    if (has_next && tid < BT) {
      // tile t+1's coefficients into the buffer tile t-1 used
      float na = 0.f, nb_ = 0.f, nc = 0.f;
      if (nv_ok) nv.coefs(p, na, nb_, nc);
      SKL_LDS float* cn = coef + (buf ^ 1) * 3 * BT;
      cn[tid] = na;
      cn[BT + tid] = nb_;
      cn[2 * BT + tid] = nc;
    }
    if (has_next) {
      // tile t+1's Q rows by LDS DMA; tile t+2's raw row values into registers
      SKL_LDS char* nb = lds + (buf ^ 1) * 2 * TILE;
      ts.issue(q1, q0 + BT, p.n_q, nb, tid, wave);
      ts.issue(q2, q0 + BT, p.n_q, nb + TILE, tid, wave);
    }
    nv_ok = t + 2 < ntiles && tid < BT && q0 + 2 * BT + tid < p.n_q;
    if (nv_ok) nv.load(p, hq + q0 + 2 * BT + tid);
    const SKL_LDS char* tsrc = SETTING == 1 ? t2 : t1;   // the setting's Q
    if constexpr (!C::TR) {
      build_transposed<T, D, BT, 8, NW * 64>(qt, tid, [&](int r, int cc) {
        return *(const SKL_LDS u32x4*)(tsrc + lds_chunk_off<T, D>(r, cc));
      });
      __syncthreads();
    }
    const int qlast = min(q0 + BT, p.n_q) - 1;
    const bool skip = wave_idle || (p.causal && kw0 > qlast + off);
    // dS kept in registers until every wave is done with the Q tiles it will overwrite
    float dsk[C::kDsInTiles ? NQB : 1][16];
    if constexpr (FUSED && C::kDsInTiles) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) dsk[qb][r] = 0.f;
    }
    if (!skip) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        f32x16 s1 = f32x16{}, s2 = f32x16{};
        __builtin_amdgcn_s_setprio(1);   // MFMA phase first when two waves share a SIMD
#pragma unroll
        for (int g = 0; g < G::kGroups; ++g) {
          const int ob = pair_off(pb, g) + qb * 32 * G::kRowBytes;
          s1 = mfma_chunk<T>(*(const SKL_LDS u32x4*)(t1 + ob), kf1[g], s1);
          s2 = mfma_chunk<T>(*(const SKL_LDS u32x4*)(t2 + ob), kf2[g], s2);
        }
        if constexpr (sizeof(T) == 2) sched_lds_mfma_pipeline<2 * G::kGroups, 4>();
        __builtin_amdgcn_s_setprio(0);
        float ds[16];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int qi = qb * 32 + 8 * m + 4 * h;   // first of four consecutive queries
          const f32x4 ca = *(const SKL_LDS f32x4*)(cf + qi);
          f32x4 cb, cc;
          if constexpr (SETTING == 1 || HAS_G)
            cb = *(const SKL_LDS f32x4*)(cf + BT + qi);
          else
            cb = f32x4{p.scale, p.scale, p.scale, p.scale};
          if constexpr (SETTING == 2 || HAS_G)
            cc = *(const SKL_LDS f32x4*)(cf + 2 * BT + qi);
          else
            cc = f32x4{1.f, 1.f, 1.f, 1.f};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * m + e;
            float v = dlogit<SETTING, HAS_G>(s1[r], s2[r], c, ca[e], cb[e], cc[e]);
            if (MASK) {
              const int q = q0 + qi + e;
              const bool ok = (q < p.n_q) & (key < p.n_k) & ((p.causal == 0) | (key <= q + off));
              v = ok ? v : 0.f;
            }
            ds[r] = v;
          }
        }
        // dK^T(d, keys) += Q^T(d, queries) dS(queries, keys)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          if constexpr (C::TR)
            dkt[db] = kgroup_mfma_tr<D>(tsrc, qb * 32, db, tb, ds, dkt[db]);
          else
            dkt[db] = kgroup_mfma<T>(qt + (db * 32 + col) * C::QT::kStride, qb * 32, h, ds, dkt[db]);
        }
        if constexpr (FUSED && C::kDsInTiles) {
#pragma unroll
          for (int r = 0; r < 16; ++r) dsk[qb][r] = ds[r];
        } else if (FUSED) {
          // this dS block -> LDS as [query][key]
          const int kl = wave * 32 + col;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int ql = qb * 32 + acc_row(r, h);
            *(SKL_LDS T*)(dst + ql * C::DS::kStride + kl * (int)sizeof(T)) = (T)ds[r];
          }
        }
      }
    } else if (FUSED && !C::kDsInTiles) {
      // nothing to add from these keys: their dS columns are zero
      const int kl = wave * 32 + col;
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ql = qb * 32 + acc_row(r, h);
          *(SKL_LDS T*)(dst + ql * C::DS::kStride + kl * (int)sizeof(T)) = (T)0.f;
        }
    }
    if constexpr (FUSED && C::kDsInTiles) {
      __syncthreads();   // every wave's scores are done: the Q tiles may be overwritten
      const int kl = wave * 32 + col;
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ql = qb * 32 + acc_row(r, h);
          *(SKL_LDS T*)(dsb + ql * C::DS::kStride + kl * (int)sizeof(T)) = (T)dsk[qb][r];
        }
    }
    if (FUSED) {
      __syncthreads();
      // dQ(queries, d) = dS(queries, keys) K(keys, d) over this block's keys
      constexpr int NB = NQB * DB;
      constexpr int DSG = C::BKW * (int)sizeof(T) / 32;   // chunk pairs along the keys
#pragma unroll
      for (int b = wave; b < NB; b += NW) {
        const int qblk = b / DB, db = b % DB;
        f32x16 acc = f32x16{};
        const SKL_LDS char* arow = dsb + (qblk * 32 + col) * C::DS::kStride + h * 16;
        const SKL_LDS char* brow = kt + (db * 32 + col) * C::KT::kStride + h * 16;
#pragma unroll
        for (int g = 0; g < DSG; ++g)
          acc = mfma_chunk<T>(*(const SKL_LDS u32x4*)(arow + g * 32), *(const SKL_LDS u32x4*)(brow + g * 32), acc);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int q = q0 + qblk * 32 + acc_row(r, h);
          if (q < p.n_q) atomicAdd(p.dq + (hq + q) * D + db * 32 + col, p.scale * acc[r]);
        }
      }
    }
  };
  settle_scalar_loads();
  int t = 0;
  for (; t < ntiles && tile_needs_mask(t); ++t) tile(t, std::true_type{});
  for (; t < ntiles && !tile_needs_mask(t); ++t) tile(t, std::false_type{});
  for (; t < ntiles; ++t) tile(t, std::true_type{});

  // dK rows of this lane's key: registers 4m..4m+3 are four consecutive d
  if (key < p.n_k) {
    float* out = p.dk + (hk + key) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int d = db * 32 + 8 * m + 4 * h;
        *(f32x4*)(out + d) = f32x4{p.scale * dkt[db][4 * m], p.scale * dkt[db][4 * m + 1],
                                   p.scale * dkt[db][4 * m + 2], p.scale * dkt[db][4 * m + 3]};
      }
  }
}

// ---- query-block kernel: dQ of the separate path -----------------------------------

template <typename T, int D, int SETTING, bool SPLIT, bool HAS_G>
__global__ __launch_bounds__(256) void bwd_q_kernel(BwdParams p) {
  using G = Geom<T, D>;
  using C = QCfg<T, D>;
  constexpr int NW = C::NW, BQ = C::BQ, BK = C::BK, NKB = C::NKB, TILE = C::TILE, DB = D / 32;
  __shared__ __attribute__((aligned(16))) char smem[C::kLds];
  SKL_LDS char* lds = (SKL_LDS char*)smem;
  SKL_LDS char* kt = lds + 4 * TILE;   // fp32 only

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int col = lane & 31;

  const int nqb = (p.n_q + BQ - 1) / BQ;
  int bid = blockIdx.x;
  int head, split = 0;
  if (SPLIT) {
    // work items (head, key range, query block), query block fastest, dealt
    // to the XCDs in contiguous runs: the workgroups that share one key range
    // run side by side on one XCD and stream its tiles through one L2
    const int total = p.heads * p.dq_splits * nqb;
    const int w = xcd_work_index(bid, total);
    if (w >= total) return;
    bid = w % nqb;
    split = (w / nqb) % p.dq_splits;
    head = w / (nqb * p.dq_splits);
  } else {
    const int w = xcd_work_index(bid, p.heads * nqb);
    if (w >= p.heads * nqb) return;
    head = w / nqb;
    bid = w % nqb;
  }
  const int qb = p.causal ? (nqb - 1 - bid) : bid;
  const int off = p.n_k - p.n_q;
  const int q0 = qb * BQ;
  const int qw0 = q0 + wave * 32;
  const int qrow = qw0 + col;
  const float c = p.c;
  const int pb = pair_base<T, D>(col, h);                              // operand reads of S
  const int tb[2] = {tr_base<D>(lane, 0), tr_base<D>(lane, 1)};        // transposing reads

  int kbeg = 0, klimit = p.n_k;
  if (SPLIT) {
    const int per = ((p.n_k + BK - 1) / BK + p.dq_splits - 1) / p.dq_splits * BK;
    kbeg = split * per;
    klimit = min(p.n_k, kbeg + per);
  }
  int kend = klimit;
  if (p.causal) kend = min(kend, min(q0 + BQ, p.n_q) + off);
  const int ntiles = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;
  int wtiles = 0;
  if (qw0 < p.n_q) {
    const int wend = p.causal ? min(klimit, min(qw0 + 32, p.n_q) + off) : klimit;
    wtiles = wend > kbeg ? min(ntiles, (wend - kbeg + BK - 1) / BK) : 0;
  }
  wtiles = __builtin_amdgcn_readfirstlane(wtiles);

  const size_t hq = (size_t)head * p.n_q;
  const size_t hk = (size_t)head * p.n_k;
  const char* k1 = p.k1 + hk * G::kRowBytes;
  const char* k2 = p.k2 + hk * G::kRowBytes;

  u32x4 qf1[G::kGroups], qf2[G::kGroups];
  const int qr = min(qrow, p.n_q - 1);
  {
    const char* a1 = p.q1 + (hq + qr) * G::kRowBytes + h * 16;
    const char* a2 = p.q2 + (hq + qr) * G::kRowBytes + h * 16;
#pragma unroll
    for (int g = 0; g < G::kGroups; ++g) {
      qf1[g] = *(const u32x4*)(a1 + g * 32);
      qf2[g] = *(const u32x4*)(a2 + g * 32);
    }
  }
  float ca, cb, cc;
  row_coefs<SETTING, HAS_G>(p, hq + qr, ca, cb, cc);

  f32x16 dqt[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) dqt[i] = f32x16{};

  TileStream<T, D, BK, NW> ts;
  ts.init(tid);
  if (ntiles > 0) {
    issue_tile_async<T, D, BK, NW>(k1, kbeg, p.n_k, lds, tid, wave);
    issue_tile_async<T, D, BK, NW>(k2, kbeg, p.n_k, lds + TILE, tid, wave);
  }
  // Masked tiles: the last ones (causal diagonal, key tail) or all of them
  // (query tail); three loops as in the key-block kernel.
  auto tile_needs_mask = [&](int t) {
    const int k0 = kbeg + t * BK;
    return (k0 + BK > klimit) || (qw0 + 32 > p.n_q) || (p.causal && k0 + BK - 1 > qw0 + off);
  };
  auto tile = [&](int t, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int buf = t & 1;
    const SKL_LDS char* t1 = lds + buf * 2 * TILE;
    const SKL_LDS char* t2 = t1 + TILE;
    wait_async_loads();
    __syncthreads();
    if (t + 1 < ntiles) {
      SKL_LDS char* nb = lds + (buf ^ 1) * 2 * TILE;
      ts.issue(k1, kbeg + (t + 1) * BK, p.n_k, nb, tid, wave);
      ts.issue(k2, kbeg + (t + 1) * BK, p.n_k, nb + TILE, tid, wave);
    }
    const SKL_LDS char* tsrc = SETTING == 1 ? t2 : t1;   // the setting's K
    if constexpr (!C::TR) {
      build_transposed<T, D, BK, 8, NW * 64>(kt, tid, [&](int r, int cc2) {
        return *(const SKL_LDS u32x4*)(tsrc + lds_chunk_off<T, D>(r, cc2));
      });
      __syncthreads();
    }
    if (t >= wtiles) return;  // wave-uniform: past this wave's frontier
    const int k0 = kbeg + t * BK;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      f32x16 s1 = f32x16{}, s2 = f32x16{};
      __builtin_amdgcn_s_setprio(1);   // MFMA phase first when two waves share a SIMD
#pragma unroll
      for (int g = 0; g < G::kGroups; ++g) {
        const int ob = pair_off(pb, g) + kb * 32 * G::kRowBytes;
        s1 = mfma_chunk<T>(*(const SKL_LDS u32x4*)(t1 + ob), qf1[g], s1);
        s2 = mfma_chunk<T>(*(const SKL_LDS u32x4*)(t2 + ob), qf2[g], s2);
      }
      if constexpr (sizeof(T) == 2) sched_lds_mfma_pipeline<2 * G::kGroups, 4>();
      __builtin_amdgcn_s_setprio(0);
      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = dlogit<SETTING, HAS_G>(s1[r], s2[r], c, ca, cb, cc);
        if (MASK) {
          const int kk = k0 + kb * 32 + acc_row(r, h);
          const bool ok = (kk < klimit) & (qrow < p.n_q) & ((p.causal == 0) | (kk <= qrow + off));
          v = ok ? v : 0.f;
        }
        ds[r] = v;
      }
      // dQ^T(d, queries) += K^T(d, keys) dS^T(keys, queries)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        if constexpr (C::TR)
          dqt[db] = kgroup_mfma_tr<D>(tsrc, kb * 32, db, tb, ds, dqt[db]);
        else
          dqt[db] = kgroup_mfma<T>(kt + (db * 32 + col) * C::KT::kStride, kb * 32, h, ds, dqt[db]);
      }
    }
  };
  settle_scalar_loads();
  int t = 0;
  for (; t < ntiles && tile_needs_mask(t); ++t) tile(t, std::true_type{});
  for (; t < ntiles && !tile_needs_mask(t); ++t) tile(t, std::false_type{});
  for (; t < ntiles; ++t) tile(t, std::true_type{});

  if (qrow < p.n_q) {
    float* out = p.dq + (hq + qrow) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int d = db * 32 + 8 * m + 4 * h;
        if (SPLIT) {
#pragma unroll
          for (int e = 0; e < 4; ++e) atomicAdd(out + d + e, p.scale * dqt[db][4 * m + e]);
        } else {
          *(f32x4*)(out + d) = f32x4{p.scale * dqt[db][4 * m], p.scale * dqt[db][4 * m + 1],
                                     p.scale * dqt[db][4 * m + 2], p.scale * dqt[db][4 * m + 3]};
        }
      }
  }
}

__global__ __launch_bounds__(256) void zero_fill_kernel(float4* p, size_t n4) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n4; i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// ---- launches ---------------------------------------------------------------------
hipError_t zero_fill(float* p, size_t n, hipStream_t s) {
  // n is a multiple of 4 (head_dim is 64 or 128) and p is 16-byte aligned
  const size_t n4 = n / 4;
  const unsigned blocks = (unsigned)((n4 + 255) / 256 < 4096 ? (n4 + 255) / 256 : 4096);
  hipLaunchKernelGGL(zero_fill_kernel, dim3(blocks), dim3(256), 0, s, (float4*)p, n4);
  return hipGetLastError();
}

template <typename T, int D, int SETTING, bool HAS_G>
static hipError_t sep(const BwdParams& p, bool do_dk, bool do_dq, hipStream_t s) {
  using KC = KvCfg<T, D>;
  using QC = QCfg<T, D>;
  hipError_t e = hipSuccess;
  if (do_dk) {
    const int nkb = (p.n_k + KC::BKW - 1) / KC::BKW;
    hipLaunchKernelGGL((bwd_kv_kernel<T, D, SETTING, false, HAS_G>), dim3(xcd_grid(p.heads * nkb)), dim3(256), 0, s,
                       p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!do_dq) return e;
  const int nqb = (p.n_q + QC::BQ - 1) / QC::BQ;
  if (p.dq_splits > 1) {
    e = zero_fill(p.dq, (size_t)p.heads * p.n_q * D, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_q_kernel<T, D, SETTING, true, HAS_G>), dim3(xcd_grid(p.heads * nqb * p.dq_splits)), dim3(256), 0, s,
                       p);
  } else {
    hipLaunchKernelGGL((bwd_q_kernel<T, D, SETTING, false, HAS_G>), dim3(xcd_grid(p.heads * nqb)), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

template <typename T, int D, int SETTING, bool HAS_G>
static hipError_t fused(const BwdParams& p, hipStream_t s) {
  using KC = KvCfg<T, D>;
  hipError_t e = zero_fill(p.dq, (size_t)p.heads * p.n_q * D, s);
  if (e != hipSuccess) return e;
  const int nkb = (p.n_k + KC::BKW - 1) / KC::BKW;
  hipLaunchKernelGGL((bwd_kv_kernel<T, D, SETTING, true, HAS_G>), dim3(xcd_grid(p.heads * nkb)), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <template <typename, int, int> class F>
static hipError_t dispatch(const BwdParams& p, int dtype, int head_dim, int mode, hipStream_t s) {
  if (dtype == 0) {
    if (head_dim == 64) return p.setting == 1 ? F<__bf16, 64, 1>::run(p, mode, s) : F<__bf16, 64, 2>::run(p, mode, s);
    return p.setting == 1 ? F<__bf16, 128, 1>::run(p, mode, s) : F<__bf16, 128, 2>::run(p, mode, s);
  }
  if (head_dim == 64) return p.setting == 1 ? F<float, 64, 1>::run(p, mode, s) : F<float, 64, 2>::run(p, mode, s);
  return p.setting == 1 ? F<float, 128, 1>::run(p, mode, s) : F<float, 128, 2>::run(p, mode, s);
}

template <typename T, int D, int S>
struct SepRun {
  static hipError_t run(const BwdParams& p, int mode, hipStream_t s) {
    // with no upstream weights the kernels skip the per-row factor g
    if (p.dkl) return sep<T, D, S, true>(p, (mode & 1) != 0, (mode & 2) != 0, s);
    return sep<T, D, S, false>(p, (mode & 1) != 0, (mode & 2) != 0, s);
  }
};
template <typename T, int D, int S>
struct FusedRun {
  static hipError_t run(const BwdParams& p, int, hipStream_t s) {
    if constexpr (KvCfg<T, D>::kLdsFused > 160 * 1024) {
      return hipErrorNotSupported;
    } else {
      return p.dkl ? fused<T, D, S, true>(p, s) : fused<T, D, S, false>(p, s);
    }
  }
};

hipError_t launch_bwd_separate(const BwdParams& p, int dtype, int head_dim, bool dk, bool dq, hipStream_t stream) {
  return dispatch<SepRun>(p, dtype, head_dim, (dk ? 1 : 0) | (dq ? 2 : 0), stream);
}

hipError_t launch_bwd_fused(const BwdParams& p, int dtype, int head_dim, hipStream_t stream) {
  return dispatch<FusedRun>(p, dtype, head_dim, 0, stream);
}

bool fused_supported(int dtype, int head_dim) {
  if (dtype == 0) return true;
  return head_dim == 64 ? KvCfg<float, 64>::kLdsFused <= 160 * 1024 : KvCfg<float, 128>::kLdsFused <= 160 * 1024;
}

}  // namespace skl
