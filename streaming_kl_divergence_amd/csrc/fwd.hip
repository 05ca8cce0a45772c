// Fused one-pass forward of the attention KL divergence, and its split-K form.
//
// "StreamKL: Fast and Memory-Efficient KL Divergence for Boosting Attention
// Distillation" (gist.science technical summary):
//   Methodology 1, Online Formulation - five running scalars per row
//     (maxima m1, m2; exp-sums l1, l2; acc, the P1-weighted logit
//     difference), one pass over key tiles, row loss acc/l1 + LSE2 - LSE1,
//     LSE_t = m_t + log l_t; acc is one value per row (not a B_Q x d block),
//     so each tile rescales it once; causal key tiles past the frontier are
//     never loaded.
//   Methodology 3, Split-K Variant - for few queries the key range is cut
//     into pieces handled by different workgroups, whose partial states are
//     merged afterwards.
//
// gfx950 mapping
//   * Workgroup = NW waves; each wave owns 32 query rows of one head.  Its Q1
//     and Q2 rows stay in VGPRs for the whole pass (the B operand).
//   * K1 and K2 tiles of 64 keys stream through double-buffered LDS, copied
//     with global_load_lds_dwordx4 (no VGPR staging) in a swizzled layout.
//   * The MFMA computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16, so each
//     lane holds one query and 16 of every 32 keys.  A lane keeps its own
//     five-scalar state for its half of the keys; the two halves are merged
//     once at the end (the same merge as split-K), so the tile loop has no
//     cross-lane reductions.
//   * Scores stay in raw units; exp2 takes fma(S, c, -m*c) with
//     c = scale*log2(e); acc is kept in raw units and scaled once at the end.
//   * Causal: Q blocks are launched heaviest first; tiles past a wave's
//     frontier are skipped; only tiles that cross the diagonal or the end of
//     the key range take the masked code path.
//   * Each XCD walks a contiguous run of (head, query block) items, one head
//     at a time (xcd_work_index), so the workgroups resident on an XCD stream
//     the same K tiles through its L2; split-K walks (head, key range, query
//     block) items, so the workgroups of one key range run side by side.
//   * When a head has a single query block (decode and other short query
//     sets) every key is read by one workgroup only, and the tiles are loaded
//     with the non-temporal cache policy.
#include <limits.h>

#include <mutex>

#include "common.hpp"
#include "kernels.hpp"

namespace skl {

// Running five-scalar state of one lane (one query, half of the keys), with
// the exponent offsets -m1 c and -m2 c kept beside the maxima (they change
// only when a maximum does).
struct RowState {
  float m1, m2, l1, l2, acc;
  float nmc1, nmc2;
};

// S1, S2 (raw units) of one 64-key tile for this lane's query: 2 blocks of 16.
// pb: the lane's pair_base.
template <typename T, int D, int NKB>
__device__ __forceinline__ void tile_scores(const SKL_LDS char* t1, const SKL_LDS char* t2, const u32x4* qf1,
                                            const u32x4* qf2, int pb, f32x16* s1, f32x16* s2) {
  using G = Geom<T, D>;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    s1[kb] = f32x16{};
    s2[kb] = f32x16{};
#pragma unroll
    for (int g = 0; g < G::kGroups; ++g) {
      const int ob = pair_off(pb, g) + kb * 32 * G::kRowBytes;
      s1[kb] = mfma_chunk<T>(*(const SKL_LDS u32x4*)(t1 + ob), qf1[g], s1[kb]);
      s2[kb] = mfma_chunk<T>(*(const SKL_LDS u32x4*)(t2 + ob), qf2[g], s2[kb]);
    }
  }
}

// Fold one tile of scores into the running state.  MASK: the tile crosses the
// causal diagonal or the end of the key range, so some pairs are excluded.
template <bool MASK, int NKB>
__device__ __forceinline__ void tile_update(RowState& st, f32x16* s1, f32x16* s2, float c, int k0, int h,
                                            int klimit, int causal, int qlim) {
  if (MASK) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + kb * 32 + acc_row(r, h);
        const bool ok = (key < klimit) & ((causal == 0) | (key <= qlim));
        s1[kb][r] = ok ? s1[kb][r] : -INFINITY;
        s2[kb][r] = ok ? s2[kb][r] : -INFINITY;
      }
  }
  float tm1 = -INFINITY, tm2 = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      tm1 = fmaxf(tm1, s1[kb][r]);
      tm2 = fmaxf(tm2, s2[kb][r]);
    }
  const float n1 = fmaxf(st.m1, tm1), n2 = fmaxf(st.m2, tm2);
  const float a1 = fast_exp2((st.m1 - n1) * c), a2 = fast_exp2((st.m2 - n2) * c);
  st.m1 = n1;
  st.m2 = n2;
  st.nmc1 = -(n1 * c);
  st.nmc2 = -(n2 * c);
  float sl1[4], sl2[4], sa[4];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float x1 = s1[kb][r], x2 = s2[kb][r];
      float e1 = fast_exp2(fmaf(x1, c, st.nmc1));
      float e2 = fast_exp2(fmaf(x2, c, st.nmc2));
      float d = x1 - x2;
      if (MASK) {
        const bool ok = x1 != -INFINITY;  // real scores are finite
        e1 = ok ? e1 : 0.f;
        e2 = ok ? e2 : 0.f;
        d = ok ? d : 0.f;
      }
      const int j = r & 3;
      if (kb == 0 && r < 4) {   // the first term of each partial sum starts it
        sl1[j] = e1;
        sl2[j] = e2;
        sa[j] = e1 * d;
      } else {
        sl1[j] += e1;
        sl2[j] += e2;
        sa[j] = fmaf(e1, d, sa[j]);
      }
    }
  st.l1 = fmaf(a1, st.l1, (sl1[0] + sl1[1]) + (sl1[2] + sl1[3]));
  st.l2 = fmaf(a2, st.l2, (sl2[0] + sl2[1]) + (sl2[2] + sl2[3]));
  st.acc = fmaf(a1, st.acc, (sa[0] + sa[1]) + (sa[2] + sa[3]));
}

// Unmasked tile folded against the current offsets m1, m2, without this
// tile's maxima.  The sums are scale-free, so any offset gives the same
// result as long as no term overflows: the fold is accepted when every lane's
// tile sum of 2^(x c - m c) stays below 2^64 (no score more than ~64 binary
// orders above its offset).  Otherwise nothing is changed and the caller runs
// the exact online update of the pages' Methodology 1 on the tile
// (tile_update: offsets raised to the tile maxima, l and acc rescaled), lane
// by lane, which cannot overflow.  An offset never exceeds the true running
// maximum, so nothing underflows that the exact update would keep.  The
// first tile of a lane always takes the exact update (its offset is the
// initial -1e30).  Saves the per-tile max reduction.  A lane whose scores
// are not finite (NaN or infinite inputs) also fails the test; the exact
// update then makes that lane's row non-finite and leaves every other lane's
// row exact.
template <int NKB>
__device__ __forceinline__ bool tile_fold_at_offsets(RowState& st, const f32x16* s1, const f32x16* s2, float c) {
  float sl1[4], sl2[4], sa[4];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float x1 = s1[kb][r], x2 = s2[kb][r];
      const int j = r & 3;
      const float e1 = fast_exp2(fmaf(x1, c, st.nmc1));
      const float e2 = fast_exp2(fmaf(x2, c, st.nmc2));
      if (kb == 0 && r < 4) {   // the first term of each partial sum starts it
        sl1[j] = e1;
        sl2[j] = e2;
        sa[j] = e1 * (x1 - x2);
      } else {
        sl1[j] += e1;
        sl2[j] += e2;
        sa[j] = fmaf(e1, x1 - x2, sa[j]);
      }
    }
  const float t1 = (sl1[0] + sl1[1]) + (sl1[2] + sl1[3]);
  const float t2 = (sl2[0] + sl2[1]) + (sl2[2] + sl2[3]);
  // the comparisons are false for inf and NaN too
  const uint64_t bad = __builtin_amdgcn_ballot_w64(!(t1 < 0x1p64f)) | __builtin_amdgcn_ballot_w64(!(t2 < 0x1p64f));
  if (bad != 0) return false;
  st.l1 += t1;
  st.l2 += t2;
  st.acc += (sa[0] + sa[1]) + (sa[2] + sa[3]);
  return true;
}

template <typename T, int D, int NW, bool SPLIT, bool STREAM>
__global__ __launch_bounds__(NW * 64) void fwd_kernel(FwdParams p) {
  using G = Geom<T, D>;
  constexpr int BK = kFwdKeyTile;
  constexpr int BQ = 32 * NW;
  constexpr int NKB = BK / 32;
  constexpr int TILE = BK * G::kRowBytes;
  __shared__ __attribute__((aligned(16))) char smem[2 * 2 * TILE];  // [buffer][K1, K2]
  SKL_LDS char* lds = (SKL_LDS char*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int col = lane & 31;

  const int nqb = (p.n_q + BQ - 1) / BQ;
  int bid = blockIdx.x;
  int head, split = 0;
  if (SPLIT) {
    // work items (head, split, query block), query block fastest, dealt to
    // the XCDs in contiguous runs: the workgroups that share one key range
    // run side by side on one XCD and stream its tiles through one L2
    const int total = p.heads * p.splits * nqb;
    const int w = xcd_work_index(bid, total);
    if (w >= total) return;
    bid = w % nqb;
    split = (w / nqb) % p.splits;
    head = w / (nqb * p.splits);
  } else {
    const int w = xcd_work_index(bid, p.heads * nqb);
    if (w >= p.heads * nqb) return;
    head = w / nqb;
    bid = w % nqb;
  }
  const int qb = p.causal ? (nqb - 1 - bid) : bid;   // causal: heaviest blocks first

  const int off = p.n_k - p.n_q;
  const int q0 = qb * BQ;
  const int qw0 = q0 + wave * 32;
  const int qrow = qw0 + col;

  // key range of this workgroup: [kbeg, klimit), cut at the causal frontier
  int kbeg = 0, klimit = p.n_k;
  if (SPLIT) {
    kbeg = split * p.split_keys;
    klimit = min(p.n_k, kbeg + p.split_keys);
  }
  int kend = klimit;
  if (p.causal) kend = min(kend, min(q0 + BQ, p.n_q) + off);
  const int ntiles = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;
  // tiles holding at least one key visible to this wave's real queries
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

  // this lane's query row: the chunks 2g + h of Q1 and Q2
  u32x4 qf1[G::kGroups], qf2[G::kGroups];
  {
    const int qr = min(qrow, p.n_q - 1);
    const char* a1 = p.q1 + (hq + qr) * G::kRowBytes + h * 16;
    const char* a2 = p.q2 + (hq + qr) * G::kRowBytes + h * 16;
#pragma unroll
    for (int g = 0; g < G::kGroups; ++g) {
      qf1[g] = *(const u32x4*)(a1 + g * 32);
      qf2[g] = *(const u32x4*)(a2 + g * 32);
    }
  }

  RowState st{kMaxInit, kMaxInit, 0.f, 0.f, 0.f, -(kMaxInit * p.c), -(kMaxInit * p.c)};
  const float c = p.c;
  const int qlim = qrow + off;   // last key this lane's query may see (causal)
  const int pb = pair_base<T, D>(col, h);

  // Two waves per SIMD (212 VGPRs each) overlap one wave's MFMAs with the other's VALU.
  f32x16 s1[NKB], s2[NKB];
  // STREAM: this workgroup holds every query of its head (one query block
  // per head: decode and other short query sets), so no other workgroup reads
  // its keys and they are streamed with non-temporal loads.  Otherwise the
  // head's workgroups share its keys through the XCD's L2 and the loads keep
  // the default cache policy.
  TileStream<T, D, BK, NW, STREAM> ts;
  ts.init(tid);
  if (ntiles > 0) {
    issue_tile_async<T, D, BK, NW, STREAM>(k1, kbeg, p.n_k, lds, tid, wave);
    issue_tile_async<T, D, BK, NW, STREAM>(k2, kbeg, p.n_k, lds + TILE, tid, wave);
  }
  // The last key this wave's first query may see: a tile holding a key past
  // it crosses the causal diagonal (wave-uniform).
  const int wdiag = p.causal ? qw0 + off : INT_MAX;
  for (int t = 0; t < ntiles; ++t) {
    wait_async_loads();
    __syncthreads();  // tile t visible; buffer t+1 free again
    const int buf = t & 1;
    if (t + 1 < ntiles) {
      SKL_LDS char* nb = lds + (buf ^ 1) * 2 * TILE;
      ts.issue2(k1, k2, kbeg + (t + 1) * BK, p.n_k, nb, nb + TILE, tid, wave);
    }
    if (t >= wtiles) continue;
    const int k0 = kbeg + t * BK;
    const bool need_mask = (k0 + BK > klimit) | (k0 + BK - 1 > wdiag);
    // one copy of the MFMA phase per LDS buffer, so that each operand address
    // is a per-lane base plus an immediate offset
    __builtin_amdgcn_s_setprio(1);   // MFMA phase first when two waves share a SIMD
    if (buf)
      tile_scores<T, D, NKB>(lds + 2 * TILE, lds + 3 * TILE, qf1, qf2, pb, s1, s2);
    else
      tile_scores<T, D, NKB>(lds, lds + TILE, qf1, qf2, pb, s1, s2);
    __builtin_amdgcn_s_setprio(0);
    if (need_mask) {
      tile_update<true, NKB>(st, s1, s2, c, k0, h, klimit, p.causal, qlim);
    } else if (!tile_fold_at_offsets<NKB>(st, s1, s2, c)) {
      tile_update<false, NKB>(st, s1, s2, c, k0, h, klimit, p.causal, qlim);
    }
  }

  // merge the two lane halves: same query, disjoint key subsets
  const float om1 = __shfl_xor(st.m1, 32), ol1 = __shfl_xor(st.l1, 32), oacc = __shfl_xor(st.acc, 32);
  const float om2 = __shfl_xor(st.m2, 32), ol2 = __shfl_xor(st.l2, 32);
  const float M1 = fmaxf(st.m1, om1), M2 = fmaxf(st.m2, om2);
  const float w = fast_exp2((st.m1 - M1) * c), ow = fast_exp2((om1 - M1) * c);
  const float v = fast_exp2((st.m2 - M2) * c), ov = fast_exp2((om2 - M2) * c);
  const float L1 = st.l1 * w + ol1 * ow;
  const float ACC = st.acc * w + oacc * ow;
  const float L2 = st.l2 * v + ol2 * ov;
  if (h == 0 && qrow < p.n_q) {
    if (SPLIT) {
      float* o = p.part + (((size_t)split * p.heads + head) * p.n_q + qrow) * 5;
      o[0] = M1;
      o[1] = L1;
      o[2] = ACC;
      o[3] = M2;
      o[4] = L2;
    } else {
      const float lse1 = M1 * p.scale + log2f(L1) * kLn2;
      const float lse2 = M2 * p.scale + log2f(L2) * kLn2;
      p.kl[hq + qrow] = p.scale * ACC / L1 + lse2 - lse1;
      p.lse1[hq + qrow] = lse1;
      p.lse2[hq + qrow] = lse2;
    }
  }
}

// Merge the partial states of all key ranges of each row and finish the row
// (the merge of the pages' Methodology 3, Split-K Variant).  One wave per row:
// lane l takes ranges l, l + 64, ...; the maxima and then the rescaled sums
// are reduced across the wave.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int x = 32; x >= 1; x >>= 1) v = fmaxf(v, __shfl_xor(v, x));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int x = 32; x >= 1; x >>= 1) v += __shfl_xor(v, x);
  return v;
}

__global__ __launch_bounds__(256) void splitk_combine_kernel(FwdParams p) {
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);   // row; the same for the whole wave
  const int rows = p.heads * p.n_q;
  if (i >= rows) return;
  const float c = p.c;
  float M1 = kMaxInit, M2 = kMaxInit;
  for (int s = lane; s < p.splits; s += 64) {
    const float* st = p.part + ((size_t)s * rows + i) * 5;
    M1 = fmaxf(M1, st[0]);
    M2 = fmaxf(M2, st[3]);
  }
  M1 = wave_max(M1);
  M2 = wave_max(M2);
  float L1 = 0.f, L2 = 0.f, ACC = 0.f;
  for (int s = lane; s < p.splits; s += 64) {
    const float* st = p.part + ((size_t)s * rows + i) * 5;
    const float w1 = fast_exp2((st[0] - M1) * c);
    const float w2 = fast_exp2((st[3] - M2) * c);
    L1 = fmaf(st[1], w1, L1);
    ACC = fmaf(st[2], w1, ACC);
    L2 = fmaf(st[4], w2, L2);
  }
  L1 = wave_sum(L1);
  ACC = wave_sum(ACC);
  L2 = wave_sum(L2);
  if (lane == 0) {
    const float lse1 = M1 * p.scale + log2f(L1) * kLn2;
    const float lse2 = M2 * p.scale + log2f(L2) * kLn2;
    p.kl[i] = p.scale * ACC / L1 + lse2 - lse1;
    p.lse1[i] = lse1;
    p.lse2[i] = lse2;
  }
}

template <typename T, int D, int NW, bool SPLIT>
static hipError_t launch_one(const FwdParams& p, hipStream_t stream) {
  const int nqb = (p.n_q + 32 * NW - 1) / (32 * NW);
  const long long blocks = xcd_grid(SPLIT ? p.heads * nqb * p.splits : p.heads * nqb);
  // one query block per head: every key byte is read by a single workgroup.
  // One-wave workgroups are used only for such shapes (at most 32 queries).
  if constexpr (NW == 1)
    hipLaunchKernelGGL((fwd_kernel<T, D, 1, SPLIT, true>), dim3((unsigned)blocks), dim3(64), 0, stream, p);
  else if (nqb == 1)
    hipLaunchKernelGGL((fwd_kernel<T, D, NW, SPLIT, true>), dim3((unsigned)blocks), dim3(NW * 64), 0, stream, p);
  else
    hipLaunchKernelGGL((fwd_kernel<T, D, NW, SPLIT, false>), dim3((unsigned)blocks), dim3(NW * 64), 0, stream, p);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_nw(const FwdParams& p, int nw, bool split, hipStream_t stream) {
  if (nw == 1) return split ? launch_one<T, D, 1, true>(p, stream) : launch_one<T, D, 1, false>(p, stream);
  return split ? launch_one<T, D, 4, true>(p, stream) : launch_one<T, D, 4, false>(p, stream);
}

hipError_t launch_fwd(const FwdParams& p, int dtype, int head_dim, int nw, bool split, hipStream_t stream) {
  if (dtype == 0) {
    return head_dim == 64 ? launch_nw<__bf16, 64>(p, nw, split, stream)
                          : launch_nw<__bf16, 128>(p, nw, split, stream);
  }
  return head_dim == 64 ? launch_nw<float, 64>(p, nw, split, stream)
                        : launch_nw<float, 128>(p, nw, split, stream);
}

hipError_t launch_splitk_combine(const FwdParams& p, hipStream_t stream) {
  const int rows = p.heads * p.n_q;
  hipLaunchKernelGGL(splitk_combine_kernel, dim3((rows + 3) / 4), dim3(256), 0, stream, p);
  return hipGetLastError();
}

// Fixed device scratch for the split-K partial states of the entry point that
// allocates nothing (streamkl_fwd_splitk_noalloc).  Every GPU the library runs
// on holds its own copy until the process ends.  In host code `scratch` names
// a host-side stand-in, not device memory, so kernels only ever receive the
// device address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
float* g_scratch_ptr[kMaxDevices];   // guarded by g_scratch_mutex
}  // namespace

hipError_t noalloc_scratch(float** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    // first call on this device, with it current: look the array up once
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = (float*)ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace skl
