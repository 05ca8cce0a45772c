// Backward of the attention KL divergence for both settings at once.
//
// "StreamKL: Fast and Memory-Efficient KL Divergence for Boosting Attention
// Distillation" (gist.science technical summary), Methodology 2: Setting 1
// (gradients to Q2, K2) and Setting 2 (gradients to Q1, K1) of the same loss,
// each recomputing P from the saved LSEs.  When both are wanted, one
// recomputation of S1, S2 and P1 per (query, key) pair serves the two.
//
// Compiled without the VGPR-only MFMA form: MFMA results go to the
// accumulation registers (AGPRs; the scores are read back with one
// v_accvgpr_read per value), which leaves the VGPRs to the resident operand
// rows and the dS work, so that both settings' gradient accumulators fit one
// wave.
#include "bwd_shared.hpp"

namespace skl {

// ---- both settings from one recomputation ----------------------------------------
// A step that trains on both distributions needs Setting 1's dS2 = g (P2 - P1)
// and Setting 2's dS1 = g P1 ((S1 - LSE1) - (S2 - LSE2) - KL) for the same
// (query, key) pairs.  Both come from the same S1, S2 and P1, so one
// recomputation serves the two: per pair 4·d flop of scores and 2 exps
// instead of 8·d and 3.  Per row: a = LSE1 log2e, b = LSE2 log2e,
// c3 = -g (LSE1 - LSE2 + KL) and g (1 without upstream weights).
// A wave's two gradient accumulators (2 x 32 rows x d fp32) next to its
// resident operand rows need more than 256 registers, so these kernels run one
// wave per SIMD; the two settings' matrix and vector work inside one wave take
// the place of a second wave.  bf16 only (the transposing LDS reads).
template <bool HAS_G>
struct BothVals {
  float l1 = 0.f, l2 = 0.f, kl = 0.f, g = 1.f;
  __device__ __forceinline__ void load(const BwdParams& p, size_t row) {
    l1 = p.lse1[row];
    l2 = p.lse2[row];
    kl = p.kl[row];
    if (HAS_G) g = p.dkl[row];
  }
  __device__ __forceinline__ void coefs(float& a, float& b, float& c3, float& gg) const {
    a = l1 * kLog2e;
    b = l2 * kLog2e;
    c3 = -g * (l1 - l2 + kl);
    gg = g;
  }
};

// dS2 (Setting 1) and dS1 (Setting 2) of one pair from the raw scores x1, x2.
template <bool HAS_G>
__device__ __forceinline__ void dlogit_both(float x1, float x2, float c, float scale, float a, float b, float c3,
                                            float g, float& d2, float& d1) {
  const float p1 = fast_exp2(fmaf(x1, c, -a));
  const float p2 = fast_exp2(fmaf(x2, c, -b));
  d2 = HAS_G ? g * (p2 - p1) : p2 - p1;
  d1 = p1 * fmaf(HAS_G ? g * scale : scale, x1 - x2, c3);
}

// The transposing reads of one 32-row block's gradient operands for both
// settings (tile ta for acca, tbt for accb), issued ahead of use.
template <int D>
struct GradOps {
  u32x2 a[2][D / 32][2], b[2][D / 32][2];
  __device__ __forceinline__ void load(const SKL_LDS char* ta, const SKL_LDS char* tbt, int rbase, const int* tb) {
    constexpr int RB = D * 2;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int o = (rbase + 16 * t) * RB;
        a[t][db][0] = read_tr4_at(ta + o + (tb[0] ^ (64 * db)));
        a[t][db][1] = read_tr4_at(ta + o + (tb[1] ^ (64 * db)));
        b[t][db][0] = read_tr4_at(tbt + o + (tb[0] ^ (64 * db)));
        b[t][db][1] = read_tr4_at(tbt + o + (tb[1] ^ (64 * db)));
      }
  }
  __device__ __forceinline__ void run(const PackedDS& pa, const PackedDS& pbk, f32x16* acca, f32x16* accb) const {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        acca[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, u32x4{a[t][db][0].x, a[t][db][0].y, a[t][db][1].x, a[t][db][1].y}), pa.b[t],
            acca[db], 0, 0, 0);
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        accb[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, u32x4{b[t][db][0].x, b[t][db][0].y, b[t][db][1].x, b[t][db][1].y}), pbk.b[t],
            accb[db], 0, 0, 0);
    }
  }
};

// Key-block kernel, both settings: dK2 = scale dS2^T Q2 and dK1 = scale dS1^T Q1
// for this workgroup's 128 keys (the layout of bwd_kv_kernel, one wave per SIMD).
template <int D, bool HAS_G>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1)))
void bwd_kv_both_kernel(BwdParams p) {
  using T = __bf16;
  using G = Geom<T, D>;
  using C = KvCfg<T, D>;
  // 128-query tiles (twice the single-setting kernel's): one workgroup per CU
  // holds them double-buffered, and each barrier and tile copy covers more work
  constexpr int NW = C::NW, BT = 2 * C::BT, NQB = 2 * C::NQB, TILE = 2 * C::TILE, DB = D / 32;
  constexpr int NC = 4;   // per-row arrays in LDS: a, b, c3, g
  __shared__ __attribute__((aligned(16))) char smem[4 * TILE + 2 * NC * BT * 4];
  SKL_LDS char* lds = (SKL_LDS char*)smem;
  SKL_LDS float* coef = (SKL_LDS float*)(lds + 4 * TILE);   // [2][NC][BT]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int col = lane & 31;

  const int nkb = (p.n_k + C::BKW - 1) / C::BKW;
  const int w = xcd_work_index(blockIdx.x, p.heads * nkb);
  if (w >= p.heads * nkb) return;
  const int head = w / nkb;
  const int kb = w % nkb;
  const int k0 = kb * C::BKW;
  const int kw0 = k0 + wave * 32;
  const int key = kw0 + col;
  const int off = p.n_k - p.n_q;
  const float c = p.c;
  const int pb = pair_base<T, D>(col, h);
  const int tb[2] = {tr_base<D>(lane, 0), tr_base<D>(lane, 1)};

  const size_t hq = (size_t)head * p.n_q;
  const size_t hk = (size_t)head * p.n_k;
  const char* q1 = p.q1 + hq * G::kRowBytes;
  const char* q2 = p.q2 + hq * G::kRowBytes;

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

  f32x16 dk2t[DB], dk1t[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) {
    dk2t[i] = f32x16{};
    dk1t[i] = f32x16{};
  }

  const int qfirst = p.causal ? max(0, k0 - off) : 0;
  const int t0 = qfirst / BT;
  const int ntiles = (p.n_q + BT - 1) / BT - t0;
  const bool wave_idle = kw0 >= p.n_k;

  auto store_coefs = [&](const BothVals<HAS_G>& v, bool ok, SKL_LDS float* cf) {
    float a = 0.f, b = 0.f, c3 = 0.f, g = 0.f;
    if (ok) v.coefs(a, b, c3, g);
    cf[tid] = a;
    cf[BT + tid] = b;
    cf[2 * BT + tid] = c3;
    cf[3 * BT + tid] = g;
  };
  TileStream<T, D, BT, NW> ts;
  ts.init(tid);
  // per-row values one tile ahead of use, as in bwd_kv_kernel
  BothVals<HAS_G> nv;
  bool nv_ok = false;
  if (ntiles > 0) {
    issue_tile_async<T, D, BT, NW>(q1, t0 * BT, p.n_q, lds, tid, wave);
    issue_tile_async<T, D, BT, NW>(q2, t0 * BT, p.n_q, lds + TILE, tid, wave);
    if (tid < BT) {
      BothVals<HAS_G> v0;
      const bool ok = t0 * BT + tid < p.n_q;
      if (ok) v0.load(p, hq + t0 * BT + tid);
      store_coefs(v0, ok, coef);
    }
    nv_ok = ntiles > 1 && tid < BT && (t0 + 1) * BT + tid < p.n_q;
    if (nv_ok) nv.load(p, hq + (t0 + 1) * BT + tid);
  }
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
    const SKL_LDS float* cf = coef + buf * NC * BT;
    wait_async_loads();
    __syncthreads();  // tile t and its per-row values visible; tile t-1's readers done
    const bool has_next = t + 1 < ntiles;
    if (has_next && tid < BT) store_coefs(nv, nv_ok, coef + (buf ^ 1) * NC * BT);
    if (has_next) {
      SKL_LDS char* nb = lds + (buf ^ 1) * 2 * TILE;
      ts.issue(q1, q0 + BT, p.n_q, nb, tid, wave);
      ts.issue(q2, q0 + BT, p.n_q, nb + TILE, tid, wave);
    }
    nv_ok = t + 2 < ntiles && tid < BT && q0 + 2 * BT + tid < p.n_q;
    if (nv_ok) nv.load(p, hq + q0 + 2 * BT + tid);
    const int qlast = min(q0 + BT, p.n_q) - 1;
    if (wave_idle || (p.causal && kw0 > qlast + off)) return;
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      GradOps<D> go;
      go.load(t2, t1, qb * 32, tb);
      __builtin_amdgcn_sched_barrier(0);
      f32x16 s1 = f32x16{}, s2 = f32x16{};
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int g = 0; g < G::kGroups; ++g) {
        const int ob = pair_off(pb, g) + qb * 32 * G::kRowBytes;
        s1 = mfma_chunk<T>(*(const SKL_LDS u32x4*)(t1 + ob), kf1[g], s1);
        s2 = mfma_chunk<T>(*(const SKL_LDS u32x4*)(t2 + ob), kf2[g], s2);
      }
      sched_lds_mfma_pipeline<2 * G::kGroups, 4>();
      __builtin_amdgcn_s_setprio(0);
      float d2[16], d1[16];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int qi = qb * 32 + 8 * m + 4 * h;
        const f32x4 ca = *(const SKL_LDS f32x4*)(cf + qi);
        const f32x4 cb = *(const SKL_LDS f32x4*)(cf + BT + qi);
        const f32x4 cc = *(const SKL_LDS f32x4*)(cf + 2 * BT + qi);
        f32x4 cg = f32x4{1.f, 1.f, 1.f, 1.f};
        if constexpr (HAS_G) cg = *(const SKL_LDS f32x4*)(cf + 3 * BT + qi);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * m + e;
          float v2, v1;
          dlogit_both<HAS_G>(s1[r], s2[r], c, p.scale, ca[e], cb[e], cc[e], cg[e], v2, v1);
          if (MASK) {
            const int q = q0 + qi + e;
            const bool ok = (q < p.n_q) & (key < p.n_k) & ((p.causal == 0) | (key <= q + off));
            v2 = ok ? v2 : 0.f;
            v1 = ok ? v1 : 0.f;
          }
          d2[r] = v2;
          d1[r] = v1;
        }
      }
      // dK2^T += Q2^T dS2, dK1^T += Q1^T dS1
      const PackedDS pd2 = pack_ds(d2), pd1 = pack_ds(d1);
      go.run(pd2, pd1, dk2t, dk1t);
    }
  };
  settle_scalar_loads();
  int t = 0;
  for (; t < ntiles && tile_needs_mask(t); ++t) tile(t, std::true_type{});
  for (; t < ntiles && !tile_needs_mask(t); ++t) tile(t, std::false_type{});
  for (; t < ntiles; ++t) tile(t, std::true_type{});

  if (key < p.n_k) {
    float* out2 = p.dk + (hk + key) * D;
    float* out1 = p.dk1 + (hk + key) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int d = db * 32 + 8 * m + 4 * h;
        *(f32x4*)(out2 + d) = f32x4{p.scale * dk2t[db][4 * m], p.scale * dk2t[db][4 * m + 1],
                                    p.scale * dk2t[db][4 * m + 2], p.scale * dk2t[db][4 * m + 3]};
        *(f32x4*)(out1 + d) = f32x4{p.scale * dk1t[db][4 * m], p.scale * dk1t[db][4 * m + 1],
                                    p.scale * dk1t[db][4 * m + 2], p.scale * dk1t[db][4 * m + 3]};
      }
  }
}

// Query-block kernel, both settings: dQ2 = scale dS2 K2 and dQ1 = scale dS1 K1
// for this workgroup's 128 queries (the layout of bwd_q_kernel; SPLIT: a key
// range per workgroup, added atomically).
template <int D, bool SPLIT, bool HAS_G>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1)))
void bwd_q_both_kernel(BwdParams p) {
  using T = __bf16;
  using G = Geom<T, D>;
  using C = QCfg<T, D>;
  // 128-key tiles, as in the key-block kernel above
  constexpr int NW = C::NW, BQ = C::BQ, BK = 2 * C::BK, NKB = 2 * C::NKB, TILE = 2 * C::TILE, DB = D / 32;
  __shared__ __attribute__((aligned(16))) char smem[4 * TILE];
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
  const int pb = pair_base<T, D>(col, h);
  const int tb[2] = {tr_base<D>(lane, 0), tr_base<D>(lane, 1)};

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
  float ca, cb, cc, cg;
  {
    BothVals<HAS_G> v;
    v.load(p, hq + qr);
    v.coefs(ca, cb, cc, cg);
  }

  f32x16 dq2t[DB], dq1t[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) {
    dq2t[i] = f32x16{};
    dq1t[i] = f32x16{};
  }

  TileStream<T, D, BK, NW> ts;
  ts.init(tid);
  if (ntiles > 0) {
    issue_tile_async<T, D, BK, NW>(k1, kbeg, p.n_k, lds, tid, wave);
    issue_tile_async<T, D, BK, NW>(k2, kbeg, p.n_k, lds + TILE, tid, wave);
  }
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
    if (t >= wtiles) return;
    const int k0 = kbeg + t * BK;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      GradOps<D> go;
      go.load(t2, t1, kb * 32, tb);
      __builtin_amdgcn_sched_barrier(0);
      f32x16 s1 = f32x16{}, s2 = f32x16{};
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int g = 0; g < G::kGroups; ++g) {
        const int ob = pair_off(pb, g) + kb * 32 * G::kRowBytes;
        s1 = mfma_chunk<T>(*(const SKL_LDS u32x4*)(t1 + ob), qf1[g], s1);
        s2 = mfma_chunk<T>(*(const SKL_LDS u32x4*)(t2 + ob), qf2[g], s2);
      }
      sched_lds_mfma_pipeline<2 * G::kGroups, 4>();
      __builtin_amdgcn_s_setprio(0);
      float d2[16], d1[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v2, v1;
        dlogit_both<HAS_G>(s1[r], s2[r], c, p.scale, ca, cb, cc, cg, v2, v1);
        if (MASK) {
          const int kk = k0 + kb * 32 + acc_row(r, h);
          const bool ok = (kk < klimit) & (qrow < p.n_q) & ((p.causal == 0) | (kk <= qrow + off));
          v2 = ok ? v2 : 0.f;
          v1 = ok ? v1 : 0.f;
        }
        d2[r] = v2;
        d1[r] = v1;
      }
      // dQ2^T += K2^T dS2^T, dQ1^T += K1^T dS1^T
      const PackedDS pd2 = pack_ds(d2), pd1 = pack_ds(d1);
      go.run(pd2, pd1, dq2t, dq1t);
    }
  };
  settle_scalar_loads();
  int t = 0;
  for (; t < ntiles && tile_needs_mask(t); ++t) tile(t, std::true_type{});
  for (; t < ntiles && !tile_needs_mask(t); ++t) tile(t, std::false_type{});
  for (; t < ntiles; ++t) tile(t, std::true_type{});

  if (qrow < p.n_q) {
    float* out2 = p.dq + (hq + qrow) * D;
    float* out1 = p.dq1 + (hq + qrow) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int d = db * 32 + 8 * m + 4 * h;
        if (SPLIT) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            atomicAdd(out2 + d + e, p.scale * dq2t[db][4 * m + e]);
            atomicAdd(out1 + d + e, p.scale * dq1t[db][4 * m + e]);
          }
        } else {
          *(f32x4*)(out2 + d) = f32x4{p.scale * dq2t[db][4 * m], p.scale * dq2t[db][4 * m + 1],
                                      p.scale * dq2t[db][4 * m + 2], p.scale * dq2t[db][4 * m + 3]};
          *(f32x4*)(out1 + d) = f32x4{p.scale * dq1t[db][4 * m], p.scale * dq1t[db][4 * m + 1],
                                      p.scale * dq1t[db][4 * m + 2], p.scale * dq1t[db][4 * m + 3]};
        }
      }
  }
}

template <int D, bool HAS_G>
static hipError_t both(const BwdParams& p, bool do_dk, bool do_dq, hipStream_t s) {
  using KC = KvCfg<__bf16, D>;
  using QC = QCfg<__bf16, D>;
  hipError_t e = hipSuccess;
  if (do_dk) {
    const int nkb = (p.n_k + KC::BKW - 1) / KC::BKW;
    hipLaunchKernelGGL((bwd_kv_both_kernel<D, HAS_G>), dim3(xcd_grid(p.heads * nkb)), dim3(256), 0, s, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!do_dq) return e;
  const int nqb = (p.n_q + QC::BQ - 1) / QC::BQ;
  if (p.dq_splits > 1) {
    e = zero_fill(p.dq, (size_t)p.heads * p.n_q * D, s);
    if (e != hipSuccess) return e;
    e = zero_fill(p.dq1, (size_t)p.heads * p.n_q * D, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_q_both_kernel<D, true, HAS_G>), dim3(xcd_grid(p.heads * nqb * p.dq_splits)), dim3(256), 0, s, p);
  } else {
    hipLaunchKernelGGL((bwd_q_both_kernel<D, false, HAS_G>), dim3(xcd_grid(p.heads * nqb)), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_both(const BwdParams& p, int dtype, int head_dim, bool dk, bool dq, hipStream_t stream) {
  if (dtype == 0) {
    if (head_dim == 64) return p.dkl ? both<64, true>(p, dk, dq, stream) : both<64, false>(p, dk, dq, stream);
    return p.dkl ? both<128, true>(p, dk, dq, stream) : both<128, false>(p, dk, dq, stream);
  }
  // fp32: the two settings one after the other
  BwdParams a = p;
  a.setting = 1;
  hipError_t e = launch_bwd_separate(a, dtype, head_dim, dk, dq, stream);
  if (e != hipSuccess) return e;
  BwdParams b = p;
  b.setting = 2;
  b.dq = p.dq1;
  b.dk = p.dk1;
  return launch_bwd_separate(b, dtype, head_dim, dk, dq, stream);
}

}  // namespace skl
