// C ABI of the attention-KL library: argument validation, workspace sizing,
// kernel choice and launches.  The operations are defined in streamkl.h; the
// kernels live in fwd.hip and bwd.hip.
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>

#include "kernels.hpp"
#include "streamkl.h"

namespace {

constexpr int kMaxSplits = 1024;
// Largest split-K grid: the kernel indexes its (head, split, query block)
// work items with 32-bit integers (and pads the grid to a multiple of 8).
constexpr long long kMaxWorkgroups = (1LL << 31) - 64;

// Experiment overrides and dispatch logging, read from the environment once per
// process, at the first call that needs them:
//   STREAMKL_LOG=1                     one stderr line per compute call: shape,
//                                      what was chosen, status;
//   STREAMKL_SPLITS=n                  split count when a split-K call passes 0;
//   STREAMKL_BWD_PATH=fused|separate   path when a single-setting backward
//                                      passes AUTO.
// A value that does not parse is ignored, with a warning on stderr.
struct EnvConfig {
  bool log = false;
  int splits = 0;                   // 0: the heuristic
  int bwd_path = STREAMKL_BWD_AUTO; // AUTO: the measured rule
};

const EnvConfig& env_config() {
  static const EnvConfig cfg = [] {
    EnvConfig c;
    const char* s = getenv("STREAMKL_LOG");
    c.log = s && *s && strcmp(s, "0") != 0;
    s = getenv("STREAMKL_SPLITS");
    if (s && *s) {
      char* end = nullptr;
      const long v = strtol(s, &end, 10);
      if (*end == '\0' && v >= 1 && v <= kMaxSplits)
        c.splits = (int)v;
      else
        fprintf(stderr, "streamkl: STREAMKL_SPLITS=%s ignored (want an integer from 1 to %d)\n", s, kMaxSplits);
    }
    s = getenv("STREAMKL_BWD_PATH");
    if (s && *s) {
      if (strcmp(s, "separate") == 0)
        c.bwd_path = STREAMKL_BWD_SEPARATE;
      else if (strcmp(s, "fused") == 0)
        c.bwd_path = STREAMKL_BWD_FUSED;
      else
        fprintf(stderr, "streamkl: STREAMKL_BWD_PATH=%s ignored (want fused or separate)\n", s);
    }
    return c;
  }();
  return cfg;
}

const char* dtype_name(int dtype) {
  return dtype == STREAMKL_BF16 ? "bf16" : dtype == STREAMKL_FP32 ? "fp32" : "dtype?";
}

const char* path_name(int path) {
  switch (path) {
    case STREAMKL_BWD_AUTO: return "auto";
    case STREAMKL_BWD_FUSED: return "fused";
    case STREAMKL_BWD_SEPARATE: return "separate";
    case STREAMKL_BWD_DK_ONLY: return "dk_only";
    case STREAMKL_BWD_DQ_ONLY: return "dq_only";
    default: return "path?";
  }
}

// The dispatch-log line of one compute call.  choose() records what was
// chosen; done() prints the line when STREAMKL_LOG is set and passes the
// status through, so every return of an entry point goes through it.
class CallLog {
 public:
  CallLog(const char* fn, int n_q, int n_k, int heads, int head_dim, int causal, int dtype)
      : fn_(fn), n_q_(n_q), n_k_(n_k), heads_(heads), head_dim_(head_dim), causal_(causal), dtype_(dtype) {
    choice_[0] = '\0';
  }
  __attribute__((format(printf, 2, 3))) void choose(const char* fmt, ...) {
    if (!env_config().log) return;
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(choice_, sizeof(choice_), fmt, ap);
    va_end(ap);
  }
  int done(int status) const {
    if (env_config().log)
      fprintf(stderr, "streamkl: %s heads=%d n_q=%d n_k=%d d=%d causal=%d %s%s%s -> %s\n", fn_, heads_, n_q_, n_k_,
              head_dim_, causal_, dtype_name(dtype_), choice_[0] ? " " : "", choice_, streamkl_strerror(status));
    return status;
  }

 private:
  const char* fn_;
  int n_q_, n_k_, heads_, head_dim_, causal_, dtype_;
  char choice_[200];
};

long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }

int device_cus() {
  // Compute units of the current device (cached per device id, 64 devices;
  // racing first calls store the same value).
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_common(const void* q1, const void* k1, const void* q2, const void* k2, int n_q, int n_k,
                 int heads, int head_dim, int causal, float scale, int dtype) {
  if (!q1 || !k1 || !q2 || !k2) return STREAMKL_ERR_NULL;
  if (n_q < 1 || n_k < 1 || heads < 1) return STREAMKL_ERR_SHAPE;
  if ((long long)heads * n_q >= (1LL << 31) || (long long)heads * n_k >= (1LL << 31)) return STREAMKL_ERR_SHAPE;
  if (causal && n_q > n_k) return STREAMKL_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return STREAMKL_ERR_UNSUPPORTED;
  if (dtype != STREAMKL_BF16 && dtype != STREAMKL_FP32) return STREAMKL_ERR_UNSUPPORTED;
  if (!isfinite(scale) || scale < 0.f) return STREAMKL_ERR_SCALE;
  if (!aligned16(q1) || !aligned16(k1) || !aligned16(q2) || !aligned16(k2)) return STREAMKL_ERR_ALIGN;
  return STREAMKL_OK;
}

skl::FwdParams fwd_params(const void* q1, const void* k1, const void* q2, const void* k2, int n_q, int n_k,
                          int heads, int causal, float scale, float* kl, float* lse1, float* lse2) {
  skl::FwdParams p;
  memset(&p, 0, sizeof(p));
  p.q1 = (const char*)q1;
  p.k1 = (const char*)k1;
  p.q2 = (const char*)q2;
  p.k2 = (const char*)k2;
  p.n_q = n_q;
  p.n_k = n_k;
  p.heads = heads;
  p.causal = causal ? 1 : 0;
  p.scale = scale;
  p.c = scale * 1.4426950408889634f;
  p.kl = kl;
  p.lse1 = lse1;
  p.lse2 = lse2;
  p.splits = 1;
  p.split_keys = n_k;
  return p;
}

// keys per split for `splits` ranges, rounded up to whole key tiles
int split_keys_for(int n_k, int splits) {
  const int t = skl::kFwdKeyTile;
  const int tiles = (n_k + t - 1) / t;
  const int per = (tiles + splits - 1) / splits;
  return per * t;
}

// number of non-empty ranges once rounded to whole tiles
int effective_splits(int n_k, int splits) {
  const int keys = split_keys_for(n_k, splits);
  return (n_k + keys - 1) / keys;
}

int status_of(hipError_t e) { return e == hipSuccess ? STREAMKL_OK : STREAMKL_ERR_HIP; }

// Split count of a validated split-K call, and the partial-state bytes it needs.
int splitk_count(int n_q, int n_k, int heads, int head_dim, int num_splits, size_t* need) {
  const int splits = num_splits == 0 ? streamkl_splitk_auto(n_q, n_k, heads, head_dim)
                                     : effective_splits(n_k, num_splits);
  *need = (size_t)splits * heads * n_q * 5 * sizeof(float);
  return splits;
}

const char* splits_source(int num_splits) {
  return num_splits ? "given" : env_config().splits ? "STREAMKL_SPLITS" : "auto";
}

// Workgroup count of the forward kernel for `splits` key ranges.
long long fwd_workgroups(int n_q, int heads, int splits) {
  return (long long)heads * ceil_div(n_q, skl::fwd_queries_per_block(skl::fwd_waves(n_q))) * splits;
}

// The partial kernel, then the combine, on `stream`, with the partial states in `part`.
int splitk_launch(const void* q1, const void* k1, const void* q2, const void* k2, int n_q, int n_k, int heads,
                  int head_dim, int causal, float scale, streamkl_dtype dtype, int splits, float* kl, float* lse1,
                  float* lse2, float* part, hipStream_t stream) {
  skl::FwdParams p = fwd_params(q1, k1, q2, k2, n_q, n_k, heads, causal, scale, kl, lse1, lse2);
  p.part = part;
  p.splits = splits;
  p.split_keys = split_keys_for(n_k, splits);
  hipError_t e = skl::launch_fwd(p, (int)dtype, head_dim, skl::fwd_waves(n_q), true, stream);
  if (e != hipSuccess) return STREAMKL_ERR_HIP;
  return status_of(skl::launch_splitk_combine(p, stream));
}

}  // namespace

extern "C" {

int streamkl_splitk_auto(int n_q, int n_k, int heads, int head_dim) {
  (void)head_dim;
  if (n_q < 1 || n_k < 1 || heads < 1) return 1;
  if (env_config().splits) return effective_splits(n_k, env_config().splits);
  const int nw = skl::fwd_waves(n_q);
  const long long blocks = (long long)heads * ((n_q + skl::fwd_queries_per_block(nw) - 1) /
                                               skl::fwd_queries_per_block(nw));
  // aim for about 8 workgroups per compute unit, each streaming >= 8 key tiles
  const long long want = 8LL * device_cus();
  long long s = (want + blocks - 1) / blocks;
  const long long max_by_len = (n_k + 8 * skl::kFwdKeyTile - 1) / (8 * skl::kFwdKeyTile);
  if (s > max_by_len) s = max_by_len;
  if (s < 1) s = 1;
  if (s > kMaxSplits) s = kMaxSplits;
  return effective_splits(n_k, (int)s);
}

size_t streamkl_workspace_bytes(int op, int n_q, int n_k, int heads, int head_dim, int num_splits,
                                streamkl_bwd_path path) {
  if (n_q < 1 || n_k < 1 || heads < 1 || (head_dim != 64 && head_dim != 128)) return (size_t)-1;
  if (op == 0) {
    if (num_splits < 0 || num_splits > kMaxSplits) return (size_t)-1;
    size_t need = 0;
    splitk_count(n_q, n_k, heads, head_dim, num_splits, &need);
    return need;
  }
  if (op == 1 || op == 2) {
    if ((int)path < STREAMKL_BWD_AUTO || (int)path > STREAMKL_BWD_DQ_ONLY) return (size_t)-1;
    return 0;
  }
  return (size_t)-1;
}

int streamkl_fwd(const void* q1, const void* k1, const void* q2, const void* k2, int n_q, int n_k,
                 int heads, int head_dim, int causal, float scale, streamkl_dtype dtype, float* kl,
                 float* lse1, float* lse2, hipStream_t stream) {
  CallLog lg("streamkl_fwd", n_q, n_k, heads, head_dim, causal, (int)dtype);
  int st = check_common(q1, k1, q2, k2, n_q, n_k, heads, head_dim, causal, scale, (int)dtype);
  if (st) return lg.done(st);
  if (!kl || !lse1 || !lse2) return lg.done(STREAMKL_ERR_NULL);
  skl::FwdParams p = fwd_params(q1, k1, q2, k2, n_q, n_k, heads, causal, scale, kl, lse1, lse2);
  lg.choose("one-pass waves=%d workgroups=%lld", skl::fwd_waves(n_q), fwd_workgroups(n_q, heads, 1));
  return lg.done(status_of(skl::launch_fwd(p, (int)dtype, head_dim, skl::fwd_waves(n_q), false, stream)));
}

int streamkl_fwd_splitk(const void* q1, const void* k1, const void* q2, const void* k2, int n_q, int n_k,
                        int heads, int head_dim, int causal, float scale, streamkl_dtype dtype,
                        int num_splits, float* kl, float* lse1, float* lse2, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  CallLog lg("streamkl_fwd_splitk", n_q, n_k, heads, head_dim, causal, (int)dtype);
  int st = check_common(q1, k1, q2, k2, n_q, n_k, heads, head_dim, causal, scale, (int)dtype);
  if (st) return lg.done(st);
  if (!kl || !lse1 || !lse2) return lg.done(STREAMKL_ERR_NULL);
  if (num_splits < 0 || num_splits > kMaxSplits) return lg.done(STREAMKL_ERR_UNSUPPORTED);
  size_t need = 0;
  const int splits = splitk_count(n_q, n_k, heads, head_dim, num_splits, &need);
  if (fwd_workgroups(n_q, heads, splits) > kMaxWorkgroups) return lg.done(STREAMKL_ERR_SHAPE);
  lg.choose("splits=%d (%s) keys_per_split=%d workgroups=%lld workspace=%zu/%zu", splits,
            splits_source(num_splits), split_keys_for(n_k, splits), fwd_workgroups(n_q, heads, splits), need,
            workspace_bytes);
  if (!workspace || workspace_bytes < need) return lg.done(STREAMKL_ERR_WORKSPACE);
  if (!aligned16(workspace)) return lg.done(STREAMKL_ERR_ALIGN);
  return lg.done(splitk_launch(q1, k1, q2, k2, n_q, n_k, heads, head_dim, causal, scale, dtype, splits, kl, lse1,
                               lse2, (float*)workspace, stream));
}

int streamkl_fwd_splitk_noalloc(const void* q1, const void* k1, const void* q2, const void* k2, int n_q,
                                int n_k, int heads, int head_dim, int causal, float scale, streamkl_dtype dtype,
                                int num_splits, float* kl, float* lse1, float* lse2, hipStream_t stream) {
  CallLog lg("streamkl_fwd_splitk_noalloc", n_q, n_k, heads, head_dim, causal, (int)dtype);
  int st = check_common(q1, k1, q2, k2, n_q, n_k, heads, head_dim, causal, scale, (int)dtype);
  if (st) return lg.done(st);
  if (!kl || !lse1 || !lse2) return lg.done(STREAMKL_ERR_NULL);
  if (num_splits < 0 || num_splits > kMaxSplits) return lg.done(STREAMKL_ERR_UNSUPPORTED);
  size_t need = 0;
  const int splits = splitk_count(n_q, n_k, heads, head_dim, num_splits, &need);
  if (fwd_workgroups(n_q, heads, splits) > kMaxWorkgroups) return lg.done(STREAMKL_ERR_SHAPE);
  lg.choose("splits=%d (%s) keys_per_split=%d workgroups=%lld scratch=%zu/%zu", splits, splits_source(num_splits),
            split_keys_for(n_k, splits), fwd_workgroups(n_q, heads, splits), need, skl::kNoAllocScratchBytes);
  if (need > skl::kNoAllocScratchBytes) return lg.done(STREAMKL_ERR_TOO_LARGE);
  // The partial kernel writes every (range, head, query) state the combine
  // reads, so the scratch needs no clearing between calls.
  float* part = nullptr;
  if (skl::noalloc_scratch(&part) != hipSuccess) return lg.done(STREAMKL_ERR_HIP);
  return lg.done(splitk_launch(q1, k1, q2, k2, n_q, n_k, heads, head_dim, causal, scale, dtype, splits, kl, lse1,
                               lse2, part, stream));
}

int streamkl_bwd_select(int n_q, int n_k, int heads, int head_dim, int causal) {
  (void)n_q;
  (void)n_k;
  (void)heads;
  (void)head_dim;
  (void)causal;
  // The pages' rule (Methodology 2, Recomputation Strategy, Kernel Fusion
  // paragraph) takes the fused kernel while dQ fits the cache.  On MI355X the
  // fused kernel moves 4*d/128 bytes of fp32 atomics per (query, key) pair,
  // about six times the time of the score recomputation it saves, and
  // measured slower than the separate kernels at every size tried: 0.94x at
  // 64 queries x 128K keys (dQ 1 MiB) down to 0.44x at 16K queries, both
  // settings.  So AUTO takes the separate kernels whatever the shape; the
  // fused path stays available on request (or through STREAMKL_BWD_PATH).
  if (env_config().bwd_path != STREAMKL_BWD_AUTO) return env_config().bwd_path;
  return STREAMKL_BWD_SEPARATE;
}

// Key ranges for the separate path's dQ kernel: enough workgroups to fill the
// chip when there are few query blocks (each range adds into dQ atomically).
static int dq_splits_for(int n_q, int n_k, int heads) {
  const long long blocks = (long long)heads * ((n_q + skl::kBwdQueriesPerBlock - 1) / skl::kBwdQueriesPerBlock);
  const long long want = 4LL * device_cus();
  if (blocks >= want) return 1;
  long long s = (want + blocks - 1) / blocks;
  const long long max_by_len = (n_k + 1023) / 1024;   // at least ~16 key tiles per range
  if (s > max_by_len) s = max_by_len;
  if (s > 64) s = 64;
  return s < 1 ? 1 : (int)s;
}

static int bwd_common(int setting, const void* q1, const void* k1, const void* q2, const void* k2, int n_q,
                      int n_k, int heads, int head_dim, int causal, float scale, streamkl_dtype dtype,
                      const float* lse1, const float* lse2, const float* kl, const float* dkl, float* dq,
                      float* dk, streamkl_bwd_path path, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  (void)workspace;
  (void)workspace_bytes;
  CallLog lg(setting == 1 ? "streamkl_bwd_set1" : "streamkl_bwd_set2", n_q, n_k, heads, head_dim, causal, (int)dtype);
  int st = check_common(q1, k1, q2, k2, n_q, n_k, heads, head_dim, causal, scale, (int)dtype);
  if (st) return lg.done(st);
  if ((int)path < STREAMKL_BWD_AUTO || (int)path > STREAMKL_BWD_DQ_ONLY) return lg.done(STREAMKL_ERR_UNSUPPORTED);
  const bool want_dq = path != STREAMKL_BWD_DK_ONLY, want_dk = path != STREAMKL_BWD_DQ_ONLY;
  if (!lse1 || !lse2 || (want_dq && !dq) || (want_dk && !dk) || (setting == 2 && !kl))
    return lg.done(STREAMKL_ERR_NULL);
  if ((want_dq && !aligned16(dq)) || (want_dk && !aligned16(dk))) return lg.done(STREAMKL_ERR_ALIGN);
  const streamkl_bwd_path asked = path;
  if (path == STREAMKL_BWD_AUTO) {
    path = (streamkl_bwd_path)streamkl_bwd_select(n_q, n_k, heads, head_dim, causal);
    if (path == STREAMKL_BWD_FUSED && !skl::fused_supported((int)dtype, head_dim)) path = STREAMKL_BWD_SEPARATE;
  }
  if (path == STREAMKL_BWD_FUSED && !skl::fused_supported((int)dtype, head_dim))
    return lg.done(STREAMKL_ERR_UNSUPPORTED);
  skl::BwdParams p;
  memset(&p, 0, sizeof(p));
  p.q1 = (const char*)q1;
  p.k1 = (const char*)k1;
  p.q2 = (const char*)q2;
  p.k2 = (const char*)k2;
  p.n_q = n_q;
  p.n_k = n_k;
  p.heads = heads;
  p.causal = causal ? 1 : 0;
  p.scale = scale;
  p.c = scale * 1.4426950408889634f;
  p.lse1 = lse1;
  p.lse2 = lse2;
  p.kl = kl;
  p.dkl = dkl;
  p.dq = dq;
  p.dk = dk;
  p.setting = setting;
  p.dq_splits = path == STREAMKL_BWD_FUSED ? 1 : dq_splits_for(n_q, n_k, heads);
  const long long key_blocks = heads * ceil_div(n_k, skl::kBwdKeysPerBlock);
  const long long query_blocks = heads * ceil_div(n_q, skl::kBwdQueriesPerBlock);
  if (path == STREAMKL_BWD_FUSED) {
    lg.choose("path=fused (asked %s%s) workgroups=%lld", path_name(asked),
              asked == STREAMKL_BWD_AUTO && env_config().bwd_path ? ", STREAMKL_BWD_PATH" : "", key_blocks);
    return lg.done(status_of(skl::launch_bwd_fused(p, (int)dtype, head_dim, stream)));
  }
  lg.choose("path=%s (asked %s%s) dk_workgroups=%lld dq_workgroups=%lld dq_splits=%d",
            path_name(path), path_name(asked),
            asked == STREAMKL_BWD_AUTO && env_config().bwd_path ? ", STREAMKL_BWD_PATH" : "",
            want_dk ? key_blocks : 0LL, want_dq ? query_blocks * p.dq_splits : 0LL, p.dq_splits);
  return lg.done(status_of(skl::launch_bwd_separate(p, (int)dtype, head_dim, want_dk, want_dq, stream)));
}

int streamkl_bwd_set1(const void* q1, const void* k1, const void* q2, const void* k2, int n_q, int n_k,
                      int heads, int head_dim, int causal, float scale, streamkl_dtype dtype,
                      const float* lse1, const float* lse2, const float* dkl, float* dq2, float* dk2,
                      streamkl_bwd_path path, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return bwd_common(1, q1, k1, q2, k2, n_q, n_k, heads, head_dim, causal, scale, dtype, lse1, lse2, nullptr,
                    dkl, dq2, dk2, path, workspace, workspace_bytes, stream);
}

int streamkl_bwd_set2(const void* q1, const void* k1, const void* q2, const void* k2, int n_q, int n_k,
                      int heads, int head_dim, int causal, float scale, streamkl_dtype dtype,
                      const float* lse1, const float* lse2, const float* kl, const float* dkl, float* dq1,
                      float* dk1, streamkl_bwd_path path, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  return bwd_common(2, q1, k1, q2, k2, n_q, n_k, heads, head_dim, causal, scale, dtype, lse1, lse2, kl, dkl,
                    dq1, dk1, path, workspace, workspace_bytes, stream);
}

int streamkl_bwd_both(const void* q1, const void* k1, const void* q2, const void* k2, int n_q, int n_k,
                      int heads, int head_dim, int causal, float scale, streamkl_dtype dtype,
                      const float* lse1, const float* lse2, const float* kl, const float* dkl, float* dq1,
                      float* dk1, float* dq2, float* dk2, streamkl_bwd_path path, hipStream_t stream) {
  CallLog lg("streamkl_bwd_both", n_q, n_k, heads, head_dim, causal, (int)dtype);
  int st = check_common(q1, k1, q2, k2, n_q, n_k, heads, head_dim, causal, scale, (int)dtype);
  if (st) return lg.done(st);
  if ((int)path < STREAMKL_BWD_AUTO || (int)path > STREAMKL_BWD_DQ_ONLY || path == STREAMKL_BWD_FUSED)
    return lg.done(STREAMKL_ERR_UNSUPPORTED);
  const bool want_dq = path != STREAMKL_BWD_DK_ONLY, want_dk = path != STREAMKL_BWD_DQ_ONLY;
  if (!lse1 || !lse2 || !kl || (want_dq && (!dq1 || !dq2)) || (want_dk && (!dk1 || !dk2)))
    return lg.done(STREAMKL_ERR_NULL);
  if ((want_dq && (!aligned16(dq1) || !aligned16(dq2))) || (want_dk && (!aligned16(dk1) || !aligned16(dk2))))
    return lg.done(STREAMKL_ERR_ALIGN);
  skl::BwdParams p;
  memset(&p, 0, sizeof(p));
  p.q1 = (const char*)q1;
  p.k1 = (const char*)k1;
  p.q2 = (const char*)q2;
  p.k2 = (const char*)k2;
  p.n_q = n_q;
  p.n_k = n_k;
  p.heads = heads;
  p.causal = causal ? 1 : 0;
  p.scale = scale;
  p.c = scale * 1.4426950408889634f;
  p.lse1 = lse1;
  p.lse2 = lse2;
  p.kl = kl;
  p.dkl = dkl;
  p.dq = dq2;
  p.dk = dk2;
  p.dq1 = dq1;
  p.dk1 = dk1;
  p.dq_splits = dq_splits_for(n_q, n_k, heads);
  lg.choose("path=%s dk_workgroups=%lld dq_workgroups=%lld dq_splits=%d",
            path == STREAMKL_BWD_AUTO ? "separate" : path_name(path),
            want_dk ? heads * ceil_div(n_k, skl::kBwdKeysPerBlock) : 0LL,
            want_dq ? heads * ceil_div(n_q, skl::kBwdQueriesPerBlock) * p.dq_splits : 0LL, p.dq_splits);
  return lg.done(status_of(skl::launch_bwd_both(p, (int)dtype, head_dim, want_dk, want_dq, stream)));
}

const char* streamkl_strerror(int status) {
  switch (status) {
    case STREAMKL_OK: return "ok";
    case STREAMKL_ERR_NULL: return "a required pointer is NULL";
    case STREAMKL_ERR_SHAPE: return "invalid shape (n_q, n_k, heads < 1, too large, or causal with n_q > n_k)";
    case STREAMKL_ERR_UNSUPPORTED: return "unsupported head_dim, dtype, path or split count";
    case STREAMKL_ERR_SCALE: return "scale must be finite and >= 0";
    case STREAMKL_ERR_WORKSPACE: return "workspace missing or too small";
    case STREAMKL_ERR_HIP: return "HIP launch error";
    case STREAMKL_ERR_ALIGN: return "array not 16-byte aligned";
    case STREAMKL_ERR_TOO_LARGE: return "split-K partial states exceed the 8 MiB scratch of streamkl_fwd_splitk_noalloc";
    default: return "unknown status";
  }
}

}  // extern "C"
