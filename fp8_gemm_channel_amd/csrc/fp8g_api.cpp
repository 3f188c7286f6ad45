// fp8g_api.cpp -- C ABI of libfp8g.so: argument checks, the launch planner and
// the entry points declared in include/fp8g.h.
//
// The planner picks a path by the M regime, as the pages' kernels do: the
// decode-shaped M (a handful of rows) is memory-bound and runs as split-K over
// the streamed weight ("Claude Fable 5", Triton split-K cell, for a small M;
// "Kimi K3 (256k)", SM90 WGMMA and SM120 cells, skinny split-K paths; here up
// to M = 128, where measurements put the boundary on MI355X), and
// everything else runs as one tiled MFMA kernel whose tile shrinks for small
// problems so the launch still fills the chip.  Configurations are fixed per
// shape class, never tuned at run time ("GLM-5.2", B200 TMA Triton cell and
// single-Triton-kernel cell: pinned per-regime configs).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "fp8g.h"
#include "fp8g_internal.h"

namespace {

thread_local std::string g_last_error;
// Call ids for the split-K tickets.  A ticket left in the (uninitialized)
// workspace by an earlier call, or any other stale bytes there, must not look
// like this call's: ids are a counter passed through the splitmix64 finalizer
// (a bijection), so consecutive ids differ in about half their 56 bits and no
// simple pattern (zero, small integers, float bits) is likely to match one.
// Ids keep 48 bits: a ticket holds (id << 16 | arrivals); no id is 0.
std::atomic<unsigned long long> g_call_counter{0};

unsigned long long call_id() {
  unsigned long long z = g_call_counter.fetch_add(1, std::memory_order_relaxed) + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  z &= (1ull << 48) - 1;
  return z ? z : 1;  // 0 marks a released ticket
}

int fail(int status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int hip_fail(hipError_t e, const char *what) {
  return fail(FP8G_ERR_HIP, "%s: %s (%s)", what, hipGetErrorName(e), hipGetErrorString(e));
}

// Workspace memory (split-K partials and tickets, stream-K partials):
// stream-ordered allocations from one memory pool per device.  The pool keeps
// up to kPoolKeepBytes of freed blocks for reuse across synchronisations and
// returns anything above that: with a pool that returns all memory at every
// synchronisation, each call mapped fresh pages (a 34 MB workspace measured
// ~25 us of extra call time), while an unbounded one would keep the largest
// workspace ever used for the life of the process.  Created on first use.
constexpr uint64_t kPoolKeepBytes = uint64_t(64) << 20;
constexpr int kMaxDevices = 64;
std::mutex g_pool_mutex;
hipMemPool_t g_pools[kMaxDevices] = {};

hipError_t workspace_alloc(void **ptr, size_t bytes, hipStream_t stream) {
  // the pool of the device the stream runs on (the kernels run there too,
  // whatever device is current)
  hipDevice_t dev = -1;
  hipError_t e = hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  hipMemPool_t pool;
  {
    std::lock_guard<std::mutex> lock(g_pool_mutex);
    if (!g_pools[dev]) {
      hipMemPoolProps props;
      memset(&props, 0, sizeof props);
      props.allocType = hipMemAllocationTypePinned;
      props.location.type = hipMemLocationTypeDevice;
      props.location.id = dev;
      hipMemPool_t created;
      e = hipMemPoolCreate(&created, &props);
      if (e != hipSuccess) return e;
      uint64_t keep = kPoolKeepBytes;
      e = hipMemPoolSetAttribute(created, hipMemPoolAttrReleaseThreshold, &keep);
      if (e != hipSuccess) {
        (void)hipMemPoolDestroy(created);
        return e;
      }
      g_pools[dev] = created;
    }
    pool = g_pools[dev];
  }
  return hipMallocFromPoolAsync(ptr, bytes, pool, stream);
}

constexpr int kNumCUs = 256;          // MI355X compute units
// The split-K path takes M <= 128 and is the default there.  Measured on MI355X
// for 65 <= M <= 128 (cold, events attached): faster than the best main-path
// tile on 16 of 24 shapes, by up to 4.5x (1024 x 28672), at most 5% slower
// on the others (N >= 12288 with K = 4096, where the main path has the
// workgroups too).
constexpr int kSkinnyMaxM = 128;
constexpr int kSkinnyAutoM = 128;
constexpr int kMaxSplit = 64;
constexpr int kMaxStreamK = 2048;    // stream-K workgroups (2 partial tiles each must stay below 2 GiB)

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Threads per workgroup of each kernel configuration.
int64_t block_threads(int32_t path, int32_t variant) {
  if (path == FP8G_PATH_SPLITK) return variant > 20 ? 512 : 256;
  if (variant == 27) return 64;
  return (variant == 3 || variant == 19 || variant == 20) ? 256 : 512;
}

// A launch's work-items along x must stay below 2^32 (HIP's grid limit).
int check_grid(const fp8g_plan &p, int64_t grid_x) {
  if (grid_x * block_threads(p.path, p.variant) > (int64_t)UINT32_MAX)
    return fail(FP8G_ERR_UNSUPPORTED, "launch of %lld workgroups exceeds the grid limit", (long long)grid_x);
  return FP8G_OK;
}

// Bytes of split-K tickets (one 128-byte line per column tile), padded so the
// partials that follow start 256-byte aligned.
int64_t splitk_ticket_bytes(int64_t tiles) { return cdiv(tiles * 8 * fp8g::kTicketStride, 256) * 256; }

int check_dims(int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K < 0) return fail(FP8G_ERR_INVALID_ARG, "negative dimension (M=%lld N=%lld K=%lld)",
                                           (long long)M, (long long)N, (long long)K);
  if (M > FP8G_MAX_MN || N > FP8G_MAX_MN)
    return fail(FP8G_ERR_INVALID_ARG, "M or N above %lld", (long long)FP8G_MAX_MN);
  if (K > FP8G_MAX_K) return fail(FP8G_ERR_INVALID_ARG, "K=%lld above %lld", (long long)K, (long long)FP8G_MAX_K);
  return FP8G_OK;
}

// Main-path configuration for (M, N, K) when not forced.  Few tiles: 64 x 64
// (variant 3, several workgroups per compute unit).  Otherwise the cheapest of
// three tile sizes by  waves of tiles x flops per tile / sustained rate of one
// compute unit, the rates measured on MI355X with full waves (cold cache):
// 256 x 256 (variant 10) ~10.4 TFLOP/s (8192^3), 128 x 256 (variant 17) ~7.0
// (1024 x 8192 x 8192), 128 x 128 with eight waves (variant 18) ~4.9
// (512 x 8192 x 8192).  On the shapes measured this picks the fastest variant:
// 4096^3, 8192^3, 3072^3 -> 10; 1024 x 8192^2, 1536 x 4096^2, 512 x 12288 x
// 4096 -> 17; 512 x 8192^2, 768 x 4096^2, 2048^3 -> 18; 128 x 8192^2 -> 3.
int auto_main_variant(int64_t M, int64_t N, int64_t K) {
  // Tiny problems (at most 256 blocks of 16 x 16 and two K steps): the
  // register-tile kernel, one memory round trip with nothing staged in LDS.
  // Measured on MI355X against variant 3 (interleaved, cold, outputs
  // identical): 256^3 -2.9%, 240^2 x 256 -11.5%, 144 x 256 x 256 -3.9%, level at
  // K = 128 and 256 x 384 x 256; slower from K = 384 (+6%) or 320^2 (+4%) on.
  if (K <= 256 && K % 16 == 0 && cdiv(M, 16) * cdiv(N, 16) <= 256) return 27;
  if (cdiv(M, 128) * cdiv(N, 128) < kNumCUs / 2) return 3;
  struct Cand {
    int variant, bm, bn;
    double tflops_per_cu;
  };
  static const Cand cands[] = {{10, 256, 256, 10.4}, {17, 128, 256, 7.0}, {18, 128, 128, 4.9}};
  const double kp = (double)cdiv(K, 128) * 128;
  int best = 10;
  double best_t = -1;
  for (const Cand &c : cands) {
    const int64_t waves = cdiv(cdiv(M, c.bm) * cdiv(N, c.bn), kNumCUs);
    const double t = (double)waves * 2.0 * c.bm * c.bn * kp / (c.tflops_per_cu * 1e12);
    if (best_t < 0 || t < best_t) {
      best_t = t;
      best = c.variant;
    }
  }
  return best;
}

int64_t slice_bytes(int64_t K, int64_t S) {
  const int64_t chunk = fp8g::skinny_chunk_bytes();
  return cdiv(cdiv(K, S), chunk) * chunk;
}

// Rows per workgroup (16 * rb), K slices S and kernel of the split-K path when
// nothing is forced.  Rules fitted to measurements on MI355X (cold cache,
// every configuration of a shape timed in interleaved rounds; M = 1 .. 64,
// N = 1024 .. 28672, K = 2048 .. 28672; within 1.3% of the best configuration
// on geometric mean, 9% at worst): up to 32 rows of x, the 8-wave kernel with
// the most w rows per workgroup that still gives at least 160 workgroups
// without splitting K (a K split costs ~3 us of partial hand-off); otherwise
// the most rows for which K slices of at least 4 KiB reach 160 workgroups;
// otherwise 16 rows unsplit.  With 33 .. 64 rows of x (re-read from L2 by
// every workgroup), the 4-wave kernel with 32 rows, or 16 when 32 cannot
// reach 160 workgroups, splitting K while slices keep at least 2 KiB per 16
// rows.
void auto_splitk(int64_t M, int64_t N, int64_t K, int64_t *rb_out, int64_t *S_out, int *kind_base) {
  auto grow = [&](int64_t nb, int64_t target, int64_t min_slice) {
    int64_t S = 1;
    while (nb * S < target && S < kMaxSplit && slice_bytes(K, 2 * S) >= min_slice) S *= 2;
    return S;
  };
  constexpr int64_t kMinWorkgroups = 160;
  if (M <= 32) {
    const int max_rb = fp8g::skinny_max_row_blocks((int)M, fp8g::SkinnyKind::kRing8);
    *kind_base = 20;
    for (int rb = max_rb; rb >= 2; --rb)
      if (cdiv(N, 16 * rb) >= kMinWorkgroups) {
        *rb_out = rb;
        *S_out = 1;
        return;
      }
    for (int rb = max_rb; rb >= 1; --rb) {
      const int64_t nb = cdiv(N, 16 * rb), S = grow(nb, kMinWorkgroups, 4096);
      if (nb * S >= kMinWorkgroups) {
        *rb_out = rb;
        *S_out = S;
        return;
      }
    }
    *rb_out = 1;
    *S_out = 1;
    return;
  }
  *kind_base = 0;
  for (int rb = 2; rb >= 1; --rb) {
    const int64_t nb = cdiv(N, 16 * rb), S = grow(nb, kMinWorkgroups, 2048 * rb);
    if (nb * S >= kMinWorkgroups || rb == 1) {
      *rb_out = rb;
      *S_out = S;
      return;
    }
  }
}

int plan_impl(int64_t M, int64_t N, int64_t K, int32_t path, int32_t variant, int32_t split_k, fp8g_plan *p) {
  if (!p) return fail(FP8G_ERR_INVALID_ARG, "plan output pointer is null");
  int st = check_dims(M, N, K);
  if (st) return st;
  memset(p, 0, sizeof *p);
  p->split_k = 1;
  p->k_slice = K;
  if (path != 0 && path != FP8G_PATH_MAIN && path != FP8G_PATH_SPLITK)
    return fail(FP8G_ERR_INVALID_ARG, "unknown path override %d", path);
  if (split_k < 0 || split_k > kMaxStreamK)
    return fail(FP8G_ERR_INVALID_ARG, "split_k=%d outside 0..%d", split_k, kMaxStreamK);
  if (variant < 0) return fail(FP8G_ERR_INVALID_ARG, "negative variant %d", variant);
  if (M == 0 || N == 0) {
    p->path = FP8G_PATH_NONE;
    return FP8G_OK;
  }
  if (K == 0) {
    p->path = FP8G_PATH_ZERO;
    p->grid = 1;
    return FP8G_OK;
  }
  if (path == 0) path = (M <= kSkinnyAutoM) ? FP8G_PATH_SPLITK : FP8G_PATH_MAIN;
  if (path == FP8G_PATH_SPLITK) {
    if (M > kSkinnyMaxM) return fail(FP8G_ERR_INVALID_ARG, "split-K path needs M <= %d (M=%lld)", kSkinnyMaxM, (long long)M);
    if (split_k > kMaxSplit)
      return fail(FP8G_ERR_INVALID_ARG, "split-K path takes split_k 0..%d (split_k=%d)", kMaxSplit, split_k);
    // Variants 1-5 force the LDS-ring kernel with 16 * variant w rows per
    // workgroup and 4 waves, 21-24 the same kernel with 8 waves and
    // 16 * (variant - 20) rows; 0 lets the planner choose.
    const fp8g::SkinnyKind kind = variant > 20 ? fp8g::SkinnyKind::kRing8 : fp8g::SkinnyKind::kRing4;
    const int kind_base = variant > 20 ? 20 : 0;
    const int forced_rb = variant - kind_base;
    const int max_rb = fp8g::skinny_max_row_blocks((int)M, kind);
    if (forced_rb > max_rb || (variant > 5 && variant < 21) || variant > 24)
      return fail(FP8G_ERR_INVALID_ARG, "split-K variant %d not available for M=%lld", variant, (long long)M);
    const int64_t chunk = fp8g::skinny_chunk_bytes();
    const int64_t nchunks = cdiv(K, chunk);
    const int64_t m_rows = M <= 16 ? 16 : (M <= 32 ? 32 : (M <= 64 ? 64 : 128));  // x rows staged per chunk
    // Choose rows per workgroup (16 * rb) and the number of K slices S by a
    // bandwidth model: workgroups run in rounds of one per compute unit; a round
    // costs the w bytes one workgroup streams plus a quarter of its x bytes (x
    // is re-read from L2); S > 1 adds the partials round trip and the final
    // reduction by one workgroup per column tile (about 2 us of one CU's share
    // of HBM bandwidth, ~48 KiB).
    int64_t best_cost = -1, best_rb = 1, best_S = 1;
    int kbase = kind_base;
    if (variant == 0 && split_k == 0) {
      auto_splitk(M, N, K, &best_rb, &best_S, &kbase);
      best_cost = 0;  // chosen: skip the model below
    }
    for (int rb = 1; rb <= max_rb && best_cost != 0; ++rb) {
      if (forced_rb != 0 && rb != forced_rb) continue;
      const int64_t nb = cdiv(N, 16 * rb);
      for (int64_t S0 = 1; S0 <= kMaxSplit; S0 *= 2) {
        int64_t S = split_k ? split_k : S0;
        if (split_k && S0 > 1) break;
        const int64_t k_slice = cdiv(cdiv(K, S), chunk) * chunk;
        S = cdiv(K, k_slice);
        const int64_t rounds = cdiv(nb * S, kNumCUs);
        int64_t cost = rounds * (16 * rb * k_slice + m_rows * k_slice / 4);
        if (S > 1) cost += 48 * 1024 + (2 * S * M * N * 4 + M * N * 2) / kNumCUs;
        if (best_cost < 0 || cost < best_cost) {
          best_cost = cost;
          best_rb = rb;
          best_S = S;
        }
        if (S >= nchunks) break;
      }
    }
    const fp8g::SkinnyConfig *c = fp8g::skinny_config((int)best_rb + kbase);
    if (!c) return fail(FP8G_ERR_INVALID_ARG, "unknown split-K variant %d", variant);
    const int64_t k_slice = cdiv(cdiv(K, best_S), chunk) * chunk;
    const int64_t S = cdiv(K, k_slice);  // no empty slices
    p->path = FP8G_PATH_SPLITK;
    p->variant = c->id;
    p->tile_m = (int32_t)m_rows;
    p->tile_n = fp8g::skinny_tile_n(*c);
    p->tile_k = (int32_t)chunk;
    p->split_k = (int32_t)S;
    p->k_slice = k_slice;
    p->k_tail = (K % chunk) != 0;
    p->grid = cdiv(N, p->tile_n) * S;
    // one ticket line per column tile (padded to 256 bytes), then the fp32
    // partials, tile-major: [column tile][S][M][tile_n]
    p->workspace_bytes = S > 1 ? splitk_ticket_bytes(cdiv(N, p->tile_n)) +
                                     cdiv(N, p->tile_n) * S * M * p->tile_n * (int64_t)sizeof(float)
                               : 0;
    return check_grid(*p, cdiv(N, p->tile_n));  // the launch grid is (column tiles, S)
  }
  const bool auto_variant = variant == 0;
  if (auto_variant) variant = auto_main_variant(M, N, K);
  if (split_k != 0 && variant != 16)
    return fail(FP8G_ERR_INVALID_ARG, "main variant %d takes no split_k (split_k=%d)", variant, split_k);

  const fp8g::MainConfig *c = fp8g::main_config(variant);
  if (!c) return fail(FP8G_ERR_INVALID_ARG, "unknown main variant %d", variant);
  const int64_t tiles_m = cdiv(M, c->bm), tiles_n = cdiv(N, c->bn);
  if (tiles_m * tiles_n > INT32_MAX) return fail(FP8G_ERR_UNSUPPORTED, "too many tiles");
  p->path = FP8G_PATH_MAIN;
  p->variant = variant;
  p->tile_m = c->bm;
  p->tile_n = c->bn;
  p->tile_k = c->bk;
  p->group_m = (int32_t)(tiles_m < 8 ? tiles_m : 8);
  // Operand rows are always read where they are: K need not be a multiple of
  // anything, and the last K step is masked inside the kernel (bytes at or
  // past K load as zeros).  Nothing is copied or padded.
  p->k_tail = (K % c->bk) != 0;
  // Where the 256 x 256 tiles are chosen and there is no K tail (K % 128 ==
  // 0), the one-wave-per-SIMD kernel runs them: same tiles and the same sums
  // in the same order, measured faster or level (interleaved with variant 10
  // on one MI355X: 8192^3 393 vs 418 us, 1536 x 8192^2 100.5 vs 108.0,
  // 2560 x 4096^2 50.7 vs 52.8, 3072^3 42.0 vs 42.7, 4096^3 level within 1%).
  if (auto_variant && variant == 10 && !p->k_tail) {
    variant = 19;
    p->variant = 19;
  }
  if (variant == 19 && p->k_tail)
    return fail(FP8G_ERR_INVALID_ARG, "main variant 19 needs K %% 128 == 0 (K=%lld)", (long long)K);
  // Variant 20 (rows fetched as whole cache lines, realigned in registers) needs
  // odd K above 128 (two K steps at least), the last row of each operand to end
  // on a 16-byte boundary (M K and N K multiples of 16) and 128-byte-aligned
  // operands (checked by the call, which runs variant 10 instead when the plan
  // was the planner's choice).  Where it
  // applies it replaces variant 10 for odd K: measured on MI355X at 4096^2 x
  // 4127, 74.6 us against 89.2 us for variant 10 streaming the rows as they lie.
  const bool lines_ok = (M * K) % 16 == 0 && (N * K) % 16 == 0;
  if (auto_variant && variant == 10 && K % 2 == 1 && K > 128 && lines_ok) {
    variant = 20;
    p->variant = 20;
  }
  if (variant == 27 && K % 16 != 0)
    return fail(FP8G_ERR_INVALID_ARG, "main variant 27 needs K %% 16 == 0 (K=%lld)", (long long)K);
  if (variant == 20 && (K % 2 == 0 || K <= 128))
    return fail(FP8G_ERR_INVALID_ARG, "main variant 20 needs odd K above 128 (K=%lld)", (long long)K);
  if (variant == 20 && !lines_ok)
    return fail(FP8G_ERR_INVALID_ARG, "main variant 20 needs M*K and N*K multiples of 16 (M=%lld N=%lld K=%lld)",
                (long long)M, (long long)N, (long long)K);
  p->grid = tiles_m * tiles_n;
  p->dp_tiles = (int32_t)(tiles_m * tiles_n);
  if (variant == 16) {
    // Stream-K: whole waves of tiles stay one tile per workgroup except the
    // last, which joins the partial wave; one workgroup per compute unit then
    // splits the (tile, K step) units of those tiles evenly, so every compute
    // unit gets between one and two tiles' worth (less than one when the tiles
    // do not fill a wave).  split_k forces the number of stream-K workgroups.
    const int64_t T = tiles_m * tiles_n, nk = cdiv(K, c->bk);
    const int64_t n_dp = T > kNumCUs ? (T / kNumCUs - 1) * kNumCUs : 0;
    if (T * nk >= INT32_MAX) return fail(FP8G_ERR_UNSUPPORTED, "stream-K needs tiles x K steps below 2^31");
    int64_t n_sk = split_k > 0 ? split_k : kNumCUs;
    if (n_sk > (T - n_dp) * nk) n_sk = (T - n_dp) * nk;  // at least one unit each
    p->dp_tiles = (int32_t)n_dp;
    p->sk_groups = (int32_t)n_sk;
    p->grid = n_dp + n_sk;
    p->workspace_bytes = splitk_ticket_bytes(T - n_dp) + 2 * n_sk * fp8g::kMainPartialBytes;
  }
  return check_grid(*p, p->grid);
}

bool overlaps(const void *a, size_t an, const void *b, size_t bn) {
  if (!a || !b || an == 0 || bn == 0) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + bn && b0 < a0 + an;
}

// Every configuration is built for every operand format except stream-K
// (main variant 16, E4M3 only).
bool supports_formats(const fp8g_plan &p) { return !(p.path == FP8G_PATH_MAIN && p.variant == 16); }

// Workspace of one call: from the pool (stream-ordered allocation, freed on
// the stream after the kernel), or -- with `fixed` -- the caller's buffer.
hipError_t call_workspace(const fp8g::FixedWorkspace *fixed, void **ws, size_t bytes, hipStream_t stream) {
  return fixed ? fixed->get(stream, ws) : workspace_alloc(ws, bytes, stream);
}
hipError_t release_workspace(const fp8g::FixedWorkspace *fixed, void *ws, hipStream_t stream) {
  return (fixed || !ws) ? hipSuccess : hipFreeAsync(ws, stream);
}

int run(const void *x, const void *w, const float *scale, const float *bias, void *y, int64_t M, int64_t N,
        int64_t K, int32_t x_format, int32_t w_format, int32_t act, int32_t path, int32_t variant, int32_t split_k,
        void *stream_ptr, void *start_event = nullptr, void *stop_event = nullptr,
        const fp8g::FixedWorkspace *fixed = nullptr) {
  g_last_error.clear();
  if ((x_format != FP8G_FMT_E4M3 && x_format != FP8G_FMT_E5M2) ||
      (w_format != FP8G_FMT_E4M3 && w_format != FP8G_FMT_E5M2))
    return fail(FP8G_ERR_INVALID_ARG, "unknown operand format (x_format=%d w_format=%d)", x_format, w_format);
  if (act < FP8G_ACT_NONE || act > FP8G_ACT_GELU_TANH) return fail(FP8G_ERR_INVALID_ARG, "unknown activation %d", act);
  const int fmt = (w_format << 1) | x_format;
  fp8g_plan p;
  int st = plan_impl(M, N, K, path, variant, split_k, &p);
  if (st) return st;
  if (fixed && (uint64_t)p.workspace_bytes > fixed->capacity)
    return fail(FP8G_ERR_UNSUPPORTED,
                "the plan needs %lld bytes of workspace; the allocation-free entry point has %llu "
                "(choose fewer K slices or stream-K workgroups)",
                (long long)p.workspace_bytes, (unsigned long long)fixed->capacity);
  if (fmt != 0 && !supports_formats(p))
    return fail(FP8G_ERR_INVALID_ARG, "%s variant %d is built for E4M3 operands only", p.path == FP8G_PATH_MAIN ? "main" : "split-K",
                p.variant);
  hipStream_t stream = (hipStream_t)stream_ptr;
  const fp8g::DispatchEvents events{(hipEvent_t)start_event, (hipEvent_t)stop_event};
  if (p.path == FP8G_PATH_NONE) {
    // no kernel to attach the events to: record them on the stream instead
    hipError_t e = hipSuccess;
    if (events.start) e = hipEventRecord(events.start, stream);
    if (e == hipSuccess && events.stop) e = hipEventRecord(events.stop, stream);
    return e == hipSuccess ? FP8G_OK : hip_fail(e, "hipEventRecord (empty extent)");
  }
  if (!y) return fail(FP8G_ERR_INVALID_ARG, "y is null");
  if (!scale) return fail(FP8G_ERR_INVALID_ARG, "scale is null");
  if (K > 0 && (!x || !w)) return fail(FP8G_ERR_INVALID_ARG, "x or w is null");
  if ((uintptr_t)scale % 4) return fail(FP8G_ERR_INVALID_ARG, "scale is not 4-byte aligned");
  if ((uintptr_t)y % 2) return fail(FP8G_ERR_INVALID_ARG, "y is not 2-byte aligned");
  if ((uintptr_t)bias % 4) return fail(FP8G_ERR_INVALID_ARG, "bias is not 4-byte aligned");
  const size_t ybytes = (size_t)M * (size_t)N * 2;
  if (overlaps(y, ybytes, x, (size_t)M * (size_t)K) || overlaps(y, ybytes, w, (size_t)N * (size_t)K) ||
      overlaps(y, ybytes, scale, (size_t)N * 4) || overlaps(y, ybytes, bias, (size_t)N * 4))
    return fail(FP8G_ERR_INVALID_ARG, "y overlaps an input");

  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");

  const bool vec = (N % 4 == 0) && ((uintptr_t)y % 8 == 0);
  if (p.path == FP8G_PATH_ZERO) {
    // K = 0: the empty sum is +0; with a bias or an activation y = act(bias)
    if (bias || act != FP8G_ACT_NONE) e = fp8g::launch_empty_k((uint16_t *)y, bias, act, M, N, stream, events);
    else e = fp8g::launch_zero((uint16_t *)y, M * N, stream, events);
    return e == hipSuccess ? FP8G_OK : hip_fail(e, "K = 0 launch");
  }
  if (p.path == FP8G_PATH_MAIN && p.variant == 20 && (((uintptr_t)x | (uintptr_t)w) & 127u)) {
    // whole-line fetches would start before an operand that is not 128-byte aligned
    if (variant != 0)
      return fail(FP8G_ERR_INVALID_ARG, "main variant 20 needs x and w 128-byte aligned");
    p.variant = 10;
  }
  if (p.path == FP8G_PATH_MAIN) {
    const int ystore = (N % 8 == 0 && (uintptr_t)y % 16 == 0) ? 16 : vec ? 8 : 2;
    fp8g::MainLaunch l{(const uint8_t *)x, (const uint8_t *)w, scale, (uint16_t *)y, (int)M, (int)N, (int)K,
                       (int)cdiv(M, p.tile_m), (int)cdiv(N, p.tile_n), p.group_m, p.variant, p.k_tail != 0, ystore};
    l.bias = bias;
    l.act = act;
    l.fmt = fmt;
    l.ywb = cdiv(M, p.tile_m) * cdiv(N, p.tile_n) > kNumCUs ? 1 : 0;
    l.ev = events;
    void *ws = nullptr;
    if (p.workspace_bytes > 0) {
      // stream-K: the tickets of the stream-K tiles, then two partial tiles per
      // stream-K workgroup; uninitialized (tickets carry the call id, partials
      // are written before they are read)
      e = call_workspace(fixed, &ws, (size_t)p.workspace_bytes, stream);
      if (e != hipSuccess) return hip_fail(e, "workspace (main path)");
      const int64_t sk_tiles = cdiv(M, p.tile_m) * cdiv(N, p.tile_n) - p.dp_tiles;
      l.n_dp = p.dp_tiles;
      l.n_sk = p.sk_groups;
      l.tickets = (unsigned long long *)ws;
      l.partials = (float *)((char *)ws + splitk_ticket_bytes(sk_tiles));
      l.epoch = call_id();
    }
    if (e == hipSuccess) e = fp8g::launch_main(l, stream);
    const hipError_t f = release_workspace(fixed, ws, stream);
    if (e == hipSuccess && f != hipSuccess) return hip_fail(f, "hipFreeAsync(main-path workspace)");
    return e == hipSuccess ? FP8G_OK : hip_fail(e, "main kernel launch");
  }
  // split-K
  void *ws = nullptr;
  float *partials = nullptr;
  unsigned long long *tickets = nullptr;
  if (p.split_k > 1) {
    e = call_workspace(fixed, &ws, (size_t)p.workspace_bytes, stream);
    if (e != hipSuccess) return hip_fail(e, "workspace (split-K)");
    // The workspace is not initialized: a ticket carries the call id, so stale
    // values are harmless, and every partial is written before it is read.
    tickets = (unsigned long long *)ws;
    partials = (float *)((char *)ws + splitk_ticket_bytes(cdiv(N, p.tile_n)));
  }
  const unsigned long long epoch = call_id();
  fp8g::SkinnyLaunch l{(const uint8_t *)x, (const uint8_t *)w, scale, (uint16_t *)y, partials, tickets, epoch,
                       (int)M, (int)N, (int)K, (int)p.k_slice, p.split_k, p.variant, vec};
  l.bias = bias;
  l.act = act;
  l.fmt = fmt;
  l.ev = events;
  e = fp8g::launch_skinny(l, stream);
  const hipError_t f = release_workspace(fixed, ws, stream);
  if (e == hipSuccess && f != hipSuccess) return hip_fail(f, "hipFreeAsync(split-K workspace)");
  return e == hipSuccess ? FP8G_OK : hip_fail(e, "split-K kernel launch");
}

}  // namespace

namespace fp8g {
int run_fixed_workspace(const void *x, const void *w, const float *scale, void *y, int64_t M, int64_t N, int64_t K,
                        int32_t path, int32_t variant, int32_t split_k, void *stream, const FixedWorkspace &ws) {
  return run(x, w, scale, nullptr, y, M, N, K, FP8G_FMT_E4M3, FP8G_FMT_E4M3, FP8G_ACT_NONE, path, variant, split_k,
             stream, nullptr, nullptr, &ws);
}
}  // namespace fp8g

extern "C" {

int fp8_gemm_scaled(const void *x, const void *w, const float *scale, void *y, int64_t M, int64_t N, int64_t K,
                    void *stream) {
  return run(x, w, scale, nullptr, y, M, N, K, FP8G_FMT_E4M3, FP8G_FMT_E4M3, FP8G_ACT_NONE, 0, 0, 0, stream);
}

int fp8_gemm_scaled_ex(const void *x, const void *w, const float *scale, void *y, int64_t M, int64_t N, int64_t K,
                       int32_t path, int32_t variant, int32_t split_k, void *stream) {
  return run(x, w, scale, nullptr, y, M, N, K, FP8G_FMT_E4M3, FP8G_FMT_E4M3, FP8G_ACT_NONE, path, variant, split_k,
             stream);
}

int fp8_gemm_scaled_act(const void *x, const void *w, const float *scale, const float *bias, void *y, int64_t M,
                        int64_t N, int64_t K, int32_t x_format, int32_t w_format, int32_t activation, void *stream) {
  return run(x, w, scale, bias, y, M, N, K, x_format, w_format, activation, 0, 0, 0, stream);
}

int fp8_gemm_scaled_act_ex(const void *x, const void *w, const float *scale, const float *bias, void *y, int64_t M,
                           int64_t N, int64_t K, int32_t x_format, int32_t w_format, int32_t activation,
                           int32_t path, int32_t variant, int32_t split_k, void *stream) {
  return run(x, w, scale, bias, y, M, N, K, x_format, w_format, activation, path, variant, split_k, stream);
}

int fp8_gemm_scaled_act_timed(const void *x, const void *w, const float *scale, const float *bias, void *y,
                              int64_t M, int64_t N, int64_t K, int32_t x_format, int32_t w_format,
                              int32_t activation, int32_t path, int32_t variant, int32_t split_k, void *stream,
                              void *start_event, void *stop_event) {
  return run(x, w, scale, bias, y, M, N, K, x_format, w_format, activation, path, variant, split_k, stream,
             start_event, stop_event);
}

int fp8_gemm_plan(int64_t M, int64_t N, int64_t K, fp8g_plan *out) {
  g_last_error.clear();
  return plan_impl(M, N, K, 0, 0, 0, out);
}

int fp8_gemm_plan_ex(int64_t M, int64_t N, int64_t K, int32_t path, int32_t variant, int32_t split_k,
                     fp8g_plan *out) {
  g_last_error.clear();
  return plan_impl(M, N, K, path, variant, split_k, out);
}

const char *fp8_gemm_strerror(int status) {
  switch (status) {
    case FP8G_OK: return "success";
    case FP8G_ERR_INVALID_ARG: return "invalid argument";
    case FP8G_ERR_UNSUPPORTED: return "unsupported configuration";
    case FP8G_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char *fp8_gemm_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
