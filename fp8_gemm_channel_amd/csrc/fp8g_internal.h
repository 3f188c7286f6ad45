// fp8g_internal.h -- declarations shared by the host API (fp8g_api.cpp) and the
// kernel launchers (fp8g_kernels.hip) of libfp8g.so.  Not installed, not part
// of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8g {

// One launch of the main (tiled MFMA) kernel.
// Events attached to one kernel's own dispatch (hipExtLaunchKernel): `start` is
// recorded when the kernel begins and `stop` when it has ended; null = none.
struct DispatchEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

struct MainLaunch {
  const uint8_t *x;
  const uint8_t *w;
  const float *scale;
  uint16_t *y;
  int M, N, K;
  int tiles_m, tiles_n, group_m;
  int variant;   // main-path configuration id
  bool k_tail;   // K % tile_k != 0
  int ystore;    // widest y store: 16 (N % 8 == 0, y 16-byte aligned), 8 (N % 4 == 0, y 8-byte aligned) or 2
  int ywb = 0;   // y stores write-back (more tiles than compute units) or non-temporal
  const float *bias = nullptr;  // per-column bias [N], or null
  int act = 0;                  // epilogue activation (FP8G_ACT_*)
  int fmt = 0;                  // (w format << 1) | x format, 0 = E4M3, 1 = E5M2
  // variant 16 (stream-K) only:
  int n_dp = 0, n_sk = 0;                 // whole-tile workgroups, stream-K workgroups
  float *partials = nullptr;              // 2 * n_sk partial tiles of kMainPartialBytes
  unsigned long long *tickets = nullptr;  // one per stream-K tile, kTicketStride apart (any initial value)
  unsigned long long epoch = 0;           // id of this call, < 2^48
  DispatchEvents ev;                      // attached to the main kernel's dispatch
};

// One launch of the skinny split-K kernel (with S > 1 the last workgroup of each
// column tile adds the slices' partials and writes y in the same launch).
struct SkinnyLaunch {
  const uint8_t *x;
  const uint8_t *w;
  const float *scale;
  uint16_t *y;
  float *partials;  // [column tile][S][M][tile_n] fp32, only when S > 1
  unsigned long long *tickets;  // one per column tile, kTicketStride apart, only when S > 1 (any initial value)
  unsigned long long epoch;     // id of this call, < 2^48
  int M, N, K;
  int k_slice, S;
  int variant;      // skinny configuration id
  bool vec;         // N % 4 == 0 and y 8-byte aligned
  const float *bias = nullptr;  // per-column bias [N], or null
  int act = 0;                  // epilogue activation (FP8G_ACT_*)
  int fmt = 0;                  // (w format << 1) | x format, 0 = E4M3, 1 = E5M2
  DispatchEvents ev;            // attached to the kernel's dispatch
};

// Split-K tickets sit one 128-byte cache line apart (in 8-byte units): the
// atomics of different column tiles then never queue on the same line.
constexpr int kTicketStride = 16;
// One partial 256 x 256 fp32 tile of the stream-K main kernel.
constexpr int64_t kMainPartialBytes = 256 * 256 * 4;

// Kernel-side tile geometry of each configuration id (also used by the planner).
struct MainConfig {
  int id, bm, bn, bk, stages;
};
struct SkinnyConfig {
  int id, row_blocks;  // w rows per workgroup = 16 * row_blocks
};

const MainConfig *main_config(int id);      // nullptr if unknown
const SkinnyConfig *skinny_config(int id);  // nullptr if unknown
int skinny_tile_n(const SkinnyConfig &c);   // output columns per workgroup
// The split-K kernel: LDS rings with 4 waves (variants 1-5) or 8 waves (21-24).
enum class SkinnyKind { kRing4, kRing8 };
int skinny_max_row_blocks(int M, SkinnyKind kind);  // limit on row_blocks for this M and kernel
int skinny_chunk_bytes();                   // K granularity of one wave iteration

// A workspace the caller owns, in place of the library's pool: `get` returns
// its device address for the stream's device; `capacity` is its size.
struct FixedWorkspace {
  uint64_t capacity;
  hipError_t (*get)(hipStream_t stream, void **ptr);
};
// fp8_gemm_scaled_ex with the call's workspace taken from `ws` (no
// allocation); plans that need more than ws.capacity bytes are refused with
// FP8G_ERR_UNSUPPORTED before anything is enqueued.
int run_fixed_workspace(const void *x, const void *w, const float *scale, void *y, int64_t M, int64_t N, int64_t K,
                        int32_t path, int32_t variant, int32_t split_k, void *stream, const FixedWorkspace &ws);

hipError_t launch_main(const MainLaunch &l, hipStream_t stream);
hipError_t launch_main5(const MainLaunch &l, hipStream_t stream);            // variants 10, 16
hipError_t launch_main5_epi(const MainLaunch &l, hipStream_t stream);        // variant 10, bias / activation
hipError_t launch_main4w(const MainLaunch &l, hipStream_t stream);           // variant 19
hipError_t launch_main4w_epi(const MainLaunch &l, hipStream_t stream);       // variant 19, bias / activation
hipError_t launch_main4wr(const MainLaunch &l, hipStream_t stream);          // variant 20
hipError_t launch_main4wr_epi(const MainLaunch &l, hipStream_t stream);      // variant 20, bias / activation
hipError_t launch_main_tiles(const MainLaunch &l, hipStream_t stream);       // variants 3, 17, 18
hipError_t launch_main_tiles_epi(const MainLaunch &l, hipStream_t stream);   // the same, bias / activation
hipError_t launch_direct(const MainLaunch &l, hipStream_t stream);           // variant 27 (register tiles)
hipError_t launch_skinny_epi(const SkinnyLaunch &l, hipStream_t stream);     // bias / activation
hipError_t launch_skinny(const SkinnyLaunch &l, hipStream_t stream);
hipError_t launch_zero(uint16_t *y, int64_t count, hipStream_t stream, const DispatchEvents &ev);
// K = 0 with a bias or an activation: y[m, n] = bf16(act(bias[n])).
hipError_t launch_empty_k(uint16_t *y, const float *bias, int act, int64_t M, int64_t N, hipStream_t stream,
                          const DispatchEvents &ev);

}  // namespace fp8g
