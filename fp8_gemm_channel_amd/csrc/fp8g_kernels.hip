// fp8g_kernels.hip -- gfx950 (CDNA4) kernels of the scaled FP8 GEMM
//
//     y[m,n] = bf16_rne( (sum_k x[m,k] * w[n,k]) * scale[n] )
//
// x [M,K] and w [N,K] are FP8 E4M3 (OCP) codes, row-major; scale [N] fp32;
// y [M,N] bf16.  The products run on the CDNA4 f8f6f4 matrix cores
// (V_MFMA_F32_32X32X64_F8F6F4, format code 0 = E4M3 for both operands, no block
// scale) into fp32 accumulators; the per-output-channel scale multiplies each
// finished fp32 sum once in the epilogue, which rounds to bf16 (nearest, ties
// to even).  Sources on the pages (kernelbench.com model pages, cells named by
// the kernel they audit): fp8 x fp8 with fp32 accumulation and bf16 output,
// "DeepSeek V4 Flash (0731)", CUTLASS 3.x SM90 cell; scale applied in the
// epilogue before the bf16 store, "Kimi K3 (256k)", SM120 warp-specialised
// cell; skinny M as split-K with fp32 partials and a fused reduce/scale/cast
// kernel, "Claude Fable 5", Triton split-K cell.
//
// Operand roles.  Every MFMA takes w rows as its A operand (output rows = n)
// and x rows as its B operand (output columns = m), i.e. it computes y^T
// blocks.  A lane then holds four consecutive n of one m, so one 8-byte store
// writes four adjacent bf16 outputs of a y row.
//
// MFMA 32x32x64 register layout on gfx950 (checked on the hardware):
//   A/B operand: lane l supplies row (l % 32) and 32 consecutive K bytes of
//                K-group (l / 32) in its 8 VGPRs;
//   accumulator: lane l, element e holds row 8*(e/4) + 4*(l/32) + (e%4),
//                column l % 32.
// Only the pairing matters for a dot product: A and B are loaded with the same
// (lane, byte) -> k map, so any permutation of K inside one MFMA is harmless.
//
// Memory access.  All global reads are raw buffer loads.  A buffer's range is
// set to the valid rows of the tile, so rows past M or N read as zero without
// branches, and a fully out-of-range 16-byte load returns zeros.  Loads need no
// alignment: rows of an odd K (e.g. K = 4127) start at any byte.  The K tail
// (a K step that ends past K) is assembled in registers with the bytes past K
// forced to zero: zero bytes add nothing to a dot product, which is why the
// pages could pad with zeros ("Kimi K3 (256k)", SM100 persistent-TMA Triton
// cell); here nothing is copied and nothing is padded in memory.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8g_internal.h"

namespace fp8g {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

// LLVM's raw buffer intrinsics, taking the 128-bit descriptor as <4 x i32>.
__device__ v4i llvm_buffer_load_v4i32(v4i rsrc, uint32_t voffset, uint32_t soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.v4i32");
__device__ char llvm_buffer_load_i8(v4i rsrc, uint32_t voffset, uint32_t soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.i8");
__device__ float llvm_buffer_load_f32(v4i rsrc, uint32_t voffset, uint32_t soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.f32");

// Buffer descriptor: base address, stride 0 (raw), range `bytes`, and the
// gfx9 data-format word (32-bit elements, bounds-checked raw access).
__device__ __forceinline__ v4i make_rsrc(const void *base, uint32_t bytes) {
  uint64_t a = (uint64_t)(uintptr_t)base;
  v4i r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xFFFFu));
  r.z = __builtin_amdgcn_readfirstlane((int)bytes);
  r.w = 0x00020000;
  return r;
}

__device__ __forceinline__ uint4 as_u4(v4i v) {
  return make_uint4((uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w);
}

// 16 bytes at `off`, of which only the first `valid` (< 16) may be read; the
// rest are zero.  Byte loads: each one is range-checked on its own.
__device__ __noinline__ uint4 load16_partial(v4i rsrc, uint32_t off, int valid) {
  uint32_t d[4] = {0u, 0u, 0u, 0u};
  for (int j = 0; j < valid; ++j) {
    uint32_t b = (uint8_t)llvm_buffer_load_i8(rsrc, off + j, 0, 0);
    d[j >> 2] |= b << (8 * (j & 3));
  }
  return make_uint4(d[0], d[1], d[2], d[3]);
}

// 16 bytes at `off` with `valid` bytes before the end of the row (any value).
__device__ __forceinline__ uint4 load16_masked(v4i rsrc, uint32_t off, int valid) {
  if (valid >= 16) return as_u4(llvm_buffer_load_v4i32(rsrc, off, 0, 0));
  if (valid <= 0) return make_uint4(0u, 0u, 0u, 0u);
  return load16_partial(rsrc, off, valid);
}

// LDS-DMA: 16 bytes per lane from global (voffset + soffset) into LDS at
// lds_base + 16 * lane.  Written as inline asm so the compiler does not treat
// it as an LDS store it must wait for before every LDS read; completion is
// tracked by hand with vm_wait() below.  m0 is set inside the same statement.
// (m0 is otherwise unused by these kernels, so clobbering it is safe.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(v4i rsrc, uint32_t lds_base, uint32_t voffset, uint32_t soffset) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds_base), "v"(voffset), "s"(rsrc), "s"(soffset)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt vmcnt(N), other counters untouched (gfx9 encoding).
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// fp32 -> bf16 bits, round to nearest, ties to even; NaN -> 0x7FC0.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ v16f mfma32(const v8i &a, const v8i &b, const v16f &c) {
  // Zero scale operands select the unscaled V_MFMA_F32_32X32X64_F8F6F4.
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// ------------------------------------------------------------------ main path
//
// One workgroup computes a BM (m) x BN (n) tile of y with WM x WN waves; each
// wave owns a (BM/WM) x (BN/WN) sub-tile as 32x32 MFMA blocks.  The K loop
// stages BK-byte slices of the BN w rows and BM x rows through a STAGES-deep
// ring of LDS buffers filled by LDS-DMA (16 B per lane, 1 KiB per wave
// instruction), so the global -> LDS copy needs no VGPRs and overlaps the MFMAs
// of the stages already resident.
//
// LDS layout of one stage: w rows [0, BN) then x rows [0, BM), BK bytes each.
// Within a row the 16-byte chunk c is stored at chunk position c ^ swz(r).  The
// MFMA operand reads (lane l reads row l % 32) then touch eight different
// chunk positions in every eight consecutive lanes and sixteen different
// (bank half, position) pairs in every sixteen, so they are free of bank
// conflicts whether LDS serves 128 or 256 bytes per cycle.  A DMA instruction
// writes 1 KiB contiguously; the swizzle is applied on the global side by
// choosing which chunk each lane fetches.
template <int BK>
__device__ __forceinline__ int swz(int r) {
  if constexpr (BK == 128) return (r & 7) ^ ((r >> 3) & 1);
  else return ((r >> 1) ^ (r >> 2)) & 3;  // BK == 64: four chunks per row
}

struct MainArgs {
  const uint8_t *x;
  const uint8_t *w;
  const float *scale;
  uint16_t *y;
  int M, N, K;
  int tiles_m, tiles_n, group_m;
};

template <int BM, int BN, int BK, int STAGES, int WM, int WN, bool KTAIL, bool VEC>
__global__ __launch_bounds__(WM * WN * 64, 1) void fp8g_main_kernel(MainArgs a) {
  constexpr int NWAVES = WM * WN;
  constexpr int TM = BM / WM, TN = BN / WN;  // wave sub-tile
  constexpr int FM = TM / 32, FN = TN / 32;  // 32x32 blocks per wave
  constexpr int CH = BK / 16;                // 16-byte chunks per row
  constexpr int ROWS_PER_KB = 1024 / BK;     // rows in one 1 KiB DMA block
  constexpr int STAGE_BYTES = (BM + BN) * BK;
  constexpr int BLOCKS = STAGE_BYTES / 1024;
  constexpr int DPW = BLOCKS / NWAVES;       // DMA instructions per wave per stage
  constexpr int W_DPW = (BN / ROWS_PER_KB) / NWAVES;  // of which fill w rows
  static_assert(BK == 64 || BK == 128, "BK");
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile");
  static_assert(BLOCKS % NWAVES == 0 && (BN / ROWS_PER_KB) % NWAVES == 0, "DMA split");
  static_assert(STAGES >= 2 && (STAGES - 2) * DPW < 64, "pipeline depth");

  __shared__ __attribute__((aligned(1024))) uint8_t smem[STAGES * STAGE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wave_m = wave % WM, wave_n = wave / WM;

  // Workgroup -> tile.  Workgroup ids are dispatched round-robin over the 8
  // XCDs (each with its own L2), so first renumber them so that every XCD works
  // on a contiguous range of tiles, then walk that range in groups of group_m
  // tile rows (all tile columns of a group before the next group) so the x rows
  // and w rows a group shares stay in the XCD's L2.
  const int total = a.tiles_m * a.tiles_n;
  const int pid = blockIdx.x;
  const int xcd = pid & 7, q8 = total >> 3, r8 = total & 7;
  const int lpid = xcd * q8 + min(xcd, r8) + (pid >> 3);
  const int per_group = a.group_m * a.tiles_n;
  const int gid = lpid / per_group;
  const int first_m = gid * a.group_m;
  const int gsize = min(a.tiles_m - first_m, a.group_m);
  const int within = lpid - gid * per_group;
  const int tm = first_m + within % gsize;
  const int tn = within / gsize;

  const int K = a.K;
  const int m0 = tm * BM, n0 = tn * BN;
  const int rows_x = min(BM, a.M - m0), rows_w = min(BN, a.N - n0);
  const v4i rsrc_x = make_rsrc(a.x + (size_t)m0 * K, (uint32_t)rows_x * (uint32_t)K);
  const v4i rsrc_w = make_rsrc(a.w + (size_t)n0 * K, (uint32_t)rows_w * (uint32_t)K);

  // Per-lane source offsets (without the K step) for each DMA instruction.
  // Instruction t of this wave fills 1 KiB block b = t * NWAVES + wave.
  uint32_t src_off[DPW];
  uint32_t src_chunk[DPW];  // byte offset of the logical chunk within the K step
  {
    const int rsub = lane / CH, p = lane % CH;
#pragma unroll
    for (int t = 0; t < DPW; ++t) {
      const int b = t * NWAVES + wave;
      const int R = b * ROWS_PER_KB + rsub;
      const int r = (t < W_DPW) ? R : R - BN;
      const int c = p ^ swz<BK>(r);
      src_chunk[t] = (uint32_t)c * 16u;
      src_off[t] = (uint32_t)r * (uint32_t)K + src_chunk[t];
    }
  }
  const uint32_t smem_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)smem;

  // Full K step kt -> stage buffer `st` via LDS-DMA.
  auto issue_full = [&](int kt, int st) {
    const uint32_t k0 = (uint32_t)kt * BK;
    const uint32_t sb = smem_base + (uint32_t)st * STAGE_BYTES;
#pragma unroll
    for (int t = 0; t < DPW; ++t) {
      const uint32_t lds = sb + (uint32_t)(t * NWAVES + wave) * 1024u;
      dma16(t < W_DPW ? rsrc_w : rsrc_x, lds, src_off[t], k0);
    }
  };
  // Last, partial K step -> stage buffer `st` through registers, bytes at or
  // past K zeroed.  Same block/lane mapping as the DMA path.
  auto issue_tail = [&](int kt, int st) {
    const int k0 = kt * BK;
    uint8_t *sb = smem + st * STAGE_BYTES;
#pragma unroll
    for (int t = 0; t < DPW; ++t) {
      const int valid = K - (k0 + (int)src_chunk[t]);
      const uint4 v = load16_masked(t < W_DPW ? rsrc_w : rsrc_x, src_off[t] + (uint32_t)k0, valid);
      *(uint4 *)(sb + (t * NWAVES + wave) * 1024 + lane * 16) = v;
    }
  };

  // Fragment read offsets.  Lane l reads row (l % 32) of each 32-row block and
  // the two chunks 4j + 2(l/32) + {0,1} of 64-byte sub-step j.
  const int g = lane >> 5, lr = lane & 31;
  const int aw_row = wave_n * TN + lr;  // w row of block 0 (block i adds 32 i rows)
  const int bx_row = wave_m * TM + lr;  // x row of block 0
  const int sa = swz<BK>(aw_row), sbx = swz<BK>(bx_row);  // 32 i leaves the swizzle unchanged

  v16f acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  auto compute = [&](int st) {
    const uint8_t *sw_ = smem + st * STAGE_BYTES;
    const uint8_t *sx_ = sw_ + BN * BK;
#pragma unroll
    for (int j = 0; j < BK / 64; ++j) {
      const int c0 = 4 * j + 2 * g;
      v8i af[FN], bf[FM];
#pragma unroll
      for (int i = 0; i < FN; ++i) {
        const uint8_t *row = sw_ + (aw_row + 32 * i) * BK;
        const uint4 lo = *(const uint4 *)(row + ((c0 ^ sa) << 4));
        const uint4 hi = *(const uint4 *)(row + (((c0 + 1) ^ sa) << 4));
        af[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int jm = 0; jm < FM; ++jm) {
        const uint8_t *row = sx_ + (bx_row + 32 * jm) * BK;
        const uint4 lo = *(const uint4 *)(row + ((c0 ^ sbx) << 4));
        const uint4 hi = *(const uint4 *)(row + (((c0 + 1) ^ sbx) << 4));
        bf[jm] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int jm = 0; jm < FM; ++jm) acc[i][jm] = mfma32(af[i], bf[jm], acc[i][jm]);
    }
  };

  const int nk_full = K / BK;
  const int nk = nk_full + (KTAIL ? 1 : 0);

  // Prologue: fill the first STAGES-1 buffers.
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s) {
    if (s < nk_full) issue_full(s, s);
    else if (KTAIL && s == nk_full) issue_tail(s, s);
  }

  for (int kt = 0; kt < nk; ++kt) {
    // Wait until this wave's DMA for step kt has landed.  Stages issued after
    // kt may stay in flight.  (When the register-loaded tail stage has been
    // issued, the compiler has already waited for all earlier vector memory
    // operations, which complete in order, so the count below never
    // under-waits.)
    const int ahead = min(STAGES - 2, nk - 1 - kt);
    if constexpr (STAGES >= 4) {
      if (ahead >= 2) vm_wait<2 * DPW>();
      else if (ahead == 1) vm_wait<DPW>();
      else vm_wait<0>();
    } else if constexpr (STAGES == 3) {
      if (ahead >= 1) vm_wait<DPW>();
      else vm_wait<0>();
    } else {
      vm_wait<0>();
    }
    // Every wave's part of step kt is in LDS, and every wave has finished
    // reading the buffer of step kt-1, which is refilled next.
    __syncthreads();
    const int kn = kt + STAGES - 1;
    if (kn < nk_full) issue_full(kn, kn % STAGES);
    else if (KTAIL && kn == nk_full) issue_tail(kn, kn % STAGES);
    compute(kt % STAGES);
  }

  // Epilogue: y[m, n..n+3] = bf16(acc * scale[n..n+3]).
  const v4i rsrc_s = make_rsrc(a.scale, (uint32_t)a.N * 4u);
#pragma unroll
  for (int i = 0; i < FN; ++i) {
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      const int n = n0 + wave_n * TN + 32 * i + 8 * qd + 4 * g;
      float s[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) s[e] = llvm_buffer_load_f32(rsrc_s, (uint32_t)(n + e) * 4u, 0, 0);
#pragma unroll
      for (int jm = 0; jm < FM; ++jm) {
        const int m = m0 + wave_m * TM + 32 * jm + lr;
        if (m >= a.M) continue;
        uint16_t *yr = a.y + (size_t)m * a.N;
        const uint32_t b0 = bf16_rne(acc[i][jm][4 * qd + 0] * s[0]);
        const uint32_t b1 = bf16_rne(acc[i][jm][4 * qd + 1] * s[1]);
        const uint32_t b2 = bf16_rne(acc[i][jm][4 * qd + 2] * s[2]);
        const uint32_t b3 = bf16_rne(acc[i][jm][4 * qd + 3] * s[3]);
        if (VEC) {
          if (n < a.N) *(uint2 *)(yr + n) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
        } else {
          if (n + 0 < a.N) yr[n + 0] = (uint16_t)b0;
          if (n + 1 < a.N) yr[n + 1] = (uint16_t)b1;
          if (n + 2 < a.N) yr[n + 2] = (uint16_t)b2;
          if (n + 3 < a.N) yr[n + 3] = (uint16_t)b3;
        }
      }
    }
  }
}

// ---------------------------------------------------------------- skinny path
//
// M <= 64.  The workgroup's four waves are arranged 4/WK along n (32 w rows
// each) by WK along K.  Each wave streams its w rows and the x rows straight
// from global memory into MFMA operand registers (no LDS staging: w is read
// exactly once, x is small and stays in L2), U 128-byte K chunks per
// iteration.  Lane l reads 64 contiguous bytes of its row per chunk; MFMA j of
// the chunk consumes bytes [32 j, 32 j + 32) of them, which is the same
// (lane, byte) -> k map for both operands.
//
// blockIdx.y selects the K slice [s * k_slice, min(K, (s+1) * k_slice)).  With
// one slice the kernel applies the scale and writes bf16 y directly; with
// several it writes unscaled fp32 partials P[s, m, n] that the reduce kernel
// sums in slice order.  Waves sharing a column block add their accumulators
// through LDS in wave order, so results are deterministic.
struct SkinnyArgs {
  const uint8_t *x;
  const uint8_t *w;
  const float *scale;
  uint16_t *y;
  float *P;
  int M, N, K;
  int k_slice;
};

constexpr int kSkinnyU = 4;  // 128-byte chunks per wave iteration

template <int MB, int WK, bool PARTIAL, bool VEC>
__global__ __launch_bounds__(256) void fp8g_splitk_partial_kernel(SkinnyArgs a) {
  constexpr int WN = 4 / WK;
  constexpr int U = kSkinnyU;
  static_assert(WK == 1 || WK == 2 || WK == 4, "WK");
  __shared__ float red[(WK > 1) ? (WK - 1) * WN * MB * 16 * 64 : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave % WN, wk = wave / WN;
  const int g = lane >> 5, lr = lane & 31;
  const int K = a.K;

  const int nw0 = blockIdx.x * (32 * WN) + wn * 32;
  const int rows_w = max(0, min(32, a.N - nw0));
  const int s = blockIdx.y;
  const int kbeg = s * a.k_slice;
  const int kend = min(K, kbeg + a.k_slice);

  const v4i rsrc_w = make_rsrc(a.w + (size_t)min(nw0, a.N) * K, (uint32_t)rows_w * (uint32_t)K);
  const v4i rsrc_x = make_rsrc(a.x, (uint32_t)a.M * (uint32_t)K);
  const uint32_t w_off = (uint32_t)lr * (uint32_t)K + 64u * g;
  uint32_t x_off[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) x_off[mb] = (uint32_t)(lr + 32 * mb) * (uint32_t)K + 64u * g;

  v16f acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[mb][e] = 0.0f;

  const int step = WK * U * 128;
  for (int kc = kbeg + wk * U * 128; kc < kend; kc += step) {
    uint4 wv[U][4], xv[MB][U][4];
    if (kc + U * 128 <= kend) {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const uint32_t ko = (uint32_t)(kc + u * 128 + 16 * h);
          wv[u][h] = as_u4(llvm_buffer_load_v4i32(rsrc_w, w_off + ko, 0, 0));
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) xv[mb][u][h] = as_u4(llvm_buffer_load_v4i32(rsrc_x, x_off[mb] + ko, 0, 0));
        }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const int kb = kc + u * 128 + 64 * g + 16 * h;  // this lane's chunk start
          const int valid = kend - kb;
          const uint32_t ko = (uint32_t)(kc + u * 128 + 16 * h);
          wv[u][h] = load16_masked(rsrc_w, w_off + ko, valid);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) xv[mb][u][h] = load16_masked(rsrc_x, x_off[mb] + ko, valid);
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint4 a0 = wv[u][2 * j], a1 = wv[u][2 * j + 1];
        const v8i af = v8i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const uint4 b0 = xv[mb][u][2 * j], b1 = xv[mb][u][2 * j + 1];
          const v8i bf = v8i{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
          acc[mb] = mfma32(af, bf, acc[mb]);
        }
      }
  }

  if constexpr (WK > 1) {
    if (wk > 0) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) red[((((wk - 1) * WN + wn) * MB + mb) * 16 + e) * 64 + lane] = acc[mb][e];
    }
    __syncthreads();
    if (wk > 0) return;
#pragma unroll
    for (int o = 1; o < WK; ++o)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[mb][e] += red[((((o - 1) * WN + wn) * MB + mb) * 16 + e) * 64 + lane];
  }

  const v4i rsrc_s = make_rsrc(a.scale, (uint32_t)a.N * 4u);
#pragma unroll
  for (int qd = 0; qd < 4; ++qd) {
    const int n = nw0 + 8 * qd + 4 * g;
    float sc[4];
    if (!PARTIAL) {
#pragma unroll
      for (int e = 0; e < 4; ++e) sc[e] = llvm_buffer_load_f32(rsrc_s, (uint32_t)(n + e) * 4u, 0, 0);
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int m = 32 * mb + lr;
      if (m >= a.M) continue;
      const float v0 = acc[mb][4 * qd + 0], v1 = acc[mb][4 * qd + 1];
      const float v2 = acc[mb][4 * qd + 2], v3 = acc[mb][4 * qd + 3];
      if (PARTIAL) {
        float *pr = a.P + ((size_t)s * a.M + m) * a.N;
        if (VEC) {
          if (n < a.N) *(float4 *)(pr + n) = make_float4(v0, v1, v2, v3);
        } else {
          if (n + 0 < a.N) pr[n + 0] = v0;
          if (n + 1 < a.N) pr[n + 1] = v1;
          if (n + 2 < a.N) pr[n + 2] = v2;
          if (n + 3 < a.N) pr[n + 3] = v3;
        }
      } else {
        uint16_t *yr = a.y + (size_t)m * a.N;
        const uint32_t b0 = bf16_rne(v0 * sc[0]), b1 = bf16_rne(v1 * sc[1]);
        const uint32_t b2 = bf16_rne(v2 * sc[2]), b3 = bf16_rne(v3 * sc[3]);
        if (VEC) {
          if (n < a.N) *(uint2 *)(yr + n) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
        } else {
          if (n + 0 < a.N) yr[n + 0] = (uint16_t)b0;
          if (n + 1 < a.N) yr[n + 1] = (uint16_t)b1;
          if (n + 2 < a.N) yr[n + 2] = (uint16_t)b2;
          if (n + 3 < a.N) yr[n + 3] = (uint16_t)b3;
        }
      }
    }
  }
}

// y[m, n..n+3] = bf16((sum_{s<S} P[s, m, n..n+3]) * scale[n..n+3]), slices
// added in order s = 0, 1, ..., S-1.  One thread per four outputs of a row.
template <bool VEC>
__global__ __launch_bounds__(256) void fp8g_splitk_reduce_kernel(const float *__restrict__ P,
                                                                 const float *__restrict__ scale,
                                                                 uint16_t *__restrict__ y, int M, int N, int S) {
  const int n4 = (N + 3) / 4;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)M * n4) return;
  const int m = (int)(idx / n4);
  const int n = (int)(idx - (int64_t)m * n4) * 4;
  const size_t plane = (size_t)M * N;
  const float *p = P + (size_t)m * N + n;
  uint16_t *yr = y + (size_t)m * N;
  if (VEC) {
    float4 acc = *(const float4 *)p;
    for (int s = 1; s < S; ++s) {
      const float4 v = *(const float4 *)(p + s * plane);
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    // scale is only guaranteed 4-byte aligned
    const uint32_t b0 = bf16_rne(acc.x * scale[n + 0]), b1 = bf16_rne(acc.y * scale[n + 1]);
    const uint32_t b2 = bf16_rne(acc.z * scale[n + 2]), b3 = bf16_rne(acc.w * scale[n + 3]);
    *(uint2 *)(yr + n) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
  } else {
    for (int e = 0; e < 4 && n + e < N; ++e) {
      float acc = p[e];
      for (int s = 1; s < S; ++s) acc += p[s * plane + e];
      yr[n + e] = (uint16_t)bf16_rne(acc * scale[n + e]);
    }
  }
}

__global__ __launch_bounds__(256) void fp8g_zero_kernel(uint16_t *__restrict__ y, int64_t count) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) y[i] = 0;
}

// ------------------------------------------------------------------ launchers
static const MainConfig kMainConfigs[] = {
    {1, 256, 256, 128, 2},
    {2, 128, 128, 128, 2},
    {3, 64, 64, 128, 2},
    {4, 256, 256, 64, 4},
};
static const SkinnyConfig kSkinnyConfigs[] = {
    {1, 4},
    {2, 2},
    {3, 1},
};

const MainConfig *main_config(int id) {
  for (const auto &c : kMainConfigs)
    if (c.id == id) return &c;
  return nullptr;
}
const SkinnyConfig *skinny_config(int id) {
  for (const auto &c : kSkinnyConfigs)
    if (c.id == id) return &c;
  return nullptr;
}
int skinny_tile_n(const SkinnyConfig &c) { return 32 * (4 / c.waves_k); }
int skinny_chunk_bytes() { return 128; }

template <int BM, int BN, int BK, int STAGES, int WM, int WN>
static hipError_t launch_main_cfg(const MainLaunch &l, hipStream_t stream) {
  MainArgs a{l.x, l.w, l.scale, l.y, l.M, l.N, l.K, l.tiles_m, l.tiles_n, l.group_m};
  const dim3 grid((unsigned)(l.tiles_m * l.tiles_n)), block(WM * WN * 64);
  if (l.k_tail) {
    if (l.vec) fp8g_main_kernel<BM, BN, BK, STAGES, WM, WN, true, true><<<grid, block, 0, stream>>>(a);
    else fp8g_main_kernel<BM, BN, BK, STAGES, WM, WN, true, false><<<grid, block, 0, stream>>>(a);
  } else {
    if (l.vec) fp8g_main_kernel<BM, BN, BK, STAGES, WM, WN, false, true><<<grid, block, 0, stream>>>(a);
    else fp8g_main_kernel<BM, BN, BK, STAGES, WM, WN, false, false><<<grid, block, 0, stream>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_main(const MainLaunch &l, hipStream_t stream) {
  switch (l.variant) {
    case 1: return launch_main_cfg<256, 256, 128, 2, 2, 2>(l, stream);
    case 2: return launch_main_cfg<128, 128, 128, 2, 2, 2>(l, stream);
    case 3: return launch_main_cfg<64, 64, 128, 2, 2, 2>(l, stream);
    case 4: return launch_main_cfg<256, 256, 64, 4, 2, 2>(l, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int MB, int WK>
static hipError_t launch_skinny_cfg(const SkinnyLaunch &l, hipStream_t stream) {
  SkinnyArgs a{l.x, l.w, l.scale, l.y, l.partials, l.M, l.N, l.K, l.k_slice};
  constexpr int tile_n = 32 * (4 / WK);
  const dim3 grid((unsigned)((l.N + tile_n - 1) / tile_n), (unsigned)l.S), block(256);
  const bool partial = l.S > 1;
  if (partial) {
    if (l.N % 4 == 0) fp8g_splitk_partial_kernel<MB, WK, true, true><<<grid, block, 0, stream>>>(a);
    else fp8g_splitk_partial_kernel<MB, WK, true, false><<<grid, block, 0, stream>>>(a);
  } else {
    if (l.vec) fp8g_splitk_partial_kernel<MB, WK, false, true><<<grid, block, 0, stream>>>(a);
    else fp8g_splitk_partial_kernel<MB, WK, false, false><<<grid, block, 0, stream>>>(a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !partial) return e;
  const int64_t threads = (int64_t)l.M * ((l.N + 3) / 4);
  const dim3 rgrid((unsigned)((threads + 255) / 256));
  if (l.vec) fp8g_splitk_reduce_kernel<true><<<rgrid, block, 0, stream>>>(l.partials, l.scale, l.y, l.M, l.N, l.S);
  else fp8g_splitk_reduce_kernel<false><<<rgrid, block, 0, stream>>>(l.partials, l.scale, l.y, l.M, l.N, l.S);
  return hipGetLastError();
}

hipError_t launch_skinny(const SkinnyLaunch &l, hipStream_t stream) {
  const bool two = l.M > 32;
  switch (l.variant) {
    case 1: return two ? launch_skinny_cfg<2, 4>(l, stream) : launch_skinny_cfg<1, 4>(l, stream);
    case 2: return two ? launch_skinny_cfg<2, 2>(l, stream) : launch_skinny_cfg<1, 2>(l, stream);
    case 3: return two ? launch_skinny_cfg<2, 1>(l, stream) : launch_skinny_cfg<1, 1>(l, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_zero(uint16_t *y, int64_t count, hipStream_t stream) {
  int64_t blocks = (count + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  fp8g_zero_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(y, count);
  return hipGetLastError();
}

}  // namespace fp8g
