// fp8g_kernels.hpp -- device code of libfp8g.so: kernel templates and the
// helpers they share.  Included by the translation units that instantiate
// and launch them (fp8g_kernels.hip and fp8g_launch_*.hip), which are built
// in parallel; everything here is a template or inline.
//
//     y[m,n] = bf16_rne( (sum_k x[m,k] * w[n,k]) * scale[n] )
//
// x [M,K] and w [N,K] are FP8 E4M3 (OCP) codes, row-major; scale [N] fp32;
// y [M,N] bf16.  The products run on the CDNA4 f8f6f4 matrix cores
// (V_MFMA_F32_32X32X64_F8F6F4 or V_MFMA_F32_16X16X128_F8F6F4, format code 0 =
// E4M3 for both operands, no block scale) into fp32 accumulators; the per-output-channel scale multiplies each
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
// branches, and a fully out-of-range 16-byte load returns zeros.  Operand rows
// are read where they lie: rows of an odd K (e.g. K = 4127) start at any byte
// and no kernel needs them aligned.  The K tail (a K step that ends past K) is
// masked inside the kernel, the bytes past K entering as zeros: zero bytes add
// nothing to a dot product, which is why the pages could pad with zeros
// ("Kimi K3 (256k)", SM100 persistent-TMA Triton cell).  No operand is ever
// copied, padded or cached.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "fp8g_internal.h"

namespace fp8g {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));

// LLVM's raw buffer intrinsics, taking the 128-bit descriptor as <4 x i32>.
__device__ v4i llvm_buffer_load_v4i32(v4i rsrc, uint32_t voffset, uint32_t soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.v4i32");
__device__ char llvm_buffer_load_i8(v4i rsrc, uint32_t voffset, uint32_t soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.i8");
__device__ float llvm_buffer_load_f32(v4i rsrc, uint32_t voffset, uint32_t soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.f32");
__device__ v4f llvm_buffer_load_v4f32(v4i rsrc, uint32_t voffset, uint32_t soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.v4f32");
__device__ void llvm_buffer_store_v4f32(v4f data, v4i rsrc, uint32_t voffset, uint32_t soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.store.v4f32");
__device__ void llvm_buffer_store_f32(float data, v4i rsrc, uint32_t voffset, uint32_t soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.store.f32");

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
__device__ __forceinline__ uint4 load16_partial(v4i rsrc, uint32_t off, int valid) {
  uint32_t d[4] = {0u, 0u, 0u, 0u};
  for (int j = 0; j < valid; ++j) {
    uint32_t b = (uint8_t)llvm_buffer_load_i8(rsrc, off + j, 0, 0);
    d[j >> 2] |= b << (8 * (j & 3));
  }
  return make_uint4(d[0], d[1], d[2], d[3]);
}

// The same for 0 < valid < 16 when the row holds at least 16 bytes up to
// off + valid (i.e. K >= 16): one 16-byte load that ends at the last valid
// byte, moved down by 16 - valid bytes (whole dwords first, then the byte
// remainder with a funnel shift) so the bytes past the row come in as zeros.
// One memory round trip instead of `valid` dependent byte loads.
__device__ __forceinline__ uint4 load16_tail(v4i rsrc, uint32_t off, int valid) {
  const v4i v = llvm_buffer_load_v4i32(rsrc, off + (uint32_t)valid - 16u, 0, 0);
  const int sh = 16 - valid;  // 1 .. 15
  const int q = sh >> 2, r = sh & 3;
  const uint32_t d0 = (uint32_t)v.x, d1 = (uint32_t)v.y, d2 = (uint32_t)v.z, d3 = (uint32_t)v.w;
  const uint32_t e0 = q == 0 ? d0 : q == 1 ? d1 : q == 2 ? d2 : d3;
  const uint32_t e1 = q == 0 ? d1 : q == 1 ? d2 : q == 2 ? d3 : 0u;
  const uint32_t e2 = q == 0 ? d2 : q == 1 ? d3 : 0u;
  const uint32_t e3 = q == 0 ? d3 : 0u;
  // alignbyte(hi, lo, r) = low 32 bits of ({hi, lo} >> 8r)
  return make_uint4(__builtin_amdgcn_alignbyte(e1, e0, r), __builtin_amdgcn_alignbyte(e2, e1, r),
                    __builtin_amdgcn_alignbyte(e3, e2, r), __builtin_amdgcn_alignbyte(0u, e3, r));
}

// 16 bytes at `off` with `valid` bytes before the end of the row (any value);
// K is the row length.
__device__ __forceinline__ uint4 load16_masked(v4i rsrc, uint32_t off, int valid, int K) {
  if (valid >= 16) return as_u4(llvm_buffer_load_v4i32(rsrc, off, 0, 0));
  if (valid <= 0) return make_uint4(0u, 0u, 0u, 0u);
  if (K >= 16) return load16_tail(rsrc, off, valid);
  return load16_partial(rsrc, off, valid);
}

// Debug build (FP8G_LDS_POISON): before every LDS-DMA, each lane writes 16
// bytes of 0xFF -- a NaN as E4M3, as E5M2 and as fp32 -- where its DMA will
// land, and waits until that write is done.  A read that runs ahead of its
// DMA (a miscounted vm_wait, a missing barrier) then sees NaN operands or
// scales instead of stale bytes that might pass by luck, and parity tests
// fail on the NaN outputs.  Off in the product build.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_poison16(uint32_t lds_base) {
#ifdef FP8G_LDS_POISON
  const uint32_t at = lds_base + 16u * __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const v4i nan = {-1, -1, -1, -1};
  asm volatile("ds_write_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : : "v"(at), "v"(nan) : "memory");
#else
  (void)lds_base;
#endif
}

// LDS-DMA: 16 bytes per lane from global (voffset + soffset) into LDS at
// lds_base + 16 * lane.  Written as inline asm so the compiler does not treat
// it as an LDS store it must wait for before every LDS read; completion is
// tracked by hand with vm_wait() below.  m0 is set inside the same statement.
// (m0 is otherwise unused by these kernels, so clobbering it is safe.)
__device__ __forceinline__ void dma16(v4i rsrc, uint32_t lds_base, uint32_t voffset, uint32_t soffset) {
  lds_poison16(lds_base);
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

// fp32 pair -> bf16 bits packed (lo in bits 0-15), round to nearest, ties to
// even, NaN stays NaN: one V_CVT_PK_BF16_F32 (bf16 keeps the fp32 exponent
// range, so only the mantissa is rounded; denormals are kept).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}
// One value: the low half of the pair.
__device__ __forceinline__ uint32_t bf16_rne(float f) { return bf16x2_rne(f, 0.0f) & 0xFFFFu; }

// Operand formats of the f8f6f4 MFMAs as one template parameter:
// FMT = (w format << 1) | x format, with 0 = E4M3 and 1 = E5M2 (the
// instruction's format codes for FP8 and BF8).  A operands are w rows, B
// operands x rows.
template <int FMT>
__device__ __forceinline__ v16f mfma32(const v8i &a, const v8i &b, const v16f &c) {
  // Zero scale operands select the unscaled V_MFMA_F32_32X32X64_F8F6F4.
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FMT >> 1, FMT & 1, 0, 0, 0, 0);
}

// Epilogue activations (applied after scale and bias).
constexpr int kActNone = 0, kActRelu = 1, kActSilu = 2, kActGeluTanh = 3;

// act(z) in fp32.  NaN stays NaN; at +-inf each takes its limit (+inf, and 0
// for ReLU, -0 for SiLU and GELU).  Both SiLU and the tanh form of GELU are
// z * sigmoid(t): SiLU with t = z, GELU with t = 2 u, u = sqrt(2/pi) (z +
// 0.044715 z^3), since 0.5 (1 + tanh(u)) = 1 / (1 + e^(-2u)).  The sigmoid is
// one hardware exp2 (argument pre-multiplied by log2 e, folded into the
// polynomial for GELU) and one hardware reciprocal: a few ulp of fp32, far
// below the bf16 rounding that follows.  No clamping is needed: for large z
// e^(-t) underflows to 0 (giving z), for very negative z it overflows to inf and
// the reciprocal gives 0 (giving -0); only z = -inf needs its limit selected
// (the product would be -inf * 0).  The value at z < -80 (SiLU) or < -10
// (GELU) is below 1e-33 in magnitude and taken as -0.
constexpr float kLog2e = 1.44269504088896341f;
constexpr float kGeluA = -2.0f * 0.7978845608028654f * kLog2e;             // -2 sqrt(2/pi) log2 e
constexpr float kGeluB = -2.0f * 0.7978845608028654f * 0.044715f * kLog2e;  // ... times 0.044715
template <int ACT>
__device__ __forceinline__ float activation(float z) {
  if constexpr (ACT == kActRelu) {
    return (z > 0.0f || z != z) ? z : 0.0f;
  } else if constexpr (ACT == kActSilu) {
    const float r = z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-kLog2e * z));
    return z < -80.0f ? -0.0f : r;
  } else if constexpr (ACT == kActGeluTanh) {
    const float v = z * fmaf(kGeluB, z * z, kGeluA);  // -2 u log2 e
    const float r = z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(v));
    return z < -10.0f ? -0.0f : r;
  } else {
    return z;
  }
}
__device__ __forceinline__ float activation_rt(float z, int act) {
  switch (act) {
    case kActRelu: return activation<kActRelu>(z);
    case kActSilu: return activation<kActSilu>(z);
    case kActGeluTanh: return activation<kActGeluTanh>(z);
    default: return z;
  }
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
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

struct MainArgs {
  const uint8_t *x;
  const uint8_t *w;
  const float *scale;
  uint16_t *y;
  int M, N, K;
  int tiles_m, tiles_n, group_m;
  int ystore;  // widest y store allowed by N and y's alignment: 16, 8 or 2 bytes
  const float *bias;  // per-column bias [N] added after the scale, or null
  int act;            // activation applied last: kActNone, kActRelu, kActSilu, kActGeluTanh
  // Stream-K (five-slot kernel only; zero elsewhere).  Workgroups 0 .. n_dp-1
  // each compute one whole tile, the first n_dp tiles of the raster order; the
  // n_sk workgroups after them split the (tile, K step) units of the remaining
  // tiles evenly.
  int n_dp, n_sk;
  float *P;                      // 2 partial-tile slots per stream-K workgroup
  unsigned long long *tickets;   // one per stream-K tile, kTicketStride apart
  unsigned long long epoch;      // this call's id (< 2^48)
  // y stores: ordinary (write-back) when the launch has more tiles than the GPU
  // has compute units, non-temporal otherwise (see store_tile_rows).
  int ywb;
};

// Cache policy of partial sums that pass between workgroups: device scope
// (SC1), the encoding the compiler gives agent-scope atomic loads and stores.
// Stores write through the XCD's L2 to the device coherence point and loads do
// not hit stale lines, so partials move between XCDs without flushing or
// invalidating whole caches.
constexpr int kDeviceScope = 16;
constexpr uint32_t kOut = 0x80000000u;  // a buffer offset past every descriptor's range: reads 0

// Last-arrival hand-off: every workgroup that contributes to an output tile
// takes the tile's ticket once, after its partial sums are visible device-wide;
// the one that brings the count to `target` finishes the tile.  A ticket holds
// (call id << 16 | arrivals); a ticket left by another call (or any stale
// bytes) restarts at one arrival, so tickets need no zeroing before a launch.
// The last arrival sets the ticket back to 0 (no call id is 0): a replay of a
// captured launch -- same call id, same workspace -- then starts from a clean
// ticket instead of counting on from the previous replay's total.  The
// compare-and-swap loop is lock-free: a failed attempt means another
// workgroup's succeeded.
__device__ __forceinline__ bool take_ticket(unsigned long long *t, unsigned long long epoch, int target) {
  unsigned long long old = __hip_atomic_load(t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  unsigned long long want;
  for (;;) {
    want = (old >> 16) == epoch ? old + 1 : (epoch << 16) | 1ull;
    if (__hip_atomic_compare_exchange_strong(t, &old, want, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT))
      break;
  }
  const bool last = (int)(want & 0xFFFFull) == target;
  // every contributor has arrived: nobody else touches this ticket in this launch
  if (last) __hip_atomic_store(t, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return last;
}

// Scheduling pattern for NM MFMAs and NR LDS reads spread evenly: MFMA q is
// followed by reads [q*NR/NM, (q+1)*NR/NM).
template <int Q, int NM, int NR>
__device__ __forceinline__ void interleave_mfma_reads() {
  if constexpr (Q < NM) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr ((Q + 1) * NR / NM - Q * NR / NM > 0)
      __builtin_amdgcn_sched_group_barrier(0x100, (Q + 1) * NR / NM - Q * NR / NM, 0);
    interleave_mfma_reads<Q + 1, NM, NR>();
  }
}

// Workgroup -> tile.  Workgroup ids are dispatched round-robin over the 8 XCDs
// (each with its own L2), so first renumber them so that every XCD works on a
// contiguous range of tiles, then walk that range in groups of group_m tile
// rows (all tile columns of a group before the next group) so the x rows and
// w rows a group shares stay in the XCD's L2.
__device__ __forceinline__ int xcd_remap(int pid, int count) {
  const int xcd = pid & 7, q8 = count >> 3, r8 = count & 7;
  return xcd * q8 + min(xcd, r8) + (pid >> 3);
}
__device__ __forceinline__ void raster(const MainArgs &a, int lpid, int &tm, int &tn) {
  const int per_group = a.group_m * a.tiles_n;
  const int gid = lpid / per_group;
  const int first_m = gid * a.group_m;
  const int gsize = min(a.tiles_m - first_m, a.group_m);
  const int within = lpid - gid * per_group;
  tm = first_m + within % gsize;
  tn = within / gsize;
}
__device__ __forceinline__ void tile_coords(const MainArgs &a, int &tm, int &tn) {
  raster(a, xcd_remap(blockIdx.x, a.tiles_m * a.tiles_n), tm, tn);
}

// The bf16 tile staged in LDS by the main epilogues (row pitch 2*BN bytes,
// 16-byte chunk c of row r at c ^ (r % (BN/8))) written to y row by row, 16
// bytes per lane, so one store instruction covers whole rows of the tile.
// A whole tile with 16-byte stores goes in batches of eight LDS reads, then
// their eight stores (a read-then-store loop waits out the LDS latency on every
// chunk); the rest (tile edges, narrower stores) chunk by chunk.
//
// Cache policy (a.ywb).  Every compute unit finishes its tile at about the same
// moment, so a wave of tiles writes its whole y at once (32 MiB for 256 tiles of
// 256 x 256).  With more tiles to come, ordinary stores let each XCD's L2 take
// the burst and write it back while the next tiles compute (measured on MI355X:
// 8192^2 x 1024 9-10% and 8192^3 1.3-2.8% faster than non-temporal stores);
// with one wave of tiles nothing overlaps the write, and non-temporal stores,
// which do not displace cached lines, are as fast or slightly faster (4096^3).
__device__ __forceinline__ void store16(const MainArgs &a, v4i v, uint16_t *dst) {
  if (a.ywb) *(v4i *)dst = v;
  else __builtin_nontemporal_store(v, (v4i *)dst);
}
template <int BM, int BN, int NTHREADS>
__device__ __forceinline__ void store_tile_rows(const MainArgs &a, const uint8_t *smem, int m0, int n0, int tid) {
  constexpr int CPR = BN / 8, PITCH = 2 * BN, TOTAL = BM * CPR;
  auto sw = [](int r) __attribute__((always_inline)) { return r & (CPR - 1); };
  if constexpr (TOTAL % NTHREADS == 0 && NTHREADS % CPR == 0) {
    constexpr int ITERS = TOTAL / NTHREADS, B = ITERS < 8 ? ITERS : 8;
    static_assert(ITERS % B == 0, "whole batches");
    if (a.ystore == 16 && m0 + BM <= a.M && n0 + BN <= a.N) {
      const int c = tid % CPR, r0 = tid / CPR;
      constexpr int RSTEP = NTHREADS / CPR;
#pragma unroll
      for (int j0 = 0; j0 < ITERS; j0 += B) {
        v4i v[B];
#pragma unroll
        for (int b = 0; b < B; ++b) {
          const int r = r0 + (j0 + b) * RSTEP;
          v[b] = *(const v4i *)(smem + r * PITCH + ((c ^ sw(r)) << 4));
        }
#pragma unroll
        for (int b = 0; b < B; ++b) {
          const int r = r0 + (j0 + b) * RSTEP;
          store16(a, v[b], a.y + (size_t)(m0 + r) * a.N + n0 + 8 * c);
        }
      }
      return;
    }
  }
  for (int idx = tid; idx < TOTAL; idx += NTHREADS) {
    const int r = idx / CPR, c = idx % CPR;
    const int m = m0 + r, n = n0 + 8 * c;
    if (m >= a.M || n >= a.N) continue;
    const uint4 v = *(const uint4 *)(smem + r * PITCH + ((c ^ sw(r)) << 4));
    uint16_t *dst = a.y + (size_t)m * a.N + n;
    if (a.ystore == 16) {  // N % 8 == 0 and y 16-byte aligned: the chunk is whole
      store16(a, v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w}, dst);
    } else if (a.ystore == 8) {  // N % 4 == 0 and y 8-byte aligned
      *(uint2 *)dst = make_uint2(v.x, v.y);
      if (n + 4 < a.N) *(uint2 *)(dst + 4) = make_uint2(v.z, v.w);
    } else {
      const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (n + e < a.N) dst[e] = (uint16_t)(d[e >> 1] >> (16 * (e & 1)));
    }
  }
}

// Epilogue of the main kernels: y[m, n..n+3] = bf16(acc * scale[n..n+3]) for a
// BM x BN tile computed by WM x WN waves (wave tile (BM/WM) x (BN/WN) as 32x32
// blocks), with the tile's scales at s_lds[0 .. BN) and at least 2*BM*BN bytes
// of LDS at smem that no wave uses any more after the first barrier.
template <int BM, int BN, int WM, int WN, int ACT, bool BIAS>
__device__ __forceinline__ void main_epilogue_t(const v16f (&acc)[BN / WN / 32][BM / WM / 32], const MainArgs &a,
                                                uint8_t *smem, const float *s_lds, const float *b_lds, int m0,
                                                int n0, int wave, int lane, int tid) {
  constexpr int NWAVES = WM * WN, TM = BM / WM, TN = BN / WN, FM = TM / 32, FN = TN / 32;
  // Epilogue: y[m, n..n+3] = bf16(acc * scale[n..n+3]), written through LDS so
  // that y leaves in whole rows.  A lane's results are four consecutive n of
  // one m, so stored directly every store instruction would touch 32 rows with
  // 16 bytes each and every 128-byte line of y would be assembled from eight
  // partial writes.  Instead the waves put the bf16 tile into the (now idle)
  // stage buffers -- row pitch 2*BN bytes, 16-byte chunk c of row r at
  // c ^ (r % CPR), which keeps both the 32-row writes and the row reads nearly
  // free of bank conflicts -- and then write it out row by row, 16 bytes per
  // lane, so one store instruction covers whole rows of the tile.
  constexpr int CPR = BN / 8;  // 16-byte chunks per tile row
  constexpr int PITCH = 2 * BN;
  constexpr int NTHREADS = NWAVES * 64;
  const int g = lane >> 5, lr = lane & 31;
  const int wave_m = wave % WM, wave_n = wave / WM;
  __syncthreads();  // every wave is done with the stage buffers (and s_lds is published)
#pragma unroll
  for (int i = 0; i < FN; ++i) {
#pragma unroll
    for (int qd = 0; qd < 4; ++qd) {
      const int nl = wave_n * TN + 32 * i + 8 * qd + 4 * g;
      const float4 sc = *(const float4 *)(s_lds + nl);
      float4 bi = make_float4(0.f, 0.f, 0.f, 0.f);
      if constexpr (BIAS) bi = *(const float4 *)(b_lds + nl);
      // z = acc * scale (+ bias), then the activation, in fp32
      auto val = [&](float v, float scl, float bs) __attribute__((always_inline)) {
        float z = v * scl;
        if constexpr (BIAS) z += bs;
        return activation<ACT>(z);
      };
#pragma unroll
      for (int jm = 0; jm < FM; ++jm) {
        const int ml = wave_m * TM + 32 * jm + lr;
        const uint32_t p01 = bf16x2_rne(val(acc[i][jm][4 * qd + 0], sc.x, bi.x), val(acc[i][jm][4 * qd + 1], sc.y, bi.y));
        const uint32_t p23 = bf16x2_rne(val(acc[i][jm][4 * qd + 2], sc.z, bi.z), val(acc[i][jm][4 * qd + 3], sc.w, bi.w));
        const int off = ml * PITCH + (((nl >> 3) ^ (ml & (CPR - 1))) << 4) + ((nl & 7) << 1);
        *(uint2 *)(smem + off) = make_uint2(p01, p23);
      }
    }
  }
  __syncthreads();
  store_tile_rows<BM, BN, NTHREADS>(a, smem, m0, n0, tid);
}

// main_epilogue_t for the call's activation and bias (one uniform switch).
// b_lds holds the tile's BN biases when a.bias is set.  Kernels built without
// EPI (no bias, no activation: the plain operation) compile only that case.
template <int BM, int BN, int WM, int WN, bool EPI>
__device__ __forceinline__ void main_epilogue(const v16f (&acc)[BN / WN / 32][BM / WM / 32], const MainArgs &a,
                                              uint8_t *smem, const float *s_lds, const float *b_lds, int m0,
                                              int n0, int wave, int lane, int tid) {
  if constexpr (!EPI) {
    main_epilogue_t<BM, BN, WM, WN, kActNone, false>(acc, a, smem, s_lds, b_lds, m0, n0, wave, lane, tid);
    return;
  }
  const int sel = a.act * 2 + (a.bias != nullptr ? 1 : 0);
#define FP8G_EPI(ACT, BIAS) \
  main_epilogue_t<BM, BN, WM, WN, ACT, BIAS>(acc, a, smem, s_lds, b_lds, m0, n0, wave, lane, tid)
  switch (sel) {
    case 1: FP8G_EPI(kActNone, true); break;
    case 2: FP8G_EPI(kActRelu, false); break;
    case 3: FP8G_EPI(kActRelu, true); break;
    case 4: FP8G_EPI(kActSilu, false); break;
    case 5: FP8G_EPI(kActSilu, true); break;
    case 6: FP8G_EPI(kActGeluTanh, false); break;
    case 7: FP8G_EPI(kActGeluTanh, true); break;
    default: FP8G_EPI(kActNone, false); break;
  }
#undef FP8G_EPI
}

// Software pipeline.  A K step is 128 bytes (one stage buffer), worked as two
// 64-byte MFMA sub-steps; F[u & 1] holds the operands of sub-step u.  Sub-step u:
//
//     [last sub-step of step s only] wait for this wave's DMA of step s+1,
//         workgroup barrier, LDS-DMA of step s+DIST into a retired buffer
//     MFMAs of sub-step u (operands in F[u & 1]), interleaved with the LDS
//     reads of sub-step u+1's operands into F[(u+1) & 1]
//
// The barrier publishes step s+1 (every wave's DMA has landed) and retires the
// buffer of step s (every wave has read its operands).  128-byte steps (rather
// than 64) halve the barriers and have each DMA instruction fetch 8 rows x 128
// bytes instead of 16 rows x 64 bytes, which the global-to-LDS path serves
// faster (measured on MI355X: ~7% on 4096^3 and 8192^3).
// With 8 waves per workgroup two waves share each SIMD, so one wave's MFMAs
// cover the other's barrier and LDS waits; a single wave per SIMD can neither
// keep the matrix pipe full nor keep enough LDS reads in flight (measured on
// MI355X: ~4.0-4.5 vs ~4.8 PFLOP/s for back-to-back MFMAs, ~110 vs ~200
// B/clk/CU for 16-byte LDS reads).
template <int BM, int BN, int STAGES, int WM, int WN, bool KTAIL, int FMT = 0, bool EPI = false>
__global__ __launch_bounds__(WM * WN * 64, 1) void fp8g_main_kernel(MainArgs a) {
  constexpr int BK = 128;
  constexpr int NWAVES = WM * WN;
  constexpr int TM = BM / WM, TN = BN / WN;  // wave sub-tile
  constexpr int FM = TM / 32, FN = TN / 32;  // 32x32 blocks per wave
  constexpr int SUB = BK / 64;               // MFMA sub-steps per K step
  constexpr int CH = BK / 16;                // 16-byte chunks per row
  constexpr int ROWS_PER_KB = 1024 / BK;     // rows in one 1 KiB DMA block
  constexpr int STAGE_BYTES = (BM + BN) * BK;
  constexpr int BLOCKS = STAGE_BYTES / 1024;
  constexpr int DPW = BLOCKS / NWAVES;       // DMA instructions per wave per stage
  constexpr int W_DPW = (BN / ROWS_PER_KB) / NWAVES;  // of which fill w rows
  constexpr int NMFMA = FN * FM;             // MFMAs per wave per 64-byte sub-step
  constexpr int NREAD = (FN + FM) * 2;       // 16-byte LDS reads per wave per sub-step
  // Prefetch distance in steps: step k+STAGES goes into the buffer of step k
  // itself, which a step's last sub-step retires.
  constexpr int DIST = STAGES;
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile");
  static_assert(BLOCKS % NWAVES == 0 && (BN / ROWS_PER_KB) % NWAVES == 0, "DMA split");
  static_assert(DIST >= 2 && DIST <= 5 && (DIST - 1) * DPW < 64, "vmcnt range");
  static_assert(BN <= 256, "one DMA instruction stages the tile's scales");

  // Stage ring, then the tile's BN scales, then its BN biases.
  __shared__ __attribute__((aligned(1024))) uint8_t smem[STAGES * STAGE_BYTES + 2048];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wave_m = wave % WM, wave_n = wave / WM;

  int tm, tn;
  tile_coords(a, tm, tn);

  const int K = a.K;
  const int m0 = tm * BM, n0 = tn * BN;
  const int rows_x = min(BM, a.M - m0), rows_w = min(BN, a.N - n0);
  // A tile's rows form one range of at most 256 * (2^24 - 1) bytes, so an
  // offset equal to it never wraps 32 bits; rows past M / N read zero.
  const uint32_t range_x = (uint32_t)rows_x * (uint32_t)K, range_w = (uint32_t)rows_w * (uint32_t)K;

  const int g = lane >> 5, lr = lane & 31;
  const uint32_t smem_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)smem;
  const uint32_t scale_lds = smem_base + STAGES * STAGE_BYTES;
  // The tile's scales scale[n0 .. n0+BN) go to LDS now (wave 0, one DMA; columns
  // past N read as zero), so the epilogue does not wait on global memory.  This
  // is wave 0's oldest vector-memory operation, so its first stage wait covers
  // it, and every barrier after that publishes it.
  // The biases (if any) follow the same way, one DMA after the scales.
  if (wave == 0) {
    const v4i rsrc_s = make_rsrc(a.scale + n0, (uint32_t)(a.N - n0) * 4u);
    dma16(rsrc_s, scale_lds, (uint32_t)lane * 16u, 0u);
    if (EPI && a.bias) {
      const v4i rsrc_b = make_rsrc(a.bias + n0, (uint32_t)(a.N - n0) * 4u);
      dma16(rsrc_b, scale_lds + 1024u, (uint32_t)lane * 16u, 0u);
    }
  }

  // DMA instruction t of a wave fills 1 KiB block t*NWAVES + wave of a stage
  // (w rows first, then x rows): ROWS_PER_KB rows of BK bytes, lane l taking
  // row l / CH of the block and logical chunk (l % CH) ^ swz(row).  Blocks
  // start at multiples of ROWS_PER_KB rows and NWAVES is even, so the row bits
  // the swizzle reads are the same in every block: each lane has one source
  // offset relative to its block and one chunk for all t, and block t gets
  // its own descriptor (base moved to the block's first row, range cut to
  // match, so rows past M / N still read zero).
  static_assert(NWAVES % 2 == 0 && BN % 16 == 0, "block-invariant swizzle");
  const int dma_lrow = wave * ROWS_PER_KB + lane / CH;  // row within block t = 0
  const int dma_chunk = (lane % CH) ^ swz(dma_lrow);
  const uint32_t laneff = (uint32_t)dma_lrow * (uint32_t)K + (uint32_t)dma_chunk * 16u;
  const uint32_t blk_stride = (uint32_t)(NWAVES * ROWS_PER_KB) * (uint32_t)K;
  v4i rs[DPW];
#pragma unroll
  for (int t = 0; t < DPW; ++t) {
    const int tt = t < W_DPW ? t : t - W_DPW;
    const uint32_t range = t < W_DPW ? range_w : range_x;
    const uint32_t skip = (uint32_t)tt * blk_stride;  // < 256 * K: no wrap
    const uint8_t *base = t < W_DPW ? a.w + (size_t)n0 * K : a.x + (size_t)m0 * K;
    rs[t] = make_rsrc(base + skip, range > skip ? range - skip : 0u);
  }

  const int nk_full_c = K / BK;  // K steps that lie entirely before K

  // Full K step kt -> stage buffer `st` via LDS-DMA.
  auto issue_full = [&](int kt, int st) __attribute__((always_inline)) {
    const uint32_t k0 = (uint32_t)kt * BK;
    const uint32_t sb = smem_base + (uint32_t)st * STAGE_BYTES;
#pragma unroll
    for (int t = 0; t < DPW; ++t) dma16(rs[t], sb + (uint32_t)(t * NWAVES + wave) * 1024u, laneff, k0);
  };
  // Last, partial K step (k0 + BK > K) -> stage buffer `st`, also by LDS-DMA:
  // chunks entirely before K load as usual, chunks at or past K are pointed out
  // of range and land as zeros, and the one chunk per row that straddles K is
  // zeroed the same way here and rebuilt later by fix_tail.
  auto issue_tail = [&](int kt, int st) __attribute__((always_inline)) {
    const int k0 = kt * BK;
    const uint32_t sb = smem_base + (uint32_t)st * STAGE_BYTES;
    const int valid = K - (k0 + 16 * dma_chunk);
    // range_w / range_x bound every block's cut range from above
    const uint32_t off_w = valid >= 16 ? laneff + (uint32_t)k0 : range_w;
    const uint32_t off_x = valid >= 16 ? laneff + (uint32_t)k0 : range_x;
#pragma unroll
    for (int t = 0; t < DPW; ++t) dma16(rs[t], sb + (uint32_t)(t * NWAVES + wave) * 1024u, t < W_DPW ? off_w : off_x, 0u);
  };
  // Rebuild the straddling chunks of the tail stage (one shifted 16-byte load
  // each, or byte loads when K < 16), bytes at or past K zero.  Called once every DMA
  // of the tail stage has landed and before the barrier that publishes it; the
  // barrier's LDS wait covers these writes.
  auto fix_tail = [&](int st) __attribute__((always_inline)) {
    const int k0 = nk_full_c * BK;
    uint8_t *sb = smem + st * STAGE_BYTES;
    const int valid = K - (k0 + 16 * dma_chunk);
    if (valid > 0 && valid < 16) {
#pragma unroll
      for (int t = 0; t < DPW; ++t) {
        const uint4 v = K >= 16 ? load16_tail(rs[t], laneff + (uint32_t)k0, valid)
                                : load16_partial(rs[t], laneff + (uint32_t)k0, valid);
        *(uint4 *)(sb + (t * NWAVES + wave) * 1024 + lane * 16) = v;
      }
    }
  };
  const int nk = nk_full_c + (KTAIL ? 1 : 0);
  const int nk_full = nk_full_c;
  auto issue = [&](int kt) __attribute__((always_inline)) {
    if (kt < nk_full) issue_full(kt, kt % STAGES);
    else if (KTAIL && kt == nk_full) issue_tail(kt, kt % STAGES);
  };

  // Fragment reads.  Lane l reads row (l % 32) of each 32-row block and the two
  // chunks 4j + 2(l/32) + {0,1} of 64-byte sub-step j.
  const int aw_row = wave_n * TN + lr;  // w row of block 0 (block i adds 32 i rows)
  const int bx_row = wave_m * TM + lr;  // x row of block 0
  const int sa = swz(aw_row), sbx = swz(bx_row);  // 32 i leaves the swizzle unchanged

  // Operand registers of two sub-steps: F[u & 1] holds sub-step u.
  v8i fa[2][FN], fb[2][FM];
  // LDS read number q (q in [0, NREAD)) of sub-step j of stage `st`: low then
  // high 16 bytes of each block, blocks in the order the MFMAs first use them
  // (w block 0, all FM x blocks, then w blocks 1 .. FN-1).
  auto read_one = [&](int st, int j, int q, v8i (&af)[FN], v8i (&bf)[FM]) __attribute__((always_inline)) {
    const int ord = q / 2, half = q % 2;
    const int blk = ord == 0 ? 0 : (ord <= FM ? FN + ord - 1 : ord - FM);
    const int c = 4 * j + 2 * g + half;
    const uint8_t *sw_ = smem + st * STAGE_BYTES;
    if (blk < FN) {
      const uint8_t *row = sw_ + (aw_row + 32 * blk) * BK;
      const uint4 v = *(const uint4 *)(row + ((c ^ sa) << 4));
      af[blk][4 * half + 0] = (int)v.x; af[blk][4 * half + 1] = (int)v.y;
      af[blk][4 * half + 2] = (int)v.z; af[blk][4 * half + 3] = (int)v.w;
    } else {
      const uint8_t *row = sw_ + BN * BK + (bx_row + 32 * (blk - FN)) * BK;
      const uint4 v = *(const uint4 *)(row + ((c ^ sbx) << 4));
      bf[blk - FN][4 * half + 0] = (int)v.x; bf[blk - FN][4 * half + 1] = (int)v.y;
      bf[blk - FN][4 * half + 2] = (int)v.z; bf[blk - FN][4 * half + 3] = (int)v.w;
    }
  };

  v16f acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // Wait until this wave's DMA of a step has landed while the `ahead` (<= 4)
  // steps issued after it may stay in flight (vmcnt completes in order).
  auto wait_ahead = [&](int ahead) __attribute__((always_inline)) {
    if (ahead >= 4) vm_wait<4 * DPW>();
    else if (ahead == 3) vm_wait<3 * DPW>();
    else if (ahead == 2) vm_wait<2 * DPW>();
    else if (ahead == 1) vm_wait<DPW>();
    else vm_wait<0>();
  };

  // Prologue: DMA of steps 0 .. DIST-1, then sub-step 0's operands.
#pragma unroll
  for (int s = 0; s < DIST; ++s) issue(s);
  wait_ahead(min(DIST - 1, nk - 1));
  if (KTAIL && nk_full == 0) {  // the tail is step 0: every DMA issued so far has landed
    vm_wait<0>();
    fix_tail(0);
  }
  __syncthreads();

#pragma unroll
  for (int q = 0; q < NREAD; ++q) read_one(0, 0, q, fa[0], fb[0]);

  // Sub-step u (step s = u / SUB, part j = u % SUB): MFMAs on F[cur],
  // interleaved with the reads of sub-step u+1 into F[cur ^ 1].  The last
  // sub-step of a step is a boundary: before it, step s+1 must be published.
  const int nsub = nk * SUB;
  auto substep = [&](const int u, const int cur, const bool boundary) __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    const int s = u / SUB;
    if (boundary) {
      // Own DMA of step s+1 must have landed; steps s+2 .. s+DIST-1 (issued
      // earlier) may stay in flight.
      wait_ahead(min(DIST - 2, nk - 2 - s));
      // step s+1 is the tail: the wait above covered its DMA (nothing is
      // issued after the tail), so rebuild its straddling chunks before
      // publishing it
      if (KTAIL && s + 1 == nk_full) fix_tail((s + 1) % STAGES);
      // After this barrier every wave has read all operands of step s (the
      // last of them during the previous sub-step), so its buffer is free;
      // so is the buffer of step s-1.  Step s+DIST goes into one of them.
      __syncthreads();
      issue(s + DIST);
      __builtin_amdgcn_sched_barrier(0);
    }
    const bool more = u + 1 < nsub;
    const int un = u + 1;
    const int st = (un / SUB) % STAGES, jn = un % SUB;
#pragma unroll
    for (int q = 0; q < NMFMA; ++q) {
      const int i = q / FM, jm = q % FM;
      acc[i][jm] = mfma32<FMT>(fa[cur][i], fb[cur][jm], acc[i][jm]);
      if (more) {
#pragma unroll
        for (int r = q * NREAD / NMFMA; r < (q + 1) * NREAD / NMFMA; ++r) read_one(st, jn, r, fa[cur ^ 1], fb[cur ^ 1]);
      }
    }
    interleave_mfma_reads<0, NMFMA, NREAD>();
    __builtin_amdgcn_sched_barrier(0);
  };
  for (int s = 0; s < nk; ++s) {
    substep(2 * s, 0, false);
    substep(2 * s + 1, 1, true);
  }

  static_assert(2 * BM * BN <= STAGES * STAGE_BYTES, "the bf16 tile fits in the stage buffers");
  main_epilogue<BM, BN, WM, WN, EPI>(acc, a, smem, (const float *)(smem + STAGES * STAGE_BYTES),
                                (const float *)(smem + STAGES * STAGE_BYTES + 1024), m0, n0, wave, lane,
                                (int)threadIdx.x);
}

// ------------------------------------------------- main path, five LDS slots
//
// 256 x 256 tiles, 128-byte K steps, 8 waves with 64 (m) x 128 (n) wave tiles,
// as variant 6 of the kernel above, but with a deeper feed.  Measured on
// MI355X, the global-to-LDS copy of a K step (64 KiB per workgroup, 64 LDS-DMA
// instructions) is limited by how fast the compute unit accepts DMA
// instructions (about one per 20-25 cycles): issued in one burst after the
// barrier, the second wave of every SIMD stalls for ~1400 cycles before it can
// issue its MFMAs.  Spreading the instructions over the step needs them to be
// issued earlier, i.e. more buffering than two 64 KiB stages in 160 KiB of LDS.
//
// So a stage is split in halves: LDS holds five 32 KiB slots, each one K step
// of either the tile's w rows or its x rows -- w of step k in slot k % 2, x of
// step k in slot 2 + k % 3.  x (whose rows are shared by fewer of the tiles an
// XCD runs at once, so it misses L2 more often) is fetched two steps ahead and
// w one step ahead, and every DMA instruction is issued between two MFMAs, so
// no wave waits long for the instruction queue.  The epilogue's
// scales no longer fit in LDS during the K loop: thread t < 256 keeps
// scale[n0 + t] in a register and writes it to LDS after the loop.
// Stream-K work split (variant 16).  Units are (tile, K step) pairs numbered
// tile * nk + step over the stream-K tiles only; stream-K workgroup i takes the
// units [sk_start(i), sk_start(i + 1)).
// The host keeps every unit number below 2^31.
__device__ __forceinline__ int sk_start(int i, int units, int n_sk) { return (int)((int64_t)i * units / n_sk); }
// The stream-K workgroup whose range holds unit u (the largest i with sk_start(i) <= u).
__device__ __forceinline__ int sk_owner(int u, int units, int n_sk) {
  return (int)(((int64_t)(u + 1) * n_sk - 1) / units);
}
// Bytes of one partial tile: 512 threads x 128 fp32 accumulators, stored in
// register order (thread t's float4 q at (q * 512 + t) * 16), since only the
// same thread of another workgroup of this kernel reads it back.
constexpr uint32_t kPartialBytes = (uint32_t)kMainPartialBytes;

template <bool KTAIL, bool SK, int FMT = 0, bool EPI = false>
__global__ __launch_bounds__(512, 1) void fp8g_main5_kernel(MainArgs a) {
  constexpr int BM = 256, BN = 256, BK = 128, WM = 4, WN = 2, NWAVES = 8;
  constexpr int TM = BM / WM, TN = BN / WN, FM = TM / 32, FN = TN / 32;
  constexpr int CH = BK / 16, ROWS_PER_KB = 1024 / BK;
  constexpr int SLOT = 256 * BK;                         // one half step: 256 rows x 128 bytes
  constexpr int HDPW = SLOT / 1024 / NWAVES;             // DMA instructions per wave per half step (4)
  constexpr int NMFMA = FN * FM, NREAD = (FN + FM) * 2;  // per wave per 64-byte sub-step
  static_assert(HDPW == 4 && NMFMA == 8, "x DMAs are spread two per sub-step, after MFMAs 1 and 5");
  static_assert(2 * BM * BN + 2 * BN * 4 <= 5 * SLOT, "epilogue tile, scales and biases fit");
  static_assert(FN * FM * 16 == 128 && NWAVES * 64 * 128 * 4 == (int)kPartialBytes, "partial tile layout");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[5 * SLOT];

  const int K = a.K;
  const uint32_t smem_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)smem;
  const int total = a.tiles_m * a.tiles_n;
  const int nk_full = K / BK;
  const int nk = nk_full + (KTAIL ? 1 : 0);  // K steps of a tile
  auto slot_w = [&](int k) __attribute__((always_inline)) { return (uint32_t)((k & 1) * SLOT); };
  auto slot_x = [&](int k) __attribute__((always_inline)) { return (uint32_t)((2 + k % 3) * SLOT); };

  // This workgroup's units [u0, u1), unit = tile * nk + K step with tiles in
  // raster order: one whole tile, or (stream-K) a contiguous range that may
  // cover the end of one tile, whole tiles, and the start of another.
  // Without stream-K only the tile is used (u0 = tile, one segment of nk
  // steps); with it the host keeps all unit numbers below 2^31.
  int u0, u1;
  int sk_i = 0;
  if (!SK || (int)blockIdx.x < a.n_dp) {
    const int t = xcd_remap(blockIdx.x, SK ? a.n_dp : total);
    u0 = SK ? t * nk : t;
    u1 = SK ? u0 + nk : t + 1;
  } else {
    // consecutive ranges share a tile, so keep them on one XCD
    sk_i = xcd_remap(blockIdx.x - a.n_dp, a.n_sk);
    const int units = (total - a.n_dp) * nk;
    u0 = a.n_dp * nk + sk_start(sk_i, units, a.n_sk);
    u1 = a.n_dp * nk + sk_start(sk_i + 1, units, a.n_sk);
  }

  for (int u = u0; u < u1;) {
    // Segment: steps [kb, ke) of one tile.
    const int tile = SK ? u / nk : u0;
    const int kb = SK ? u - tile * nk : 0;
    const int ke = SK ? min(nk, kb + (u1 - u)) : nk;
    const bool first_seg = u == u0;
    u += SK ? ke - kb : 1;
    if (SK && !first_seg) {
      // the previous segment's last LDS reads (epilogue or ticket flag) and
      // stores are done before this one's DMAs refill the slots
      vm_wait<0>();
      __syncthreads();
    }
    const int nkl = ke - kb;  // steps of this segment; local step s is K step kb + s

    // Thread ids.  With stream-K they pass through an empty asm, so the
    // compiler cannot see through them and computes what derives from them
    // (DMA offsets, LDS fragment addresses, epilogue addresses) in each
    // segment instead of hoisting it out of the segment loop and keeping it
    // live -- spilled -- across every K loop.
    int tid = threadIdx.x;
    int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    if constexpr (SK) {
      asm volatile("" : "+v"(tid));
      asm volatile("" : "+s"(wave));
    }
    const int lane = tid & 63;
    const int wave_m = wave % WM, wave_n = wave / WM;
    const int g = lane >> 5, lr = lane & 31;

    // DMA instruction t (0..3) of a wave fills 1 KiB block t*8 + wave of a half
    // step: 8 rows of 128 bytes, lane l taking row l / 8 and logical chunk
    // (l % 8) ^ swz(row); descriptor t starts at the block's first row (rows past
    // M / N read zero).
    const int dma_lrow = wave * ROWS_PER_KB + lane / CH;
    const int dma_chunk = (lane % CH) ^ swz(dma_lrow);
    const uint32_t laneff = (uint32_t)dma_lrow * (uint32_t)K + (uint32_t)dma_chunk * 16u;
    const uint32_t blk_stride = (uint32_t)(NWAVES * ROWS_PER_KB) * (uint32_t)K;
    // Fragment reads: lane l reads row (l % 32) of each 32-row block, chunks
    // 4j + 2(l/32) + {0,1} of 64-byte sub-step j; blocks in first-use order.
    const int aw_row = wave_n * TN + lr, bx_row = wave_m * TM + lr;
    const int sa = swz(aw_row), sbx = swz(bx_row);
    int tm, tn;
    raster(a, tile, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int rows_x = min(BM, a.M - m0), rows_w = min(BN, a.N - n0);
    const uint32_t range_x = (uint32_t)rows_x * (uint32_t)K, range_w = (uint32_t)rows_w * (uint32_t)K;

    // The epilogue's scale (and bias) for column n0 + tid (zero past N); these
    // loads are the oldest vector-memory operations, so every DMA wait below
    // also covers them.
    float my_scale = 0.0f, my_bias = 0.0f;
    if (tid < BN)
      my_scale = llvm_buffer_load_f32(make_rsrc(a.scale + n0, (uint32_t)(a.N - n0) * 4u), (uint32_t)tid * 4u, 0, 0);
    // (the stream-K kernel has no register to spare: it reads the bias after the loop)
    if (EPI && !SK && a.bias && tid < BN)
      my_bias = llvm_buffer_load_f32(make_rsrc(a.bias + n0, (uint32_t)(a.N - n0) * 4u), (uint32_t)tid * 4u, 0, 0);

    v4i rw[HDPW], rx[HDPW];
#pragma unroll
    for (int t = 0; t < HDPW; ++t) {
      const uint32_t skip = (uint32_t)t * blk_stride;
      rw[t] = make_rsrc(a.w + (size_t)n0 * K + skip, range_w > skip ? range_w - skip : 0u);
      rx[t] = make_rsrc(a.x + (size_t)m0 * K + skip, range_x > skip ? range_x - skip : 0u);
    }

    // DMA instruction t of local step kt's w (or x) half; nothing past the
    // segment is fetched.  The tile's tail step points chunks at or past K out
    // of range (zeros) and fix_tail rebuilds the straddling one.
    auto dma_half = [&](const v4i &rs, uint32_t range, uint32_t slot, int kt, int t) __attribute__((always_inline)) {
      const uint32_t lds = smem_base + slot + (uint32_t)(t * NWAVES + wave) * 1024u;
      if (kt < nkl) {
        const int kg = kb + kt;
        if (!KTAIL || kg < nk_full) {
          dma16(rs, lds, laneff, (uint32_t)kg * BK);
        } else {
          const int valid = K - (kg * BK + 16 * dma_chunk);
          dma16(rs, lds, valid >= 16 ? laneff + (uint32_t)(kg * BK) : range, 0u);
        }
      }
    };
    auto issue_w = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
      for (int t = 0; t < HDPW; ++t) dma_half(rw[t], range_w, slot_w(kt), kt, t);
    };
    auto issue_x = [&](int kt, int t) __attribute__((always_inline)) { dma_half(rx[t], range_x, slot_x(kt), kt, t); };
    auto fix_tail = [&](int kt) __attribute__((always_inline)) {
      const int k0 = (kb + kt) * BK;
      const int valid = K - (k0 + 16 * dma_chunk);
      if (valid > 0 && valid < 16) {
#pragma unroll
        for (int t = 0; t < 2 * HDPW; ++t) {  // w blocks, then x blocks, one at a time (runs once)
          const v4i &rs = t < HDPW ? rw[t % HDPW] : rx[t % HDPW];
          const uint4 v = K >= 16 ? load16_tail(rs, laneff + (uint32_t)k0, valid)
                                  : load16_partial(rs, laneff + (uint32_t)k0, valid);
          const uint32_t slot = t < HDPW ? slot_w(kt) : slot_x(kt);
          *(uint4 *)(smem + slot + ((t % HDPW) * NWAVES + wave) * 1024 + lane * 16) = v;
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };

    v8i fa[2][FN], fb[2][FM];
    auto read_one = [&](int k, int j, int q, v8i (&af)[FN], v8i (&bf)[FM]) __attribute__((always_inline)) {
      const int ord = q / 2, half = q % 2;
      const int blk = ord == 0 ? 0 : (ord <= FM ? FN + ord - 1 : ord - FM);
      const int c = 4 * j + 2 * g + half;
      if (blk < FN) {
        const uint8_t *row = smem + slot_w(k) + (aw_row + 32 * blk) * BK;
        const uint4 v = *(const uint4 *)(row + ((c ^ sa) << 4));
        af[blk][4 * half + 0] = (int)v.x; af[blk][4 * half + 1] = (int)v.y;
        af[blk][4 * half + 2] = (int)v.z; af[blk][4 * half + 3] = (int)v.w;
      } else {
        const uint8_t *row = smem + slot_x(k) + (bx_row + 32 * (blk - FN)) * BK;
        const uint4 v = *(const uint4 *)(row + ((c ^ sbx) << 4));
        bf[blk - FN][4 * half + 0] = (int)v.x; bf[blk - FN][4 * half + 1] = (int)v.y;
        bf[blk - FN][4 * half + 2] = (int)v.z; bf[blk - FN][4 * half + 3] = (int)v.w;
      }
    };

    v16f acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int j = 0; j < FM; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    // Prologue: w(0), x(0), x(1), w(1), x(2) -- the steady-state issue order --
    // then wait for step 0 (what was issued after x(0) may stay in flight).
    issue_w(0);
#pragma unroll
    for (int t = 0; t < HDPW; ++t) issue_x(0, t);
#pragma unroll
    for (int t = 0; t < HDPW; ++t) issue_x(1, t);
    issue_w(1);
#pragma unroll
    for (int t = 0; t < HDPW; ++t) issue_x(2, t);
    if (nkl >= 3) vm_wait<3 * HDPW>();
    else if (nkl == 2) vm_wait<2 * HDPW>();
    else vm_wait<0>();
    if (KTAIL && kb == nk_full) fix_tail(0);  // the segment is the tail step alone: everything issued has landed
    __syncthreads();
#pragma unroll
    for (int q = 0; q < NREAD; ++q) read_one(0, 0, q, fa[0], fb[0]);

    // Sub-step u = 2s + j of local step s.  j = 1 is the boundary: wait for
    // this wave's DMA of w(s+1) and x(s+1), barrier (publishes step s+1, retires
    // step s's slots), then, spread over the MFMAs, w(s+2) into the slot of w(s)
    // and the first half of x(s+3) into the slot of x(s); sub-step 2s+2 issues
    // the second half of x(s+3).
    const int nsub = 2 * nkl;
    auto substep = [&](const int us, const int cur) __attribute__((always_inline)) {
      __builtin_amdgcn_sched_barrier(0);
      const int s = us >> 1, j = us & 1;
      if (j == 1) {
        // This wave's last DMA of w(s+1) came after MFMA 6 of sub-step 2s-1;
        // after it only x(s+2) instructions 1 (after MFMA 7), 2 and 3 (sub-step
        // 2s) were issued, so at most 3 may stay in flight.  (At s = 0 the
        // prologue issued all of x(2) after w(1): waiting for 3 is stricter.)
        if (s + 2 < nkl) vm_wait<HDPW - 1>();
        else vm_wait<0>();
        if (KTAIL && kb + s + 1 == nk_full) fix_tail(s + 1);
        __syncthreads();
        __builtin_amdgcn_sched_barrier(0);
      }
      const int xk = j == 1 ? s + 3 : s + 2;  // x step whose DMAs this sub-step spreads
      const int xt = j == 1 ? 0 : 2;          // ... instructions xt and xt + 1
      const bool xdma = j == 1 || s >= 1;
      const bool more = us + 1 < nsub;
      const int un = us + 1;
#pragma unroll
      for (int q = 0; q < NMFMA; ++q) {
        const int i = q / FM, jm = q % FM;
        acc[i][jm] = mfma32<FMT>(fa[cur][i], fb[cur][jm], acc[i][jm]);
        if (more) {
#pragma unroll
          for (int r = q * NREAD / NMFMA; r < (q + 1) * NREAD / NMFMA; ++r)
            read_one(un >> 1, un & 1, r, fa[cur ^ 1], fb[cur ^ 1]);
        }
        // w(s+2) after MFMAs 0, 2, 4, 6 of the boundary sub-step, x after MFMAs 3
        // and 7 (measured best among the placements tried: a burst of DMA
        // instructions right after the barrier stalls the issuing waves)
        if (j == 1 && (q & 1) == 0) dma_half(rw[q >> 1], range_w, slot_w(s + 2), s + 2, q >> 1);
        if ((q == 3 || q == 7) && xdma) issue_x(xk, xt + (q == 7 ? 1 : 0));
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    for (int s = 0; s < nkl; ++s) {
      substep(2 * s, 0);
      substep(2 * s + 1, 1);
    }

    if constexpr (SK) {
      if (kb != 0 || ke != nk) {
        // Part of a tile.  Contributors are the stream-K workgroups c0 .. c1
        // whose ranges meet the tile, in K order.  Each stores its partial sums
        // (slot 2i if the segment opens the workgroup's range, else 2i+1: a
        // range holds at most one opening and one closing partial segment),
        // and the last to take the tile's ticket adds them all.
        const int tt = tile - a.n_dp;
        const int units = (total - a.n_dp) * nk;
        const int tu0 = tt * nk;
        const int c0 = sk_owner(tu0, units, a.n_sk), c1 = sk_owner(tu0 + nk - 1, units, a.n_sk);
        auto slot_of = [&](int i) __attribute__((always_inline)) {
          return (uint32_t)(2 * i + (sk_start(i, units, a.n_sk) >= tu0 ? 0 : 1)) * kPartialBytes;
        };
        const v4i rsrc_p = make_rsrc(a.P, (uint32_t)a.n_sk * 2u * kPartialBytes);
        // Thread t's float4 q of a partial tile sits at slot + q * 8 KiB + t * 16:
        // the per-thread part is the one VGPR offset, the rest goes in the
        // (uniform) scalar offset, so no address registers live across the loop.
        const uint32_t toff = (uint32_t)tid * 16u;
        auto own4 = [&](int q) __attribute__((always_inline)) {
          const int i = q / (4 * FM), jm = (q / 4) % FM, e = 4 * (q % 4);
          return v4f{acc[i][jm][e], acc[i][jm][e + 1], acc[i][jm][e + 2], acc[i][jm][e + 3]};
        };
        {
          const uint32_t mine = slot_of(sk_i);
#pragma unroll
          for (int q = 0; q < 32; ++q)
            llvm_buffer_store_v4f32(own4(q), rsrc_p, toff, mine + (uint32_t)q * 8192u, kDeviceScope);
        }
        asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
        __syncthreads();  // all partial stores acknowledged; every wave is done with the slots
        int *flag = (int *)smem;
        if (tid == 0) *flag = take_ticket(a.tickets + (size_t)tt * kTicketStride, a.epoch, c1 - c0 + 1);
        __syncthreads();
        const bool last = *flag != 0;
        if (!last) continue;
        asm volatile("" : : : "memory");
        // acc = P[c0] + P[c0+1] + ... + P[c1], added in that order whoever
        // finishes (the own part comes from registers), so the result does
        // not depend on arrival order.  Four float4 per thread at a time.
#pragma unroll
        for (int q0 = 0; q0 < 32; q0 += 4) {
          __builtin_amdgcn_sched_barrier(0);
          v4f t[4];
          if (c0 == sk_i) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) t[jj] = own4(q0 + jj);
          } else {
            const uint32_t base = slot_of(c0);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
              t[jj] = llvm_buffer_load_v4f32(rsrc_p, toff, base + (uint32_t)(q0 + jj) * 8192u, kDeviceScope);
          }
          for (int c = c0 + 1; c <= c1; ++c) {
            if (c == sk_i) {
#pragma unroll
              for (int jj = 0; jj < 4; ++jj) t[jj] += own4(q0 + jj);
            } else {
              const uint32_t base = slot_of(c);
              v4f v[4];
#pragma unroll
              for (int jj = 0; jj < 4; ++jj)
                v[jj] = llvm_buffer_load_v4f32(rsrc_p, toff, base + (uint32_t)(q0 + jj) * 8192u, kDeviceScope);
#pragma unroll
              for (int jj = 0; jj < 4; ++jj) t[jj] += v[jj];
            }
          }
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int q = q0 + jj, i = q / (4 * FM), jm = (q / 4) % FM, e = 4 * (q % 4);
            acc[i][jm][e] = t[jj].x; acc[i][jm][e + 1] = t[jj].y;
            acc[i][jm][e + 2] = t[jj].z; acc[i][jm][e + 3] = t[jj].w;
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }

    // Scales and biases into LDS past the bf16 tile, published by the
    // epilogue's first barrier.
    float *s_lds = (float *)(smem + 2 * BM * BN);
    float *b_lds = s_lds + BN;
    if (EPI && SK && a.bias && tid < BN)
      my_bias = llvm_buffer_load_f32(make_rsrc(a.bias + n0, (uint32_t)(a.N - n0) * 4u), (uint32_t)tid * 4u, 0, 0);
    __syncthreads();  // every wave is done with the slots (and the ticket flag)
    if (tid < BN) {
      s_lds[tid] = my_scale;
      b_lds[tid] = my_bias;
    }
    main_epilogue<BM, BN, WM, WN, EPI>(acc, a, smem, s_lds, b_lds, m0, n0, wave, lane, tid);
  }
}

// ---------------------------------------------------------------- skinny path
//
// M <= 128 (decode-shaped): the time is the stream of w through HBM.  A workgroup
// owns R = 16*RB rows of w (output columns) and one K slice.  Its NW waves (4 or
// 8) take the slice's 128-byte K chunks round-robin (wave v: chunks v, v+NW, ...), so
// together they read every w row front to back.  Each wave streams its chunks --
// R rows of w and 16*MB rows of x, 128 bytes each -- into a private ring of D LDS
// slots with LDS-DMA, one 1 KiB instruction per 8 rows, and multiplies them with
// V_MFMA_F32_16X16X128_F8F6F4 (A = 16 w rows, B = 16 x rows).  w is loaded with
// the non-temporal policy (read once; on gfx950 this roughly doubles streaming
// read bandwidth), x without it (every workgroup re-reads x, so it should stay in
// L2).  No barrier is needed in the K loop because no wave reads another wave's
// slots; completion is tracked with vmcnt.  At the end the per-wave sums are
// added through LDS in wave order, so results are deterministic.
//
// MFMA 16x16x128 layout (gfx950, checked on the hardware): operand lane l supplies
// row l % 16 and the 32 bytes of K-group l / 16; accumulator lane l, element e is
// row 4*(l/16) + e, column l % 16.  Rows here are w rows (n), columns x rows (m).
//
// blockIdx.y selects the K slice [s * k_slice, min(K, (s+1) * k_slice)).  With one
// slice the kernel scales and writes bf16 y; with several it writes unscaled fp32
// partials that the last workgroup of the column tile adds in slice order
// (splitk_finish).
struct SkinnyArgs {
  const uint8_t *x;
  const uint8_t *w;
  const float *scale;
  uint16_t *y;
  float *P;                  // fp32 partials [column tile][S][M][16*RB] (S > 1)
  unsigned long long *tickets;  // one per column tile, kTicketStride apart (S > 1), any initial value
  unsigned long long epoch;  // this call's id (< 2^48)
  int M, N, K;
  int k_slice;
  int vec;            // y rows allow 8-byte stores (N % 4 == 0, y 8-byte aligned)
  const float *bias;  // per-column bias [N] added after the scale, or null
  int act;            // activation applied last (kAct*)
};

template <int RB, int MB, int WAVES = 4>
struct SkinnyShape {
  static constexpr int NW = WAVES;         // waves per workgroup
  static constexpr int R = 16 * RB;        // w rows per workgroup
  static constexpr int MX = 16 * MB;       // x rows staged per chunk
  static constexpr int ROWS = R + MX;
  static constexpr int SLOT = ROWS * 128;  // bytes per ring slot
  static constexpr int OPS = ROWS / 8;     // 1 KiB DMA instructions per chunk
  // ring depth (chunks in flight per wave): 3 with 4 waves, 2 with 8 or with 128 x rows
  static constexpr int D = NW * 3 * SLOT <= 160 * 1024 ? 3 : 2;
  static constexpr int WAVE_LDS = D * SLOT;
  static_assert(NW * WAVE_LDS <= 160 * 1024, "LDS");
  static_assert((D - 1) * OPS < 64, "vmcnt range");
};

// 128-byte rows, 16-row MFMA reads: chunk c of row r lives at position c ^ swz16(r);
// every 8 consecutive rows use 8 different positions, every 16 rows 16 different
// (bank half, position) pairs.
__device__ __forceinline__ int swz16(int r) { return (r & 7) ^ ((r >> 3) & 1); }

__device__ __forceinline__ void dma16_nt(v4i rsrc, uint32_t lds_base, uint32_t voffset, uint32_t soffset) {
  lds_poison16(lds_base);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds"
               :
               : "s"(lds_base), "v"(voffset), "s"(rsrc), "s"(soffset)
               : "memory", "m0");
}

// s_waitcnt vmcnt(N) / lgkmcnt(0) as compiler memory barriers: LDS reads of data
// written by LDS-DMA must not be moved above the wait that covers the DMA.
template <int N>
__device__ __forceinline__ void vm_wait_fence() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
__device__ __forceinline__ void lgkm_wait_fence() { asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory"); }

template <int FMT>
__device__ __forceinline__ v4f mfma16(const v8i &a, const v8i &b, const v4f &c) {
  // Zero scale operands select the unscaled V_MFMA_F32_16X16X128_F8F6F4
  // (format codes as for mfma32).
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FMT >> 1, FMT & 1, 0, 0, 0, 0);
}

// Split-K with S > 1 slices, in the same launch.  Every workgroup of a column
// tile has stored its unscaled fp32 partials (tile-major: the tile's S slices
// of M x 16*RB floats are contiguous); the last of the tile's S workgroups to
// finish adds them in slice order s = 0, 1, ..., S-1, scales, rounds to bf16 and
// writes y, so the result does not depend on the order the workgroups ran in.
// "Last" is decided on the tile's ticket (take_ticket).  Ordering: each wave
// waits until its device-scope partial stores are acknowledged, the workgroup
// meets at a barrier, and only then does one thread take the ticket; the last
// workgroup reads with device scope after its ticket.  No L2 write-back or
// invalidate is needed for these accesses.
template <int RB, bool EPI>
__device__ __forceinline__ void splitk_finish(const SkinnyArgs &a, int n0, int *flag) {
  constexpr int R = 16 * RB;
  const int S = (int)gridDim.y;
  asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
  __syncthreads();
  if (threadIdx.x == 0) *flag = take_ticket(a.tickets + (size_t)blockIdx.x * kTicketStride, a.epoch, S);
  __syncthreads();
  if (!*flag) return;
  asm volatile("" : : : "memory");
  const v4i rsrc_p = make_rsrc(a.P + (size_t)blockIdx.x * S * a.M * R, (uint32_t)(S * a.M * R) * 4u);
  const uint32_t slice_bytes = (uint32_t)(a.M * R) * 4u;
  constexpr int q4 = R / 4;  // four-column groups in the tile
  // Each thread sums IT items (four columns of one row), IT * SB loads in flight
  // at a time; loads that fall past S or past the items read zero and are unused.
  constexpr int IT = 2, SB = 8;
  const int items = a.M * q4;
  const v4i rsrc_s = make_rsrc(a.scale + n0, (uint32_t)min(R, a.N - n0) * 4u);
  const v4i rsrc_b = make_rsrc(a.bias ? a.bias + n0 : nullptr, a.bias ? (uint32_t)min(R, a.N - n0) * 4u : 0u);
  for (int i0 = threadIdx.x; i0 < items; i0 += IT * (int)blockDim.x) {
    uint32_t off[IT];
    v4f acc[IT], sc[IT], bs[IT];
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int idx = i0 + i * (int)blockDim.x;
      off[i] = idx < items ? (uint32_t)((idx / q4) * R + 4 * (idx % q4)) * 4u : kOut;
      // scale of the item's four columns, requested before the partials
      sc[i] = llvm_buffer_load_v4f32(rsrc_s, idx < items ? (uint32_t)(4 * (idx % q4)) * 4u : kOut, 0, 0);
      // without a bias the descriptor's range is 0: every read is zero
      bs[i] = llvm_buffer_load_v4f32(rsrc_b, idx < items ? (uint32_t)(4 * (idx % q4)) * 4u : kOut, 0, 0);
      acc[i] = v4f{0.f, 0.f, 0.f, 0.f};
    }
    for (int s0 = 0; s0 < S; s0 += SB) {
      v4f v[IT][SB];
#pragma unroll
      for (int j = 0; j < SB; ++j)
#pragma unroll
        for (int i = 0; i < IT; ++i)
          v[i][j] = llvm_buffer_load_v4f32(rsrc_p, s0 + j < S ? off[i] + (uint32_t)(s0 + j) * slice_bytes : kOut, 0,
                                           kDeviceScope);
#pragma unroll
      for (int j = 0; j < SB; ++j)
#pragma unroll
        for (int i = 0; i < IT; ++i) {
          if (s0 + j >= S) continue;
          // slice 0 starts the sum (keeps its sign of zero), the others add in order
          if (s0 + j == 0) acc[i] = v[i][j];
          else { acc[i].x += v[i][j].x; acc[i].y += v[i][j].y; acc[i].z += v[i][j].z; acc[i].w += v[i][j].w; }
        }
    }
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int idx = i0 + i * (int)blockDim.x;
      if (idx >= items) continue;
      const int m = idx / q4, n = n0 + 4 * (idx % q4);
      if (n >= a.N) continue;
      uint16_t *yr = a.y + (size_t)m * a.N;
      auto val = [&](float v, float scl, float bb) __attribute__((always_inline)) {
        float z = v * scl;
        if constexpr (EPI) {
          if (a.bias) z += bb;
          z = activation_rt(z, a.act);
        }
        return bf16_rne(z);
      };
      const uint32_t b0 = val(acc[i].x, sc[i].x, bs[i].x), b1 = val(acc[i].y, sc[i].y, bs[i].y);
      const uint32_t b2 = val(acc[i].z, sc[i].z, bs[i].z), b3 = val(acc[i].w, sc[i].w, bs[i].w);
      if (a.vec) {
        *(uint2 *)(yr + n) = make_uint2(b0 | (b1 << 16), b2 | (b3 << 16));
      } else {
        const uint32_t b[4] = {b0, b1, b2, b3};
        for (int e = 0; e < 4 && n + e < a.N; ++e) yr[n + e] = (uint16_t)b[e];
      }
    }
  }
}

// End of a skinny workgroup: the NW waves' sums are added through LDS (`red`,
// NW*RB*MB*4*64 floats) in wave order, so the result does not depend on timing;
// wave v finishes blocks v, v+NW, ...  One K slice: scale and bf16 store;
// several: unscaled fp32 partials, which the column tile's last workgroup adds.
template <int RB, int MB, bool EPI, int NW = 4>
__device__ __forceinline__ void skinny_finish(const v4f (&acc)[RB][MB], const SkinnyArgs &a, float *red, int n0,
                                              int s, int wave, int lane, const v4f *esc, const v4f *ebi) {
  const int g = lane >> 4, lr = lane & 15;
  __syncthreads();
  // red[wave][block][lane] holds the lane's four sums of a block (16 bytes):
  // one 16-byte write per block, one 16-byte read per wave and block below.
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) *(v4f *)&red[(((wave * RB + rb) * MB + mb) * 64 + lane) * 4] = acc[rb][mb];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < (RB * MB + NW - 1) / NW; ++i) {
    const int b = wave + i * NW;
    if (b >= RB * MB) break;
    const int rb = b / MB, mb = b % MB;
    float v[4];
    {
      v4f t = *(const v4f *)&red[(b * 64 + lane) * 4];
#pragma unroll
      for (int o = 1; o < NW; ++o) {
        const v4f u = *(const v4f *)&red[((o * RB * MB + b) * 64 + lane) * 4];
        t[0] += u[0]; t[1] += u[1]; t[2] += u[2]; t[3] += u[3];
      }
      v[0] = t[0]; v[1] = t[1]; v[2] = t[2]; v[3] = t[3];
    }
    const int n = n0 + 16 * rb + 4 * g;
    const int m = 16 * mb + lr;
    if (m >= a.M) continue;
    if (gridDim.y > 1) {
      // all 16*RB columns of the tile are stored, also those past N (never read)
      const v4i rsrc_p = make_rsrc(a.P + ((size_t)blockIdx.x * gridDim.y + s) * a.M * (16 * RB),
                                   (uint32_t)(a.M * 16 * RB) * 4u);
      llvm_buffer_store_v4f32(v4f{v[0], v[1], v[2], v[3]}, rsrc_p, (uint32_t)(m * 16 * RB + (n - n0)) * 4u, 0,
                              kDeviceScope);
    } else {
      uint16_t *yr = a.y + (size_t)m * a.N;
      uint32_t bits[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float z = v[e] * esc[i][e];
        if constexpr (EPI) {
          if (a.bias) z += ebi[i][e];
          z = activation_rt(z, a.act);
        }
        bits[e] = bf16_rne(z);
      }
      if (a.vec) {
        if (n < a.N) *(uint2 *)(yr + n) = make_uint2(bits[0] | (bits[1] << 16), bits[2] | (bits[3] << 16));
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n + e < a.N) yr[n + e] = (uint16_t)bits[e];
      }
    }
  }
  if (gridDim.y > 1) splitk_finish<RB, EPI>(a, n0, (int *)red);
}

template <int RB, int MB, int FMT = 0, bool EPI = false, int NW = 4>
__global__ __launch_bounds__(64 * NW, 1) void fp8g_splitk_partial_kernel(SkinnyArgs a) {
  using S = SkinnyShape<RB, MB, NW>;
  constexpr int R = S::R, OPS = S::OPS, D = S::D, SLOT = S::SLOT, W_OPS = R / 8;
  static_assert(NW * RB * MB * 4 * 64 * 4 <= NW * S::WAVE_LDS, "the cross-wave sum fits in the ring");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NW * S::WAVE_LDS];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int K = a.K;
  const int n0 = blockIdx.x * R;
  const int rows_w = min(R, a.N - n0);
  const int s = blockIdx.y;
  const int kbeg = s * a.k_slice;
  const int kend = min(K, kbeg + a.k_slice);
  const int nch = (kend - kbeg + 127) >> 7;
  const int my = nch > wave ? (nch - wave + NW - 1) / NW : 0;  // chunks of this wave

  const v4i rsrc_w = make_rsrc(a.w + (size_t)n0 * K, (uint32_t)rows_w * (uint32_t)K);
  const v4i rsrc_x = make_rsrc(a.x, (uint32_t)a.M * (uint32_t)K);

  // With one K slice, the epilogue's scales (and biases) for the blocks this
  // wave finishes -- columns n .. n+3 of block b = wave + i NW, n = n0 + 16 (b /
  // MB) + 4 (lane / 16) -- requested before any DMA, so the kernel's end does
  // not wait for a cold read (columns at or past N read as zero).  With several
  // slices the column tile's last workgroup scales in splitk_finish.
  constexpr int BPW = (RB * MB + NW - 1) / NW;
  v4f esc[BPW], ebi[BPW];
  {
    const bool one = gridDim.y == 1;
    const v4i rsrc_s = make_rsrc(a.scale, one ? (uint32_t)a.N * 4u : 0u);
    const v4i rsrc_b = make_rsrc(a.bias, EPI && one && a.bias ? (uint32_t)a.N * 4u : 0u);
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const int b = wave + i * NW;
      const uint32_t at = b < RB * MB ? (uint32_t)(n0 + 16 * (b / MB) + 4 * (lane >> 4)) * 4u : kOut;
      esc[i] = llvm_buffer_load_v4f32(rsrc_s, at, 0, 0);
      ebi[i] = EPI ? llvm_buffer_load_v4f32(rsrc_b, at, 0, 0) : v4f{0.f, 0.f, 0.f, 0.f};
    }
  }

  // DMA instruction t moves rows 8t .. 8t+7 of a slot (w rows, then x rows).
  uint32_t src_off[OPS], src_chunk[OPS];
#pragma unroll
  for (int t = 0; t < OPS; ++t) {
    const int row = 8 * t + (lane >> 3);
    const int r = t < W_OPS ? row : row - R;
    const int c = (lane & 7) ^ swz16(r);
    src_chunk[t] = (uint32_t)c * 16u;
    src_off[t] = (uint32_t)r * (uint32_t)K + src_chunk[t];
  }
  const uint32_t ring_base =
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)smem + (uint32_t)wave * S::WAVE_LDS;
  uint8_t *ring = smem + wave * S::WAVE_LDS;

  // Local chunk j (global chunk wave + NW j) -> slot j % D.
  auto issue = [&](int j) __attribute__((always_inline)) {
    const int kc = kbeg + ((wave + NW * j) << 7);
    const int slot = j % D;
    if (kc + 128 <= kend) {
#pragma unroll
      for (int t = 0; t < OPS; ++t) {
        const uint32_t lds = ring_base + (uint32_t)(slot * SLOT + t * 1024);
        if (t < W_OPS) dma16_nt(rsrc_w, lds, src_off[t], (uint32_t)kc);
        else dma16(rsrc_x, lds, src_off[t], (uint32_t)kc);
      }
    } else {
      // the last chunk of K: bytes at or past K are zero
#pragma unroll
      for (int t = 0; t < OPS; ++t) {
        const uint4 v = load16_masked(t < W_OPS ? rsrc_w : rsrc_x, src_off[t] + (uint32_t)kc,
                                      kend - (kc + (int)src_chunk[t]), K);
        *(uint4 *)(ring + slot * SLOT + t * 1024 + lane * 16) = v;
      }
    }
  };

  v4f acc[RB][MB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[rb][mb] = v4f{0.f, 0.f, 0.f, 0.f};

  const int g = lane >> 4, lr = lane & 15;
  const int sw = swz16(lr);  // 16 rb and 16 mb leave the swizzle unchanged
  const int c0 = (2 * g) ^ sw, c1 = (2 * g + 1) ^ sw;

  for (int j = 0; j < D && j < my; ++j) issue(j);
  for (int j = 0; j < my; ++j) {
    const int ahead = min(D - 1, my - 1 - j);  // chunks issued after j
    if (ahead >= 2) vm_wait_fence<2 * OPS>();
    else if (ahead == 1) vm_wait_fence<OPS>();
    else vm_wait_fence<0>();
    const uint8_t *sl = ring + (j % D) * SLOT;
    v8i af[RB], bf[MB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const uint8_t *row = sl + (16 * rb + lr) * 128;
      const uint4 lo = *(const uint4 *)(row + (c0 << 4)), hi = *(const uint4 *)(row + (c1 << 4));
      af[rb] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const uint8_t *row = sl + (R + 16 * mb + lr) * 128;
      const uint4 lo = *(const uint4 *)(row + (c0 << 4)), hi = *(const uint4 *)(row + (c1 << 4));
      bf[mb] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
    if (j + D < my) {
      lgkm_wait_fence();  // this slot's reads are done before it is refilled
      issue(j + D);
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[rb][mb] = mfma16<FMT>(af[rb], bf[mb], acc[rb][mb]);
  }

  skinny_finish<RB, MB, EPI, NW>(acc, a, (float *)smem, n0, s, wave, lane, esc, ebi);
}

// Epilogue for accumulators of V_MFMA_F32_16X16X128_F8F6F4 (A = w, B = x):
// lane l, element e of block (i, j) is n = 16 i + 4 (l / 16) + e and
// m = 16 j + l % 16 of the wave tile, four consecutive n of one m.  Same
// arithmetic (scale, bias, activation in fp32), staging through LDS and
// whole-row stores as main_epilogue_t.
template <int BM, int BN, int WM, int WN, int ACT, bool BIAS>
__device__ __forceinline__ void main_epilogue16_t(const v4f (&acc)[BN / WN / 16][BM / WM / 16], const MainArgs &a,
                                                  uint8_t *smem, const float *s_lds, const float *b_lds, int m0,
                                                  int n0, int wave, int lane, int tid) {
  constexpr int NWAVES = WM * WN, TM = BM / WM, TN = BN / WN, FM = TM / 16, FN = TN / 16;
  constexpr int CPR = BN / 8, PITCH = 2 * BN, NTHREADS = NWAVES * 64;
  const int g = lane >> 4, l16 = lane & 15;
  const int wave_m = wave % WM, wave_n = wave / WM;
  __syncthreads();  // s_lds (and b_lds) are published
#pragma unroll
  for (int i = 0; i < FN; ++i) {
    const int nl = wave_n * TN + 16 * i + 4 * g;
    const float4 sc = *(const float4 *)(s_lds + nl);
    float4 bi = make_float4(0.f, 0.f, 0.f, 0.f);
    if constexpr (BIAS) bi = *(const float4 *)(b_lds + nl);
    auto val = [&](float v, float scl, float bs) __attribute__((always_inline)) {
      float z = v * scl;
      if constexpr (BIAS) z += bs;
      return activation<ACT>(z);
    };
#pragma unroll
    for (int j = 0; j < FM; ++j) {
      const int ml = wave_m * TM + 16 * j + l16;
      const uint32_t p01 = bf16x2_rne(val(acc[i][j][0], sc.x, bi.x), val(acc[i][j][1], sc.y, bi.y));
      const uint32_t p23 = bf16x2_rne(val(acc[i][j][2], sc.z, bi.z), val(acc[i][j][3], sc.w, bi.w));
      const int off = ml * PITCH + (((nl >> 3) ^ (ml & (CPR - 1))) << 4) + ((nl & 7) << 1);
      *(uint2 *)(smem + off) = make_uint2(p01, p23);
    }
  }
  __syncthreads();
  store_tile_rows<BM, BN, NTHREADS>(a, smem, m0, n0, tid);
}

// main_epilogue16_t for the call's activation and bias (one uniform switch);
// built without EPI, only the plain operation is compiled.
template <int BM, int BN, int WM, int WN, bool EPI>
__device__ __forceinline__ void main_epilogue16(const v4f (&acc)[BN / WN / 16][BM / WM / 16], const MainArgs &a,
                                                uint8_t *smem, const float *s_lds, const float *b_lds, int m0,
                                                int n0, int wave, int lane, int tid) {
  if constexpr (!EPI) {
    main_epilogue16_t<BM, BN, WM, WN, kActNone, false>(acc, a, smem, s_lds, b_lds, m0, n0, wave, lane, tid);
    return;
  }
  const int sel = a.act * 2 + (a.bias != nullptr ? 1 : 0);
#define FP8G_EPI(ACT, BIAS) \
  main_epilogue16_t<BM, BN, WM, WN, ACT, BIAS>(acc, a, smem, s_lds, b_lds, m0, n0, wave, lane, tid)
  switch (sel) {
    case 1: FP8G_EPI(kActNone, true); break;
    case 2: FP8G_EPI(kActRelu, false); break;
    case 3: FP8G_EPI(kActRelu, true); break;
    case 4: FP8G_EPI(kActSilu, false); break;
    case 5: FP8G_EPI(kActSilu, true); break;
    case 6: FP8G_EPI(kActGeluTanh, false); break;
    case 7: FP8G_EPI(kActGeluTanh, true); break;
    default: FP8G_EPI(kActNone, false); break;
  }
#undef FP8G_EPI
}

// Epilogue of variant 20, whose operand blocks carry tile rows in a per-call
// order (fp8g_main4wr_kernel).  Lane row i of a 16-row block carries the tile
// row perm(b, h, i); rows 2j and 2j + 1 are 128 apart.  So lane l (l16 = l % 16,
// g = l / 16) holds, in accumulator block (nb, mb), row mrow[mb] (its own l16 in
// x block mb) and, for elements e = 0, 1, 2, 3, columns pa[nb], pa[nb] + 128,
// pb[nb], pb[nb] + 128 (lane rows 4 g + e of w block nb): scattered rows and
// columns, but in pairs 128 apart.
//
// The bf16 tile is staged as column pairs: dword p (0..127) of row r holds
// columns p (low half) and p + 128 (high half), so each element pair is one
// 4-byte write.  Row pitch 512 bytes; pair chunk c = p / 4 of row r at position c
// ^ pswz(r), pswz(r) = ((r / 16) ^ r) mod 16.  One write instruction stores one
// pair p_g per lane group g for sixteen rows that agree mod 16 and differ in r /
// 16 (sixteen chunk positions); the four p_g agree mod 32, so two of the groups
// share a bank (2-way conflicts, in exchange for whole-line stores below).
__device__ __forceinline__ int pswz(int r) { return ((r >> 4) ^ r) & 15; }

// Writes the 256 x 256 bf16 tile staged by main_epilogue_perm_t to y (256
// threads).  Pass q (0..15) takes column group G = 8 (q % 2) + t % 8 of row 32 (q
// / 2) + t / 8 (thread t): pair chunks 2G and 2G + 1, i.e. columns 8 G .. 8 G + 7
// (low halves) and 128 + 8 G .. (high halves), one 16-byte store each, so eight
// lanes store one whole 128-byte line of a row; the two rows a 16-lane group
// reads differ in pswz's low bit, so its reads hit sixteen chunk positions.
__device__ __forceinline__ void store_tile_pairs(const MainArgs &a, const uint8_t *smem, int m0, int n0, int tid) {
  constexpr int PITCH = 512;
  auto grp = [&](int q) __attribute__((always_inline)) { return 8 * (q & 1) + (tid & 7); };
  auto row = [&](int q) __attribute__((always_inline)) { return 32 * (q >> 1) + (tid >> 3); };
  // columns 8 G .. + 7 (lo) and 128 + 8 G .. + 7 (hi) of row r
  auto fetch = [&](int r, int G, v4i &lo, v4i &hi) __attribute__((always_inline)) {
    const v4i d0 = *(const v4i *)(smem + r * PITCH + (((2 * G) ^ pswz(r)) << 4));
    const v4i d1 = *(const v4i *)(smem + r * PITCH + (((2 * G + 1) ^ pswz(r)) << 4));
    const uint32_t p[8] = {(uint32_t)d0[0], (uint32_t)d0[1], (uint32_t)d0[2], (uint32_t)d0[3],
                           (uint32_t)d1[0], (uint32_t)d1[1], (uint32_t)d1[2], (uint32_t)d1[3]};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      lo[k] = (int)__builtin_amdgcn_perm(p[2 * k + 1], p[2 * k], 0x05040100u);  // low halves
      hi[k] = (int)__builtin_amdgcn_perm(p[2 * k + 1], p[2 * k], 0x07060302u);  // high halves
    }
  };
  if (a.ystore == 16 && m0 + 256 <= a.M && n0 + 256 <= a.N) {
#pragma unroll
    for (int q0 = 0; q0 < 16; q0 += 4) {
      v4i lo[4], hi[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) fetch(row(q0 + b), grp(q0 + b), lo[b], hi[b]);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        uint16_t *yr = a.y + (size_t)(m0 + row(q0 + b)) * a.N + n0;
        store16(a, lo[b], yr + 8 * grp(q0 + b));
        store16(a, hi[b], yr + 128 + 8 * grp(q0 + b));
      }
    }
    return;
  }
  for (int q = 0; q < 16; ++q) {
    const int r = row(q), G = grp(q);
    const int m = m0 + r;
    if (m >= a.M || n0 + 8 * G >= a.N) continue;
    v4i lo, hi;
    fetch(r, G, lo, hi);
    uint16_t *yr = a.y + (size_t)m * a.N + n0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int n = n0 + 128 * h + 8 * G;
      if (n >= a.N) continue;
      const v4i v = h ? hi : lo;
      uint16_t *dst = yr + 128 * h + 8 * G;
      if (a.ystore == 16) {  // N % 8 == 0 and y 16-byte aligned: the chunk is whole
        store16(a, v, dst);
      } else if (a.ystore == 8) {  // N % 4 == 0 and y 8-byte aligned
        *(uint2 *)dst = make_uint2((uint32_t)v[0], (uint32_t)v[1]);
        if (n + 4 < a.N) *(uint2 *)(dst + 4) = make_uint2((uint32_t)v[2], (uint32_t)v[3]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (n + e < a.N) dst[e] = (uint16_t)((uint32_t)v[e >> 1] >> (16 * (e & 1)));
      }
    }
  }
}

template <int ACT, bool BIAS>
__device__ __forceinline__ void main_epilogue_perm_t(const v4f (&acc)[8][8], const MainArgs &a, uint8_t *smem,
                                                     const float *s_lds, const float *b_lds, int m0, int n0,
                                                     const int (&mrow)[8], const int (&pa)[8], const int (&pb)[8],
                                                     int tid) {
  constexpr int PITCH = 512;
  __syncthreads();  // s_lds (and b_lds) are published
  uint32_t rbase[8], rsw[8];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) {
    rbase[mb] = (uint32_t)mrow[mb] * PITCH;
    rsw[mb] = (uint32_t)pswz(mrow[mb]) << 4;
  }
  auto val = [&](float v, float scl, float bs) __attribute__((always_inline)) {
    float z = v * scl;
    if constexpr (BIAS) z += bs;
    return activation<ACT>(z);
  };
  // byte offset of pair p within its row, before the row's chunk swizzle
  auto at = [](int p) __attribute__((always_inline)) { return (uint32_t)p << 2; };
  // Every scale (and bias) this lane needs is read before the first write: LDS
  // operations complete in order, so a read behind writes waits for all of them.
  float sc[8][4], bi[8][4];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
    const int col[4] = {pa[nb], pa[nb] + 128, pb[nb], pb[nb] + 128};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sc[nb][e] = s_lds[col[e]];
      bi[nb][e] = BIAS ? b_lds[col[e]] : 0.0f;
    }
  }
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
    const uint32_t ca = at(pa[nb]), cb = at(pb[nb]);
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const v4f &v = acc[nb][mb];
      *(uint32_t *)(smem + (rbase[mb] | (ca ^ rsw[mb]))) =
          bf16x2_rne(val(v[0], sc[nb][0], bi[nb][0]), val(v[1], sc[nb][1], bi[nb][1]));
      *(uint32_t *)(smem + (rbase[mb] | (cb ^ rsw[mb]))) =
          bf16x2_rne(val(v[2], sc[nb][2], bi[nb][2]), val(v[3], sc[nb][3], bi[nb][3]));
    }
  }
  __syncthreads();
  store_tile_pairs(a, smem, m0, n0, tid);
}
template <bool EPI>
__device__ __forceinline__ void main_epilogue_perm(const v4f (&acc)[8][8], const MainArgs &a, uint8_t *smem,
                                                   const float *s_lds, const float *b_lds, int m0, int n0,
                                                   const int (&mrow)[8], const int (&pa)[8], const int (&pb)[8],
                                                   int tid) {
  if constexpr (!EPI) {
    main_epilogue_perm_t<kActNone, false>(acc, a, smem, s_lds, b_lds, m0, n0, mrow, pa, pb, tid);
    return;
  }
  const int sel = a.act * 2 + (a.bias != nullptr ? 1 : 0);
#define FP8G_EPI(ACT, BIAS) main_epilogue_perm_t<ACT, BIAS>(acc, a, smem, s_lds, b_lds, m0, n0, mrow, pa, pb, tid)
  switch (sel) {
    case 1: FP8G_EPI(kActNone, true); break;
    case 2: FP8G_EPI(kActRelu, false); break;
    case 3: FP8G_EPI(kActRelu, true); break;
    case 4: FP8G_EPI(kActSilu, false); break;
    case 5: FP8G_EPI(kActSilu, true); break;
    case 6: FP8G_EPI(kActGeluTanh, false); break;
    case 7: FP8G_EPI(kActGeluTanh, true); break;
    default: FP8G_EPI(kActNone, false); break;
  }
#undef FP8G_EPI
}

// ------------------------------------------- main path, one wave per SIMD
//
// 256 x 256 tiles and 128-byte K steps with four waves, each owning a 128 (m) x
// 128 (n) quarter of the tile as 8 x 8 blocks of V_MFMA_F32_16X16X128_F8F6F4.
// Per K step a quarter reads 32 KiB of operands from LDS, where two 64 x 128
// wave tiles read 48 KiB.
//
// With one wave per SIMD nothing covers a wave's waits, so the feed must run
// further ahead, in the same 160 KiB.  LDS holds ten 16 KiB units; a unit is
// one K step of half the tile's w rows or half its x rows: L = rows 0-63 and
// 128-191 (blocks 0-3 of both wave tiles), H = rows 64-127 and 192-255 (blocks
// 4-7).  A step runs as four quadrants of 16 MFMAs, with a barrier after the
// second and after the fourth:
//
//     Q1  w L x x L   reads x H (s)          DMA L units of s + 2 (first half)
//     Q2  w L x x H   reads w H (s)          DMA L units of s + 2 (second half)
//         barrier M_s: publishes w L, x L (s + 1); retires the H units of s
//     Q3  w H x x L   reads w L (s + 1)      DMA H units of s + 3 (first half)
//     Q4  w H x x H   reads x L (s + 1)      DMA H units of s + 3 (second half)
//         barrier E_s: publishes the H units of s + 1; retires the L units of s + 1
//
// Operands are single-buffered in registers (A[8] w blocks, B[8] x blocks):
// each read overwrites a block after its last use in the step.  An H unit is
// requested 2-2.5 steps before it is published and an L unit 1-1.5 steps (H
// units cycle through three slots per operand, L units through two: 3 + 3 + 2
// + 2 = 10).  Every read and DMA is pinned next to its MFMA by a scheduling
// barrier: left to the compiler, a quadrant's DMAs went out in one burst at its
// start and the issuing wave -- the only one on its SIMD -- stalled behind
// them (the kernel ran 8% slower).  Rows of a unit are stored with the 16-row
// swizzle swz16.  K % 128 == 0 only (other K run on the five-slot kernel).
template <int FMT = 0, bool EPI = false>
__global__ __launch_bounds__(256, 1) void fp8g_main4w_kernel(MainArgs a) {
  constexpr int BM = 256, BN = 256, BK = 128, WM = 2, WN = 2, NWAVES = 4;
  constexpr int TM = BM / WM, TN = BN / WN, FM = TM / 16, FN = TN / 16;
  constexpr int UNIT = 128 * BK;               // 16 KiB
  constexpr int UDPW = UNIT / 1024 / NWAVES;   // LDS-DMA instructions per wave per unit (4)
  static_assert(FM == 8 && FN == 8 && UDPW == 4, "the quadrant schedule assumes 8 x 8 blocks");
  static_assert(2 * BM * BN + 2 * BN * 4 <= 10 * UNIT, "epilogue tile, scales and biases fit");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[10 * UNIT];

  const int K = a.K;
  const int nk = K / BK;
  const uint32_t smem_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)smem;
  auto u_wl = [&](int k) __attribute__((always_inline)) { return (uint32_t)((k & 1) * UNIT); };
  auto u_xl = [&](int k) __attribute__((always_inline)) { return (uint32_t)((2 + (k & 1)) * UNIT); };
  auto u_wh = [&](int k) __attribute__((always_inline)) { return (uint32_t)((4 + k % 3) * UNIT); };
  auto u_xh = [&](int k) __attribute__((always_inline)) { return (uint32_t)((7 + k % 3) * UNIT); };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wave_m = wave % WM, wave_n = wave / WM;
  int tm, tn;
  tile_coords(a, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int rows_x = min(BM, a.M - m0), rows_w = min(BN, a.N - n0);
  // A tile's rows form one buffer range; rows past M or N read zero.
  const v4i rw = make_rsrc(a.w + (size_t)n0 * K, (uint32_t)rows_w * (uint32_t)K);
  const v4i rx = make_rsrc(a.x + (size_t)m0 * K, (uint32_t)rows_x * (uint32_t)K);
  // The epilogue's scale for column n0 + tid (the oldest vector-memory load:
  // every DMA wait below covers it).
  const float my_scale = llvm_buffer_load_f32(make_rsrc(a.scale + n0, (uint32_t)(a.N - n0) * 4u), (uint32_t)tid * 4u, 0, 0);
  float my_bias = 0.0f;
  if (EPI && a.bias)
    my_bias = llvm_buffer_load_f32(make_rsrc(a.bias + n0, (uint32_t)(a.N - n0) * 4u), (uint32_t)tid * 4u, 0, 0);

  // DMA instruction t of a wave fills unit rows (4t + wave) * 8 .. + 7, lane l
  // taking row (4t + wave) * 8 + l / 8 and logical chunk (l % 8) ^ swz16(row).
  // Unit row i is tile row i (i < 64) or i + 64, plus 64 for an H unit; the row
  // offset sits in the VGPR offset, which the buffer range check sees.
  const int urow = wave * 8 + (lane >> 3);
  const uint32_t dchunk = (uint32_t)(((lane & 7) ^ swz16(urow)) << 4);
  uint32_t vo_l[UDPW], vo_h[UDPW];
#pragma unroll
  for (int t = 0; t < UDPW; ++t) {
    const int i = t * NWAVES * 8 + urow;
    vo_l[t] = (uint32_t)(i + (i >= 64 ? 64 : 0)) * (uint32_t)K + dchunk;
    vo_h[t] = vo_l[t] + 64u * (uint32_t)K;
  }
  auto dma_l = [&](const v4i &rs, uint32_t unit, int k, int t) __attribute__((always_inline)) {
    dma16(rs, smem_base + unit + (uint32_t)(t * NWAVES + wave) * 1024u, vo_l[t], (uint32_t)k * BK);
  };
  auto dma_h = [&](const v4i &rs, uint32_t unit, int k, int t) __attribute__((always_inline)) {
    dma16(rs, smem_base + unit + (uint32_t)(t * NWAVES + wave) * 1024u, vo_h[t], (uint32_t)k * BK);
  };
  // The eight DMA instructions of a step's L (or H) units: w then x.
  auto issue_l = [&](int k, int q) __attribute__((always_inline)) {
    if (q < UDPW) dma_l(rw, u_wl(k), k, q);
    else dma_l(rx, u_xl(k), k, q - UDPW);
  };
  auto issue_h = [&](int k, int q) __attribute__((always_inline)) {
    if (q < UDPW) dma_h(rw, u_wh(k), k, q);
    else dma_h(rx, u_xh(k), k, q - UDPW);
  };

  // Operand reads: lane l takes row l % 16 of a 16-row block and logical chunks
  // 2g, 2g + 1 (g = l / 16), the 32 K bytes of its K group.  Block b of a wave
  // tile is unit row (wave half) * 64 + (b % 4) * 16 + l % 16.
  const int g = lane >> 4, l16 = lane & 15;
  const int sw = swz16(l16);
  const uint32_t c0 = (uint32_t)(((2 * g) ^ sw) << 4), c1 = (uint32_t)(((2 * g + 1) ^ sw) << 4);
  const uint32_t ra = (uint32_t)(wave_n * 64 + l16) * BK, rb = (uint32_t)(wave_m * 64 + l16) * BK;
  auto half16 = [&](uint32_t at, int hf, v8i &f) __attribute__((always_inline)) {
    const uint4 v = *(const uint4 *)(smem + at + (hf ? c1 : c0));
    f[4 * hf + 0] = (int)v.x; f[4 * hf + 1] = (int)v.y; f[4 * hf + 2] = (int)v.z; f[4 * hf + 3] = (int)v.w;
  };
  // The same read in the K loop: one VALU add of the unit's base (an SGPR) to
  // the lane's loop-invariant row and chunk offset per quadrant and chunk half,
  // the block as the instruction's immediate offset.  The add is written out so
  // the compiler cannot reassociate it: left to itself it spread the k % 3 of
  // the rotating units over the lane offsets, 30 VALU instructions a step, each
  // taking issue cycles from the MFMAs of this one wave per SIMD.
  const uint32_t oa[2] = {ra + c0, ra + c1}, ob[2] = {rb + c0, rb + c1};
  auto lane_at = [](uint32_t unit, uint32_t off) __attribute__((always_inline)) {
    uint32_t r;
    asm("v_add_u32 %0, %1, %2" : "=v"(r) : "s"(unit), "v"(off));
    return r;
  };
  auto rd16 = [&](uint32_t unit, const uint32_t (&o)[2], int blk, int hf, v8i &f) __attribute__((always_inline)) {
    const uint4 v = *(const uint4 *)(smem + lane_at(unit, o[hf]) + blk * 16 * BK);
    f[4 * hf + 0] = (int)v.x; f[4 * hf + 1] = (int)v.y; f[4 * hf + 2] = (int)v.z; f[4 * hf + 3] = (int)v.w;
  };

  v4f acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  v8i A[FN], B[FM];

  // Prologue in the steady state's issue order: H(0), L(0), H(1), L(1), H(2);
  // then wait for H(0) and L(0) (what came after them may stay in flight).
#pragma unroll
  for (int q = 0; q < 2 * UDPW; ++q) issue_h(0, q);
#pragma unroll
  for (int q = 0; q < 2 * UDPW; ++q) issue_l(0, q);
  if (nk > 1) {
#pragma unroll
    for (int q = 0; q < 2 * UDPW; ++q) issue_h(1, q);
#pragma unroll
    for (int q = 0; q < 2 * UDPW; ++q) issue_l(1, q);
  }
  if (nk > 2) {
#pragma unroll
    for (int q = 0; q < 2 * UDPW; ++q) issue_h(2, q);
  }
  if (nk > 2) vm_wait<6 * UDPW>();
  else if (nk > 1) vm_wait<4 * UDPW>();
  else vm_wait<0>();
  __syncthreads();
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    half16(u_wl(0) + ra + b * 16 * BK, 0, A[b]);
    half16(u_wl(0) + ra + b * 16 * BK, 1, A[b]);
    half16(u_xl(0) + rb + b * 16 * BK, 0, B[b]);
    half16(u_xl(0) + rb + b * 16 * BK, 1, B[b]);
  }

  // Step s.  STEADY (s + 3 < nk): every read and DMA of the schedule exists,
  // so the body has no branches; the last three steps take the guarded body.
  // In each quadrant the eight reads go out with its first eight MFMAs (so they
  // have landed by the barrier that retires their unit) and its four DMAs with
  // MFMAs 2, 6, 10, 14 (measured on MI355X, interleaved: 0.2-1.0% faster than
  // with MFMAs 1, 5, 9, 13 on five shapes); the MFMAs take their blocks in the
  // order the previous quadrant read them, so every block is read at least
  // eight MFMAs before its first use.
  auto step = [&](const int s, auto steady) __attribute__((always_inline)) {
    constexpr bool STEADY = decltype(steady)::value;
    const bool more = STEADY || s + 1 < nk;
    const bool more2 = STEADY || s + 2 < nk, more3 = STEADY || s + 3 < nk;
    // Q1: w L x x L (x block-major: B[0..3] arrived in that order); read x H (s)
    // into B[4..7]; DMA half of the L units of s + 2.
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int mb = q >> 2, nb = q & 3;
      acc[nb][mb] = mfma16<FMT>(A[nb], B[mb], acc[nb][mb]);
      if (q < 8) rd16(u_xh(s), ob, q >> 1, q & 1, B[4 + (q >> 1)]);
      if ((q & 3) == 2 && more2) issue_l(s + 2, q >> 2);
      __builtin_amdgcn_sched_barrier(0);  // keep the spread as written
    }
    // Q2: w L x x H (x block-major); read w H (s) into A[4..7]; DMA the other
    // half of the L units of s + 2.
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int mb = 4 + (q >> 2), nb = q & 3;
      acc[nb][mb] = mfma16<FMT>(A[nb], B[mb], acc[nb][mb]);
      if (q < 8) rd16(u_wh(s), oa, q >> 1, q & 1, A[4 + (q >> 1)]);
      if ((q & 3) == 2 && more2) issue_l(s + 2, 4 + (q >> 2));
      __builtin_amdgcn_sched_barrier(0);
    }
    if (more) {
      // M_s publishes the L units of s + 1 (this wave issued H(s + 2) and L(s + 2)
      // after them) and retires the H units of s (read in Q1 and Q2).
      if (more2) vm_wait<4 * UDPW>();
      else vm_wait<0>();
      __syncthreads();
    }
    __builtin_amdgcn_sched_barrier(0);
    // Q3: w H x x L (w block-major: A[4..7] arrived in that order); read w L
    // (s + 1) into A[0..3]; DMA half of the H units of s + 3.
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int nb = 4 + (q >> 2), mb = q & 3;
      acc[nb][mb] = mfma16<FMT>(A[nb], B[mb], acc[nb][mb]);
      if (more && q < 8) rd16(u_wl(s + 1), oa, q >> 1, q & 1, A[q >> 1]);
      if ((q & 3) == 2 && more3) issue_h(s + 3, q >> 2);
      __builtin_amdgcn_sched_barrier(0);
    }
    // Q4: w H x x H; read x L (s + 1) into B[0..3]; DMA the other half of the
    // H units of s + 3.
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int nb = 4 + (q >> 2), mb = 4 + (q & 3);
      acc[nb][mb] = mfma16<FMT>(A[nb], B[mb], acc[nb][mb]);
      if (more && q < 8) rd16(u_xl(s + 1), ob, q >> 1, q & 1, B[q >> 1]);
      if ((q & 3) == 2 && more3) issue_h(s + 3, 4 + (q >> 2));
      __builtin_amdgcn_sched_barrier(0);
    }
    if (more) {
      // E_s publishes the H units of s + 1; issued after them: L(s + 1), and
      // H(s + 2), L(s + 2), H(s + 3) where they exist.  Retires the L units of
      // s + 1 (read in Q3 and Q4).
      if (more3) vm_wait<8 * UDPW>();
      else if (more2) vm_wait<6 * UDPW>();
      else vm_wait<2 * UDPW>();
      __syncthreads();
    }
  };
  int s = 0;
  for (; s + 3 < nk; ++s) step(s, std::true_type{});
  float *s_lds = (float *)(smem + 2 * BM * BN), *b_lds = s_lds + BN;

  if constexpr (!EPI) {
    // Plain epilogue: the accumulators of w blocks 0-3 are final after Q2 of the
    // last step, and no operand is read from LDS after it, so half of the bf16
    // tile is staged between the MFMAs of Q3 and Q4 (one block per MFMA) and
    // only the other half after them (the same arithmetic as main_epilogue16:
    // y = bf16(acc * scale); measured on MI355X: 4096^3 -0.9%, 8192^2 x 1024
    // -3.1%, 8192^3 -0.3%).
    for (; s + 1 < nk; ++s) step(s, std::false_type{});
    constexpr int CPR = BN / 8, PITCH = 2 * BN;
    auto stage = [&](int i, int j, const float4 &sc) __attribute__((always_inline)) {
      const int nl = wave_n * TN + 16 * i + 4 * g;
      const int ml = wave_m * TM + 16 * j + l16;
      const uint32_t p01 = bf16x2_rne(acc[i][j][0] * sc.x, acc[i][j][1] * sc.y);
      const uint32_t p23 = bf16x2_rne(acc[i][j][2] * sc.z, acc[i][j][3] * sc.w);
      const int off = ml * PITCH + (((nl >> 3) ^ (ml & (CPR - 1))) << 4) + ((nl & 7) << 1);
      *(uint2 *)(smem + off) = make_uint2(p01, p23);
    };
    // last step: Q1 and Q2 read the H units of s (no DMA is in flight)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int mb = q >> 2, nb = q & 3;
      acc[nb][mb] = mfma16<FMT>(A[nb], B[mb], acc[nb][mb]);
      if (q < 8) rd16(u_xh(s), ob, q >> 1, q & 1, B[4 + (q >> 1)]);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int mb = 4 + (q >> 2), nb = q & 3;
      acc[nb][mb] = mfma16<FMT>(A[nb], B[mb], acc[nb][mb]);
      if (q < 8) rd16(u_wh(s), oa, q >> 1, q & 1, A[4 + (q >> 1)]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // every wave has read its operands: the units hold the bf16 tile from here
    __syncthreads();
    s_lds[tid] = my_scale;
    __syncthreads();
    float4 sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] = *(const float4 *)(s_lds + wave_n * TN + 16 * i + 4 * g);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int nb = 4 + (q >> 2), mb = q & 3;
      acc[nb][mb] = mfma16<FMT>(A[nb], B[mb], acc[nb][mb]);
      stage(q >> 3, q & 7, sc[q >> 3]);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int nb = 4 + (q >> 2), mb = 4 + (q & 3);
      acc[nb][mb] = mfma16<FMT>(A[nb], B[mb], acc[nb][mb]);
      stage(2 + (q >> 3), q & 7, sc[2 + (q >> 3)]);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 4; i < FN; ++i) {
      const float4 c = *(const float4 *)(s_lds + wave_n * TN + 16 * i + 4 * g);
#pragma unroll
      for (int j = 0; j < FM; ++j) stage(i, j, c);
    }
    __syncthreads();
    store_tile_rows<BM, BN, NWAVES * 64>(a, smem, m0, n0, tid);
    (void)b_lds;
    (void)my_bias;
  } else {
    for (; s < nk; ++s) step(s, std::false_type{});
    // Scales (and biases) into LDS past the bf16 tile once every wave is done
    // with the units.
    __syncthreads();
    s_lds[tid] = my_scale;
    b_lds[tid] = my_bias;
    main_epilogue16<BM, BN, WM, WN, EPI>(acc, a, smem, s_lds, b_lds, m0, n0, wave, lane, tid);
  }
}

// ------------------------- main path, one wave per SIMD, cache-line rows (odd K)
//
// Variant 19's tiles, waves and MFMA order for odd K, where rows do not start on
// the 128-byte line grid.  A 128-byte K window of such a row spans two cache
// lines, and streaming it as it lies costs the global-to-LDS path about twice
// the line traffic of an aligned row (measured on MI355X, 4096^2 x 4127: 85-91
// us against 62 us for the same steps on aligned rows).  Here every row is
// fetched as whole aligned lines, one line per row per K step, and each lane
// rebuilds its operand bytes from two lines in registers.
//
// Row r of a tile starts o_r = a0 + r K bytes past the line holding the tile's
// first byte (a0 = that byte's address mod 128); write o_r mod 128 = 16 c_r +
// beta_r (chunk c_r, byte beta_r of its line).  The K window of step t is then
// the nine 16-byte chunks c_r .. c_r + 8 of the row's lines t and t + 1, shifted
// down by beta_r bytes.
//
// Row order.  For odd K, r -> o_r mod 128 is a bijection of r mod 128, so tile
// rows can be dealt to MFMA block lanes by (c, beta): lane row i (0..15) of
// block b (0..7) of wave half h carries the row with c = i / 2 and beta = 2 b +
// h (lane rows 2 j and 2 j + 1 take the two rows of that class, 128 apart):
//
//     perm(b, h, i) = ((16 (i / 2) + 2 b + h - a0) K^-1 mod 128) + 128 (i mod 2)
//
// A block's shift is then beta / 4 = b / 2 whole dwords, known at compile time,
// plus beta mod 4 = 2 (b mod 2) + h bytes, a wave-uniform value: eight
// V_ALIGNBYTE_B32 per 32-byte window and no branch.  Where a lane finds its
// chunks in LDS does not depend on the call either.  The epilogue puts the rows
// back in order (main_epilogue_perm).
//
// LDS holds ten 16 KiB units, each one line of half the tile's rows of one
// operand (L = blocks 0-3 of both wave halves, H = blocks 4-7; unit row 64 h + 16
// (b mod 4) + i); x lines cycle through three units per half, w lines through
// two.  A step runs four quadrants of 16 MFMAs, each followed by a barrier, and
// every unit is read in one quadrant only:
//
//     Q1  w L x x L   reads x H window (t)       DMA x L line t + 3
//     Q2  w L x x H   reads w H window (t)       DMA x H line t + 3
//     Q3  w H x x L   reads w L window (t + 1)   DMA w H line t + 2
//     Q4  w H x x H   reads x L window (t + 1)   DMA w L line t + 3
//
// A line is published by the barrier before its first reading quadrant and
// retired by the barrier after its second (1.25 steps later); its DMA goes out in
// the quadrant after the barrier that retired the line it replaces, 1.75 steps
// (x) or 0.75 steps (w) before it is published.
//
// In a unit, row i's window chunk v (line chunk (c + v) mod 8) sits at position
// v ^ swz16(i).  Lane l (i = l mod 16, K group g = l / 16) reads window chunks
// 2 g, 2 g + 1 and 2 g + 2, the last ones from the unit of line t + 1 once c + v
// reaches 8: positions and unit choice depend on the lane alone.  The reads go
// out in one quadrant and the shift is applied in the next, just before the
// block's first MFMA; in the last step the bytes at or past K are cleared in
// both operands.
//
// Requirements (checked by the host): K odd and above 128; x and w 128-byte aligned, so no
// line starts before an operand; M K and N K multiples of 16, so the last row
// of either operand ends on a 16-byte boundary and a tile's buffer range never
// cuts a chunk (bytes past the range read as zero; bytes of the next row that a
// line carries past K are cleared).
template <int N, typename F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
// f(std::integral_constant<int, 0>{}) .. f(std::integral_constant<int, N - 1>{}).
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  static_for_impl<N>(f, std::make_integer_sequence<int, N>{});
}

template <int FMT = 0, bool EPI = false>
__global__ __launch_bounds__(256, 1) void fp8g_main4wr_kernel(MainArgs a) {
  constexpr int BM = 256, BN = 256, BK = 128, WM = 2, WN = 2, NWAVES = 4;
  constexpr int TM = BM / WM, TN = BN / WN, FM = TM / 16, FN = TN / 16;
  constexpr int UNIT = 128 * BK;              // 16 KiB: one line of 128 rows
  constexpr int UDPW = UNIT / 1024 / NWAVES;  // LDS-DMA instructions per wave per unit (4)
  static_assert(FM == 8 && FN == 8 && UDPW == 4, "the quadrant schedule assumes 8 x 8 blocks");
  static_assert(2 * BM * BN + 2 * BN * 4 <= 10 * UNIT, "epilogue tile, scales and biases fit");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[10 * UNIT];

  const int K = a.K;
  const int nk = (K + BK - 1) / BK;  // K steps; lines 0 .. nk of every row are fetched
  const uint32_t smem_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)smem;
  // unit of line j: x L 0-2, x H 3-5, w L 6-7, w H 8-9 (uniform: scalar arithmetic)
  auto mod3 = [&](int j) __attribute__((always_inline)) { return j - 3 * (int)(((uint32_t)j * 0xAAABu) >> 17); };
  auto u_xl = [&](int j) __attribute__((always_inline)) { return (uint32_t)(mod3(j) * UNIT); };
  auto u_xh = [&](int j) __attribute__((always_inline)) { return (uint32_t)((3 + mod3(j)) * UNIT); };
  auto u_wl = [&](int j) __attribute__((always_inline)) { return (uint32_t)((6 + (j & 1)) * UNIT); };
  auto u_wh = [&](int j) __attribute__((always_inline)) { return (uint32_t)((8 + (j & 1)) * UNIT); };
  auto exists = [&](int j) __attribute__((always_inline)) { return j <= nk; };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wave_m = wave % WM, wave_n = wave / WM;
  int tm, tn;
  tile_coords(a, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int rows_x = min(BM, a.M - m0), rows_w = min(BN, a.N - n0);
  // Each tile's rows as one buffer from the line holding its first byte to the
  // end of its last valid row (a multiple of 16 bytes: see above).
  const uint8_t *bx = a.x + (size_t)m0 * K, *bw = a.w + (size_t)n0 * K;
  const uint32_t ax0 = (uint32_t)((uintptr_t)bx & 127u), aw0 = (uint32_t)((uintptr_t)bw & 127u);
  const v4i rx = make_rsrc(bx - ax0, ax0 + (uint32_t)rows_x * (uint32_t)K);
  const v4i rw = make_rsrc(bw - aw0, aw0 + (uint32_t)rows_w * (uint32_t)K);
  const float my_scale = llvm_buffer_load_f32(make_rsrc(a.scale + n0, (uint32_t)(a.N - n0) * 4u), (uint32_t)tid * 4u, 0, 0);
  float my_bias = 0.0f;
  if (EPI && a.bias)
    my_bias = llvm_buffer_load_f32(make_rsrc(a.bias + n0, (uint32_t)(a.N - n0) * 4u), (uint32_t)tid * 4u, 0, 0);

  // K^-1 mod 128 (K odd): K K = 1 mod 8, and each Newton step x (2 - K x)
  // doubles the number of correct low bits (3 -> 6 -> 12).
  uint32_t kinv = (uint32_t)K;
  kinv *= 2u - (uint32_t)K * kinv;
  kinv *= 2u - (uint32_t)K * kinv;
  // Tile row carried by lane row i of block b of wave half h (a0: ax0 or aw0).
  auto perm = [&](uint32_t a0, int b, int h, int i) __attribute__((always_inline)) {
    return (int)((((uint32_t)(16 * (i >> 1) + 2 * b + h) - a0) * kinv) & 127u) + 128 * (i & 1);
  };

  // DMA instruction t of a wave fills unit rows (4t + wave) * 8 .. + 7 of a
  // line: lane l takes unit row u = (4t + wave) * 8 + l / 8 and position p = l %
  // 8, i.e. window chunk p ^ swz16(u % 16) = line chunk (c + that) mod 8.  The
  // line's start sits in the VGPR offset, the line index times 128 in the SGPR
  // offset.
  uint32_t vdx[2][UDPW], vdw[2][UDPW];
#pragma unroll
  for (int hu = 0; hu < 2; ++hu)
#pragma unroll
    for (int t = 0; t < UDPW; ++t) {
      const int u = (t * NWAVES + wave) * 8 + (lane >> 3);
      const int h = u >> 6, b = ((u >> 4) & 3) + 4 * hu, i = u & 15;
      const uint32_t v = (uint32_t)((lane & 7) ^ swz16(i));
      const uint32_t ox = ax0 + (uint32_t)perm(ax0, b, h, i) * (uint32_t)K;
      const uint32_t ow = aw0 + (uint32_t)perm(aw0, b, h, i) * (uint32_t)K;
      vdx[hu][t] = (ox & ~127u) + 16u * ((((ox >> 4) & 7u) + v) & 7u);
      vdw[hu][t] = (ow & ~127u) + 16u * ((((ow >> 4) & 7u) + v) & 7u);
    }
  auto dma_unit = [&](const v4i &rs, uint32_t unit, const uint32_t (&vo)[UDPW], int j, int t)
      __attribute__((always_inline)) {
    dma16(rs, smem_base + unit + (uint32_t)(t * NWAVES + wave) * 1024u, vo[t], (uint32_t)j * BK);
  };
  // The four DMA groups of the schedule (4 instructions per wave each); the one
  // for quadrant q of step s carries line s + 3 (x L, x H, w L) or s + 2 (w H).
  auto issue = [&](int q, int s, int t) __attribute__((always_inline)) {
    if (q == 1) dma_unit(rx, u_xl(s + 3), vdx[0], s + 3, t);
    else if (q == 2) dma_unit(rx, u_xh(s + 3), vdx[1], s + 3, t);
    else if (q == 3) dma_unit(rw, u_wh(s + 2), vdw[1], s + 2, t);
    else dma_unit(rw, u_wl(s + 3), vdw[0], s + 3, t);
  };
  auto group_exists = [&](int q, int s) __attribute__((always_inline)) { return exists(q == 3 ? s + 2 : s + 3); };

  // Operand reads.  Read k (0..2) of lane l is window chunk v = 2 g + k of unit
  // row 64 h + 16 (b mod 4) + l16: LDS offset lp[k] + 2048 (b mod 4) from the
  // unit of line t, or of line t + 1 where sel[k] is set.
  const int g = lane >> 4, l16 = lane & 15;
  uint32_t lpx[3], lpw[3], sel[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const int v = 2 * g + k;
    const uint32_t pos = (uint32_t)l16 * BK + (uint32_t)(((v & 7) ^ swz16(l16)) << 4);
    lpx[k] = (uint32_t)wave_m * 64u * BK + pos;
    lpw[k] = (uint32_t)wave_n * 64u * BK + pos;
    sel[k] = (l16 >> 1) + v >= 8 ? ~0u : 0u;
  }
  // The three addresses of a window read from units S0 (line t) and S1 (line t + 1):
  // two VALU instructions each, written out so the compiler cannot reassociate
  // the wave-uniform unit bases into the lane offsets (it spent about three more
  // a window that way, and each VALU instruction takes issue cycles from the
  // MFMAs of this one wave per SIMD).
  auto win = [&](uint32_t S0, uint32_t S1, const uint32_t (&lp)[3], uint32_t (&at)[3])
      __attribute__((always_inline)) {
    const uint32_t d = S1 - S0;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      uint32_t m;
      asm("v_and_b32 %0, %1, %2" : "=v"(m) : "s"(d), "v"(sel[k]));
      asm("v_add3_u32 %0, %1, %2, %3" : "=v"(at[k]) : "v"(lp[k]), "s"(S0), "v"(m));
    }
  };
  // Read k of block b mod 4 = bl: chunks 0 and 1 into f, chunk 2 into x3.
  auto read_blk = [&](const uint32_t (&at)[3], int bl, int k, v8i &f, v4i &x3) __attribute__((always_inline)) {
    const uint4 v = *(const uint4 *)(smem + at[k] + (uint32_t)bl * 16u * BK);
    if (k < 2) {
      f[4 * k + 0] = (int)v.x; f[4 * k + 1] = (int)v.y; f[4 * k + 2] = (int)v.z; f[4 * k + 3] = (int)v.w;
    } else {
      x3 = v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
    }
  };
  // Shift block b's window into place: bytes [beta, beta + 32) of the 48 read,
  // beta = 2 b + h, i.e. registers from b / 2 on and sh[b % 2] = beta mod 4
  // bytes.  With `tail` (the guarded last steps only) bytes at or past K are
  // then cleared when t is the last step.
  const uint32_t shx[2] = {(uint32_t)wave_m, 2u + (uint32_t)wave_m};
  const uint32_t shw[2] = {(uint32_t)wave_n, 2u + (uint32_t)wave_n};
  auto realign = [&](v8i &f, const v4i &x3, auto bc, const uint32_t (&sh)[2], int t, auto tail)
      __attribute__((always_inline)) {
    constexpr int b = decltype(bc)::value, D = b >> 1;
    const uint32_t r[12] = {(uint32_t)f[0], (uint32_t)f[1], (uint32_t)f[2], (uint32_t)f[3], (uint32_t)f[4],
                            (uint32_t)f[5], (uint32_t)f[6], (uint32_t)f[7], (uint32_t)x3.x, (uint32_t)x3.y,
                            (uint32_t)x3.z, (uint32_t)x3.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = (int)__builtin_amdgcn_alignbyte(r[e + D + 1], r[e + D], sh[b & 1]);
    // The dwords the shift does not use are consumed here, so the compiler keeps
    // every read at 16 bytes: narrower reads are serviced for more lanes at once,
    // and the four K groups of a block then collide on the same banks (measured:
    // 20x the bank-conflict cycles of whole-chunk reads).
#pragma unroll
    for (int i = 0; i < 12; ++i)
      if (i < D || i > D + 8) asm volatile("" : : "v"(r[i]));
    if (decltype(tail)::value && t == nk - 1) {
      const int valid = K - t * BK - 32 * g;  // bytes of this lane's 32 that lie before K
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int vb = valid - 4 * e;
        const uint32_t m = vb >= 4 ? 0xFFFFFFFFu : vb <= 0 ? 0u : (1u << (8 * vb)) - 1u;
        f[e] = (int)((uint32_t)f[e] & m);
      }
    }
  };
  using I0 = std::integral_constant<int, 0>;

  v4f acc[FN][FM];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < FM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  v8i A[FN], B[FM];
  v4i A3[FN], B3[FM];  // third chunk of each block's window until its realignment

  // vmcnt with n DMA groups allowed to stay in flight.
  auto wait_groups = [&](int n) __attribute__((always_inline)) {
    switch (n) {
      case 0: vm_wait<0>(); break;
      case 1: vm_wait<UDPW>(); break;
      case 2: vm_wait<2 * UDPW>(); break;
      case 3: vm_wait<3 * UDPW>(); break;
      case 4: vm_wait<4 * UDPW>(); break;
      case 5: vm_wait<5 * UDPW>(); break;
      default: vm_wait<6 * UDPW>(); break;
    }
  };

  // Prologue: lines 0 and 1 of every unit, and line 0 of w H; then the first
  // windows of A[0..3] and B[0..3]; then the groups the schedule places in the
  // (virtual) step -1: x L 2, x H 2, w H 1, w L 2 (w L 2 into the unit of w L 0,
  // free once the windows are read).
#pragma unroll
  for (int t = 0; t < UDPW; ++t) {
    dma_unit(rx, u_xl(0), vdx[0], 0, t);
    dma_unit(rw, u_wl(0), vdw[0], 0, t);
  }
#pragma unroll
  for (int t = 0; t < UDPW; ++t) {
    dma_unit(rx, u_xl(1), vdx[0], 1, t);
    dma_unit(rw, u_wl(1), vdw[0], 1, t);
  }
#pragma unroll
  for (int t = 0; t < UDPW; ++t) {
    dma_unit(rx, u_xh(0), vdx[1], 0, t);
    dma_unit(rx, u_xh(1), vdx[1], 1, t);
    dma_unit(rw, u_wh(0), vdw[1], 0, t);
  }
  vm_wait<0>();
  __syncthreads();
  {
    uint32_t aw[3], ax[3];
    win(u_wl(0), u_wl(1), lpw, aw);
    win(u_xl(0), u_xl(1), lpx, ax);
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        read_blk(aw, b, k, A[b], A3[b]);
        read_blk(ax, b, k, B[b], B3[b]);
      }
  }
  __syncthreads();  // the windows are read: w L 0 and x L 0 are retired
#pragma unroll
  for (int q = 1; q <= 4; ++q)
    if (group_exists(q, -1)) {
#pragma unroll
      for (int t = 0; t < UDPW; ++t) issue(q, -1, t);
    }
  // B[1..3] are realigned in step 0's first quadrant, as in every step.
  static_for<4>([&](auto bc) __attribute__((always_inline)) {
    realign(A[decltype(bc)::value], A3[decltype(bc)::value], bc, shw, 0, std::true_type{});
  });
  realign(B[0], B3[0], I0{}, shx, 0, std::true_type{});

  // Step s.  STEADY: every DMA group and read of the schedule exists (s + 3 <=
  // nk), so the body has no branches; the last steps take the guarded body.
  // Reads go out with MFMAs 0-11 of their quadrant (three per block), DMAs with
  // MFMAs 1, 5, 9, 13.  A block is realigned four MFMAs before its first use:
  // its reads went out at least a quadrant earlier, or (the first block read in
  // a quadrant) twelve MFMAs earlier.
  auto step = [&](const int s, auto steady) __attribute__((always_inline)) {
    constexpr bool STEADY = decltype(steady)::value;
    using TAILC = std::integral_constant<bool, !STEADY>;
    const bool next = STEADY || s + 1 < nk;  // the windows of step s + 1 exist
    uint32_t at[3];
    // ---- Q1: w L x x L; read x H (s) into B[4..7]; realign B[1..4]
    win(u_xh(s), u_xh(s + 1), lpx, at);
    __builtin_amdgcn_sched_barrier(0);
    static_for<16>([&](auto qc) __attribute__((always_inline)) {
      constexpr int q = decltype(qc)::value, mb = q >> 2, nb = q & 3;
      acc[nb][mb] = mfma16<FMT>(A[nb], B[mb], acc[nb][mb]);
      if constexpr ((q & 3) == 0)
        realign(B[1 + mb], B3[1 + mb], std::integral_constant<int, 1 + mb>{}, shx, s, TAILC{});
      if constexpr (q < 12) read_blk(at, q / 3, q % 3, B[4 + q / 3], B3[4 + q / 3]);
      if ((q & 3) == 1 && (STEADY || group_exists(1, s))) issue(1, s, q >> 2);
      __builtin_amdgcn_sched_barrier(0);  // keep the spread as written
    });
    // B1: publishes w H line s + 1; groups issued after it: w L s + 2, x L s + 3
    if (STEADY) vm_wait<2 * UDPW>();
    else wait_groups((int)group_exists(4, s - 1) + (int)group_exists(1, s));
    __syncthreads();
    // ---- Q2: w L x x H; read w H (s) into A[4..7]; realign B[5..7], A[4]
    win(u_wh(s), u_wh(s + 1), lpw, at);
    __builtin_amdgcn_sched_barrier(0);
    static_for<16>([&](auto qc) __attribute__((always_inline)) {
      constexpr int q = decltype(qc)::value, mb = 4 + (q >> 2), nb = q & 3;
      acc[nb][mb] = mfma16<FMT>(A[nb], B[mb], acc[nb][mb]);
      if constexpr (q < 12 && (q & 3) == 0)
        realign(B[mb + 1], B3[mb + 1], std::integral_constant<int, mb + 1>{}, shx, s, TAILC{});
      if constexpr (q == 12) realign(A[4], A3[4], std::integral_constant<int, 4>{}, shw, s, TAILC{});
      if constexpr (q < 12) read_blk(at, q / 3, q % 3, A[4 + q / 3], A3[4 + q / 3]);
      if ((q & 3) == 1 && (STEADY || group_exists(2, s))) issue(2, s, q >> 2);
      __builtin_amdgcn_sched_barrier(0);
    });
    // B2: publishes w L line s + 2; after it: x L s + 3, x H s + 3
    if (STEADY) vm_wait<2 * UDPW>();
    else wait_groups((int)group_exists(1, s) + (int)group_exists(2, s));
    __syncthreads();
    // ---- Q3: w H x x L; read w L (s + 1) into A[0..3]; realign A[5..7], A[0]
    win(u_wl(s + 1), u_wl(s + 2), lpw, at);
    __builtin_amdgcn_sched_barrier(0);
    static_for<16>([&](auto qc) __attribute__((always_inline)) {
      constexpr int q = decltype(qc)::value, nb = 4 + (q >> 2), mb = q & 3;
      acc[nb][mb] = mfma16<FMT>(A[nb], B[mb], acc[nb][mb]);
      if constexpr (q < 12 && (q & 3) == 0)
        realign(A[nb + 1], A3[nb + 1], std::integral_constant<int, nb + 1>{}, shw, s, TAILC{});
      if constexpr (q == 12) {
        if (next) realign(A[0], A3[0], I0{}, shw, s + 1, TAILC{});
      }
      if constexpr (q < 12) {
        if (next) read_blk(at, q / 3, q % 3, A[q / 3], A3[q / 3]);
      }
      if ((q & 3) == 1 && (STEADY || group_exists(3, s))) issue(3, s, q >> 2);
      __builtin_amdgcn_sched_barrier(0);
    });
    // B3: publishes x L line s + 2; after it: x H s + 2, w H s + 1, w L s + 2,
    // x L s + 3, x H s + 3, w H s + 2
    if (STEADY) vm_wait<6 * UDPW>();
    else
      wait_groups((int)group_exists(2, s - 1) + (int)group_exists(3, s - 1) + (int)group_exists(4, s - 1) +
                  (int)group_exists(1, s) + (int)group_exists(2, s) + (int)group_exists(3, s));
    __syncthreads();
    // ---- Q4: w H x x H; read x L (s + 1) into B[0..3]; realign A[1..3], B[0]
    win(u_xl(s + 1), u_xl(s + 2), lpx, at);
    __builtin_amdgcn_sched_barrier(0);
    static_for<16>([&](auto qc) __attribute__((always_inline)) {
      constexpr int q = decltype(qc)::value, nb = 4 + (q >> 2), mb = 4 + (q & 3);
      acc[nb][mb] = mfma16<FMT>(A[nb], B[mb], acc[nb][mb]);
      if constexpr (q < 12 && (q & 3) == 0) {
        if (next) realign(A[1 + (q >> 2)], A3[1 + (q >> 2)], std::integral_constant<int, 1 + (q >> 2)>{}, shw, s + 1, TAILC{});
      }
      if constexpr (q == 12) {
        if (next) realign(B[0], B3[0], I0{}, shx, s + 1, TAILC{});
      }
      if constexpr (q < 12) {
        if (next) read_blk(at, q / 3, q % 3, B[q / 3], B3[q / 3]);
      }
      if ((q & 3) == 1 && (STEADY || group_exists(4, s))) issue(4, s, q >> 2);
      __builtin_amdgcn_sched_barrier(0);
    });
    // B4: publishes x H line s + 2; after it: w H s + 1, w L s + 2, and the four
    // groups of this step
    if (STEADY) vm_wait<6 * UDPW>();
    else
      wait_groups((int)group_exists(3, s - 1) + (int)group_exists(4, s - 1) + (int)group_exists(1, s) +
                  (int)group_exists(2, s) + (int)group_exists(3, s) + (int)group_exists(4, s));
    __syncthreads();
  };
  // K > 128 (checked by the host), so the steady steps end at s = nk - 2 and
  // exactly two guarded steps follow.  In the plain kernel they are written out
  // as steps nk - 2 and nk - 1, so every guard in them folds at compile time:
  // with a loop (or a conditional step) there, the compiler routed eight
  // accumulators through AGPR copies inside the steady loop, 40 VALU
  // instructions and extra wait states a step, and with the guards left to run
  // time the two written-out steps were long branchy code (slower for small K).
  // The cost is two register spills outside the K loop (20 bytes of scratch a
  // lane).  The kernels with a bias or an activation keep the loop (written
  // out, their larger epilogue spilled more).
  int s = 0;
  for (; s + 3 <= nk; ++s) step(s, std::true_type{});
  if constexpr (EPI) {
    for (; s < nk; ++s) step(s, std::false_type{});
  } else {
    step(nk - 2, std::false_type{});
    step(nk - 1, std::false_type{});
  }

  // Every DMA has landed and every wave is done with the units: scales (and
  // biases) go into LDS past the bf16 tile.
  vm_wait<0>();
  float *s_lds = (float *)(smem + 2 * BM * BN), *b_lds = s_lds + BN;
  __syncthreads();
  s_lds[tid] = my_scale;
  if constexpr (EPI) b_lds[tid] = my_bias;
  // rows of this lane (l16 of each x block) and its column pairs (lane rows 4 g
  // and 4 g + 2 of each w block; 4 g + 1 and 4 g + 3 are those plus 128)
  int mrow[FM], pa[FN], pb[FN];
#pragma unroll
  for (int mb = 0; mb < FM; ++mb) mrow[mb] = perm(ax0, mb, wave_m, l16);
#pragma unroll
  for (int nb = 0; nb < FN; ++nb) {
    pa[nb] = perm(aw0, nb, wave_n, 4 * g);
    pb[nb] = perm(aw0, nb, wave_n, 4 * g + 2);
  }
  main_epilogue_perm<EPI>(acc, a, smem, s_lds, b_lds, m0, n0, mrow, pa, pb, tid);
}

// ------------------------------------------ main path, register tiles (tiny problems)
//
// One wave per 16 x 16 block of y and no LDS: each lane loads its operand bytes
// straight into the registers V_MFMA_F32_16X16X128_F8F6F4 takes them from (w row
// n0 + l % 16 as the A operand, x row m0 + l % 16 as the B operand, K bytes
// [32 (l / 16), + 32) of each 128-byte step: two 16-byte loads per operand and
// step), up to eight K steps in flight at once, and writes its four results of
// a row (columns n0 + 4 (l / 16) .. + 3 of row m0 + l % 16, the accumulator
// layout) as one 8-byte store.  For problems that 64 x 64 tiles cannot spread
// over the GPU, where a call is a memory round trip plus the launch: nothing is
// staged in LDS on either side of the MFMAs.  The K steps are added in the same
// order as in every other main kernel.  Requires K % 16 == 0 (checked by the
// host): a 16-byte piece of a row then lies wholly before K or wholly past it,
// and the pieces past it are read as zeros (offset out of range); rows past M
// or N lie past the tile's buffer range and read as zeros too.
template <int FMT, bool EPI>
__global__ __launch_bounds__(64) void fp8g_direct_kernel(MainArgs a) {
  constexpr int D = 8;  // K steps in flight
  const int lane = threadIdx.x, l16 = lane & 15, g = lane >> 4;
  const int tm = (int)blockIdx.x % a.tiles_m, tn = (int)blockIdx.x / a.tiles_m;
  const int m0 = 16 * tm, n0 = 16 * tn, K = a.K;
  const v4i rx = make_rsrc(a.x + (size_t)m0 * K, (uint32_t)min(16, a.M - m0) * (uint32_t)K);
  const v4i rw = make_rsrc(a.w + (size_t)n0 * K, (uint32_t)min(16, a.N - n0) * (uint32_t)K);
  const v4i rs = make_rsrc(a.scale + n0, (uint32_t)(a.N - n0) * 4u);
  const uint32_t row = (uint32_t)l16 * (uint32_t)K;
  const int nk = (K + 127) / 128;
  // piece h of this lane's K group in step s, from the operand of descriptor r
  auto piece = [&](const v4i &r, int s, int h) __attribute__((always_inline)) {
    const int k = 128 * s + 32 * g + 16 * h;
    return llvm_buffer_load_v4i32(r, k < K ? row + (uint32_t)k : kOut, 0, 0);
  };
  // the epilogue's scales (and biases), requested with the first operands
  const v4f sc = llvm_buffer_load_v4f32(rs, 16u * (uint32_t)g, 0, 0);
  v4f bi = v4f{0.f, 0.f, 0.f, 0.f};
  if (EPI && a.bias) bi = llvm_buffer_load_v4f32(make_rsrc(a.bias + n0, (uint32_t)(a.N - n0) * 4u), 16u * (uint32_t)g, 0, 0);
  v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < nk; s0 += D) {
    v8i A[D], B[D];
#pragma unroll
    for (int i = 0; i < D; ++i) {
      if (s0 + i < nk) {
        const v4i w0 = piece(rw, s0 + i, 0), w1 = piece(rw, s0 + i, 1);
        const v4i x0 = piece(rx, s0 + i, 0), x1 = piece(rx, s0 + i, 1);
        A[i] = v8i{w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
        B[i] = v8i{x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      }
    }
#pragma unroll
    for (int i = 0; i < D; ++i)
      if (s0 + i < nk) acc = mfma16<FMT>(A[i], B[i], acc);
  }
  const int m = m0 + l16, n = n0 + 4 * g;
  if (m >= a.M || n >= a.N) return;
  float z[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    z[e] = acc[e] * sc[e];
    if constexpr (EPI) {
      if (a.bias) z[e] += bi[e];  // (no +0 without a bias: it would turn -0 into +0)
      z[e] = activation_rt(z[e], a.act);
    }
  }
  uint16_t *yr = a.y + (size_t)m * a.N + n;
  if (a.ystore >= 8 && n + 4 <= a.N) {  // N % 4 == 0 and y 8-byte aligned: the four are one 8-byte piece
    *(uint2 *)yr = make_uint2(bf16x2_rne(z[0], z[1]), bf16x2_rne(z[2], z[3]));
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (n + e < a.N) yr[e] = (uint16_t)bf16_rne(z[e]);
  }
}

// ------------------------------------------------------- launch templates
// Instantiated by the fp8g_launch_*.hip units.  EPI = the call has a bias or
// an activation (kernels built without it compile only the plain epilogue).

inline bool has_epilogue(const MainLaunch &l) { return l.bias != nullptr || l.act != kActNone; }
inline bool has_epilogue(const SkinnyLaunch &l) { return l.bias != nullptr || l.act != kActNone; }

// Launches kernel(args...) on `stream`; with events set they are attached to
// this dispatch (recorded when the kernel begins and when it has ended).
template <typename... P, typename... A>
static inline hipError_t dispatch(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t stream,
                                  const DispatchEvents &ev, A... args) {
  if (ev.start || ev.stop) hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, ev.start, ev.stop, 0, args...);
  else kernel<<<grid, block, 0, stream>>>(args...);
  return hipGetLastError();
}

// Kernel arguments of a main-path launch.
static inline MainArgs main_args(const MainLaunch &l) {
  MainArgs a{l.x, l.w, l.scale, l.y, l.M, l.N, l.K, l.tiles_m, l.tiles_n, l.group_m, l.ystore};
  a.bias = l.bias;
  a.act = l.act;
  a.ywb = l.ywb;
  return a;
}

// Calls f(std::integral_constant<int, fmt>) for the launch's operand formats.
template <typename F>
static inline hipError_t with_format(int fmt, F &&f) {
  switch (fmt) {
    case 0: return f(std::integral_constant<int, 0>{});
    case 1: return f(std::integral_constant<int, 1>{});
    case 2: return f(std::integral_constant<int, 2>{});
    case 3: return f(std::integral_constant<int, 3>{});
    default: return hipErrorInvalidValue;
  }
}

// The generic main kernel for one configuration.  Operand formats other than
// E4M3 x E4M3 are built for the configurations the planner chooses (ALLFMT).
template <int BM, int BN, int STAGES, int WM, int WN, bool EPI>
static hipError_t launch_main_cfg(const MainLaunch &l, hipStream_t stream) {
  const MainArgs a = main_args(l);
  const dim3 grid((unsigned)(l.tiles_m * l.tiles_n)), block(WM * WN * 64);
  return with_format(l.fmt, [&](auto fmt) {
    constexpr int F = decltype(fmt)::value;
    if (l.k_tail) return dispatch(fp8g_main_kernel<BM, BN, STAGES, WM, WN, true, F, EPI>, grid, block, stream, l.ev, a);
    return dispatch(fp8g_main_kernel<BM, BN, STAGES, WM, WN, false, F, EPI>, grid, block, stream, l.ev, a);
  });
}

// Tile sizes the planner chooses besides 256 x 256 (variants 3, 17, 18).
template <bool EPI>
static hipError_t launch_main_tiles_t(const MainLaunch &l, hipStream_t stream) {
  switch (l.variant) {
    case 3: return launch_main_cfg<64, 64, 3, 2, 2, EPI>(l, stream);
    case 17: return launch_main_cfg<128, 256, 3, 2, 4, EPI>(l, stream);
    case 18: return launch_main_cfg<128, 128, 4, 2, 4, EPI>(l, stream);
    default: return hipErrorInvalidValue;
  }
}

// The five-slot kernel without stream-K (variant 10).
template <bool EPI>
static hipError_t launch_main4w_t(const MainLaunch &l, hipStream_t stream) {
  if (l.k_tail) return hipErrorInvalidValue;  // K % 128 == 0 only
  const MainArgs a = main_args(l);
  const dim3 grid((unsigned)(l.tiles_m * l.tiles_n)), block(256);
  return with_format(l.fmt, [&](auto fmt) {
    constexpr int F = decltype(fmt)::value;
    return dispatch(fp8g_main4w_kernel<F, EPI>, grid, block, stream, l.ev, a);
  });
}
// The cache-line-row kernel (variant 20; the host checks its requirements).
template <bool EPI>
static hipError_t launch_main4wr_t(const MainLaunch &l, hipStream_t stream) {
  // two K steps at least: the kernel runs its last two steps unconditionally
  if (l.K <= 128 || l.K % 2 == 0) return hipErrorInvalidValue;
  const MainArgs a = main_args(l);
  const dim3 grid((unsigned)(l.tiles_m * l.tiles_n)), block(256);
  return with_format(l.fmt, [&](auto fmt) {
    constexpr int F = decltype(fmt)::value;
    return dispatch(fp8g_main4wr_kernel<F, EPI>, grid, block, stream, l.ev, a);
  });
}
template <bool EPI>
static hipError_t launch_direct_t(const MainLaunch &l, hipStream_t stream) {
  if (l.K % 16 != 0) return hipErrorInvalidValue;
  const MainArgs a = main_args(l);
  const dim3 grid((unsigned)(l.tiles_m * l.tiles_n)), block(64);
  return with_format(l.fmt, [&](auto fmt) {
    constexpr int F = decltype(fmt)::value;
    return dispatch(fp8g_direct_kernel<F, EPI>, grid, block, stream, l.ev, a);
  });
}
template <bool EPI>
static hipError_t launch_main5_dp(const MainLaunch &l, hipStream_t stream) {
  const MainArgs a = main_args(l);
  const dim3 grid((unsigned)(l.tiles_m * l.tiles_n)), block(512);
  return with_format(l.fmt, [&](auto fmt) {
    constexpr int F = decltype(fmt)::value;
    if (l.k_tail) return dispatch(fp8g_main5_kernel<true, false, F, EPI>, grid, block, stream, l.ev, a);
    return dispatch(fp8g_main5_kernel<false, false, F, EPI>, grid, block, stream, l.ev, a);
  });
}

template <int RB, int MB, bool EPI, int NW = 4>
static hipError_t launch_skinny_cfg(const SkinnyLaunch &l, hipStream_t stream) {
  SkinnyArgs a{l.x, l.w, l.scale, l.y, l.partials, l.tickets, l.epoch, l.M, l.N, l.K, l.k_slice, l.vec,
               l.bias, l.act};
  const dim3 grid((unsigned)((l.N + 16 * RB - 1) / (16 * RB)), (unsigned)l.S), block(64 * NW);
  return with_format(l.fmt, [&](auto fmt) {
    constexpr int F = decltype(fmt)::value;
    return dispatch(fp8g_splitk_partial_kernel<RB, MB, F, EPI, NW>, grid, block, stream, l.ev, a);
  });
}

// Split-K variants 1-5 (LDS rings, 4 waves) and 21-24 (LDS rings two chunks
// deep, 8 waves).
template <int MB, bool EPI>
static hipError_t launch_skinny_mb(const SkinnyLaunch &l, hipStream_t stream) {
  switch (l.variant) {
    case 21: if constexpr (MB <= 4) return launch_skinny_cfg<1, MB, EPI, 8>(l, stream); else break;
    case 22: if constexpr (MB <= 2) return launch_skinny_cfg<2, MB, EPI, 8>(l, stream); else break;
    case 23: if constexpr (MB <= 2) return launch_skinny_cfg<3, MB, EPI, 8>(l, stream); else break;
    case 24: if constexpr (MB == 1) return launch_skinny_cfg<4, MB, EPI, 8>(l, stream); else break;
    case 1: return launch_skinny_cfg<1, MB, EPI>(l, stream);
    case 2: return launch_skinny_cfg<2, MB, EPI>(l, stream);
    case 3: if constexpr (MB <= 2) return launch_skinny_cfg<3, MB, EPI>(l, stream); else break;
    case 4: if constexpr (MB <= 2) return launch_skinny_cfg<4, MB, EPI>(l, stream); else break;
    case 5: if constexpr (MB == 1) return launch_skinny_cfg<5, MB, EPI>(l, stream); else break;
    default: break;
  }
  return hipErrorInvalidValue;
}

template <bool EPI>
static hipError_t launch_skinny_t(const SkinnyLaunch &l, hipStream_t stream) {
  if (l.M <= 16) return launch_skinny_mb<1, EPI>(l, stream);
  if (l.M <= 32) return launch_skinny_mb<2, EPI>(l, stream);
  if (l.M <= 64) return launch_skinny_mb<4, EPI>(l, stream);
  return launch_skinny_mb<8, EPI>(l, stream);
}

}  // namespace fp8g
