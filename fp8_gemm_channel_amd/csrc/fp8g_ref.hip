// fp8g_ref.hip -- reference kernels that measure what MI355X attains on the two
// resources the GEMM is bound by (libfp8g_ref.so, separate from libfp8g.so and
// not part of its interface): HBM streams for the memory-bound shapes, and a
// loop of back-to-back fp8 MFMAs from registers for the compute-bound ones.
//
// The streams read an N x K byte matrix -- a decode weight -- once from HBM and
// compute nothing but an XOR checksum of what they read, so a profile of the
// split-K kernel can be set beside the rate at which one launch streams the
// same bytes with nothing else to do:
//
//   mode 0  the split-K kernel's weight stream alone: 48 rows per workgroup,
//           eight waves taking 128-byte K chunks round-robin, each through a
//           private two-slot LDS ring filled by non-temporal LDS-DMA (the x rows
//           and the MFMAs of the real kernel left out)
//   mode 1  the same with 24 rows and three slots per wave: 512 workgroups, two
//           per compute unit (the fastest LDS-DMA pattern measured on MI355X)
//   mode 2  plain 16-byte non-temporal loads into registers, 1024 workgroups of
//           256 threads, eight loads in flight per thread, grid-stride
//
// The non-temporal policy matters: the same patterns with the default policy
// took twice as long on MI355X.
//
// out receives one XOR per thread; the XOR of all of them equals the XOR of the
// matrix read as 32-bit words when every word was read exactly once.
#include <hip/hip_ext.h>

#include "fp8g_kernels.hpp"

namespace fp8g {

template <int R, int NW, int D>
__global__ __launch_bounds__(64 * NW, 1) void fp8g_stream_ldsdma_kernel(const uint8_t *w, int N, int K, uint32_t *out) {
  constexpr int OPS = R / 8, SLOT = R * 128;
  static_assert(R % 8 == 0 && D >= 1 && D <= 3 && NW * D * SLOT <= 160 * 1024, "ring fits in LDS");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NW * D * SLOT];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = blockIdx.x * R;
  const v4i rs = make_rsrc(w + (size_t)n0 * K, (uint32_t)min(R, N - n0) * (uint32_t)K);
  const int nch = K >> 7;
  const int my = nch > wave ? (nch - wave + NW - 1) / NW : 0;
  uint32_t off[OPS];
#pragma unroll
  for (int t = 0; t < OPS; ++t) off[t] = (uint32_t)(8 * t + (lane >> 3)) * (uint32_t)K + (uint32_t)(lane & 7) * 16u;
  const uint32_t ring = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)smem + (uint32_t)(wave * D * SLOT);
  const uint8_t *mine = smem + wave * D * SLOT + lane * 16;

  auto issue = [&](int j) __attribute__((always_inline)) {
    const uint32_t kc = (uint32_t)(wave + NW * j) << 7;
#pragma unroll
    for (int t = 0; t < OPS; ++t) dma16_nt(rs, ring + (uint32_t)((j % D) * SLOT + t * 1024), off[t], kc);
  };
  uint32_t acc = 0;
  for (int j = 0; j < D && j < my; ++j) issue(j);
  for (int j = 0; j < my; ++j) {
    const int ahead = min(D - 1, my - 1 - j);  // chunks issued after j
    if (ahead >= 2) vm_wait_fence<2 * OPS>();
    else if (ahead == 1) vm_wait_fence<OPS>();
    else vm_wait_fence<0>();
    // every lane reads back the 16 bytes its own DMAs wrote
#pragma unroll
    for (int t = 0; t < OPS; ++t) {
      const uint4 v = *(const uint4 *)(mine + (j % D) * SLOT + t * 1024);
      acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (j + D < my) {
      lgkm_wait_fence();  // the slot's reads are done before it is refilled
      issue(j + D);
    }
  }
  out[(size_t)blockIdx.x * (64 * NW) + threadIdx.x] = acc;
}

template <int U>
__global__ __launch_bounds__(256) void fp8g_stream_vgpr_kernel(const uint8_t *w, uint32_t bytes, uint32_t *out) {
  const v4i rs = make_rsrc(w, bytes);
  constexpr uint32_t PER_ITER = 256u * 16u * U;
  const uint32_t stride = gridDim.x * PER_ITER;
  uint32_t acc = 0;
  for (uint32_t base = blockIdx.x * PER_ITER + threadIdx.x * 16u; base < bytes; base += stride) {
    v4i v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = llvm_buffer_load_v4i32(rs, base + (uint32_t)u * 4096u, 0, 2);  // nt
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= (uint32_t)(v[u].x ^ v[u].y ^ v[u].z ^ v[u].w);
  }
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = acc;
}


// Back-to-back V_MFMA_F32_16X16X128_F8F6F4 from registers, one wave per SIMD
// (256 threads, one workgroup per compute unit at most): each wave runs `iters`
// rounds of 64 independent MFMAs over eight A and eight B operand sets of
// pseudo-random E4M3 codes (bit 3 of every byte cleared: no NaN codes), the
// data the GEMM's operands look like.  No memory traffic in the loop; out gets
// one float per thread (a sum of its accumulators) so nothing is dead.  The
// MFMA rate sustained on random operands is data dependent and below the
// published peak (the chip's clock drops under this load).
__device__ __forceinline__ uint32_t ref_mix(uint32_t h) {
  h ^= h >> 16; h *= 0x7feb352dU; h ^= h >> 15; h *= 0x846ca68bU; h ^= h >> 16;  // a 32-bit integer finalizer
  return h;
}
template <typename F, int... I>
__device__ __forceinline__ void ref_for_impl(F &&f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void ref_for(F &&f) { ref_for_impl(f, std::make_integer_sequence<int, N>{}); }

__global__ __launch_bounds__(256, 1) void fp8g_mfma_ref_kernel(float *out, int iters, uint32_t seed) {
  v8i A[8], B[8];
  for (int s = 0; s < 8; ++s)
    for (int i = 0; i < 8; ++i) {
      const uint32_t ha = ref_mix(seed * 977u + threadIdx.x * 131u + blockIdx.x * 7919u + (uint32_t)(s * 17 + i));
      const uint32_t hb = ref_mix(ha ^ 0x9e3779b9u);
      A[s][i] = (int)(ha & 0xF7F7F7F7u);
      B[s][i] = (int)(hb & 0xF7F7F7F7u);
    }
  v4f acc[64];
  ref_for<64>([&](auto jc) __attribute__((always_inline)) { acc[decltype(jc)::value] = v4f{0.f, 0.f, 0.f, 0.f}; });
  for (int it = 0; it < iters; ++it)
    ref_for<64>([&](auto jc) __attribute__((always_inline)) {
      constexpr int j = decltype(jc)::value;
      acc[j] = mfma16<0>(A[j & 7], B[(j >> 3) & 7], acc[j]);
    });
  float t = 0.f;
  ref_for<64>([&](auto jc) __attribute__((always_inline)) {
    constexpr int j = decltype(jc)::value;
    t += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  });
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = t;
}

}  // namespace fp8g

// Launch stream `mode` over the N x K matrix w (device pointer, row-major,
// 16-byte aligned).  out: device buffer of fp8g_stream_out_words(mode, N, K)
// 32-bit words.  Events e0/e1 (may be null) are recorded around the dispatch
// itself.  Returns 0, -1 for a shape the mode does not take (N a multiple of
// 48, K a positive multiple of 128, N K below 2^31), -2 for an unknown mode,
// or the HIP error of the launch.
extern "C" long long fp8g_stream_out_words(int mode, int N, int K) {
  if (mode == 0) return (long long)(N / 48) * 512;
  if (mode == 1) return (long long)(N / 24) * 512;
  if (mode == 2) return 1024LL * 256;
  (void)K;
  return -2;
}

extern "C" int fp8g_stream_launch(int mode, const void *w, int N, int K, unsigned int *out, void *stream, void *e0,
                                  void *e1) {
  using namespace fp8g;
  if (N <= 0 || K <= 0 || N % 48 || K % 128 || (unsigned long long)N * (unsigned long long)K >= (1ull << 31))
    return -1;
  hipStream_t st = (hipStream_t)stream;
  hipEvent_t a = (hipEvent_t)e0, b = (hipEvent_t)e1;
  const uint8_t *p = (const uint8_t *)w;
  switch (mode) {
    case 0:
      hipExtLaunchKernelGGL(fp8g_stream_ldsdma_kernel<48, 8, 2>, dim3(N / 48), dim3(512), 0, st, a, b, 0, p, N, K, out);
      break;
    case 1:
      hipExtLaunchKernelGGL(fp8g_stream_ldsdma_kernel<24, 8, 3>, dim3(N / 24), dim3(512), 0, st, a, b, 0, p, N, K, out);
      break;
    case 2:
      hipExtLaunchKernelGGL(fp8g_stream_vgpr_kernel<8>, dim3(1024), dim3(256), 0, st, a, b, 0, p,
                            (uint32_t)((size_t)N * K), out);
      break;
    default:
      return -2;
  }
  return (int)hipGetLastError();
}

// Launch the MFMA loop: `grid` workgroups of 256 threads, `iters` rounds of 64
// MFMAs per wave (2 * 16 * 16 * 128 FLOPs each); out: device buffer of grid *
// 256 floats.  Events e0/e1 (may be null) are recorded around the dispatch.
// Returns 0, -1 for grid outside 1..65536 or iters outside 1..1000000, or the
// HIP error of the launch.
extern "C" int fp8g_mfma_ref_launch(float *out, int grid, int iters, unsigned int seed, void *stream, void *e0,
                                    void *e1) {
  using namespace fp8g;
  if (grid < 1 || grid > 65536 || iters < 1 || iters > 1000000) return -1;
  hipExtLaunchKernelGGL(fp8g_mfma_ref_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, (hipEvent_t)e0,
                        (hipEvent_t)e1, 0, out, iters, (uint32_t)seed);
  return (int)hipGetLastError();
}
