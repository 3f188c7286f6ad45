// fp8g_kernels.hip -- configuration tables, the K = 0 kernels and the main-path
// dispatch of libfp8g.so.  The kernel templates live in fp8g_kernels.hpp; the
// fp8g_launch_*.hip units instantiate them.
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
#include "fp8g_kernels.hpp"

namespace fp8g {

__global__ __launch_bounds__(256) void fp8g_zero_kernel(uint16_t *__restrict__ y, int64_t count) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) y[i] = 0;
}

// K = 0 with a bias or an activation: the empty sum is +0, so
// y[m, n] = bf16(act(bias[n])) (bias 0 when absent); grid-stride over y.
__global__ __launch_bounds__(256) void fp8g_empty_k_kernel(uint16_t *__restrict__ y, const float *__restrict__ bias,
                                                           int act, int64_t N, int64_t count) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += (int64_t)gridDim.x * blockDim.x) {
    const float z = bias ? bias[i % N] : 0.0f;
    y[i] = (uint16_t)bf16_rne(activation_rt(z, act));
  }
}

// ------------------------------------------------------------------ launchers
static const MainConfig kMainConfigs[] = {
    {3, 64, 64, 128, 3},   // 4 waves, small problems
    {10, 256, 256, 128, 2}, // 8 waves, five half-step LDS slots (x two steps ahead)
    {16, 256, 256, 128, 2}, // variant 10 with stream-K over the tiles past the full waves
    {17, 128, 256, 128, 3}, // 8 waves, wave tile 64 x 64: grids of 128 x 256 tiles (mid M)
    {18, 128, 128, 128, 4}, // 8 waves, wave tile 64 (m) x 32 (n): grids of 128 x 128 tiles (mid M)
    {19, 256, 256, 128, 2}, // 4 waves, wave tile 128 x 128, ten 16 KiB LDS units (K % 128 == 0)
    {20, 256, 256, 128, 2}, // variant 19 on rows fetched as whole cache lines and realigned (K % 128 != 0)
    {27, 16, 16, 128, 1},   // one wave per 16 x 16 block, operands straight into registers (tiny problems)
};
// ids 1-5: LDS-ring kernel with 4 waves, 21-24: with 8 waves; 16 * row_blocks
// w rows per workgroup
static const SkinnyConfig kSkinnyConfigs[] = {
    {1, 1}, {2, 2}, {3, 3}, {4, 4}, {5, 5}, {21, 1}, {22, 2}, {23, 3}, {24, 4},
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
int skinny_tile_n(const SkinnyConfig &c) { return 16 * c.row_blocks; }
int skinny_max_row_blocks(int M, SkinnyKind kind) {
  switch (kind) {
    case SkinnyKind::kRing8: return M <= 16 ? 4 : (M <= 32 ? 3 : (M <= 64 ? 1 : 0));  // 8 rings of 2 slots
    default: return M <= 16 ? 5 : (M <= 32 ? 4 : 2);  // 4 rings of 3 slots (2 with 128 x rows)
  }
}
int skinny_chunk_bytes() { return 128; }

hipError_t launch_main(const MainLaunch &l, hipStream_t stream) {
  switch (l.variant) {
    case 10:
    case 16: return launch_main5(l, stream);
    case 19: return launch_main4w(l, stream);
    case 20: return launch_main4wr(l, stream);
    case 27: return launch_direct(l, stream);
    case 3:
    case 17:
    case 18: return launch_main_tiles(l, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_zero(uint16_t *y, int64_t count, hipStream_t stream, const DispatchEvents &ev) {
  int64_t blocks = (count + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  return dispatch(fp8g_zero_kernel, dim3((unsigned)blocks), dim3(256), stream, ev, y, count);
}

hipError_t launch_empty_k(uint16_t *y, const float *bias, int act, int64_t M, int64_t N, hipStream_t stream,
                          const DispatchEvents &ev) {
  const int64_t count = M * N;
  int64_t blocks = (count + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  return dispatch(fp8g_empty_k_kernel, dim3((unsigned)blocks), dim3(256), stream, ev, y, bias, act, N, count);
}

}  // namespace fp8g
