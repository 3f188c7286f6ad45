// fp8g_launch_main4w.hip -- the one-wave-per-SIMD main kernel (variant 19:
// 256 x 256 tiles, 4 waves of 128 x 128, K % 128 == 0), plain epilogue, every
// operand format.
#include "fp8g_kernels.hpp"

namespace fp8g {

hipError_t launch_main4w(const MainLaunch &l, hipStream_t stream) {
  return has_epilogue(l) ? launch_main4w_epi(l, stream) : launch_main4w_t<false>(l, stream);
}

}  // namespace fp8g
