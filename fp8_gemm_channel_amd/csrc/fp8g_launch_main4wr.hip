// fp8g_launch_main4wr.hip -- the one-wave-per-SIMD main kernel on rows fetched
// as whole cache lines (variant 20: 256 x 256 tiles, K % 128 != 0), plain
// epilogue, every operand format.
#include "fp8g_kernels.hpp"

namespace fp8g {

hipError_t launch_main4wr(const MainLaunch &l, hipStream_t stream) {
  return has_epilogue(l) ? launch_main4wr_epi(l, stream) : launch_main4wr_t<false>(l, stream);
}

}  // namespace fp8g
