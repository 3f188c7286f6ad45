// fp8g_launch_main4w_epi.hip -- the one-wave-per-SIMD main kernel (variant
// 19) with a bias or an activation, every operand format.
#include "fp8g_kernels.hpp"

namespace fp8g {

hipError_t launch_main4w_epi(const MainLaunch &l, hipStream_t stream) { return launch_main4w_t<true>(l, stream); }

}  // namespace fp8g
