// fp8g_launch_main4wr_epi.hip -- the cache-line-row main kernel (variant 20)
// with a bias or an activation, every operand format.
#include "fp8g_kernels.hpp"

namespace fp8g {

hipError_t launch_main4wr_epi(const MainLaunch &l, hipStream_t stream) { return launch_main4wr_t<true>(l, stream); }

}  // namespace fp8g
