// fp8g_launch_main5_epi.hip -- the five-slot main kernel (variant 10) with a
// bias or an activation, every operand format.
#include "fp8g_kernels.hpp"

namespace fp8g {

hipError_t launch_main5_epi(const MainLaunch &l, hipStream_t stream) { return launch_main5_dp<true>(l, stream); }

}  // namespace fp8g
