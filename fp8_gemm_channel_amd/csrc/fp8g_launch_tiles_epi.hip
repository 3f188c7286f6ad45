// fp8g_launch_tiles_epi.hip -- variants 3, 17, 18 with a bias or an activation.
#include "fp8g_kernels.hpp"

namespace fp8g {

hipError_t launch_main_tiles_epi(const MainLaunch &l, hipStream_t stream) {
  return launch_main_tiles_t<true>(l, stream);
}

}  // namespace fp8g
