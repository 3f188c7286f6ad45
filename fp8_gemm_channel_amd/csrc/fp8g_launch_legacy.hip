// fp8g_launch_legacy.hip -- the other main-kernel configurations (variants 1,
// 2, 4-7, 9: E4M3 operands), built once with the general epilogue.
#include "fp8g_kernels.hpp"

namespace fp8g {

hipError_t launch_main_legacy(const MainLaunch &l, hipStream_t stream) {
  switch (l.variant) {
    case 1: return launch_main_cfg<256, 256, 64, 4, 4, 2, false, false, true>(l, stream);
    case 2: return launch_main_cfg<128, 128, 64, 4, 2, 2, false, false, true>(l, stream);
    case 4: return launch_main_cfg<256, 256, 64, 4, 2, 4, false, false, true>(l, stream);
    case 5: return launch_main_cfg<256, 256, 64, 4, 2, 2, false, false, true>(l, stream);
    case 6: return launch_main_cfg<256, 256, 128, 2, 4, 2, false, false, true>(l, stream);
    case 7: return launch_main_cfg<256, 256, 128, 2, 2, 4, false, false, true>(l, stream);
    case 9: return launch_main_cfg<256, 256, 64, 4, 4, 2, true, false, true>(l, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fp8g
