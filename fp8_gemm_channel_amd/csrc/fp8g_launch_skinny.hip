// fp8g_launch_skinny.hip -- the split-K (skinny M) kernel with the plain
// epilogue; calls with a bias or an activation go to fp8g_launch_skinny_epi.hip.
#include "fp8g_kernels.hpp"

namespace fp8g {

hipError_t launch_skinny(const SkinnyLaunch &l, hipStream_t stream) {
  if (has_epilogue(l)) return launch_skinny_epi(l, stream);
  return launch_skinny_t<false>(l, stream);
}

}  // namespace fp8g
