// fp8g_launch_skinny.hip -- the split-K (skinny M) kernels with the plain
// epilogue; calls with a bias or an activation, and the direct-to-register
// variants, go to fp8g_launch_skinny_epi.hip.
#include "fp8g_kernels.hpp"

namespace fp8g {

hipError_t launch_skinny(const SkinnyLaunch &l, hipStream_t stream) {
  if (has_epilogue(l) || (l.variant > 10 && l.variant < 21)) return launch_skinny_epi(l, stream);
  return launch_skinny_t<false>(l, stream);
}

}  // namespace fp8g
