// fp8g_launch_skinny_epi.hip -- the split-K kernel with the general epilogue
// (bias, activation).
#include "fp8g_kernels.hpp"

namespace fp8g {

hipError_t launch_skinny_epi(const SkinnyLaunch &l, hipStream_t stream) { return launch_skinny_t<true>(l, stream); }

}  // namespace fp8g
