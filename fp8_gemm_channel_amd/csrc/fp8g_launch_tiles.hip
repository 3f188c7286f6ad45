// fp8g_launch_tiles.hip -- the main kernel for the tile sizes the planner
// chooses besides 256 x 256 (variants 3, 17, 18) and the register-tile kernel
// (variant 27), every operand format.
#include "fp8g_kernels.hpp"

namespace fp8g {

hipError_t launch_main_tiles(const MainLaunch &l, hipStream_t stream) {
  return has_epilogue(l) ? launch_main_tiles_epi(l, stream) : launch_main_tiles_t<false>(l, stream);
}

hipError_t launch_direct(const MainLaunch &l, hipStream_t stream) {
  return has_epilogue(l) ? launch_direct_t<true>(l, stream) : launch_direct_t<false>(l, stream);
}

}  // namespace fp8g
