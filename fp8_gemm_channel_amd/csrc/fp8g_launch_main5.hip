// fp8g_launch_main5.hip -- launches the five-slot main kernel: variant 10
// (plain epilogue, every operand format) and variant 16 (stream-K, E4M3).
#include "fp8g_kernels.hpp"

namespace fp8g {

hipError_t launch_main5(const MainLaunch &l, hipStream_t stream) {
  if (l.variant != 16) return has_epilogue(l) ? launch_main5_epi(l, stream) : launch_main5_dp<false>(l, stream);
  if (l.fmt != 0) return hipErrorInvalidValue;
  MainArgs a = main_args(l);
  a.n_dp = l.n_dp;
  a.n_sk = l.n_sk;
  a.P = l.partials;
  a.tickets = l.tickets;
  a.epoch = l.epoch;
  const dim3 grid((unsigned)(l.n_dp + l.n_sk)), block(512);
  if (l.k_tail) return dispatch(fp8g_main5_kernel<true, true, 0, true>, grid, block, stream, l.ev, a);
  return dispatch(fp8g_main5_kernel<false, true, 0, true>, grid, block, stream, l.ev, a);
}

}  // namespace fp8g
