// Instantiations of the backward chunk kernels for one (input dtype, contraction width).
// Compiled once per pair with -DFLA_TIN_BF16=0/1 -DFLA_BWD_DY=<width>.
#include "bwd_dispatch.hpp"

#ifndef FLA_BWD_DY
#error "FLA_BWD_DY must be defined"
#endif
#ifndef FLA_TIN_BF16
#error "FLA_TIN_BF16 must be defined"
#endif

namespace fla {
namespace {

#if FLA_TIN_BF16
using TIn = __bf16;
#else
using TIn = float;
#endif
constexpr int DY = FLA_BWD_DY;

template <int ROLE, int DECAY>
hipError_t launch_impl(const BwdArgs &a, unsigned grid, hipStream_t s) {
  BwdArgs copy = a;
  void *args[] = {&copy};
  return hipLaunchKernel(reinterpret_cast<const void *>(&chunk_bwd_kernel<TIn, ROLE, DY, DECAY>),
                         dim3(grid), dim3(BwdCfg<TIn, ROLE, DY, DECAY>::NT), args, 0, s);
}

template <int ROLE, int DECAY>
BwdLauncher pick() {
  if constexpr (BwdCfg<TIn, ROLE, DY, DECAY>::FITS) return &launch_impl<ROLE, DECAY>;
  else return nullptr;
}

template <int ROLE>
BwdLauncher pick_d(int decay) {
  switch (decay) {
  case DECAY_NONE: return pick<ROLE, DECAY_NONE>();
  case DECAY_GAMMA: return pick<ROLE, DECAY_GAMMA>();
  case DECAY_GATE: return pick<ROLE, DECAY_GATE>();
  case DECAY_TOKEN: return pick<ROLE, DECAY_TOKEN>();
  default: return nullptr;
  }
}

BwdLauncher pick_r(int role, int decay) {
  switch (role) {
  case BWD_DQ: return pick_d<BWD_DQ>(decay);
  case BWD_DK: return pick_d<BWD_DK>(decay);
  case BWD_DV: return pick_d<BWD_DV>(decay);
  default: return nullptr;
  }
}

} // namespace

#define FLA_CAT3(a, b, c) a##b##_##c
#define FLA_NAME(t, d) FLA_CAT3(bwd_launcher_, t, d)
#if FLA_TIN_BF16
BwdLauncher FLA_NAME(bf16, FLA_BWD_DY)(int role, int decay) { return pick_r(role, decay); }
#else
BwdLauncher FLA_NAME(f32, FLA_BWD_DY)(int role, int decay) { return pick_r(role, decay); }
#endif

} // namespace fla
