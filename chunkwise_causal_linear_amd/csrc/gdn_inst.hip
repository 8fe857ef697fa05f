// Instantiations of the gated delta rule kernels (bf16 / fp32 inputs, dk = 64 / 128): the
// per-chunk pre-pass and the streaming state pass.
#include <hip/hip_runtime.h>

#include "gdn_fwd.hpp"

namespace fla {

using GdnLauncher = hipError_t (*)(const GdnArgs &, unsigned grid, hipStream_t);

struct GdnLaunchers {
  GdnLauncher prep, state; // both null when (dtype, dk) is not built
};

namespace {

template <typename TIn, int DK, bool PREP>
hipError_t gdn_launch_impl(const GdnArgs &a, unsigned grid, hipStream_t s) {
  GdnArgs copy = a;
  void *args[] = {&copy};
  const void *fn = PREP ? reinterpret_cast<const void *>(&gdn_prep_kernel<TIn, DK>)
                        : reinterpret_cast<const void *>(&gdn_state_kernel<TIn, DK>);
  return hipLaunchKernel(fn, dim3(grid), dim3(PREP ? GdnCfg<TIn, DK>::NT : 2 * GdnCfg<TIn, DK>::NT), args, 0, s);
}

template <typename TIn, int DK>
GdnLaunchers gdn_pick() {
  if constexpr (GdnCfg<TIn, DK>::FITS)
    return {&gdn_launch_impl<TIn, DK, true>, &gdn_launch_impl<TIn, DK, false>};
  else
    return {nullptr, nullptr};
}

} // namespace

GdnLaunchers gdn_launchers(bool bf16, int dk) {
  if (bf16) {
    if (dk == 64) return gdn_pick<__bf16, 64>();
    if (dk == 128) return gdn_pick<__bf16, 128>();
  } else {
    if (dk == 64) return gdn_pick<float, 64>();
    if (dk == 128) return gdn_pick<float, 128>();
  }
  return {nullptr, nullptr};
}

} // namespace fla
