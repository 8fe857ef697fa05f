// Instantiations of the gated delta rule chunk kernel (bf16 / fp32 inputs, dk = 64 / 128).
#include <hip/hip_runtime.h>

#include "gdn_fwd.hpp"

namespace fla {

using GdnLauncher = hipError_t (*)(const GdnArgs &, unsigned grid, hipStream_t);

namespace {

template <typename TIn, int DK>
hipError_t gdn_launch_impl(const GdnArgs &a, unsigned grid, hipStream_t s) {
  GdnArgs copy = a;
  void *args[] = {&copy};
  return hipLaunchKernel(reinterpret_cast<const void *>(&gdn_fwd_kernel<TIn, DK>), dim3(grid),
                         dim3(GdnCfg<TIn, DK>::NT), args, 0, s);
}

template <typename TIn, int DK>
GdnLauncher gdn_pick() {
  if constexpr (GdnCfg<TIn, DK>::FITS) return &gdn_launch_impl<TIn, DK>;
  else return nullptr;
}

} // namespace

// Launcher for (dtype, dk), or nullptr when unsupported.
GdnLauncher gdn_launcher(bool bf16, int dk) {
  if (bf16) {
    if (dk == 64) return gdn_pick<__bf16, 64>();
    if (dk == 128) return gdn_pick<__bf16, 128>();
  } else {
    if (dk == 64) return gdn_pick<float, 64>();
    if (dk == 128) return gdn_pick<float, 128>();
  }
  return nullptr;
}

} // namespace fla
