// Instantiations of the fused chunk kernel for one (input dtype, key dimension).
// Compiled once per pair with -DFLA_TIN_BF16=0/1 -DFLA_DK=<dk>.
#include "dispatch.hpp"

#ifndef FLA_DK
#error "FLA_DK must be defined"
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
constexpr int DK = FLA_DK;

template <int C, int DECAY, bool NORM>
hipError_t launch_impl(const ChunkArgs &a, unsigned grid, hipStream_t s) {
  ChunkArgs copy = a;
  void *args[] = {&copy};
  const void *fn;
  if (a.bthd)
    fn = a.state_only ? reinterpret_cast<const void *>(&chunk_fwd_kernel<TIn, DK, C, DECAY, NORM, true, true>)
                      : reinterpret_cast<const void *>(&chunk_fwd_kernel<TIn, DK, C, DECAY, NORM, false, true>);
  else
    fn = a.state_only ? reinterpret_cast<const void *>(&chunk_fwd_kernel<TIn, DK, C, DECAY, NORM, true, false>)
                      : reinterpret_cast<const void *>(&chunk_fwd_kernel<TIn, DK, C, DECAY, NORM, false, false>);
  return hipLaunchKernel(fn, dim3(grid), dim3(Cfg<TIn, DK, C, DECAY, NORM>::NT), args, 0, s);
}

template <int C, int DECAY, bool NORM>
ChunkLauncher pick() {
  if constexpr (Cfg<TIn, DK, C, DECAY, NORM>::FITS) return &launch_impl<C, DECAY, NORM>;
  else return nullptr;
}

template <int C>
ChunkLauncher pick_dn(int decay, bool norm) {
  switch (decay) {
  case DECAY_NONE: return norm ? pick<C, DECAY_NONE, true>() : pick<C, DECAY_NONE, false>();
  case DECAY_GAMMA: return norm ? pick<C, DECAY_GAMMA, true>() : pick<C, DECAY_GAMMA, false>();
  case DECAY_GATE: return norm ? pick<C, DECAY_GATE, true>() : pick<C, DECAY_GATE, false>();
  case DECAY_TOKEN: return norm ? pick<C, DECAY_TOKEN, true>() : pick<C, DECAY_TOKEN, false>();
  default: return nullptr;
  }
}

ChunkLauncher pick_c(int chunk, int decay, bool norm) {
  switch (chunk) {
  case 16: return pick_dn<16>(decay, norm);
  case 32: return pick_dn<32>(decay, norm);
  case 64: return pick_dn<64>(decay, norm);
  case 128: return pick_dn<128>(decay, norm);
  default: return nullptr;
  }
}

} // namespace

#define FLA_CAT3(a, b, c) a##b##_##c
#define FLA_NAME(t, d) FLA_CAT3(chunk_launcher_, t, d)
#if FLA_TIN_BF16
ChunkLauncher FLA_NAME(bf16, FLA_DK)(int chunk, int decay, bool norm) { return pick_c(chunk, decay, norm); }
#else
ChunkLauncher FLA_NAME(f32, FLA_DK)(int chunk, int decay, bool norm) { return pick_c(chunk, decay, norm); }
#endif

} // namespace fla
