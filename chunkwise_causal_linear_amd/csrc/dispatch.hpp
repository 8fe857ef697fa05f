// Launcher table of the fused chunk kernel instantiations (one translation unit per
// input dtype and key dimension, so they compile in parallel).
#pragma once

#include <hip/hip_runtime.h>

#include "chunk_fwd.hpp"

namespace fla {

using ChunkLauncher = hipError_t (*)(const ChunkArgs &, unsigned grid, hipStream_t);

// Returns the launcher for (chunk, decay kind, normaliser) or nullptr when that
// combination's tiles do not fit in LDS.
#define FLA_DECLARE_LAUNCHER(tname, dk) \
  ChunkLauncher chunk_launcher_##tname##_##dk(int chunk, int decay, bool norm);
FLA_DECLARE_LAUNCHER(bf16, 16)
FLA_DECLARE_LAUNCHER(bf16, 32)
FLA_DECLARE_LAUNCHER(bf16, 64)
FLA_DECLARE_LAUNCHER(bf16, 128)
FLA_DECLARE_LAUNCHER(bf16, 256)
FLA_DECLARE_LAUNCHER(f32, 16)
FLA_DECLARE_LAUNCHER(f32, 32)
FLA_DECLARE_LAUNCHER(f32, 64)
FLA_DECLARE_LAUNCHER(f32, 128)
FLA_DECLARE_LAUNCHER(f32, 256)
#undef FLA_DECLARE_LAUNCHER

} // namespace fla
