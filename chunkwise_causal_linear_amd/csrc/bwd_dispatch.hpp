// Launcher table of the backward chunk kernels (one translation unit per input dtype and
// contraction width, so they compile in parallel).
#pragma once

#include <hip/hip_runtime.h>

#include "chunk_bwd.hpp"

namespace fla {

using BwdLauncher = hipError_t (*)(const BwdArgs &, unsigned grid, hipStream_t);

// Launcher for (role, decay kind) with contraction width DY (dv for the dq and dk roles,
// dk for the dv role), or nullptr when that combination's tiles do not fit in LDS.
#define FLA_DECLARE_BWD(tname, dy) BwdLauncher bwd_launcher_##tname##_##dy(int role, int decay);
FLA_DECLARE_BWD(bf16, 64)
FLA_DECLARE_BWD(bf16, 128)
FLA_DECLARE_BWD(bf16, 256)
FLA_DECLARE_BWD(f32, 64)
FLA_DECLARE_BWD(f32, 128)
FLA_DECLARE_BWD(f32, 256)
#undef FLA_DECLARE_BWD

} // namespace fla
