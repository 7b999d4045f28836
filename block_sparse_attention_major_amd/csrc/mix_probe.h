// Launcher of the instruction-mix probe (mix_probe.hip), a diagnostic kept
// apart from the attention path's shared declarations.
#pragma once

#include <hip/hip_runtime.h>

namespace sa {

// waves_per_simd in 1..3 (2 with pingpong), cus >= 1, iters >= 1; cycles:
// device int64 [cus * waves_per_simd * 4], sink: device float
// [cus * waves_per_simd * 256].
hipError_t launch_mix_probe(int waves_per_simd, int pingpong, int cus, int iters, long long *cycles, float *sink,
                            hipStream_t s);

}  // namespace sa
