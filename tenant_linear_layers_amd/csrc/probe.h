// Calibration probe of the single-variant decode's loads (probe.hip); it
// computes nothing of the method.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bd {

// The decode's loads on a 4096 x 4096 bf16 matrix without its arithmetic,
// modes 0..5 (include/bitdelta.h, bitdelta_probe_decode_loads).
hipError_t launch_probe_decode_loads(const void* w, const void* signs, const void* x, int mode,
                                     uint32_t* sink, hipStream_t stream);

}  // namespace bd
