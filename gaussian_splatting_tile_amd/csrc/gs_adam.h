// Internal declaration of the fused SH Adam step (public interface:
// gs_sh_adam_step in include/gs.h).
#pragma once

#include <hip/hip_runtime.h>

#include "gs.h"

namespace gsi {

// Launches the update described by `a` (already validated) on stream s.
hipError_t launch_sh_adam(const gs_sh_adam &a, hipStream_t s);

}  // namespace gsi
