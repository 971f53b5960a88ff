// Which form the wide-tile chunk kernel runs, shared by the planner and the
// kernel's launcher (chunk_wide.hip checks it against its LDS layout).
#pragma once

#include "../../include/paged_attn.h"

namespace pa {

// The paired form (eight waves, two per SIMD: score waves and conversion
// waves) runs wherever its LDS layout fits one CU: every type pair at
// D = 128, and at D = 256 all but F16 K and V together and F16 with Q8_0
// (their raw tiles leave no room for the ring). The four-wave form takes
// those three.
constexpr bool chunk_wide_paired(int kt, int vt, int D) {
  return D == 128 || !((kt == PA_F16 && vt != PA_Q4_0) || (vt == PA_F16 && kt != PA_Q4_0));
}

}  // namespace pa
