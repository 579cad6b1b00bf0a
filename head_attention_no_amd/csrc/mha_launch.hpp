// Launchers of the attention-forward kernel instances.
//
// Each (element type, head dim) pair is instantiated in its own translation
// unit (mha_launch.hip, compiled once per pair), so the instances build in
// parallel; the C-ABI layer only sees this declaration.
#pragma once

#include <hip/hip_runtime.h>

#include "mha_common.hpp"

namespace fa355 {

// Launches the kernel for element type T (__bf16, _Float16 or float), head
// dim D and mask kind `mask` (MaskKind) on `stream`, for the p.n_items work
// items (one workgroup each, or fewer workgroups that each walk several).
template <typename T, int D>
hipError_t launch_mha(const Params &p, int mask, hipStream_t stream);

}  // namespace fa355
