// Launcher of the deferred-dequantisation decode GEMV (qmm_gemv_i8.hip).
// Kept apart from qmm_internal.h, whose contents the bf16 GEMV's recorded
// HBM traffic is keyed to.
#pragma once

#include "qmm_internal.h"

namespace qmm {

constexpr int kI8MaxD = 57344;   // the row's int8 codes and chunk sums fit 64 KiB of LDS
int launch_gemv_i8(const GemvArgs& a, void* stream);

}  // namespace qmm
