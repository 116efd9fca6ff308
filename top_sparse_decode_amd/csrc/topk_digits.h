// Radix digits of the exact top-k select, shared by the top-k kernels and
// by the index scan when it builds the first-digit histogram itself.
#pragma once

#include "device_common.h"

namespace tsd {

constexpr int kTopkB1 = 12, kTopkB2 = 10, kTopkB3 = 10;  // digit widths (bits)
constexpr int kTopkBins1 = 1 << kTopkB1;
constexpr int kTopkBins2 = 1 << kTopkB2;
constexpr int kTopkBins3 = 1 << kTopkB3;

// Digit 1 of a score's order-preserving key.
TSD_DEVICE uint32_t topk_digit1(uint32_t key) { return key >> (32 - kTopkB1); }

}  // namespace tsd
