// Kernel-variant switches from the environment (SNM_LOG, SNM_FORCE_VARIANT): see variant.cpp.
#pragma once

#include <stdint.h>

namespace snm {

enum class Variant { kNone, kWide, kLarge, kGeneric, kUnsplit, kDirect };

// The variant SNM_FORCE_VARIANT names (kNone if unset or unknown).
Variant forced_variant();
// With SNM_LOG set: one line on stderr naming the variant an operation selected.
void log_variant(const char* op, int64_t R, int64_t K, int64_t C, const char* variant);

}  // namespace snm
