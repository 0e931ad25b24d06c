// Internal helpers shared by the host solver and the device launchers of libaatc.
#pragma once

#include <cstdarg>
#include <cstddef>
#include <cstdint>

#include "aatc.h"

namespace aatc {

// Records a formatted message for aatc_last_error() and returns `s`.
aatc_status fail(aatc_status s, const char* fmt, ...);
void clear_error();

// FNV-1a 64 over a blob with its checksum field treated as zero.
uint64_t blob_checksum(const aatc_calib* c);

// Integer reverse water-filling: the `total` largest candidates sigma_i^2 4^-k (k < max_bits)
// in the order (value desc, channel asc, bit asc) -> bits[d].
void waterfill(const double* s2, int d, int total, int max_bits, uint8_t* bits);

// Layout derived from the per-channel bits (shared by calibrate and validate).
void build_layout(aatc_calib* c);

}  // namespace aatc
