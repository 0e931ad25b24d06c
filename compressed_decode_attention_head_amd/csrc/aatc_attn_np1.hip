// Decode-attention kernels with 1 K pair(s) of 128 bit-planes (see aatc_attn_kernel.h).
#include "aatc_attn_kernel.h"

namespace aatc_attn {
template AATC_LAUNCH_NP_SIG(1);
}  // namespace aatc_attn
