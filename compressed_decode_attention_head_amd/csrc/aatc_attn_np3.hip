// Decode-attention kernels with 3 K pair(s) of 128 bit-planes (see aatc_attn_kernel.h).
#include "aatc_attn_kernel.h"

namespace aatc_attn {
template hipError_t launch_np<3>(int, int, const AttnArgs&, dim3, size_t, hipStream_t, bool*);
}  // namespace aatc_attn
