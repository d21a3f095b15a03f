// Split kernels with a 512-token window (16 strided blocks of 32 tokens),
// bf16 caches, with a ring of 3 steps: the variant for grids of more
// workgroups than the device has CUs (several workgroups per CU).
#include "decode_split.h"

namespace pkv {

hipError_t launch_decode_split_w512_many(const DecodeArgs& a, int head_dim, int group, hipStream_t st,
                                         hipEvent_t e0, hipEvent_t e1) {
  return launch_decode_window<16, kRingMany>(a, head_dim, group, st, e0, e1);
}

}  // namespace pkv
