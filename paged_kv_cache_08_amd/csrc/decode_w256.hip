// Split kernels with a 256-token window (8 strided blocks of 32 tokens), bf16 caches.
#include "decode_split.h"

namespace pkv {

hipError_t launch_decode_split_w256(const DecodeArgs& a, int head_dim, int group, hipStream_t st,
                                    hipEvent_t e0, hipEvent_t e1) {
  return launch_decode_window<8>(a, head_dim, group, st, e0, e1);
}

}  // namespace pkv
